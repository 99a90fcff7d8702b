// splitzip_host.hip -- host runtime and C ABI of the SplitZip BF16 exponent-split codec.
//
// The stateful codec follows "SplitZip: Ultra-Fast Lossless KV Compression for
// Disaggregated LLM Serving" (README "Codec API"): built once per chunk size,
// calibrated once (top-16 exponent codebook, coverage), then used for any number of
// encode/decode calls whose outputs belong to that codec state.  This file owns:
//   - argument validation and status/error reporting (never throws across the ABI);
//   - codebook selection from the GPU histogram (count descending, exponent ascending),
//     one codebook or several per codec, and the exponent statistics of a histogram;
//   - per-stream workspaces: encode scratch (per-tile escape slots and counts, overflow
//     area, segmented sums), per-segment escape counts, pinned descriptor staging for
//     ragged batches;
//   - kernel launches and the one small readback that encode needs.
#include "splitzip_internal.h"

#include <splitzip.h>
#include <splitzip_tuning.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <exception>
#include <new>
#include <string>
#include <vector>

namespace {

constexpr uint32_t kCodecMagic = 0x53a2c0dcu;
constexpr int kStagingSlots = 16;


thread_local char g_last_error[512];   // no allocation: fail() cannot throw

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int fail_hip(hipError_t e, const char *what)
{
    return fail(e == hipErrorOutOfMemory ? SPLITZIP_E_NOMEM : SPLITZIP_E_DEVICE, "%s: %s", what,
                hipGetErrorString(e));
}

// Runs the body of an entry point: a C++ exception (host memory exhausted, a mutex error)
// becomes a status instead of crossing the C ABI.
template <class F>
int guarded(F &&body) noexcept
{
    try {
        return body();
    } catch (const std::bad_alloc &) {
        return fail(SPLITZIP_E_NOMEM, "host memory allocation failed");
    } catch (const std::exception &ex) {
        return fail(SPLITZIP_E_DEVICE, "internal error: %s", ex.what());
    } catch (...) {
        return fail(SPLITZIP_E_DEVICE, "internal error");
    }
}

#define SZ_HIP(call, what)                     \
    do {                                       \
        hipError_t e_ = (call);                \
        if (e_ != hipSuccess)                  \
            return fail_hip(e_, what);         \
    } while (0)

bool chunk_size_ok(uint32_t c)
{
    return c >= SPLITZIP_MIN_CHUNK && c <= SPLITZIP_MAX_CHUNK && (c & (c - 1)) == 0;
}

uint32_t log2u(uint32_t c)
{
    uint32_t l = 0;
    while ((1u << l) < c)
        ++l;
    return l;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

uint64_t ceil_div(uint64_t a, uint64_t b) { return a / b + (a % b != 0); }

// Makes the codec's device current for the duration of a call.
struct DeviceGuard {
    int prev = -1;
    bool switched = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev)
    {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            switched = err == hipSuccess;
        }
    }
    ~DeviceGuard()
    {
        if (switched)
            (void)hipSetDevice(prev);
    }
};

// Descriptor tables of one ragged-batch launch, staged through pinned memory.
struct Staging {
    sz::SegDesc *h_segs = nullptr;
    uint32_t *h_tiles = nullptr;   // the n + 1 tile starts, then the coarse segment table
    sz::SegDesc *d_segs = nullptr;
    uint32_t *d_tiles = nullptr;
    uint32_t cap = 0;              // descriptors
    uint64_t tcap = 0;             // entries of h_tiles / d_tiles
    uint32_t n = 0;                // descriptors held (h_* and d_* have the same contents)
    hipEvent_t done = nullptr;   // recorded after the last copy out of h_*
    bool used = false;
};

// Events of one profiled call: the kind of each of its n kernels and n + 1 events around them.
struct TimedCall {
    int kind[SPLITZIP_KERNELS] = {};   // kernel kind of each launch
    int n = 0;
    hipEvent_t ev[SPLITZIP_KERNELS] = {};
};

// Everything a launch on one stream needs besides the caller's buffers.
struct Workspace {
    std::mutex mu;
    hipStream_t stream = nullptr;
    // device
    uint8_t *scratch = nullptr;       // encode scratch (see EncodeScratch)
    uint64_t scratch_cap = 0;         // bytes
    unsigned long long *ovf_ctr = nullptr;   // [2], see EncodeArgs
    uint64_t *chain = nullptr;        // one-pass encode state: chain_cap status words
    uint32_t chain_cap = 0;
    uint64_t chain_launches = 0;      // one-pass launches on it (their tags)
    uint8_t *result = nullptr;        // [err u32, pad u32, seg_escapes u64 * result_cap]
    uint32_t result_cap = 0;
    // host
    uint8_t *h_result = nullptr;      // pinned mirror of `result`
    uint32_t *hint = nullptr;         // host memory mapped for the device: the escapes of the
    uint32_t *d_hint = nullptr;       // last encode's first tile (d_hint: its device address)
    bool hint_failed = false;         // no mapped host memory for it: calls go on without
    Staging staging[kStagingSlots];
    int next_slot = 0;
    // profiling
    std::vector<TimedCall> pending;
    std::vector<hipEvent_t> spare_events;
    double sum_ms[SPLITZIP_KERNELS] = {};
    uint64_t timed[SPLITZIP_KERNELS] = {};

    ~Workspace()
    {
        for (TimedCall &c : pending)
            for (int i = 0; i <= c.n; ++i)
                (void)hipEventDestroy(c.ev[i]);
        for (hipEvent_t e : spare_events)
            (void)hipEventDestroy(e);
        (void)hipFree(scratch);
        (void)hipFree(ovf_ctr);
        (void)hipFree(chain);
        (void)hipFree(result);
        (void)hipHostFree(h_result);
        (void)hipHostFree(hint);
        for (Staging &s : staging) {
            (void)hipHostFree(s.h_segs);
            (void)hipHostFree(s.h_tiles);
            (void)hipFree(s.d_segs);
            (void)hipFree(s.d_tiles);
            if (s.done)
                (void)hipEventDestroy(s.done);
        }
    }
};

// ---- scratch of the allocation-free encode -------------------------------------------------
// One fixed array per device, shared by every splitzip_encode_noalloc call on that device.
// In host code the name only stands for the array: a kernel gets the device copy's address,
// which hipGetSymbolAddress returns with that device current (noalloc_base below).
static __device__ __align__(256) uint8_t noalloc_scratch[SPLITZIP_NOALLOC_SCRATCH_BYTES];

constexpr int kNoAllocDevices = 64;
// The last bytes of the array hold the one-pass state of the allocation-free encode: the
// status words of up to kNoAllocChainTiles tiles (4 GiB of BF16), 4 MiB.  Only one-pass calls touch
// them, and the array starts zeroed (a cleared state).
constexpr uint32_t kNoAllocChainTiles = 1u << 17;
constexpr uint64_t kNoAllocChainBytes = 8ull * sz::kChainStride * kNoAllocChainTiles;
constexpr uint64_t kNoAllocScratchBytes = SPLITZIP_NOALLOC_SCRATCH_BYTES - kNoAllocChainBytes;

struct NoAllocDevice {
    std::mutex mu;             // serializes the host side of the calls on the device
    uint8_t *base = nullptr;   // the device's copy of noalloc_scratch, once resolved
    uint64_t chain_launches = 0;   // one-pass launches on its state
};

NoAllocDevice g_noalloc[kNoAllocDevices];

}  // namespace

struct splitzip_codec {
    uint32_t magic = kCodecMagic;
    uint32_t elem = sz::kElemBF16;   // element type of every tensor the codec codes
    int device = 0;
    std::atomic<bool> profiling{false};   // set by splitzip_profile, read by every call
    std::atomic<uint32_t> onepass_tiles{SPLITZIP_ONEPASS_TILES};   // calls of at most this many tiles: one pass
    std::atomic<uint32_t> small_tiles{sz::kSmallTiles};   // calls of at most this many tiles: pack + finish
    std::atomic<uint32_t> stage_tiles{sz::kStageTiles};   // larger calls: the builds for escape-heavy inputs
    std::atomic<uint64_t> private_ovf_bytes{sz::kPrivateOvfBytes};   // per-tile overflow regions up to this
    uint32_t chunk_size = 0;
    uint32_t log2_chunk = 0;
    uint32_t n_books = 0;
    std::vector<uint8_t> cbs;   // [16 * n_books] codebooks
    uint8_t *d_lut = nullptr;   // device [256 * n_books] inverse LUTs
    uint32_t *d_cbs = nullptr;  // device [4 * n_books] codebooks as little-endian dwords
    std::mutex mu;
    // one workspace per stream; a call holds a reference for its duration, so that
    // splitzip_release_stream can drop the map's reference while a call still uses it
    std::map<hipStream_t, std::shared_ptr<Workspace>> ws;
};

namespace {

int codec_check(const splitzip_codec *c)
{
    if (!c || c->magic != kCodecMagic)
        return fail(SPLITZIP_E_INVALID, "codec handle is NULL or not a codec");
    return SPLITZIP_OK;
}

bool codebook_distinct(const uint8_t cb[16])
{
    bool seen[256] = {};
    for (int k = 0; k < 16; ++k) {
        if (seen[cb[k]])
            return false;
        seen[cb[k]] = true;
    }
    return true;
}

int make_codec(const uint8_t *cbs, uint32_t n_books, uint32_t chunk_size, uint32_t elem, int device,
               hipStream_t stream, splitzip_codec **out)
{
    std::unique_ptr<splitzip_codec> c(new (std::nothrow) splitzip_codec);
    if (!c)
        return fail(SPLITZIP_E_NOMEM, "host allocation of the codec failed");
    c->elem = elem;
    c->device = device;
    c->chunk_size = chunk_size;
    c->log2_chunk = log2u(chunk_size);
    c->n_books = n_books;
    c->cbs.assign(cbs, cbs + 16 * (size_t)n_books);
    // inverse LUT of each book.  BF16: exponent -> code, or the escape entry.  E5M2: element
    // byte -> code or escape entry in bits 0..4, and the byte's 3-bit field (sign << 2) |
    // mantissa in bits 5..7, so one lookup serves the codes, the flags and the field stream.
    std::vector<uint8_t> lut(256 * (size_t)n_books, sz::kEscapeEntry);
    for (uint32_t b = 0; b < n_books; ++b) {
        uint8_t *l = &lut[256 * (size_t)b];
        uint8_t inv[256];
        std::memset(inv, sz::kEscapeEntry, sizeof inv);
        for (int k = 0; k < 16; ++k)
            inv[cbs[16 * (size_t)b + k]] = (uint8_t)k;
        for (int v = 0; v < 256; ++v)
            l[v] = elem == sz::kElemE5M2
                       ? (uint8_t)(inv[(v >> 2) & 0x1F] | ((((v >> 7) << 2) | (v & 3)) << 5))
                       : inv[v];
    }
    SZ_HIP(hipMalloc(&c->d_lut, lut.size()), "hipMalloc(codec tables)");
    hipError_t e = hipMalloc(&c->d_cbs, c->cbs.size());
    if (e == hipSuccess)
        e = hipMemcpyAsync(c->d_lut, lut.data(), lut.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(c->d_cbs, c->cbs.data(), c->cbs.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        (void)hipFree(c->d_lut);
        (void)hipFree(c->d_cbs);
        return fail_hip(e, "upload of codec tables");
    }
    *out = c.release();
    return SPLITZIP_OK;
}

// Rank all 256 exponents by count (descending), ties by exponent (ascending); the first 16
// are the codebook.  Returns how many of the counted exponents it holds.
uint64_t pick_codebook(const uint64_t hist[256], uint8_t cb[16])
{
    int order[256];
    for (int e = 0; e < 256; ++e)
        order[e] = e;
    std::stable_sort(order, order + 256, [&](int a, int b) { return hist[a] > hist[b]; });
    uint64_t covered = 0;
    for (int k = 0; k < 16; ++k) {
        cb[k] = (uint8_t)order[k];
        covered += hist[order[k]];
    }
    return covered;
}

// Exponent histograms of n_seg tensors (BF16 words or E5M2 bytes) into host
// hist[256 * n_seg]; blocks.
int run_histograms(uint32_t n_seg, const void *const *d_x, const uint64_t *n, uint32_t elem,
                   hipStream_t stream, uint64_t *hist)
{
    std::vector<sz::HistSeg> segs(n_seg);
    std::vector<uint32_t> start((size_t)n_seg + 1);
    uint64_t blocks = 0;
    for (uint32_t s = 0; s < n_seg; ++s) {
        if (n[s] > 0 && (!d_x[s] || !aligned(d_x[s], 16)))
            return fail(SPLITZIP_E_INVALID, "tensor %u: pointer NULL or not 16-byte aligned", s);
        segs[s] = sz::HistSeg{n[s] ? static_cast<const uint16_t *>(d_x[s]) : nullptr, n[s]};
        start[s] = (uint32_t)blocks;
        blocks += sz::hist_blocks(n[s]);
        if (blocks > 0x7FFFFFFFull)
            return fail(SPLITZIP_E_INVALID, "too many tensors in one call");
    }
    start[n_seg] = (uint32_t)blocks;
    // one device allocation: partial counts, histograms, then the tables
    auto up = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
    const uint64_t off_hist = up(blocks * 256 * sizeof(uint32_t));
    const uint64_t off_segs = up(off_hist + (uint64_t)n_seg * 256 * sizeof(uint64_t));
    const uint64_t off_start = up(off_segs + (uint64_t)n_seg * sizeof(sz::HistSeg));
    const uint64_t total = off_start + ((uint64_t)n_seg + 1) * sizeof(uint32_t);
    uint8_t *d = nullptr;
    SZ_HIP(hipMalloc(&d, total), "hipMalloc(histogram scratch)");
    sz::HistArgs a{};
    a.seg0 = segs[0];
    a.segs = reinterpret_cast<const sz::HistSeg *>(d + off_segs);
    a.block_start = reinterpret_cast<const uint32_t *>(d + off_start);
    a.partial = reinterpret_cast<uint32_t *>(d);
    a.hist = reinterpret_cast<uint64_t *>(d + off_hist);
    a.n_seg = n_seg;
    a.n_blocks = (uint32_t)blocks;
    a.elem = elem;
    hipError_t e = hipSuccess;
    if (n_seg > 1) {
        e = hipMemcpyAsync(d + off_segs, segs.data(), n_seg * sizeof(sz::HistSeg), hipMemcpyHostToDevice, stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(d + off_start, start.data(), start.size() * sizeof(uint32_t),
                               hipMemcpyHostToDevice, stream);
    }
    if (e == hipSuccess)
        e = sz::launch_histogram(a, stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(hist, a.hist, (size_t)n_seg * 256 * sizeof(uint64_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(stream);
    (void)hipFree(d);
    if (e != hipSuccess)
        return fail_hip(e, "exponent histogram");
    return SPLITZIP_OK;
}

// Workspace of (codec, stream), created on first use; the caller keeps *out for the call.
int get_workspace(splitzip_codec *c, hipStream_t stream, std::shared_ptr<Workspace> *out)
{
    std::lock_guard<std::mutex> lock(c->mu);
    auto it = c->ws.find(stream);
    if (it != c->ws.end()) {
        *out = it->second;
        return SPLITZIP_OK;
    }
    std::shared_ptr<Workspace> w(new (std::nothrow) Workspace);
    if (!w)
        return fail(SPLITZIP_E_NOMEM, "host allocation of a workspace failed");
    w->stream = stream;
    *out = w;
    c->ws.emplace(stream, std::move(w));
    return SPLITZIP_OK;
}

// Device bytes a workspace holds (its lock held).
uint64_t workspace_device_bytes(const Workspace &w)
{
    uint64_t b = w.scratch_cap + (w.ovf_ctr ? 2 * sizeof(unsigned long long) : 0) +
                 8ull * sz::kChainStride * w.chain_cap +
                 (w.result ? 8 + 8 * (uint64_t)w.result_cap : 0);
    for (const Staging &s : w.staging)
        b += (s.d_segs ? (uint64_t)s.cap * sizeof(sz::SegDesc) : 0) + (s.d_tiles ? s.tcap * sizeof(uint32_t) : 0);
    return b;
}

// ---- profiling: events around each launch, resolved into per-kernel totals ----------

hipEvent_t take_event(Workspace *w)
{
    if (!w->spare_events.empty()) {
        hipEvent_t e = w->spare_events.back();
        w->spare_events.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess)
        return nullptr;
    return e;
}

// Fold finished calls into the totals (all of them when `wait`).
void resolve_timings(Workspace *w, bool wait)
{
    size_t done = 0;
    for (; done < w->pending.size(); ++done) {
        TimedCall &c = w->pending[done];
        if (wait)
            (void)hipEventSynchronize(c.ev[c.n]);
        else if (hipEventQuery(c.ev[c.n]) != hipSuccess)
            break;
        for (int i = 0; i < c.n; ++i) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, c.ev[i], c.ev[i + 1]) == hipSuccess) {
                w->sum_ms[c.kind[i]] += ms;
                w->timed[c.kind[i]] += 1;
            }
        }
        for (int i = 0; i <= c.n; ++i)
            w->spare_events.push_back(c.ev[i]);
    }
    w->pending.erase(w->pending.begin(), w->pending.begin() + done);
}

// Starts a profiled call of n kernels (no-op when profiling is off or events run out).
struct CallTimer {
    Workspace *w = nullptr;
    TimedCall call;
    int recorded = 0;
    hipStream_t stream = nullptr;
    CallTimer(splitzip_codec *c, Workspace *ws, hipStream_t s, const int *kinds, int n)
    {
        if (!c->profiling || !ws || n >= SPLITZIP_KERNELS)
            return;
        resolve_timings(ws, false);
        for (int i = 0; i < n; ++i)
            call.kind[i] = kinds[i];
        call.n = n;
        for (int i = 0; i <= n; ++i)
            if (!(call.ev[i] = take_event(ws))) {
                for (int k = 0; k < i; ++k)
                    ws->spare_events.push_back(call.ev[k]);
                return;
            }
        w = ws;
        stream = s;
    }
    void mark()   // after each launch, and once before the first
    {
        if (w && recorded <= call.n)
            (void)hipEventRecord(call.ev[recorded++], stream);
    }
    ~CallTimer()
    {
        if (!w)
            return;
        if (recorded == call.n + 1) {
            w->pending.push_back(call);
        } else {
            for (int i = 0; i <= call.n; ++i)
                w->spare_events.push_back(call.ev[i]);
        }
    }
};

// Byte offsets of the encode scratch arrays for one launch.
struct EncodeScratch {
    uint64_t tile_count, tile_ovf, spill_rec, ovf_tiles, slots, block_sum, group_sum, seg_total,
        ovf, total;
    EncodeScratch(uint64_t n_tiles, uint64_t ovf_cap, uint64_t n_seg, uint64_t slot_escapes)
    {
        auto up = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
        tile_count = 0;
        tile_ovf = up(tile_count + 4 * n_tiles);
        spill_rec = up(tile_ovf + 8 * n_tiles);
        ovf_tiles = up(spill_rec + sizeof(sz::SpillRec) * n_tiles);
        slots = up(ovf_tiles + 4 * n_tiles);
        block_sum = up(slots + 4 * slot_escapes * n_tiles);
        group_sum = up(block_sum + 8 * ((n_tiles + sz::kSumTiles - 1) / sz::kSumTiles));
        seg_total = up(group_sum + 8 * ((n_tiles + sz::kPlaceTiles - 1) / sz::kPlaceTiles));
        ovf = up(seg_total + 8 * n_seg);
        total = up(ovf + 4 * ovf_cap);
    }
};

int ensure_scratch(Workspace *w, uint64_t bytes)
{
    if (!w->ovf_ctr) {
        SZ_HIP(hipMalloc(&w->ovf_ctr, 2 * sizeof(unsigned long long)), "hipMalloc(overflow counter)");
        SZ_HIP(hipMemsetAsync(w->ovf_ctr, 0, 2 * sizeof(unsigned long long), w->stream), "hipMemsetAsync(counter)");
    }
    if (w->scratch_cap >= bytes)
        return SPLITZIP_OK;
    const uint64_t cap = std::max<uint64_t>(bytes, w->scratch_cap + w->scratch_cap / 2);
    SZ_HIP(hipStreamSynchronize(w->stream), "hipStreamSynchronize");
    (void)hipFree(w->scratch);
    w->scratch = nullptr;
    w->scratch_cap = 0;
    SZ_HIP(hipMalloc(&w->scratch, cap), "hipMalloc(encode scratch)");
    w->scratch_cap = cap;
    return SPLITZIP_OK;
}

// The one-pass state of a workspace, for calls of up to n_tiles tiles; a new one starts
// cleared (no status word written).
int ensure_chain(Workspace *w, uint32_t n_tiles)
{
    if (w->chain_cap >= n_tiles)
        return SPLITZIP_OK;
    const uint32_t cap = (uint32_t)std::min<uint64_t>(0xFFFFFFFFull,
                                                      std::max<uint64_t>(n_tiles, w->chain_cap + w->chain_cap / 2));
    SZ_HIP(hipStreamSynchronize(w->stream), "hipStreamSynchronize");
    (void)hipFree(w->chain);
    w->chain = nullptr;
    w->chain_cap = 0;
    SZ_HIP(hipMalloc(&w->chain, 8ull * sz::kChainStride * cap), "hipMalloc(one-pass state)");
    SZ_HIP(sz::launch_chain_clear(w->chain, cap, w->stream), "clear of the one-pass state");
    w->chain_cap = cap;
    return SPLITZIP_OK;
}

// The workspace's hint word (see Workspace::hint), 0 when new.  Only a hint: when the mapped
// host memory cannot be had, calls go on without it (the size rule alone picks the launches).
void ensure_hint(Workspace *w)
{
    if (w->hint || w->hint_failed)
        return;
    void *h = nullptr, *d = nullptr;
    if (hipHostMalloc(&h, 64, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) {
        (void)hipGetLastError();
        w->hint_failed = true;
        return;
    }
    std::memset(h, 0, 64);
    if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipHostFree(h);
        w->hint_failed = true;
        return;
    }
    w->hint = static_cast<uint32_t *>(h);
    w->d_hint = static_cast<uint32_t *>(d);
}

// The tag of the next one-pass launch on a state of cap status words, counted in *launches;
// when the tag wraps to 0 the state is cleared first (on the stream, before that launch), so
// that no status word is older than 2^23 launches.
hipError_t chain_next_tag(uint64_t *launches, uint64_t *status, uint32_t cap, hipStream_t stream, uint32_t *tag)
{
    const uint64_t l = ++*launches;
    *tag = (uint32_t)(l & sz::kChainTagMask);
    return *tag == 0 ? sz::launch_chain_clear(status, cap, stream) : hipSuccess;
}

int ensure_result(Workspace *w, uint32_t n_seg)
{
    if (w->result_cap >= n_seg)
        return SPLITZIP_OK;
    uint32_t cap = std::max<uint32_t>(n_seg, std::max<uint32_t>(64, 2 * w->result_cap));
    SZ_HIP(hipStreamSynchronize(w->stream), "hipStreamSynchronize");
    (void)hipFree(w->result);
    (void)hipHostFree(w->h_result);
    w->result = nullptr;
    w->h_result = nullptr;
    w->result_cap = 0;
    const size_t bytes = 8 + 8 * (size_t)cap;
    SZ_HIP(hipMalloc(&w->result, bytes), "hipMalloc(results)");
    SZ_HIP(hipHostMalloc(&w->h_result, bytes, hipHostMallocDefault), "hipHostMalloc(results)");
    SZ_HIP(hipMemsetAsync(w->result, 0, bytes, w->stream), "hipMemsetAsync(results)");
    w->result_cap = cap;
    return SPLITZIP_OK;
}

// Entries of the coarse segment table of a call with these tile starts: one per group of
// 1 << kSegAtShift tiles, and the end of the last group's bracket (kernels read entries g and
// g + 1 for the group g of a tile).
uint64_t seg_at_entries(const std::vector<uint32_t> &tiles)
{
    const uint64_t n_tiles = tiles.back();
    return ((n_tiles + (1u << sz::kSegAtShift) - 1) >> sz::kSegAtShift) + 1;
}

// The coarse segment table: entry g = the segment holding tile g << kSegAtShift, then the
// last segment.
void build_seg_at(const std::vector<uint32_t> &tiles, uint32_t *out)
{
    const uint32_t n_seg = (uint32_t)tiles.size() - 1;
    const uint64_t n_tiles = tiles[n_seg];
    uint32_t s = 0;
    uint64_t g = 0;
    for (; (g << sz::kSegAtShift) < n_tiles; ++g) {
        const uint64_t t = g << sz::kSegAtShift;
        while (s + 1 < n_seg && tiles[s + 1] <= t)
            ++s;
        out[g] = s;
    }
    out[g] = n_seg - 1;
}

// Copy the descriptor tables of a ragged batch to the device through a pinned slot: the
// descriptors, the tile starts and the coarse segment table.  A batch called again with the
// same buffers (the same tables) uses the device copy a slot still holds: no copy is
// enqueued.  Slots are only rewritten by later calls on the same stream, so a kernel that
// reads one has finished before the copy that replaces it runs.
int stage_descriptors(Workspace *w, const std::vector<sz::SegDesc> &segs,
                      const std::vector<uint32_t> &tiles, const sz::SegDesc **d_segs,
                      const uint32_t **d_tiles, const uint32_t **d_seg_at)
{
    const uint32_t n = (uint32_t)segs.size();
    // the coarse table follows from the tile starts, so equal starts mean an equal table
    for (const Staging &h : w->staging)
        if (h.used && h.n == n && std::memcmp(h.h_segs, segs.data(), n * sizeof(sz::SegDesc)) == 0 &&
            std::memcmp(h.h_tiles, tiles.data(), (n + 1) * sizeof(uint32_t)) == 0) {
            *d_segs = h.d_segs;
            *d_tiles = h.d_tiles;
            *d_seg_at = h.d_tiles + n + 1;
            return SPLITZIP_OK;
        }
    const uint64_t t_entries = n + 1 + seg_at_entries(tiles);
    Staging &s = w->staging[w->next_slot];
    w->next_slot = (w->next_slot + 1) % kStagingSlots;
    s.used = false;          // until the copy below is enqueued
    if (s.done && s.n)
        SZ_HIP(hipEventSynchronize(s.done), "hipEventSynchronize(staging)");
    if (s.cap < n) {
        (void)hipHostFree(s.h_segs);
        (void)hipFree(s.d_segs);
        s.h_segs = nullptr;
        s.d_segs = nullptr;
        s.cap = 0;
        const uint32_t cap = std::max<uint32_t>(n, 64);
        SZ_HIP(hipHostMalloc(&s.h_segs, cap * sizeof(sz::SegDesc), hipHostMallocDefault), "hipHostMalloc(descriptors)");
        SZ_HIP(hipMalloc(&s.d_segs, cap * sizeof(sz::SegDesc)), "hipMalloc(descriptors)");
        s.cap = cap;
    }
    if (s.tcap < t_entries) {
        (void)hipHostFree(s.h_tiles);
        (void)hipFree(s.d_tiles);
        s.h_tiles = nullptr;
        s.d_tiles = nullptr;
        s.tcap = 0;
        const uint64_t cap = std::max<uint64_t>(t_entries, 1024);
        SZ_HIP(hipHostMalloc(&s.h_tiles, cap * sizeof(uint32_t), hipHostMallocDefault), "hipHostMalloc(tiles)");
        SZ_HIP(hipMalloc(&s.d_tiles, cap * sizeof(uint32_t)), "hipMalloc(tiles)");
        s.tcap = cap;
    }
    if (!s.done)
        SZ_HIP(hipEventCreateWithFlags(&s.done, hipEventDisableTiming), "hipEventCreate");
    std::memcpy(s.h_segs, segs.data(), n * sizeof(sz::SegDesc));
    std::memcpy(s.h_tiles, tiles.data(), (n + 1) * sizeof(uint32_t));
    build_seg_at(tiles, s.h_tiles + n + 1);
    SZ_HIP(hipMemcpyAsync(s.d_segs, s.h_segs, n * sizeof(sz::SegDesc), hipMemcpyHostToDevice, w->stream),
           "hipMemcpyAsync(descriptors)");
    SZ_HIP(hipMemcpyAsync(s.d_tiles, s.h_tiles, t_entries * sizeof(uint32_t), hipMemcpyHostToDevice, w->stream),
           "hipMemcpyAsync(tiles)");
    SZ_HIP(hipEventRecord(s.done, w->stream), "hipEventRecord(staging)");
    s.n = n;
    s.used = true;
    *d_segs = s.d_segs;
    *d_tiles = s.d_tiles;
    *d_seg_at = s.d_tiles + n + 1;
    return SPLITZIP_OK;
}

// Validation of segment i; its descriptor into out.
int check_segment(const splitzip_codec *c, uint32_t i, const splitzip_segment &g, bool encode,
                  sz::SegDesc &out)
{
    if (g.n >= sz::kMaxSegmentWords)
        return fail(SPLITZIP_E_INVALID, "segment %u: n = %llu exceeds 2^38 - 1", i,
                    (unsigned long long)g.n);
    if (!g.chunk_off || !aligned(g.chunk_off, 8))
        return fail(SPLITZIP_E_INVALID, "segment %u: chunk_off NULL or not 8-byte aligned", i);
    if (g.n > 0) {
        if (!g.data || !g.sm || !g.codes)
            return fail(SPLITZIP_E_INVALID, "segment %u: NULL data/sm/codes", i);
        if (!aligned(g.data, 16) || !aligned(g.sm, 16) || !aligned(g.codes, 16))
            return fail(SPLITZIP_E_INVALID, "segment %u: data/sm/codes not 16-byte aligned", i);
    }
    const uint64_t esc = encode ? g.esc_capacity : g.n_escapes;
    if (esc > 0 && (!g.esc_pos || !g.esc_exp || !aligned(g.esc_pos, 2)))
        return fail(SPLITZIP_E_INVALID, "segment %u: escape arrays NULL or misaligned", i);
    if (!encode && g.n_escapes > g.n)
        return fail(SPLITZIP_E_FORMAT, "segment %u: %llu escapes for %llu words", i,
                    (unsigned long long)g.n_escapes, (unsigned long long)g.n);
    if (g.book >= c->n_books)
        return fail(SPLITZIP_E_INVALID, "segment %u: book %u, the codec has %u", i, g.book,
                    c->n_books);
    out = sz::SegDesc{g.data, g.sm, g.codes, g.chunk_off, g.esc_pos, g.esc_exp, g.n, esc,
                      g.book, 0u, nullptr};
    return SPLITZIP_OK;
}

// Tiles of a segment of n elements (at least one, so that every segment has a first tile).
uint64_t segment_tiles(uint64_t n, uint64_t tile_words) { return std::max<uint64_t>(1, ceil_div(n, tile_words)); }

// Shared validation of segment arrays; builds descriptors and tile starts.
int prepare_segments_tiled(const splitzip_codec *c, uint32_t n_seg, const splitzip_segment *segs,
                           bool encode, uint64_t tile_words, std::vector<sz::SegDesc> &desc,
                           std::vector<uint32_t> &tiles)
{
    if (n_seg == 0)
        return fail(SPLITZIP_E_INVALID, "n_seg is 0");
    if (!segs)
        return fail(SPLITZIP_E_INVALID, "segs is NULL");
    desc.resize(n_seg);
    tiles.resize((size_t)n_seg + 1);
    uint64_t total = 0;
    for (uint32_t i = 0; i < n_seg; ++i) {
        const int rc = check_segment(c, i, segs[i], encode, desc[i]);
        if (rc != SPLITZIP_OK)
            return rc;
        tiles[i] = (uint32_t)total;
        total += segment_tiles(segs[i].n, tile_words);
        if (total > 0xFFFFFFF0ull)
            return fail(SPLITZIP_E_INVALID, "too many tiles in one call");
    }
    tiles[n_seg] = (uint32_t)total;
    return SPLITZIP_OK;
}

// The one book every segment uses, or -1 when they differ.
int64_t common_book(uint32_t n_seg, const splitzip_segment *segs)
{
    for (uint32_t i = 1; i < n_seg; ++i)
        if (segs[i].book != segs[0].book)
            return -1;
    return segs[0].book;
}

// Entries of a pack tile's escape slot for the codec's element type.
uint32_t slot_escapes(const splitzip_codec *c)
{
    return c->elem == sz::kElemE5M2 ? sz::kE8SlotEscapes : sz::kSlotEscapes;
}

// Elements per encode (pack) or decode tile of the codec's element type.
uint64_t tile_elements(const splitzip_codec *c, bool encode)
{
    if (c->elem == sz::kElemE5M2)
        return 1ull << (encode ? sz::kE8EncTileShift : sz::kE8DecTileShift);
    return encode ? sz::kEncTileWords : sz::kDecTileWords;
}

// log2 of the elements per pack tile of a call of n_tiles tiles of tile_elements(c, true): a
// one-pass encode of E5M2 bytes takes tiles half as long over at most kE8ShortChainTiles of
// them, or over any number when the input's escapes cluster (`clustered`: the previous
// encode's first tile was escape-heavy with its escapes falling unevenly over its waves).
uint32_t pack_tile_shift(const splitzip_codec *c, bool onepass, uint64_t n_tiles, bool clustered = false)
{
    if (c->elem == sz::kElemE5M2)
        return onepass && (n_tiles <= sz::kE8ShortChainTiles || clustered) ? sz::kE8ChainTileShift
                                                                          : sz::kE8EncTileShift;
    return sz::kEncTileShift;
}

// Canonical stream size of n elements with E escapes (0 for an invalid chunk size).
uint64_t stream_bytes(uint32_t elem, uint64_t n, uint32_t chunk_size, uint64_t E)
{
    // n and E below 2^38 keep every term, and the sum, far from 64-bit overflow
    if (!chunk_size_ok(chunk_size) || n >= sz::kMaxSegmentWords || E >= sz::kMaxSegmentWords)
        return 0;
    const uint64_t sm = elem == sz::kElemE5M2 ? ceil_div(3 * n, 8) : n;
    return SPLITZIP_HEADER_BYTES + sm + ceil_div(n, 2) + 8 * (ceil_div(n, chunk_size) + 1) + 3 * E;
}

int prepare_segments(const splitzip_codec *c, uint32_t n_seg, const splitzip_segment *segs,
                     bool encode, std::vector<sz::SegDesc> &desc, std::vector<uint32_t> &tiles)
{
    return prepare_segments_tiled(c, n_seg, segs, encode, tile_elements(c, encode), desc, tiles);
}

// Byte offsets inside a packed stream of n elements (n a multiple of 16 BF16 words, or of
// 128 E5M2 bytes): sm, codes and chunk_off at fixed places, then esc_pos[E] and esc_exp[E].
struct PackedLayout {
    uint64_t sm, codes, chunk_off, esc_pos, fixed;
    PackedLayout(uint64_t n, uint32_t chunk_size, uint32_t elem)
    {
        sm = SPLITZIP_HEADER_BYTES;
        codes = sm + (elem == sz::kElemE5M2 ? 3 * n / 8 : n);
        chunk_off = codes + n / 2;
        esc_pos = chunk_off + 8 * (ceil_div(n, chunk_size) + 1);
        fixed = esc_pos;
    }
};

// Validation of packed segments; builds descriptors (SegDesc::header set) and tile starts.
int prepare_packed(const splitzip_codec *c, uint32_t n_seg, const splitzip_packed *segs, bool encode,
                   std::vector<sz::SegDesc> &desc, std::vector<uint32_t> &tiles)
{
    if (n_seg == 0)
        return fail(SPLITZIP_E_INVALID, "n_seg is 0");
    if (!segs)
        return fail(SPLITZIP_E_INVALID, "segs is NULL");
    const uint64_t tile_words = tile_elements(c, encode);
    const uint64_t multiple = c->elem == sz::kElemE5M2 ? 128 : 16;
    desc.resize(n_seg);
    tiles.resize((size_t)n_seg + 1);
    uint64_t total = 0;
    for (uint32_t i = 0; i < n_seg; ++i) {
        const splitzip_packed &g = segs[i];
        if (g.n >= sz::kMaxSegmentWords || g.n % multiple)
            return fail(SPLITZIP_E_INVALID, "segment %u: n = %llu is not a multiple of %llu below 2^38", i,
                        (unsigned long long)g.n, (unsigned long long)multiple);
        if (!g.buf || !aligned(g.buf, 16))
            return fail(SPLITZIP_E_INVALID, "segment %u: stream buffer NULL or not 16-byte aligned", i);
        if (g.n > 0 && (!g.data || !aligned(g.data, 16)))
            return fail(SPLITZIP_E_INVALID, "segment %u: data NULL or not 16-byte aligned", i);
        if (g.book >= c->n_books)
            return fail(SPLITZIP_E_INVALID, "segment %u: book %u, the codec has %u", i, g.book,
                        c->n_books);
        const PackedLayout L(g.n, c->chunk_size, c->elem);
        if (g.buf_bytes < L.fixed)
            return fail(encode ? SPLITZIP_E_INVALID : SPLITZIP_E_FORMAT,
                        "segment %u: %llu bytes, the stream of %llu words needs at least %llu", i,
                        (unsigned long long)g.buf_bytes, (unsigned long long)g.n,
                        (unsigned long long)L.fixed);
        uint64_t esc = (g.buf_bytes - L.fixed) / 3;     // encode: escape capacity
        if (!encode) {
            if ((g.buf_bytes - L.fixed) % 3 || esc > g.n)
                return fail(SPLITZIP_E_FORMAT, "segment %u: stream length %llu does not fit %llu words", i,
                            (unsigned long long)g.buf_bytes, (unsigned long long)g.n);
        }
        uint8_t *b = g.buf;
        uint16_t *pos = reinterpret_cast<uint16_t *>(b + L.esc_pos);
        desc[i] = sz::SegDesc{g.data, b + L.sm, b + L.codes, reinterpret_cast<uint64_t *>(b + L.chunk_off),
                              pos, encode ? nullptr : b + L.esc_pos + 2 * esc, g.n, esc, g.book, 0u, b};
        tiles[i] = (uint32_t)total;
        total += std::max<uint64_t>(1, ceil_div(g.n, tile_words));
        if (total > 0xFFFFFFF0ull)
            return fail(SPLITZIP_E_INVALID, "too many tiles in one call");
    }
    tiles[n_seg] = (uint32_t)total;
    return SPLITZIP_OK;
}

int64_t common_book_packed(uint32_t n_seg, const splitzip_packed *segs)
{
    for (uint32_t i = 1; i < n_seg; ++i)
        if (segs[i].book != segs[0].book)
            return -1;
    return segs[0].book;
}

}  // namespace

// ======================================================================================
// C ABI
// ======================================================================================

namespace {

// Calibration of n_books codebooks on tensors of one element type: all exponent histograms in
// one pass, then each book = the 16 exponents ranked first by (count descending, exponent
// ascending).  hist (optional) receives hist_bins bins per book (256 for BF16, 32 for E5M2).
int calibrate_books(uint32_t elem, uint32_t n_books, const void *const *d_cal, const uint64_t *n_cal,
                    uint32_t chunk_size, void *stream_, splitzip_codec **out_codec, double *coverage,
                    uint64_t *hist, uint32_t hist_bins)
{
    g_last_error[0] = '\0';
    if (!out_codec)
        return fail(SPLITZIP_E_INVALID, "out_codec is NULL");
    if (n_books == 0 || n_books > SPLITZIP_MAX_BOOKS)
        return fail(SPLITZIP_E_INVALID, "n_books %u outside 1..%u", n_books, SPLITZIP_MAX_BOOKS);
    if (!d_cal || !n_cal)
        return fail(SPLITZIP_E_INVALID, "d_cal or n_cal is NULL");
    if (!chunk_size_ok(chunk_size))
        return fail(SPLITZIP_E_INVALID, "chunk_size %u is not a power of two in [16, 65536]", chunk_size);
    for (uint32_t b = 0; b < n_books; ++b)
        if (n_cal[b] > 0 && (!d_cal[b] || !aligned(d_cal[b], 16)))
            return fail(SPLITZIP_E_INVALID, "calibration tensor %u: pointer NULL or not 16-byte aligned", b);
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    int device = 0;
    SZ_HIP(hipGetDevice(&device), "hipGetDevice");
    std::vector<uint64_t> h(256 * (size_t)n_books);
    int rc = run_histograms(n_books, d_cal, n_cal, elem, stream, h.data());
    if (rc != SPLITZIP_OK)
        return rc;
    std::vector<uint8_t> cbs(16 * (size_t)n_books);
    std::vector<double> cov(n_books);
    for (uint32_t b = 0; b < n_books; ++b) {
        // an E5M2 histogram is 0 past bin 31, so its ranking stays inside the 32 exponents
        const uint64_t covered = pick_codebook(&h[256 * (size_t)b], &cbs[16 * (size_t)b]);
        cov[b] = n_cal[b] ? (double)covered / (double)n_cal[b] : 0.0;
    }
    splitzip_codec *c = nullptr;
    rc = make_codec(cbs.data(), n_books, chunk_size, elem, device, stream, &c);
    if (rc != SPLITZIP_OK)
        return rc;
    if (coverage)
        std::memcpy(coverage, cov.data(), n_books * sizeof(double));
    if (hist)
        for (uint32_t b = 0; b < n_books; ++b)
            std::memcpy(hist + (size_t)hist_bins * b, &h[256 * (size_t)b], hist_bins * sizeof(uint64_t));
    *out_codec = c;
    return SPLITZIP_OK;
}

int codec_from_codebooks(uint32_t elem, uint32_t n_books, const uint8_t *codebooks, uint32_t chunk_size,
                         splitzip_codec **out_codec)
{
    g_last_error[0] = '\0';
    if (!codebooks || !out_codec)
        return fail(SPLITZIP_E_INVALID, "codebooks or out_codec is NULL");
    if (n_books == 0 || n_books > SPLITZIP_MAX_BOOKS)
        return fail(SPLITZIP_E_INVALID, "n_books %u outside 1..%u", n_books, SPLITZIP_MAX_BOOKS);
    if (!chunk_size_ok(chunk_size))
        return fail(SPLITZIP_E_INVALID, "chunk_size %u is not a power of two in [16, 65536]", chunk_size);
    for (uint32_t b = 0; b < n_books; ++b) {
        if (!codebook_distinct(codebooks + 16 * (size_t)b))
            return fail(SPLITZIP_E_INVALID, "codebook %u: entries are not 16 distinct exponents", b);
        if (elem == sz::kElemE5M2)
            for (int k = 0; k < 16; ++k)
                if (codebooks[16 * (size_t)b + k] > 31)
                    return fail(SPLITZIP_E_INVALID, "codebook %u: %u is not a 5-bit E5M2 exponent", b,
                                codebooks[16 * (size_t)b + k]);
    }
    int device = 0;
    SZ_HIP(hipGetDevice(&device), "hipGetDevice");
    return make_codec(codebooks, n_books, chunk_size, elem, device, nullptr, out_codec);
}

}  // namespace

extern "C" {

int splitzip_calibrate_books(uint32_t n_books, const uint16_t *const *d_cal, const uint64_t *n_cal,
                             uint32_t chunk_size, void *stream, splitzip_codec **out_codec,
                             double *coverage, uint64_t *hist)
{
    return guarded([&]() -> int {
        return calibrate_books(sz::kElemBF16, n_books, reinterpret_cast<const void *const *>(d_cal), n_cal,
                               chunk_size, stream, out_codec, coverage, hist, 256);
    });
}

int splitzip_calibrate(const uint16_t *d_cal, uint64_t n_cal, uint32_t chunk_size, void *stream,
                       splitzip_codec **out_codec, double *out_coverage, uint64_t *out_hist)
{
    return guarded([&]() -> int {
        return splitzip_calibrate_books(1, &d_cal, &n_cal, chunk_size, stream, out_codec, out_coverage,
                                        out_hist);
    });
}

int splitzip_calibrate_books_e5m2(uint32_t n_books, const uint8_t *const *d_cal, const uint64_t *n_cal,
                                  uint32_t chunk_size, void *stream, splitzip_codec **out_codec,
                                  double *coverage, uint64_t *hist)
{
    return guarded([&]() -> int {
        return calibrate_books(sz::kElemE5M2, n_books, reinterpret_cast<const void *const *>(d_cal), n_cal,
                               chunk_size, stream, out_codec, coverage, hist, 32);
    });
}

int splitzip_calibrate_e5m2(const uint8_t *d_cal, uint64_t n_cal, uint32_t chunk_size, void *stream,
                            splitzip_codec **out_codec, double *out_coverage, uint64_t *out_hist)
{
    return guarded([&]() -> int {
        return splitzip_calibrate_books_e5m2(1, &d_cal, &n_cal, chunk_size, stream, out_codec,
                                             out_coverage, out_hist);
    });
}

int splitzip_codec_from_codebooks(uint32_t n_books, const uint8_t *codebooks, uint32_t chunk_size,
                                  splitzip_codec **out_codec)
{
    return guarded([&]() -> int {
        return codec_from_codebooks(sz::kElemBF16, n_books, codebooks, chunk_size, out_codec);
    });
}

int splitzip_codec_from_codebook(const uint8_t codebook[16], uint32_t chunk_size,
                                 splitzip_codec **out_codec)
{
    return guarded([&]() -> int {
        return splitzip_codec_from_codebooks(1, codebook, chunk_size, out_codec);
    });
}

int splitzip_codec_from_codebooks_e5m2(uint32_t n_books, const uint8_t *codebooks, uint32_t chunk_size,
                                       splitzip_codec **out_codec)
{
    return guarded([&]() -> int {
        return codec_from_codebooks(sz::kElemE5M2, n_books, codebooks, chunk_size, out_codec);
    });
}

int splitzip_codec_element(const splitzip_codec *codec, uint32_t *elem)
{
    return guarded([&]() -> int {
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        if (!elem)
            return fail(SPLITZIP_E_INVALID, "elem is NULL");
        *elem = codec->elem;
        return SPLITZIP_OK;
    });
}

int splitzip_codec_books(const splitzip_codec *codec, uint32_t *n_books, uint8_t *codebooks)
{
    return guarded([&]() -> int {
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        if (n_books)
            *n_books = codec->n_books;
        if (codebooks)
            std::memcpy(codebooks, codec->cbs.data(), codec->cbs.size());
        return SPLITZIP_OK;
    });
}

int splitzip_histogram(uint32_t n_seg, const uint16_t *const *d_x, const uint64_t *n, void *stream,
                       uint64_t *hist)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        if (n_seg == 0 || !d_x || !n || !hist)
            return fail(SPLITZIP_E_INVALID, "n_seg is 0 or an array is NULL");
        return run_histograms(n_seg, reinterpret_cast<const void *const *>(d_x), n, sz::kElemBF16,
                              static_cast<hipStream_t>(stream), hist);
    });
}

int splitzip_histogram_e5m2(uint32_t n_seg, const uint8_t *const *d_x, const uint64_t *n, void *stream,
                            uint64_t *hist)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        if (n_seg == 0 || !d_x || !n || !hist)
            return fail(SPLITZIP_E_INVALID, "n_seg is 0 or an array is NULL");
        std::vector<uint64_t> h(256 * (size_t)n_seg);
        const int rc = run_histograms(n_seg, reinterpret_cast<const void *const *>(d_x), n, sz::kElemE5M2,
                                      static_cast<hipStream_t>(stream), h.data());
        if (rc != SPLITZIP_OK)
            return rc;
        for (uint32_t s = 0; s < n_seg; ++s)
            std::memcpy(hist + 32 * (size_t)s, &h[256 * (size_t)s], 32 * sizeof(uint64_t));
        return SPLITZIP_OK;
    });
}

int splitzip_exponent_stats(const uint64_t hist[256], double *entropy_bits, double *coverage,
                            uint8_t codebook[16], uint32_t *distinct)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        if (!hist)
            return fail(SPLITZIP_E_INVALID, "hist is NULL");
        uint64_t m = 0;
        uint32_t d = 0;
        for (int e = 0; e < 256; ++e) {
            m += hist[e];
            d += hist[e] != 0;
        }
        double h = 0.0;
        for (int e = 0; e < 256; ++e)
            if (hist[e]) {
                const double p = (double)hist[e] / (double)m;
                h -= p * std::log2(p);
            }
        uint8_t cb[16];
        const uint64_t covered = pick_codebook(hist, cb);
        if (entropy_bits)
            *entropy_bits = h;
        if (coverage)
            *coverage = m ? (double)covered / (double)m : 0.0;
        if (codebook)
            std::memcpy(codebook, cb, 16);
        if (distinct)
            *distinct = d;
        return SPLITZIP_OK;
    });
}

int splitzip_codec_info(const splitzip_codec *codec, uint8_t codebook[16], uint32_t *chunk_size,
                        int *device)
{
    return guarded([&]() -> int {
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        if (codebook)
            std::memcpy(codebook, codec->cbs.data(), 16);
        if (chunk_size)
            *chunk_size = codec->chunk_size;
        if (device)
            *device = codec->device;
        return SPLITZIP_OK;
    });
}

}  // extern "C"

namespace {

// The call's shape (n_tiles pack tiles of 2^tile_shift elements), its codebook tables and the
// encode scratch arrays at `base` (laid out as `lay`; NULL for a one-pass encode) into a.
// res: the error word, then E per segment.
void set_encode_args(sz::EncodeArgs &a, const splitzip_codec *codec, uint32_t n_seg, uint32_t n_tiles,
                     uint32_t tile_shift, int64_t book, bool packed, uint8_t *base, const EncodeScratch &lay,
                     unsigned long long *ovf_ctr, uint64_t ovf_cap, bool private_ovf, uint8_t *res)
{
    // one book for the whole call: its LUT directly; several: the table, indexed per segment
    a.lut = codec->d_lut + 256 * (book < 0 ? 0 : book);
    a.multi_book = book < 0;
    a.cbs = codec->d_cbs;
    a.packed = packed;
    if (base) {     // none for a one-pass encode (base NULL)
        a.seg_total = reinterpret_cast<uint64_t *>(base + lay.seg_total);
        a.tile_count = reinterpret_cast<uint32_t *>(base + lay.tile_count);
        a.tile_ovf = reinterpret_cast<uint64_t *>(base + lay.tile_ovf);
        a.spill_rec = reinterpret_cast<sz::SpillRec *>(base + lay.spill_rec);
        a.ovf_tiles = reinterpret_cast<uint32_t *>(base + lay.ovf_tiles);
        a.slots = reinterpret_cast<uint32_t *>(base + lay.slots);
        a.block_sum = reinterpret_cast<uint64_t *>(base + lay.block_sum);
        a.group_sum = reinterpret_cast<uint64_t *>(base + lay.group_sum);
        a.ovf = reinterpret_cast<uint32_t *>(base + lay.ovf);
    }
    a.ovf_ctr = ovf_ctr;
    a.ovf_cap = ovf_cap;
    a.err = reinterpret_cast<uint32_t *>(res);
    a.seg_escapes = reinterpret_cast<uint64_t *>(res + 8);
    a.n_seg = n_seg;
    a.n_tiles = n_tiles;
    a.log2_chunk = codec->log2_chunk;
    a.elem = codec->elem;
    a.tile_shift = tile_shift;
    a.slot_escapes = codec->elem == sz::kElemE5M2 ? sz::kE8SlotEscapes : sz::kSlotEscapes;
    a.private_ovf = private_ovf ? 1u : 0u;
    a.stage = n_tiles > codec->stage_tiles.load(std::memory_order_relaxed) ? 1u : 0u;
}

// Tile starts of the segments `desc` in tiles of 2^shift elements into `out`; false when the
// call has too many such tiles.
bool tile_starts(const std::vector<sz::SegDesc> &desc, uint32_t shift, std::vector<uint32_t> &out)
{
    out.resize(desc.size() + 1);
    uint64_t total = 0;
    for (size_t i = 0; i < desc.size(); ++i) {
        out[i] = (uint32_t)total;
        total += segment_tiles(desc[i].n, 1ull << shift);
        if (total > 0xFFFFFFF0ull)
            return false;
    }
    out[desc.size()] = (uint32_t)total;
    return true;
}

// Tile starts of a one-pass encode of the segments `desc` into `out` (the launch sequences'
// `tiles` when the tile lengths agree; `clustered` as for pack_tile_shift); false when the
// call has too many such tiles.
bool onepass_tiles(const splitzip_codec *codec, const std::vector<sz::SegDesc> &desc,
                   const std::vector<uint32_t> &tiles, bool clustered, std::vector<uint32_t> &out)
{
    const uint32_t shift = pack_tile_shift(codec, true, tiles[desc.size()], clustered);
    if (shift == pack_tile_shift(codec, false, tiles[desc.size()])) {
        out = tiles;
        return true;
    }
    return tile_starts(desc, shift, out);
}

// Whether an encode of n_tiles tiles (of the launch sequences) on `stream` runs in one pass
// (see splitzip_set_onepass_tiles).  Not while the stream is being captured into a graph: a
// launch's tag is a kernel argument, and every replay of a graph would repeat it.
bool use_onepass(const splitzip_codec *codec, bool packed, uint64_t n_tiles, hipStream_t stream, bool heavy)
{
    const uint32_t limit = codec->onepass_tiles.load(std::memory_order_relaxed);
    if (packed || limit == 0 || (n_tiles > limit && !heavy))
        return false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone;
}

// The encode launches: the one-pass pack when a.chain_status is set; else pack and finish for
// calls of at most small_tiles tiles, else pack, sums, place and spill.  w (optional) times
// them when the codec is profiling.
hipError_t run_encode_stages(splitzip_codec *codec, Workspace *w, const sz::EncodeArgs &a, hipStream_t stream)
{
    if (a.chain_status) {
        static const int kOnePassKinds[] = {SPLITZIP_KERNEL_ONEPASS};
        CallTimer timer(codec, w, stream, kOnePassKinds, 1);
        timer.mark();
        const hipError_t e = sz::launch_encode_stage(sz::kStageOnePass, a, stream);
        timer.mark();
        return e;
    }
    static const int kSmallStages[] = {sz::kStagePack, sz::kStageFinish};
    static const int kSmallKinds[] = {SPLITZIP_KERNEL_PACK, SPLITZIP_KERNEL_FINISH};
    static const int kStages[] = {sz::kStagePack, sz::kStageSums, sz::kStagePlace, sz::kStageSpill};
    static const int kKinds[] = {SPLITZIP_KERNEL_PACK, SPLITZIP_KERNEL_SUMS, SPLITZIP_KERNEL_PLACE,
                                 SPLITZIP_KERNEL_SPILL};
    const bool small = a.n_tiles <= codec->small_tiles.load(std::memory_order_relaxed);
    const int *stages = small ? kSmallStages : kStages;
    const int n_stages = small ? 2 : 4;
    CallTimer timer(codec, w, stream, small ? kSmallKinds : kKinds, n_stages);
    timer.mark();
    hipError_t e = hipSuccess;
    for (int i = 0; i < n_stages && e == hipSuccess; ++i) {
        e = sz::launch_encode_stage(stages[i], a, stream);
        timer.mark();
    }
    return e;
}

// Workspace and launch shared by the blocking and non-blocking encodes (sections or packed
// streams); the caller holds the workspace lock.  d_result (optional): where the kernel
// writes its error bits and per-segment escape counts instead of the workspace's result
// buffer.  book: the one codebook of every segment, or -1 when they differ.
int encode_launch(splitzip_codec *codec, const std::vector<sz::SegDesc> &desc,
                  const std::vector<uint32_t> &tiles, int64_t book, bool packed, hipStream_t stream,
                  uint64_t *d_result, Workspace **out_ws)
{
    const uint32_t n_seg = (uint32_t)desc.size();
    std::shared_ptr<Workspace> hold;      // the caller holds its own reference too
    int rc = get_workspace(codec, stream, &hold);
    if (rc != SPLITZIP_OK)
        return rc;
    Workspace *w = hold.get();
    const uint32_t n_tiles = tiles[n_seg];
    const uint32_t tile_shift = pack_tile_shift(codec, false, n_tiles);
    ensure_hint(w);
    // an input whose first tile outgrew its slot last time is taken to be escape-heavy again:
    // the launch sequences would move its escapes through scratch
    const uint32_t hint = w->hint ? *reinterpret_cast<volatile uint32_t *>(w->hint) : 0u;
    const bool heavy = (hint & ~sz::kHintUneven) > slot_escapes(codec);
    const bool clustered = heavy && (hint & sz::kHintUneven) != 0;
    // the one-pass tiles (shorter for some E5M2 calls)
    std::vector<uint32_t> chain_tiles;
    const bool onepass = use_onepass(codec, packed, n_tiles, stream, heavy) &&
                         onepass_tiles(codec, desc, tiles, clustered, chain_tiles);
    if (onepass) {
        // no scratch: only the workspace's one-pass state
        const uint32_t n_chain = chain_tiles[n_seg];
        if ((rc = ensure_chain(w, n_chain)) != SPLITZIP_OK)
            return rc;
        if (!d_result && (rc = ensure_result(w, n_seg)) != SPLITZIP_OK)
            return rc;
        sz::EncodeArgs a{};
        a.seg0 = desc[0];
        if (n_seg > 1 &&
            (rc = stage_descriptors(w, desc, chain_tiles, &a.segs, &a.tile_start, &a.seg_at)) != SPLITZIP_OK)
            return rc;
        uint8_t *res = d_result ? reinterpret_cast<uint8_t *>(d_result) : w->result;
        set_encode_args(a, codec, n_seg, n_chain, pack_tile_shift(codec, true, n_tiles, clustered), book, packed,
                        nullptr, EncodeScratch(0, 0, 0, 0), nullptr, 0, false, res);
        a.chain_status = w->chain;
        a.chain_cap = w->chain_cap;
        a.first_tile_escapes = w->d_hint;
        hipError_t e = chain_next_tag(&w->chain_launches, w->chain, w->chain_cap, stream, &a.chain_tag);
        if (e == hipSuccess)
            e = run_encode_stages(codec, w, a, stream);
        if (e != hipSuccess)
            return fail_hip(e, "encode launch");
        *out_ws = w;
        return SPLITZIP_OK;
    }
    // every tile its own overflow region when those fit the limit; else one shared area as
    // large as the escape capacity, reserved from with an atomic counter
    const bool private_ovf = ((uint64_t)n_tiles << tile_shift) * 4 <=
                             codec->private_ovf_bytes.load(std::memory_order_relaxed);
    uint64_t ovf_cap = 1;
    for (uint32_t i = 0; i < n_seg; ++i)
        ovf_cap += desc[i].esc;
    if (private_ovf)
        ovf_cap = (uint64_t)n_tiles << tile_shift;
    const EncodeScratch lay(n_tiles, ovf_cap, n_seg, slot_escapes(codec));
    if ((rc = ensure_scratch(w, lay.total)) != SPLITZIP_OK)
        return rc;
    if (!d_result && (rc = ensure_result(w, n_seg)) != SPLITZIP_OK)
        return rc;

    sz::EncodeArgs a{};
    a.seg0 = desc[0];
    if (n_seg > 1 && (rc = stage_descriptors(w, desc, tiles, &a.segs, &a.tile_start, &a.seg_at)) != SPLITZIP_OK)
        return rc;
    uint8_t *res = d_result ? reinterpret_cast<uint8_t *>(d_result) : w->result;
    set_encode_args(a, codec, n_seg, n_tiles, tile_shift, book, packed, w->scratch, lay, w->ovf_ctr, ovf_cap,
                    private_ovf, res);
    a.first_tile_escapes = w->d_hint;
    const hipError_t e = run_encode_stages(codec, w, a, stream);
    if (e != hipSuccess) {
        // a launch that did not run to its end may leave the overflow counter set
        (void)hipMemsetAsync(w->ovf_ctr, 0, 2 * sizeof(unsigned long long), stream);
        return fail_hip(e, "encode launch");
    }
    *out_ws = w;
    return SPLITZIP_OK;
}

// Blocking readback of an encode launched on the workspace's result buffer: error bits and
// E per segment into E[], with the overflow-area bit tolerated only when some segment is
// over capacity.
int encode_readback(Workspace *w, hipStream_t stream, const std::vector<sz::SegDesc> &desc,
                    std::vector<uint64_t> &E)
{
    const uint32_t n_seg = (uint32_t)desc.size();
    hipError_t e = hipMemcpyAsync(w->h_result, w->result, 8 + 8 * (size_t)n_seg, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return fail_hip(e, "encode readback");
    uint32_t kerr = 0;
    std::memcpy(&kerr, w->h_result, 4);
    E.assign(n_seg, 0);
    std::memcpy(E.data(), w->h_result + 8, 8 * (size_t)n_seg);
    bool over_capacity = false;
    for (uint32_t i = 0; i < n_seg; ++i)
        over_capacity |= E[i] > desc[i].esc;
    if (kerr) {
        SZ_HIP(hipMemsetAsync(w->result, 0, 8, stream), "hipMemsetAsync(err)");
        if ((kerr & ~sz::kErrOverflowArea) || !over_capacity)
            return fail(SPLITZIP_E_DEVICE, "encode kernel reported error bits 0x%x", kerr);
    }
    return SPLITZIP_OK;
}

}  // namespace

extern "C" {

int splitzip_encode_async(splitzip_codec *codec, uint32_t n_seg, const splitzip_segment *segs,
                          void *stream_, uint64_t *d_result)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        if (!d_result || !aligned(d_result, 8))
            return fail(SPLITZIP_E_INVALID, "d_result NULL or not 8-byte aligned");
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        std::vector<sz::SegDesc> desc;
        std::vector<uint32_t> tiles;
        if ((rc = prepare_segments(codec, n_seg, segs, true, desc, tiles)) != SPLITZIP_OK)
            return rc;
        DeviceGuard dg(codec->device);
        if (dg.err != hipSuccess)
            return fail_hip(dg.err, "hipSetDevice");
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        std::shared_ptr<Workspace> hold;
        if ((rc = get_workspace(codec, stream, &hold)) != SPLITZIP_OK)
            return rc;
        Workspace *ws = hold.get();
        // the lock covers only the launch: nothing is read back
        std::lock_guard<std::mutex> lock(ws->mu);
        Workspace *w = nullptr;
        return encode_launch(codec, desc, tiles, common_book(n_seg, segs), false, stream, d_result, &w);
    });
}

int splitzip_encode_noalloc(splitzip_codec *codec, uint32_t n_seg, const splitzip_segment *segs,
                            void *stream_, uint64_t *d_result)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        if (!d_result || !aligned(d_result, 8))
            return fail(SPLITZIP_E_INVALID, "d_result NULL or not 8-byte aligned");
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        if (n_seg == 0 || !segs)
            return fail(SPLITZIP_E_INVALID, "n_seg is 0 or segs is NULL");
        if (n_seg > SPLITZIP_NOALLOC_MAX_SEGMENTS)
            return fail(SPLITZIP_E_INVALID, "%u segments; the allocation-free encode takes at most %u",
                        n_seg, SPLITZIP_NOALLOC_MAX_SEGMENTS);
        if (codec->device < 0 || codec->device >= kNoAllocDevices)
            return fail(SPLITZIP_E_INVALID, "device %d out of range", codec->device);
        // every segment checked, and the scratch the call needs, before anything is enqueued
        const uint64_t seq_words = tile_elements(codec, true);
        uint64_t n_tiles = 0, ovf_cap = 1;
        bool cap_over = false;
        int64_t book = segs[0].book;
        sz::SegDesc d0{};
        for (uint32_t i = 0; i < n_seg; ++i) {
            sz::SegDesc d;
            if ((rc = check_segment(codec, i, segs[i], true, d)) != SPLITZIP_OK)
                return rc;
            if (i == 0)
                d0 = d;
            n_tiles += segment_tiles(segs[i].n, seq_words);
            if (n_tiles > 0xFFFFFFF0ull)
                return fail(SPLITZIP_E_INVALID, "too many tiles in one call");
            // (the overflow area of the launch sequences is as long as the capacities)
            if (segs[i].esc_capacity > SPLITZIP_NOALLOC_SCRATCH_BYTES ||
                (ovf_cap += segs[i].esc_capacity) > SPLITZIP_NOALLOC_SCRATCH_BYTES)
                cap_over = true;
            if (segs[i].book != book)
                book = -1;
        }
        // a one-pass call needs no scratch besides its state at the end of the array
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        // a one-pass encode's tiles (shorter for small E5M2 calls)
        const uint32_t chain_shift = pack_tile_shift(codec, true, n_tiles);
        uint64_t n_chain = 0;
        for (uint32_t i = 0; i < n_seg; ++i)
            n_chain += segment_tiles(segs[i].n, 1ull << chain_shift);
        const bool onepass = use_onepass(codec, false, n_tiles, stream, false) && n_chain <= kNoAllocChainTiles;
        const uint64_t tile_words = onepass ? 1ull << chain_shift : seq_words;
        const uint32_t tile_shift = onepass ? chain_shift : pack_tile_shift(codec, false, n_tiles);
        if (onepass)
            n_tiles = n_chain;
        if (cap_over && !onepass)
            return fail(SPLITZIP_E_INVALID, "escape capacities exceed the allocation-free scratch");
        const auto up = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
        const uint64_t seg_table = n_seg > 1 ? 256 : 0;               // after the counter
        const uint64_t tile_table = up(seg_table + (n_seg > 1 ? sizeof(sz::SegDesc) * n_seg : 0));
        const uint64_t enc_base = up(
            std::max<uint64_t>(256, tile_table + (n_seg > 1 ? 4 * (n_seg + 2 + ((n_tiles + 63) >> 6)) : 0)));
        const EncodeScratch lay((uint32_t)n_tiles, ovf_cap, n_seg, slot_escapes(codec));
        if (!onepass && enc_base + lay.total > kNoAllocScratchBytes)
            return fail(SPLITZIP_E_INVALID, "the call needs %llu bytes of scratch; the allocation-free encode has %llu",
                        (unsigned long long)(enc_base + lay.total), (unsigned long long)kNoAllocScratchBytes);

        DeviceGuard dg(codec->device);
        if (dg.err != hipSuccess)
            return fail_hip(dg.err, "hipSetDevice");
        NoAllocDevice &nd = g_noalloc[codec->device];
        std::lock_guard<std::mutex> lock(nd.mu);
        if (!nd.base) {
            // once per device, with the device current: its copy of the array
            void *p = nullptr;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
            if (e != hipSuccess || !p)
                return fail_hip(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
            nd.base = static_cast<uint8_t *>(p);
        }
        uint8_t *base = nd.base;
        unsigned long long *ctr = reinterpret_cast<unsigned long long *>(base);
        sz::SegDesc *d_segs = n_seg > 1 ? reinterpret_cast<sz::SegDesc *>(base + seg_table) : nullptr;
        uint32_t *d_tiles = n_seg > 1 ? reinterpret_cast<uint32_t *>(base + tile_table) : nullptr;

        // set-up launches: the overflow counter cleared, and for several segments their
        // descriptors and tile starts (kernel arguments) written to the scratch, then the
        // coarse segment table
        hipError_t e = hipSuccess;
        sz::SetupArgs sa{};
        sa.d_segs = d_segs;
        sa.d_tiles = d_tiles;
        sa.ovf_ctr = ctr;
        if (n_seg == 1) {
            e = sz::launch_setup(sa, stream);
        } else {
            uint64_t t = 0;
            for (uint32_t first = 0; first < n_seg && e == hipSuccess; first += sz::kSetupSegs) {
                const uint32_t cnt = std::min<uint32_t>(sz::kSetupSegs, n_seg - first);
                for (uint32_t k = 0; k < cnt; ++k) {
                    (void)check_segment(codec, first + k, segs[first + k], true, sa.segs[k]);
                    sa.tiles[k] = (uint32_t)t;
                    t += segment_tiles(segs[first + k].n, tile_words);
                }
                sa.tiles[cnt] = (uint32_t)t;
                sa.first = first;
                sa.count = cnt;
                sa.last = first + cnt == n_seg ? 1u : 0u;
                e = sz::launch_setup(sa, stream);
                sa.ovf_ctr = nullptr;      // cleared by the first launch
            }
            if (e == hipSuccess)
                e = sz::launch_seg_at(d_tiles, n_seg, (uint32_t)n_tiles, d_tiles + n_seg + 1, stream);
        }
        sz::EncodeArgs a{};
        a.seg0 = d0;
        a.segs = d_segs;
        a.tile_start = d_tiles;
        a.seg_at = d_tiles ? d_tiles + n_seg + 1 : nullptr;
        if (onepass) {
            set_encode_args(a, codec, n_seg, (uint32_t)n_tiles, tile_shift, book, false, nullptr,
                            EncodeScratch(0, 0, 0, 0), nullptr, 0, false, reinterpret_cast<uint8_t *>(d_result));
            a.chain_status = reinterpret_cast<uint64_t *>(base + kNoAllocScratchBytes);
            a.chain_cap = kNoAllocChainTiles;
            if (e == hipSuccess)
                e = chain_next_tag(&nd.chain_launches, a.chain_status, a.chain_cap, stream, &a.chain_tag);
        } else {
            set_encode_args(a, codec, n_seg, (uint32_t)n_tiles, tile_shift, book, false, base + enc_base, lay, ctr,
                            ovf_cap, false, reinterpret_cast<uint8_t *>(d_result));
        }
        if (e == hipSuccess)
            e = run_encode_stages(codec, nullptr, a, stream);
        if (e != hipSuccess)
            return fail_hip(e, "allocation-free encode launch");
        return SPLITZIP_OK;
    });
}

int splitzip_encode(splitzip_codec *codec, uint32_t n_seg, splitzip_segment *segs, void *stream_)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        std::vector<sz::SegDesc> desc;
        std::vector<uint32_t> tiles;
        if ((rc = prepare_segments(codec, n_seg, segs, true, desc, tiles)) != SPLITZIP_OK)
            return rc;
        DeviceGuard dg(codec->device);
        if (dg.err != hipSuccess)
            return fail_hip(dg.err, "hipSetDevice");
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        std::shared_ptr<Workspace> hold;
        if ((rc = get_workspace(codec, stream, &hold)) != SPLITZIP_OK)
            return rc;
        Workspace *ws = hold.get();
        std::lock_guard<std::mutex> lock(ws->mu);
        Workspace *w = nullptr;
        if ((rc = encode_launch(codec, desc, tiles, common_book(n_seg, segs), false, stream, nullptr, &w)) != SPLITZIP_OK)
            return rc;
        std::vector<uint64_t> E;
        if ((rc = encode_readback(w, stream, desc, E)) != SPLITZIP_OK)
            return rc;
        for (uint32_t i = 0; i < n_seg; ++i) {
            segs[i].n_escapes = E[i];
            segs[i].compressed_bytes = stream_bytes(codec->elem, segs[i].n, codec->chunk_size, E[i]);
            if (E[i] > segs[i].esc_capacity && rc == SPLITZIP_OK)
                rc = fail(SPLITZIP_E_CAPACITY, "segment %u has %llu escapes, capacity %llu", i,
                          (unsigned long long)E[i], (unsigned long long)segs[i].esc_capacity);
        }
        return rc;
    });
}

int splitzip_encode_packed(splitzip_codec *codec, uint32_t n_seg, splitzip_packed *segs,
                           void *stream_, uint64_t *d_result)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        if (d_result && !aligned(d_result, 8))
            return fail(SPLITZIP_E_INVALID, "d_result not 8-byte aligned");
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        std::vector<sz::SegDesc> desc;
        std::vector<uint32_t> tiles;
        if ((rc = prepare_packed(codec, n_seg, segs, true, desc, tiles)) != SPLITZIP_OK)
            return rc;
        DeviceGuard dg(codec->device);
        if (dg.err != hipSuccess)
            return fail_hip(dg.err, "hipSetDevice");
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        std::shared_ptr<Workspace> hold;
        if ((rc = get_workspace(codec, stream, &hold)) != SPLITZIP_OK)
            return rc;
        Workspace *ws = hold.get();
        std::lock_guard<std::mutex> lock(ws->mu);
        Workspace *w = nullptr;
        rc = encode_launch(codec, desc, tiles, common_book_packed(n_seg, segs), true, stream, d_result, &w);
        if (rc != SPLITZIP_OK || d_result)
            return rc;
        std::vector<uint64_t> E;
        if ((rc = encode_readback(w, stream, desc, E)) != SPLITZIP_OK)
            return rc;
        for (uint32_t i = 0; i < n_seg; ++i) {
            segs[i].n_escapes = E[i];
            segs[i].stream_bytes = stream_bytes(codec->elem, segs[i].n, codec->chunk_size, E[i]);
            if (segs[i].stream_bytes > segs[i].buf_bytes && rc == SPLITZIP_OK)
                rc = fail(SPLITZIP_E_CAPACITY, "segment %u needs %llu stream bytes, buffer holds %llu", i,
                          (unsigned long long)segs[i].stream_bytes, (unsigned long long)segs[i].buf_bytes);
        }
        return rc;
    });
}

}  // extern "C"

namespace {

// Decode of the segments `desc` (tile starts `tiles`, in tiles of tile_elements(codec, false)
// elements).  An E5M2 call with more than one escape per kE8ShortDecodeDensity elements, or of
// at most kE8ShortDecodeTiles tiles, runs tiles of half that length.
int decode_launch(splitzip_codec *codec, const std::vector<sz::SegDesc> &desc,
                  const std::vector<uint32_t> &tiles_in, int64_t book, hipStream_t stream, uint32_t *d_error)
{
    const uint32_t n_seg = (uint32_t)desc.size();
    if (d_error && !aligned(d_error, 4))
        return fail(SPLITZIP_E_INVALID, "d_error not 4-byte aligned");
    uint32_t tile_shift = codec->elem == sz::kElemE5M2 ? sz::kE8DecTileShift : sz::kDecTileShift;
    std::vector<uint32_t> short_tiles;
    const std::vector<uint32_t> *tp = &tiles_in;
    if (codec->elem == sz::kElemE5M2) {
        uint64_t n = 0, E = 0;
        for (const sz::SegDesc &d : desc) {
            n += d.n;
            E += d.esc;
        }
        if ((E > n / sz::kE8ShortDecodeDensity || tiles_in[n_seg] <= sz::kE8ShortDecodeTiles) &&
            tile_starts(desc, sz::kE8DecShortTileShift, short_tiles)) {
            tile_shift = sz::kE8DecShortTileShift;
            tp = &short_tiles;
        }
    }
    const std::vector<uint32_t> &tiles = *tp;
    DeviceGuard dg(codec->device);
    if (dg.err != hipSuccess)
        return fail_hip(dg.err, "hipSetDevice");
    sz::DecodeArgs a{};
    a.seg0 = desc[0];
    std::shared_ptr<Workspace> hold;
    Workspace *w = nullptr;
    std::unique_lock<std::mutex> lock;
    int rc;
    if (n_seg > 1 || codec->profiling) {
        if ((rc = get_workspace(codec, stream, &hold)) != SPLITZIP_OK)
            return rc;
        w = hold.get();
        lock = std::unique_lock<std::mutex>(w->mu);
    }
    if (n_seg > 1 && (rc = stage_descriptors(w, desc, tiles, &a.segs, &a.tile_start, &a.seg_at)) != SPLITZIP_OK)
        return rc;
    std::memcpy(a.cb, codec->cbs.data() + 16 * (book < 0 ? 0 : book), 16);
    a.cbs = codec->d_cbs;
    a.multi_book = book < 0;
    a.err = d_error;
    a.n_seg = n_seg;
    a.n_tiles = tiles[n_seg];
    a.log2_chunk = codec->log2_chunk;
    a.elem = codec->elem;
    a.large = (uint64_t)a.n_tiles > 2ull * codec->stage_tiles.load(std::memory_order_relaxed) ? 1u : 0u;
    a.tile_shift = tile_shift;
    hipError_t e;
    {
        static const int kDecodeKind[] = {SPLITZIP_KERNEL_DECODE};
        CallTimer timer(codec, w, stream, kDecodeKind, 1);
        timer.mark();
        e = sz::launch_decode(a, stream);
        timer.mark();
    }
    if (e != hipSuccess)
        return fail_hip(e, "decode launch");
    return SPLITZIP_OK;
}

}  // namespace

extern "C" {

int splitzip_decode(splitzip_codec *codec, uint32_t n_seg, const splitzip_segment *segs,
                    void *stream_, uint32_t *d_error)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        std::vector<sz::SegDesc> desc;
        std::vector<uint32_t> tiles;
        if ((rc = prepare_segments(codec, n_seg, segs, false, desc, tiles)) != SPLITZIP_OK)
            return rc;
        return decode_launch(codec, desc, tiles, common_book(n_seg, segs), static_cast<hipStream_t>(stream_),
                             d_error);
    });
}

int splitzip_decode_packed(splitzip_codec *codec, uint32_t n_seg, const splitzip_packed *segs,
                           void *stream_, uint32_t *d_error)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        std::vector<sz::SegDesc> desc;
        std::vector<uint32_t> tiles;
        if ((rc = prepare_packed(codec, n_seg, segs, false, desc, tiles)) != SPLITZIP_OK)
            return rc;
        // each stream's codebook comes from its own header (read by the kernel)
        return decode_launch(codec, desc, tiles, 0, static_cast<hipStream_t>(stream_), d_error);
    });
}

int splitzip_set_small_tiles(splitzip_codec *codec, uint32_t max_tiles)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        if (max_tiles > sz::kSmallTiles)
            return fail(SPLITZIP_E_INVALID, "max_tiles %u exceeds %u", max_tiles, sz::kSmallTiles);
        codec->small_tiles.store(max_tiles, std::memory_order_relaxed);
        return SPLITZIP_OK;
    });
}

int splitzip_set_onepass_launches(splitzip_codec *codec, void *stream, uint64_t launches)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        std::shared_ptr<Workspace> w;
        {
            std::lock_guard<std::mutex> lock(codec->mu);
            auto it = codec->ws.find(static_cast<hipStream_t>(stream));
            if (it != codec->ws.end())
                w = it->second;
        }
        if (!w)
            return fail(SPLITZIP_E_INVALID, "the codec has no workspace for this stream");
        std::lock_guard<std::mutex> lock(w->mu);
        if (!w->chain)
            return fail(SPLITZIP_E_INVALID, "the workspace has no one-pass state");
        w->chain_launches = launches;
        return SPLITZIP_OK;
    });
}

int splitzip_set_onepass_tiles(splitzip_codec *codec, uint32_t max_tiles)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        codec->onepass_tiles.store(max_tiles, std::memory_order_relaxed);
        return SPLITZIP_OK;
    });
}

int splitzip_set_private_overflow(splitzip_codec *codec, uint64_t max_bytes)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        codec->private_ovf_bytes.store(max_bytes, std::memory_order_relaxed);
        return SPLITZIP_OK;
    });
}

int splitzip_set_stage_tiles(splitzip_codec *codec, uint32_t min_tiles)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        codec->stage_tiles.store(min_tiles, std::memory_order_relaxed);
        return SPLITZIP_OK;
    });
}

int splitzip_profile(splitzip_codec *codec, int enable)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        DeviceGuard dg(codec->device);
        std::vector<std::shared_ptr<Workspace>> all;
        {
            // workspace locks are taken without the codec lock held (calls hold them the other
            // way round)
            std::lock_guard<std::mutex> lock(codec->mu);
            codec->profiling = enable != 0;
            for (auto &kv : codec->ws)
                all.push_back(kv.second);
        }
        if (!enable) {
            for (const std::shared_ptr<Workspace> &w : all) {
                std::lock_guard<std::mutex> wl(w->mu);
                resolve_timings(w.get(), true);
                std::fill(w->sum_ms, w->sum_ms + SPLITZIP_KERNELS, 0.0);
                std::fill(w->timed, w->timed + SPLITZIP_KERNELS, 0);
            }
        }
        return SPLITZIP_OK;
    });
}

int splitzip_profile_read(splitzip_codec *codec, void *stream_, double *avg_ms, uint64_t *counts,
                          int reset)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        if (!avg_ms || !counts)
            return fail(SPLITZIP_E_INVALID, "avg_ms or counts is NULL");
        DeviceGuard dg(codec->device);
        if (dg.err != hipSuccess)
            return fail_hip(dg.err, "hipSetDevice");
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        std::shared_ptr<Workspace> hold;
        rc = get_workspace(codec, stream, &hold);
        if (rc != SPLITZIP_OK)
            return rc;
        Workspace *w = hold.get();
        std::lock_guard<std::mutex> lock(w->mu);
        SZ_HIP(hipStreamSynchronize(stream), "hipStreamSynchronize");
        resolve_timings(w, true);
        for (int k = 0; k < SPLITZIP_KERNELS; ++k) {
            counts[k] = w->timed[k];
            avg_ms[k] = w->timed[k] ? w->sum_ms[k] / (double)w->timed[k] : 0.0;
            if (reset) {
                w->sum_ms[k] = 0.0;
                w->timed[k] = 0;
            }
        }
        return SPLITZIP_OK;
    });
}

int splitzip_release_stream(splitzip_codec *codec, void *stream_)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        DeviceGuard dg(codec->device);
        if (dg.err != hipSuccess)
            return fail_hip(dg.err, "hipSetDevice");
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        std::shared_ptr<Workspace> w;
        {
            std::lock_guard<std::mutex> lock(codec->mu);
            auto it = codec->ws.find(stream);
            if (it == codec->ws.end())
                return SPLITZIP_OK;
            w = std::move(it->second);
            codec->ws.erase(it);
        }
        const hipError_t e = hipStreamSynchronize(stream);
        {
            // a call still inside the library on another thread holds the lock (and its own
            // reference, so the workspace then goes when that call returns)
            std::lock_guard<std::mutex> wl(w->mu);
        }
        w.reset();
        if (e != hipSuccess)
            return fail_hip(e, "hipStreamSynchronize");
        return SPLITZIP_OK;
    });
}

int splitzip_workspace_bytes(const splitzip_codec *codec, void *stream_, uint64_t *bytes)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        if (!bytes)
            return fail(SPLITZIP_E_INVALID, "bytes is NULL");
        splitzip_codec *c = const_cast<splitzip_codec *>(codec);   // only its locks change
        std::shared_ptr<Workspace> w;
        {
            std::lock_guard<std::mutex> lock(c->mu);
            auto it = c->ws.find(static_cast<hipStream_t>(stream_));
            if (it != c->ws.end())
                w = it->second;
        }
        *bytes = 0;
        if (w) {
            std::lock_guard<std::mutex> wl(w->mu);
            *bytes = workspace_device_bytes(*w);
        }
        return SPLITZIP_OK;
    });
}

void splitzip_free(splitzip_codec *codec)
{
    if (!codec || codec->magic != kCodecMagic)
        return;
    {
        DeviceGuard dg(codec->device);
        codec->ws.clear();
        (void)hipFree(codec->d_lut);
        (void)hipFree(codec->d_cbs);
    }
    codec->magic = 0;
    delete codec;
}

uint64_t splitzip_chunk_count(uint64_t n, uint32_t chunk_size)
{
    return chunk_size_ok(chunk_size) ? ceil_div(n, chunk_size) : 0;
}

uint64_t splitzip_compressed_bytes(uint64_t n, uint32_t chunk_size, uint64_t n_escapes)
{
    return stream_bytes(sz::kElemBF16, n, chunk_size, n_escapes);
}

uint64_t splitzip_e5m2_compressed_bytes(uint64_t n, uint32_t chunk_size, uint64_t n_escapes)
{
    return stream_bytes(sz::kElemE5M2, n, chunk_size, n_escapes);
}

static void le_put(uint8_t *p, uint64_t v, int bytes)
{
    for (int b = 0; b < bytes; ++b)
        p[b] = (uint8_t)(v >> (8 * b));
}

static uint64_t le_get(const uint8_t *p, int bytes)
{
    uint64_t v = 0;
    for (int b = 0; b < bytes; ++b)
        v |= (uint64_t)p[b] << (8 * b);
    return v;
}

int splitzip_write_header(const splitzip_codec *codec, uint32_t book, uint64_t n,
                          uint64_t n_escapes, uint8_t out[SPLITZIP_HEADER_BYTES])
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        if (!out)
            return fail(SPLITZIP_E_INVALID, "out is NULL");
        if (book >= codec->n_books)
            return fail(SPLITZIP_E_INVALID, "book %u, the codec has %u", book, codec->n_books);
        if (n >= sz::kMaxSegmentWords || n_escapes > n)
            return fail(SPLITZIP_E_INVALID, "n = %llu (below 2^38) with %llu escapes (at most n)",
                        (unsigned long long)n, (unsigned long long)n_escapes);
        std::memset(out, 0, SPLITZIP_HEADER_BYTES);
        std::memcpy(out, "SZB1", 4);
        le_put(out + 4, 1, 2);
        le_put(out + 6, SPLITZIP_HEADER_BYTES, 2);
        le_put(out + 8, codec->chunk_size, 4);
        le_put(out + 12, codec->elem, 4);
        le_put(out + 16, n, 8);
        le_put(out + 24, ceil_div(n, codec->chunk_size), 8);
        le_put(out + 32, n_escapes, 8);
        std::memcpy(out + 40, codec->cbs.data() + 16 * (size_t)book, 16);
        return SPLITZIP_OK;
    });
}

int splitzip_read_header(const uint8_t *buf, uint64_t total_len, uint64_t *n, uint32_t *chunk_size,
                         uint64_t *n_escapes, uint8_t codebook[16], uint32_t *elem)
{
    return guarded([&]() -> int {
        g_last_error[0] = '\0';
        if (!buf)
            return fail(SPLITZIP_E_INVALID, "buf is NULL");
        if (total_len < SPLITZIP_HEADER_BYTES)
            return fail(SPLITZIP_E_FORMAT, "stream shorter than its header");
        if (std::memcmp(buf, "SZB1", 4) != 0)
            return fail(SPLITZIP_E_FORMAT, "bad magic");
        const uint64_t flags = le_get(buf + 12, 4);
        if (le_get(buf + 4, 2) != 1 || le_get(buf + 6, 2) != SPLITZIP_HEADER_BYTES ||
            (flags != sz::kElemBF16 && flags != sz::kElemE5M2))
            return fail(SPLITZIP_E_FORMAT, "unsupported version, header size or flags");
        for (int i = 56; i < 64; ++i)
            if (buf[i])
                return fail(SPLITZIP_E_FORMAT, "reserved header bytes are not zero");
        const uint32_t c = (uint32_t)le_get(buf + 8, 4);
        const uint64_t nn = le_get(buf + 16, 8), nch = le_get(buf + 24, 8), e = le_get(buf + 32, 8);
        // before any size arithmetic: a larger n could wrap the size sum to the buffer length
        if (nn >= sz::kMaxSegmentWords)
            return fail(SPLITZIP_E_FORMAT, "n = %llu is not below 2^38", (unsigned long long)nn);
        if (!chunk_size_ok(c) || nch != ceil_div(nn, c))
            return fail(SPLITZIP_E_FORMAT, "bad chunk size or chunk count");
        if (e > nn || total_len != stream_bytes((uint32_t)flags, nn, c, e))
            return fail(SPLITZIP_E_FORMAT, "sizes do not match the stream length");
        if (flags == sz::kElemE5M2)
            for (int k = 0; k < 16; ++k)
                if (buf[40 + k] > 31)
                    return fail(SPLITZIP_E_FORMAT, "E5M2 codebook entry %u is not a 5-bit exponent", buf[40 + k]);
        if (n)
            *n = nn;
        if (chunk_size)
            *chunk_size = c;
        if (n_escapes)
            *n_escapes = e;
        if (codebook)
            std::memcpy(codebook, buf + 40, 16);
        if (elem)
            *elem = (uint32_t)flags;
        return SPLITZIP_OK;
    });
}

int splitzip_check_header(const splitzip_codec *codec, const uint8_t *buf, uint64_t total_len,
                          uint32_t *book)
{
    return guarded([&]() -> int {
        int rc = codec_check(codec);
        if (rc != SPLITZIP_OK)
            return rc;
        uint32_t c = 0, elem = 0;
        uint8_t cb[16];
        rc = splitzip_read_header(buf, total_len, nullptr, &c, nullptr, cb, &elem);
        if (rc != SPLITZIP_OK)
            return rc;
        if (elem != codec->elem)
            return fail(SPLITZIP_E_CODEBOOK, "stream element type %u, the codec's is %u", elem, codec->elem);
        if (c != codec->chunk_size)
            return fail(SPLITZIP_E_CODEBOOK, "stream chunk size %u, the codec's is %u", c, codec->chunk_size);
        for (uint32_t b = 0; b < codec->n_books; ++b)
            if (std::memcmp(cb, codec->cbs.data() + 16 * (size_t)b, 16) == 0) {
                if (book)
                    *book = b;
                return SPLITZIP_OK;
            }
        return fail(SPLITZIP_E_CODEBOOK, "stream codebook is none of the codec's");
    });
}

const char *splitzip_status_string(int status)
{
    switch (status) {
    case SPLITZIP_OK: return "ok";
    case SPLITZIP_E_INVALID: return "invalid argument";
    case SPLITZIP_E_NOMEM: return "out of memory";
    case SPLITZIP_E_DEVICE: return "device error";
    case SPLITZIP_E_CODEBOOK: return "codebook mismatch";
    case SPLITZIP_E_FORMAT: return "malformed stream";
    case SPLITZIP_E_CAPACITY: return "escape capacity exceeded";
    default: return "unknown status";
    }
}

const char *splitzip_last_error(void) { return g_last_error; }

}  // extern "C"
