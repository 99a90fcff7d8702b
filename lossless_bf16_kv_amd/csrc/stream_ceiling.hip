// stream_ceiling.hip -- streaming kernels that measure what the memory system delivers to
// kernels shaped like the codec's: 16-byte lane-contiguous accesses, one 256-thread workgroup
// per tile, tiles handed to the 8 XCDs in contiguous ranges, nontemporal hints.  A read, a
// write and a copy kernel; the benchmark times them beside the codec so that the codec's
// bandwidth can be set against an achievable ceiling as well as against the HBM peak.
// Built into its own library (libszceiling.so): the codec never calls it.
#include "splitzip_device.h"

namespace szc {

using sz::kThreads;

constexpr int kKindRead = 0;
constexpr int kKindWrite = 1;
constexpr int kKindCopy = 2;

// tile = kThreads lanes x U units of 16 bytes; lane l's unit u is at (u * kThreads + l)
template <int kKind, int U>
__global__ __launch_bounds__(kThreads) void stream_kernel(const uint4 *src, uint4 *dst, uint64_t units,
                                                          uint32_t n_tiles, uint32_t *sink)
{
    const uint32_t t = sz::xcd_tile(blockIdx.x, n_tiles);
    if (t >= n_tiles)
        return;
    const uint64_t base = (uint64_t)t * kThreads * U + threadIdx.x;
    uint4 v[U];
    if (kKind != kKindWrite) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t i = base + (uint64_t)u * kThreads;
            v[u] = i < units ? sz::load_stream16(src + i) : make_uint4(0, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = make_uint4(t, (uint32_t)base, u, 0x5A5A5A5Au);
    }
    if (kKind == kKindRead) {
        // fold the loaded words so the loads stay; one store per workgroup at most
        uint32_t x = 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
            x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        if (x == 0x9E3779B9u)
            sink[threadIdx.x] = x;
        return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t i = base + (uint64_t)u * kThreads;
        if (i < units)
            sz::store_stream16(dst + i, v[u].x, v[u].y, v[u].z, v[u].w);
    }
}

template <int kKind>
hipError_t launch(const void *src, void *dst, uint64_t bytes, uint32_t *sink, hipStream_t stream)
{
    constexpr int U = 8;                              // 32 KiB per tile
    const uint64_t units = bytes / 16;
    const uint64_t tiles = (units + (uint64_t)kThreads * U - 1) / ((uint64_t)kThreads * U);
    if (tiles == 0 || tiles > 0xFFFFFF00ull)
        return hipErrorInvalidValue;
    stream_kernel<kKind, U><<<sz::xcd_grid((uint32_t)tiles), kThreads, 0, stream>>>(
        static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), units, (uint32_t)tiles, sink);
    return hipGetLastError();
}

}  // namespace szc

extern "C" {

// One streaming pass over `bytes` (a multiple of 16, both buffers 16-byte aligned device
// memory): kind 0 reads src, kind 1 writes dst, kind 2 copies src to dst.  sink: device
// uint32[256] that a read may write (it normally does not).  Enqueued on `stream`; returns
// 0 or a hipError_t code.
int szc_stream(int kind, const void *src, void *dst, uint64_t bytes, uint32_t *sink, void *stream)
{
    if (bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15))
        return (int)hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (kind) {
    case szc::kKindRead:
        return src && sink ? (int)szc::launch<szc::kKindRead>(src, nullptr, bytes, sink, s) : (int)hipErrorInvalidValue;
    case szc::kKindWrite:
        return dst ? (int)szc::launch<szc::kKindWrite>(nullptr, dst, bytes, nullptr, s) : (int)hipErrorInvalidValue;
    case szc::kKindCopy:
        return src && dst ? (int)szc::launch<szc::kKindCopy>(src, dst, bytes, nullptr, s) : (int)hipErrorInvalidValue;
    default:
        return (int)hipErrorInvalidValue;
    }
}

}  // extern "C"
