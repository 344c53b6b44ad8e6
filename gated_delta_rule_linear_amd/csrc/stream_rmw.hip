// la_stream_rmw: the plain in-place read-modify-write pass that bounds a decode step
// (x <- a x over fp32 data, each element read once and written once). The decode step of
// the delta rule and of GLA streams its carried state the same way and adds only a
// reduction, so this pass over the same bytes is the step's practical ceiling.
//
// A grid of two workgroups per compute unit walks 16 KiB tiles (256 threads, four 16-byte
// pieces each). Each workgroup loads its next tile before storing the current one, so
// there is always a tile of reads in flight behind the writes. Nontemporal accesses keep
// the stream out of the caches.
#include "common.hpp"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kRmwThreads = 256;
constexpr int kRmwPieces = 4;                                   // float4 per thread per tile
constexpr uint64_t kRmwTile = uint64_t(kRmwThreads) * kRmwPieces * 4;   // floats

__global__ __launch_bounds__(kRmwThreads) void stream_rmw_kernel(float* x, uint64_t n4, float a,
                                                                 uint64_t ntiles) {
    const uint64_t stride = gridDim.x;
    uint64_t t = blockIdx.x;
    if (t >= ntiles) return;
    float4* base = reinterpret_cast<float4*>(x);
    auto idx = [&](uint64_t tile, int f) {
        return tile * (kRmwTile / 4) + uint64_t(threadIdx.x) + uint64_t(kRmwThreads) * f;
    };
    float4 cur[kRmwPieces], nxt[kRmwPieces];
#pragma unroll
    for (int f = 0; f < kRmwPieces; ++f) {
        const uint64_t i = idx(t, f);
        cur[f] = i < n4 ? load_nt4(reinterpret_cast<const float*>(base + i)) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (; t < ntiles; t += stride) {
        const uint64_t tn = t + stride;
        if (tn < ntiles) {
#pragma unroll
            for (int f = 0; f < kRmwPieces; ++f) {
                const uint64_t i = idx(tn, f);
                nxt[f] = i < n4 ? load_nt4(reinterpret_cast<const float*>(base + i)) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int f = 0; f < kRmwPieces; ++f) {
            const uint64_t i = idx(t, f);
            if (i < n4) {
                const float4 v = cur[f];
                store_nt4(reinterpret_cast<float*>(base + i), make_float4(a * v.x, a * v.y, a * v.z, a * v.w));
            }
        }
#pragma unroll
        for (int f = 0; f < kRmwPieces; ++f) cur[f] = nxt[f];
    }
}

}  // namespace
}  // namespace la

extern "C" int la_stream_rmw(float* x, uint64_t n, float a, void* stream) {
    if (n == 0) return LA_OK;
    if (x == nullptr || n % 4 != 0 || (reinterpret_cast<uintptr_t>(x) & 15) != 0) return LA_ERR_INVALID;
    const uint64_t ntiles = (n + la::kRmwTile - 1) / la::kRmwTile;
    const uint64_t grid = std::min<uint64_t>(ntiles, uint64_t(la::device_cus()) * 2);
    (void)hipGetLastError();
    la::stream_rmw_kernel<<<dim3(unsigned(grid)), dim3(la::kRmwThreads), 0, static_cast<hipStream_t>(stream)>>>(
        x, n / 4, a, ntiles);
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}
