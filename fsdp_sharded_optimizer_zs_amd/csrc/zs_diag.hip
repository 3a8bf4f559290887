// Measurement aid: the fused step's memory streams with none of its
// arithmetic, to read the step kernel against what HBM delivers for exactly
// its mix of streams (n contribution reads, p, m, v read and written, w
// written: 2 reads per write at n = 8 bf16), not only against the datasheet
// peak.
//
// Same launch shape, occupancy, tiles, lane maps, vector widths and cache
// hints as the fused kernel: two adjacent 512-element tiles per wavefront
// (whole pairs only) and one wavefront per tile pair; bf16 contributions in
// the run map (lane t: elements 8t..8t+7), their combined value moved to the
// split map (lane t: 4t..4t+3 and 256+4t..256+4t+3) through LDS; fp32
// contributions and p, m, v in the split map; non-temporal loads and stores.
// The values written are placeholders: p + m into p, v into m, p into v, and
// into w the first two words of each 16-byte XOR of the contributions (bf16:
// taken after the LDS exchange, the odd entries with 1 XORed into every word).

#include <hip/hip_ext.h>

#include "zs_internal.h"

namespace zs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 512;
constexpr int kPair = ZS_STEP_TILES;
static_assert(kThreads == kBlockThreads, "grid arithmetic assumes 256-thread workgroups");

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The streams of TP adjacent tiles from tile0: state loads first, then the
// contributions, then the stores, as in the fused kernel. BF16: contributions
// are one run-map 16-byte vector per lane; otherwise two split-map vectors.
template <bool BF16, int TP>
__device__ __forceinline__ void tiles(f32x4* __restrict__ p4, f32x4* __restrict__ m4,
                                      f32x4* __restrict__ v4, u32x2* __restrict__ w2,
                                      const PtrPack& c, int n, int64_t tile0, int lane,
                                      u32x4* slot) {
    f32x4 pa[TP], pb[TP], ma[TP], mb[TP], va[TP], vb[TP];
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        const int64_t a = (tile0 + u) * (kTile / 4) + lane, b = a + kWave;
        pa[u] = __builtin_nontemporal_load(p4 + a), pb[u] = __builtin_nontemporal_load(p4 + b);
        ma[u] = __builtin_nontemporal_load(m4 + a), mb[u] = __builtin_nontemporal_load(m4 + b);
        va[u] = __builtin_nontemporal_load(v4 + a), vb[u] = __builtin_nontemporal_load(v4 + b);
    }
    u32x4 sa[TP], sb[TP];
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        sa[u] = u32x4{0u, 0u, 0u, 0u};
        sb[u] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (BF16) {
#pragma unroll 8
            for (int q = 0; q < n; ++q)
                sa[u] ^= __builtin_nontemporal_load(static_cast<const u32x4*>(c.p[q]) +
                                                    (tile0 + u) * kWave + lane);
        } else {
#pragma unroll 8
            for (int q = 0; q < n; ++q) {
                const u32x4* cq =
                    static_cast<const u32x4*>(c.p[q]) + (tile0 + u) * (kTile / 4) + lane;
                sa[u] ^= __builtin_nontemporal_load(cq);
                sb[u] ^= __builtin_nontemporal_load(cq + kWave);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        if constexpr (BF16) {
            // the fused kernel moves 8 fp32 values (two 16-byte entries) per lane
            slot[2 * lane] = sa[u];
            slot[2 * lane + 1] = sa[u] ^ u32x4{1u, 1u, 1u, 1u};
            wave_sync();
            sa[u] = slot[lane];
            sb[u] = slot[kWave + lane];
            wave_sync();
        }
    }
    // stores stream by stream over the tile group, as in the fused kernel
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        const int64_t a = (tile0 + u) * (kTile / 4) + lane, b = a + kWave;
        __builtin_nontemporal_store(pa[u] + ma[u], p4 + a);
        __builtin_nontemporal_store(pb[u] + mb[u], p4 + b);
    }
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        const int64_t a = (tile0 + u) * (kTile / 4) + lane, b = a + kWave;
        __builtin_nontemporal_store(va[u], m4 + a);
        __builtin_nontemporal_store(vb[u], m4 + b);
    }
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        const int64_t a = (tile0 + u) * (kTile / 4) + lane, b = a + kWave;
        __builtin_nontemporal_store(pa[u], v4 + a);
        __builtin_nontemporal_store(pb[u], v4 + b);
    }
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        const int64_t a = (tile0 + u) * (kTile / 4) + lane, b = a + kWave;
        __builtin_nontemporal_store(u32x2{sa[u].x, sa[u].y}, w2 + a);
        __builtin_nontemporal_store(u32x2{sb[u].x, sb[u].y}, w2 + b);
    }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void
streams_kernel(float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
               uint16_t* __restrict__ w, int64_t npairs, PtrPack c, int n) {
    __shared__ u32x4 xpose[kWaves][kTile / 4];
    const int lane = int(threadIdx.x) % kWave;
    const int wave = int(threadIdx.x) / kWave;
    f32x4* p4 = reinterpret_cast<f32x4*>(p);
    f32x4* m4 = reinterpret_cast<f32x4*>(m);
    f32x4* v4 = reinterpret_cast<f32x4*>(v);
    u32x2* w2 = reinterpret_cast<u32x2*>(w);
    for (int64_t q = int64_t(blockIdx.x) * kWaves + wave; q < npairs;
         q += int64_t(gridDim.x) * kWaves)
        tiles<BF16, kPair>(p4, m4, v4, w2, c, n, q * kPair, lane, xpose[wave]);
}

// Single-direction, copy and triad streams, for the memory system's own
// rates: reads (two 16-byte vectors per lane in flight), writes (one 16-byte
// vector per lane), a copy and a triad (two reads per write), all
// non-temporal, in the grid-stride order of the step kernels. nvec counts
// 16-byte vectors per stream.
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4* __restrict__ a,
                                                              int64_t nvec,
                                                              u32x4* __restrict__ sink) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    for (; i + stride < nvec; i += 2 * stride) {
        const u32x4 x = __builtin_nontemporal_load(a + i);
        const u32x4 y = __builtin_nontemporal_load(a + i + stride);
        acc ^= x ^ y;
    }
    if (i < nvec) acc ^= __builtin_nontemporal_load(a + i);
    // keeps the loads; taken only when every lane's XOR is one particular value
    if ((acc.x & acc.y & acc.z & acc.w) == 0xffffffffu) sink[0] = acc;
}

__global__ __launch_bounds__(kThreads) void probe_write_kernel(u32x4* __restrict__ b,
                                                               int64_t nvec) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < nvec; i += stride)
        __builtin_nontemporal_store(u32x4{uint32_t(i), uint32_t(i >> 32), 0x5a5a5a5au, 0u}, b + i);
}

__global__ __launch_bounds__(kThreads) void probe_copy_kernel(const u32x4* __restrict__ a,
                                                              u32x4* __restrict__ b,
                                                              int64_t nvec) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < nvec; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(a + i), b + i);
}

// Two read streams for each write stream, the fused step's ratio in three
// streams: c[i] = a0[i] ^ a1[i], a0 = a[0, nvec), a1 = a[nvec, 2 nvec).
__global__ __launch_bounds__(kThreads) void probe_triad_kernel(const u32x4* __restrict__ a,
                                                               u32x4* __restrict__ c,
                                                               int64_t nvec) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < nvec; i += stride) {
        const u32x4 x = __builtin_nontemporal_load(a + i);
        const u32x4 y = __builtin_nontemporal_load(a + nvec + i);
        __builtin_nontemporal_store(x ^ y, c + i);
    }
}

}  // namespace

hipError_t launch_streams(float* p, float* m, float* v, uint16_t* w, int64_t S,
                          const PtrPack& contribs, int n, int dtype, hipStream_t stream,
                          hipEvent_t ev_start, hipEvent_t ev_stop) {
    const int64_t npairs = S / (kPair * kTile);
    const dim3 grid{unsigned(streams_grid(S, kPair))}, block{unsigned(kThreads)};
    if (ev_start != nullptr) {  // the events tied to this dispatch's start and end
        if (dtype == ZS_BF16)
            hipExtLaunchKernelGGL((streams_kernel<true>), grid, block, 0, stream, ev_start,
                                  ev_stop, 0, p, m, v, w, npairs, contribs, n);
        else
            hipExtLaunchKernelGGL((streams_kernel<false>), grid, block, 0, stream, ev_start,
                                  ev_stop, 0, p, m, v, w, npairs, contribs, n);
    } else if (dtype == ZS_BF16) {
        hipLaunchKernelGGL((streams_kernel<true>), grid, block, 0, stream, p, m, v, w, npairs,
                           contribs, n);
    } else {
        hipLaunchKernelGGL((streams_kernel<false>), grid, block, 0, stream, p, m, v, w, npairs,
                           contribs, n);
    }
    return hipGetLastError();
}

hipError_t launch_probe(int kind, void* buf, void* buf2, int64_t nvec, int per_cu,
                        hipStream_t stream) {
    // per_cu 0: a grid that covers the buffer (two vectors per lane for reads,
    // one otherwise); else a persistent grid of per_cu workgroups per CU
    const int64_t blocks =
        probe_grid(kind == ZS_PROBE_READ, nvec, per_cu, per_cu > 0 ? device_info().cu_count : 0);
    const dim3 grid{unsigned(blocks)}, block{unsigned(kThreads)};
    u32x4* a = static_cast<u32x4*>(buf);
    u32x4* b = static_cast<u32x4*>(buf2);
    if (kind == ZS_PROBE_READ)
        hipLaunchKernelGGL(probe_read_kernel, grid, block, 0, stream, a, nvec, b);
    else if (kind == ZS_PROBE_WRITE)
        hipLaunchKernelGGL(probe_write_kernel, grid, block, 0, stream, a, nvec);
    else if (kind == ZS_PROBE_TRIAD)
        hipLaunchKernelGGL(probe_triad_kernel, grid, block, 0, stream, a, b, nvec);
    else
        hipLaunchKernelGGL(probe_copy_kernel, grid, block, 0, stream, a, b, nvec);
    return hipGetLastError();
}

}  // namespace zs
