// Measurement aid: the fused step's memory streams with none of its
// arithmetic, to read the step kernel against what HBM delivers for exactly
// its mix of streams (n contribution reads, p, m, v read and written, w
// written: 2 reads per write at n = 8 bf16), not only against the datasheet
// peak.
//
// Same launch shape, lane map, vector widths and cache hints as the fused
// kernel: 8 elements per lane, non-temporal contribution loads, temporal
// state loads, non-temporal stores, a persistent grid of the same size. The
// values written are placeholders (p + m, v, p and an XOR of the
// contributions); the buffers' contents are not meaningful afterwards.

#include "zs_internal.h"

namespace zs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// VW: 16-byte vectors of one contribution per 8 elements (1 for bf16, 2 for fp32)
template <int VW>
__global__ __launch_bounds__(kThreads) void streams_kernel(float* __restrict__ p,
                                                           float* __restrict__ m,
                                                           float* __restrict__ v,
                                                           uint16_t* __restrict__ w, int64_t nvec,
                                                           PtrPack c, int n) {
    f32x4* p4 = reinterpret_cast<f32x4*>(p);
    f32x4* m4 = reinterpret_cast<f32x4*>(m);
    f32x4* v4 = reinterpret_cast<f32x4*>(v);
    u32x4* w4 = reinterpret_cast<u32x4*>(w);
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < nvec;
         i += int64_t(gridDim.x) * kThreads) {
        u32x4 s = {0u, 0u, 0u, 0u};
#pragma unroll 8
        for (int q = 0; q < n; ++q) {
            const u32x4* cq = static_cast<const u32x4*>(c.p[q]) + VW * i;
#pragma unroll
            for (int h = 0; h < VW; ++h) s ^= __builtin_nontemporal_load(cq + h);
        }
        const f32x4 pa = p4[2 * i], pb = p4[2 * i + 1];
        const f32x4 ma = m4[2 * i], mb = m4[2 * i + 1];
        const f32x4 va = v4[2 * i], vb = v4[2 * i + 1];
        __builtin_nontemporal_store(pa + ma, p4 + 2 * i);
        __builtin_nontemporal_store(pb + mb, p4 + 2 * i + 1);
        __builtin_nontemporal_store(va, m4 + 2 * i);
        __builtin_nontemporal_store(vb, m4 + 2 * i + 1);
        __builtin_nontemporal_store(pa, v4 + 2 * i);
        __builtin_nontemporal_store(pb, v4 + 2 * i + 1);
        __builtin_nontemporal_store(s, w4 + i);
    }
}

}  // namespace

hipError_t launch_streams(float* p, float* m, float* v, uint16_t* w, int64_t S,
                          const PtrPack& contribs, int n, int dtype, hipStream_t stream) {
    const int64_t nvec = S / 8;
    const int64_t cap = int64_t(device_info().cu_count) * ZS_STEP_BLOCKS_PER_CU;
    int64_t blocks = (nvec + kThreads - 1) / kThreads;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    if (dtype == ZS_BF16)
        hipLaunchKernelGGL((streams_kernel<1>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                           p, m, v, w, nvec, contribs, n);
    else
        hipLaunchKernelGGL((streams_kernel<2>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                           p, m, v, w, nvec, contribs, n);
    return hipGetLastError();
}

}  // namespace zs
