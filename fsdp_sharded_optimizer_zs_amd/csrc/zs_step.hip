// Reduce-scatter arithmetic and the fused reduce + AdamW shard step, for
// gfx950 (MI355X).
//
// Both kernels are streaming, elementwise and HBM-bound: per element they
// read the D gradient contributions (and p, m, v), do a few dozen VALU
// operations and write the results once. There is no dense contraction, so
// no MFMA and no LDS: every lane owns 8 consecutive elements, moved with
// 16-byte (dwordx4) loads and stores, and a persistent grid sized to the CU
// count walks the shard in grid-stride order, so each wavefront's accesses
// are fully coalesced 1 KiB runs per stream.
//
// The arithmetic follows the operation order fixed for the step exactly:
// contributions widened exactly and folded left to right in rank order,
// one fp32 multiply by 1/n; AdamW in fp32 with every operation rounded on
// its own. This file is compiled with -ffp-contract=off (and says so again
// below), division and sqrt are the correctly rounded IEEE operations, and
// fp32 denormals are kept.

#include "zs_internal.h"

#pragma clang fp contract(off)

// Launch shape and cache hints, chosen by measurement on MI355X over the
// 81 buckets of a 70B rank shard: 2 workgroups of 4 wavefronts per CU
// (8 wavefronts per CU) with non-temporal loads and stores was the fastest
// setting; 8 workgroups per CU, temporal stores, 4-element lanes and
// 512-element wave tiles were all equal or slower, although the wave-tile
// form writes no partial cache lines.
#ifndef ZS_STEP_BLOCKS_PER_CU
#define ZS_STEP_BLOCKS_PER_CU 2
#endif
#ifndef ZS_NT_LOADS
#define ZS_NT_LOADS 1
#endif
#ifndef ZS_NT_STORES
#define ZS_NT_STORES 1
#endif

namespace zs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 wavefronts of 64
constexpr int kVec = 8;        // elements per lane per iteration

// Streamed (read-once) loads and write-once stores.
template <typename T>
__device__ __forceinline__ T ld_once(const T* ptr) {
#if ZS_NT_LOADS
    return __builtin_nontemporal_load(ptr);
#else
    return *ptr;
#endif
}
template <typename T>
__device__ __forceinline__ void st_once(T val, T* ptr) {
#if ZS_NT_STORES
    __builtin_nontemporal_store(val, ptr);
#else
    *ptr = val;
#endif
}

// bf16 bits -> fp32: exact, the 16 bits become the high half of the word.
__device__ __forceinline__ float bf16_lo(uint32_t word) { return __uint_as_float(word << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t word) { return __uint_as_float(word & 0xffff0000u); }

// fp32 -> bf16 bits, IEEE round to nearest, ties to even. Adding 0x7fff plus
// the kept low bit carries into the kept half exactly when the dropped half
// is above one half, or equal to it with an odd kept half. NaNs keep sign
// and high payload and are made quiet.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : rounded;
}

// Contribution q's 8 elements at vector index i, widened to fp32.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t i, float (&x)[kVec]) {
    if constexpr (DT == ZS_BF16) {
        const u32x4 h = ld_once(static_cast<const u32x4*>(base) + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_lo(h[e]);
            x[2 * e + 1] = bf16_hi(h[e]);
        }
    } else {
        const f32x4* b = static_cast<const f32x4*>(base) + 2 * i;
        const f32x4 a0 = ld_once(b);
        const f32x4 a1 = ld_once(b + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a0[e];
            x[4 + e] = a1[e];
        }
    }
}

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t i) {
    if constexpr (DT == ZS_BF16) {
        return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[i]) << 16);
    } else {
        return static_cast<const float*>(base)[i];
    }
}

// g = ((c_0 + c_1) + ... + c_{n-1}) * inv_n for 8 elements, in rank order.
template <int DT, int NC>
__device__ __forceinline__ void reduce8(const PtrPack& c, int n, float inv_n, int64_t i,
                                        float (&g)[kVec]) {
    load8<DT>(c.p[0], i, g);
    if constexpr (NC > 0) {
#pragma unroll
        for (int q = 1; q < NC; ++q) {
            float x[kVec];
            load8<DT>(c.p[q], i, x);
#pragma unroll
            for (int e = 0; e < kVec; ++e) g[e] = g[e] + x[e];
        }
    } else {
#pragma unroll 4
        for (int q = 1; q < n; ++q) {
            float x[kVec];
            load8<DT>(c.p[q], i, x);
#pragma unroll
            for (int e = 0; e < kVec; ++e) g[e] = g[e] + x[e];
        }
    }
#pragma unroll
    for (int e = 0; e < kVec; ++e) g[e] = g[e] * inv_n;
}

template <int DT>
__device__ __forceinline__ float reduce1(const PtrPack& c, int n, float inv_n, int64_t i) {
    float s = load1<DT>(c.p[0], i);
    for (int q = 1; q < n; ++q) s = s + load1<DT>(c.p[q], i);
    return s * inv_n;
}

// One AdamW element, in the fixed order, every operation rounded on its own.
__device__ __forceinline__ void adamw1(float& p, float& m, float& v, float g,
                                       const AdamConsts& k) {
    const float p1 = p * k.dec;
    const float m1 = (k.b1 * m) + (k.b1c * g);
    const float v1 = (k.b2 * v) + (k.b2c * (g * g));
    const float den = (__builtin_sqrtf(v1) / k.bc2s) + k.eps;
    p = p1 - (k.ss * (m1 / den));
    m = m1;
    v = v1;
}

// ---------------------------------------------------------------- kernels

// Fused reduce + AdamW over 8-element vectors; 16-byte aligned buffers.
// The last block also handles the S % 8 tail elements one per lane.
template <int DT, int NC>
__global__ __launch_bounds__(kThreads) void adamw_vec_kernel(
    float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
    uint16_t* __restrict__ w, int64_t S, PtrPack c, int n, AdamConsts k) {
    const int64_t nvec = S / kVec;
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    f32x4* p4 = reinterpret_cast<f32x4*>(p);
    f32x4* m4 = reinterpret_cast<f32x4*>(m);
    f32x4* v4 = reinterpret_cast<f32x4*>(v);
    u32x4* w4 = reinterpret_cast<u32x4*>(w);
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < nvec; i += stride) {
        float g[kVec];
        reduce8<DT, NC>(c, n, k.inv_n, i, g);
        const f32x4 pa = p4[2 * i], pb = p4[2 * i + 1];
        const f32x4 ma = m4[2 * i], mb = m4[2 * i + 1];
        const f32x4 va = v4[2 * i], vb = v4[2 * i + 1];
        float pp[kVec], mm[kVec], vv[kVec];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pp[e] = pa[e], pp[4 + e] = pb[e];
            mm[e] = ma[e], mm[4 + e] = mb[e];
            vv[e] = va[e], vv[4 + e] = vb[e];
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) adamw1(pp[e], mm[e], vv[e], g[e], k);
        u32x4 wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[e] = f32_to_bf16(pp[2 * e]) | (f32_to_bf16(pp[2 * e + 1]) << 16);
        st_once(f32x4{pp[0], pp[1], pp[2], pp[3]}, p4 + 2 * i);
        st_once(f32x4{pp[4], pp[5], pp[6], pp[7]}, p4 + 2 * i + 1);
        st_once(f32x4{mm[0], mm[1], mm[2], mm[3]}, m4 + 2 * i);
        st_once(f32x4{mm[4], mm[5], mm[6], mm[7]}, m4 + 2 * i + 1);
        st_once(f32x4{vv[0], vv[1], vv[2], vv[3]}, v4 + 2 * i);
        st_once(f32x4{vv[4], vv[5], vv[6], vv[7]}, v4 + 2 * i + 1);
        st_once(wv, w4 + i);
    }
    const int64_t t = nvec * kVec + threadIdx.x;
    if (blockIdx.x == gridDim.x - 1 && t < S) {
        const float g = reduce1<DT>(c, n, k.inv_n, t);
        float pp = p[t], mm = m[t], vv = v[t];
        adamw1(pp, mm, vv, g, k);
        p[t] = pp;
        m[t] = mm;
        v[t] = vv;
        w[t] = uint16_t(f32_to_bf16(pp));
    }
}

// Element-at-a-time variant for buffers that are not 16-byte aligned.
template <int DT>
__global__ __launch_bounds__(kThreads) void adamw_scalar_kernel(
    float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
    uint16_t* __restrict__ w, int64_t S, PtrPack c, int n, AdamConsts k) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x; t < S; t += stride) {
        const float g = reduce1<DT>(c, n, k.inv_n, t);
        float pp = p[t], mm = m[t], vv = v[t];
        adamw1(pp, mm, vv, g, k);
        p[t] = pp;
        m[t] = mm;
        v[t] = vv;
        w[t] = uint16_t(f32_to_bf16(pp));
    }
}

// Unfused reduce: g written to HBM (fp32).
template <int DT, int NC>
__global__ __launch_bounds__(kThreads) void reduce_vec_kernel(
    float* __restrict__ out, int64_t S, PtrPack c, int n, float inv_n) {
    const int64_t nvec = S / kVec;
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    f32x4* o4 = reinterpret_cast<f32x4*>(out);
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < nvec; i += stride) {
        float g[kVec];
        reduce8<DT, NC>(c, n, inv_n, i, g);
        st_once(f32x4{g[0], g[1], g[2], g[3]}, o4 + 2 * i);
        st_once(f32x4{g[4], g[5], g[6], g[7]}, o4 + 2 * i + 1);
    }
    const int64_t t = nvec * kVec + threadIdx.x;
    if (blockIdx.x == gridDim.x - 1 && t < S) out[t] = reduce1<DT>(c, n, inv_n, t);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void reduce_scalar_kernel(
    float* __restrict__ out, int64_t S, PtrPack c, int n, float inv_n) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x; t < S; t += stride)
        out[t] = reduce1<DT>(c, n, inv_n, t);
}

// ---------------------------------------------------------------- dispatch

int grid_for(int64_t work_items) {
    const int64_t cap = int64_t(device_info().cu_count) * ZS_STEP_BLOCKS_PER_CU;
    int64_t blocks = (work_items + kThreads - 1) / kThreads;
    if (blocks > cap) blocks = cap;
    return blocks < 1 ? 1 : int(blocks);
}

template <int DT, int NC>
hipError_t adamw_vec_launch(float* p, float* m, float* v, uint16_t* w, int64_t S,
                            const PtrPack& c, int n, const AdamConsts& k,
                            hipStream_t stream) {
    hipLaunchKernelGGL((adamw_vec_kernel<DT, NC>), dim3(grid_for(S / kVec)), dim3(kThreads),
                       0, stream, p, m, v, w, S, c, n, k);
    return hipGetLastError();
}

template <int DT>
hipError_t adamw_dispatch(float* p, float* m, float* v, uint16_t* w, int64_t S,
                          const PtrPack& c, int n, const AdamConsts& k, bool aligned,
                          hipStream_t stream) {
    if (!aligned) {
        hipLaunchKernelGGL((adamw_scalar_kernel<DT>), dim3(grid_for(S)), dim3(kThreads), 0,
                           stream, p, m, v, w, S, c, n, k);
        return hipGetLastError();
    }
    switch (n) {
        case 1: return adamw_vec_launch<DT, 1>(p, m, v, w, S, c, n, k, stream);
        case 2: return adamw_vec_launch<DT, 2>(p, m, v, w, S, c, n, k, stream);
        case 4: return adamw_vec_launch<DT, 4>(p, m, v, w, S, c, n, k, stream);
        case 8: return adamw_vec_launch<DT, 8>(p, m, v, w, S, c, n, k, stream);
        case 16: return adamw_vec_launch<DT, 16>(p, m, v, w, S, c, n, k, stream);
        case 32: return adamw_vec_launch<DT, 32>(p, m, v, w, S, c, n, k, stream);
        default: return adamw_vec_launch<DT, 0>(p, m, v, w, S, c, n, k, stream);
    }
}

template <int DT, int NC>
hipError_t reduce_vec_launch(const PtrPack& c, int n, int64_t S, float inv_n, float* out,
                             hipStream_t stream) {
    hipLaunchKernelGGL((reduce_vec_kernel<DT, NC>), dim3(grid_for(S / kVec)), dim3(kThreads),
                       0, stream, out, S, c, n, inv_n);
    return hipGetLastError();
}

template <int DT>
hipError_t reduce_dispatch(const PtrPack& c, int n, int64_t S, float inv_n, float* out,
                           bool aligned, hipStream_t stream) {
    if (!aligned) {
        hipLaunchKernelGGL((reduce_scalar_kernel<DT>), dim3(grid_for(S)), dim3(kThreads), 0,
                           stream, out, S, c, n, inv_n);
        return hipGetLastError();
    }
    switch (n) {
        case 1: return reduce_vec_launch<DT, 1>(c, n, S, inv_n, out, stream);
        case 2: return reduce_vec_launch<DT, 2>(c, n, S, inv_n, out, stream);
        case 4: return reduce_vec_launch<DT, 4>(c, n, S, inv_n, out, stream);
        case 8: return reduce_vec_launch<DT, 8>(c, n, S, inv_n, out, stream);
        case 16: return reduce_vec_launch<DT, 16>(c, n, S, inv_n, out, stream);
        case 32: return reduce_vec_launch<DT, 32>(c, n, S, inv_n, out, stream);
        default: return reduce_vec_launch<DT, 0>(c, n, S, inv_n, out, stream);
    }
}

}  // namespace

hipError_t launch_adamw(float* p, float* m, float* v, uint16_t* w, int64_t S,
                        const PtrPack& contribs, int n, int dtype, const AdamConsts& k,
                        bool aligned, hipStream_t stream) {
    if (dtype == ZS_BF16)
        return adamw_dispatch<ZS_BF16>(p, m, v, w, S, contribs, n, k, aligned, stream);
    return adamw_dispatch<ZS_F32>(p, m, v, w, S, contribs, n, k, aligned, stream);
}

hipError_t launch_reduce(const PtrPack& contribs, int n, int dtype, int64_t S, float inv_n,
                         float* out, bool aligned, hipStream_t stream) {
    if (dtype == ZS_BF16)
        return reduce_dispatch<ZS_BF16>(contribs, n, S, inv_n, out, aligned, stream);
    return reduce_dispatch<ZS_F32>(contribs, n, S, inv_n, out, aligned, stream);
}

}  // namespace zs
