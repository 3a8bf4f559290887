// Reduce-scatter arithmetic and the fused reduce + AdamW shard step, for
// gfx950 (MI355X).
//
// Both kernels are streaming, elementwise and HBM-bound: per element they
// read the D gradient contributions (and p, m, v), do a few dozen VALU
// operations and write the results once. There is no dense contraction, so
// no MFMA. Work goes in 512-element tiles, 8 elements per lane; each
// wavefront takes two adjacent tiles, and the grid has one wavefront per tile
// pair. Inside a tile two lane maps are used:
//
//   run map:   lane t holds elements 8t .. 8t+7 (one 16-byte bf16 vector);
//   split map: lane t holds elements 4t .. 4t+3 and 256+4t .. 256+4t+3 (two
//              16-byte fp32 vectors).
//
// Every load and store instruction of a wavefront then covers one contiguous
// run of whole cache lines: bf16 contributions load in the run map (1 KiB),
// fp32 contributions and the state p, m, v load and store in the split map
// (1 KiB), and the bf16 working shard leaves in the split map as two 512-byte
// stores. The fp32 sums of bf16 contributions are moved from the run map to
// the split map through a 2 KiB LDS slot per wavefront. (With the run map for
// fp32 too, a lane's 32 bytes went out as two 16-byte stores and lines could
// leave L2 half written: 3.6% more HBM writes. On MI355X's 70B buckets the
// split map with tile pairs runs the step at 6.17 TB/s, against 5.94-6.04
// for the run map on a persistent grid of two workgroups per CU.)
//
// The arithmetic follows the operation order fixed for the step exactly:
// contributions widened exactly and folded left to right in rank order,
// one fp32 multiply by 1/n; AdamW in fp32 with every operation rounded on
// its own. This file is compiled with -ffp-contract=off (and says so again
// below), division and sqrt are the correctly rounded IEEE operations, and
// fp32 denormals are kept.

#include <hip/hip_ext.h>

#include "zs_internal.h"

#pragma clang fp contract(off)

// Cache hints, chosen by measurement on MI355X: every stream is touched once
// per step, so contributions and the state p, m, v are read with
// non-temporal loads and everything is written with non-temporal stores
// (70B buckets: 6.31 TB/s, against 6.16 with temporal state loads and 5.94
// with temporal contribution loads). The launch shape (ZS_STEP_TILES, one
// wavefront per tile group) is in zs_internal.h.
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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;               // 4 wavefronts of 64
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;    // wavefronts per workgroup
constexpr int kVec = 8;                     // elements per lane per tile
constexpr int kTile = kWave * kVec;         // elements per wavefront tile

// Occupancy the tiled kernels are compiled for: at most 2 wavefronts per
// SIMD, so up to 256 VGPRs each and the scheduler issues a tile pair's 28
// loads before their first use. Without it the compiler saves registers for
// a higher occupancy and serializes the loads (3.5-5.9 TB/s on MI355X); at
// most 1 wavefront per SIMD measured 3.3-3.6 TB/s.
#ifndef ZS_WAVES
#define ZS_WAVES __attribute__((amdgpu_waves_per_eu(1, 2)))
#endif

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

// One contribution's 8 elements for lane `lane` of tile `tile`, widened to
// fp32: bf16 in the run map, fp32 in the split map.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t tile, int lane,
                                      float (&x)[kVec]) {
    if constexpr (DT == ZS_BF16) {
        const u32x4 h = ld_once(static_cast<const u32x4*>(base) + tile * kWave + lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_lo(h[e]);
            x[2 * e + 1] = bf16_hi(h[e]);
        }
    } else {
        const f32x4* b = static_cast<const f32x4*>(base) + tile * (kTile / 4) + lane;
        const f32x4 a0 = ld_once(b);
        const f32x4 a1 = ld_once(b + kWave);
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

// Fold of the n contributions c.p[base .. base+n) for 8 elements, left to
// right from the first, into s (fp32, one rounding per add). Loads are
// issued in batches of up to 8 contributions ahead of their adds; the add
// order is the plain left fold whatever the batching. (A fully unrolled
// fold of 16 or 32 contributions lets the compiler interleave loads and
// adds, which measured 25% slower at 32.)
constexpr int kBatch = 8;

template <int DT, int NB>
__device__ __forceinline__ void add_batch(const PtrPack& c, int first, int64_t tile, int lane,
                                          float (&s)[kVec]) {
    float x[NB][kVec];
#pragma unroll
    for (int q = 0; q < NB; ++q) load8<DT>(c.p[first + q], tile, lane, x[q]);
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int e = 0; e < kVec; ++e) s[e] = s[e] + x[q][e];
}

// c_base .. c_base+NB-1 into s: s = c_base, then the other NB - 1 added in
// order, all NB loads issued before the first add.
template <int DT, int NB>
__device__ __forceinline__ void first_batch(const PtrPack& c, int base, int64_t tile, int lane,
                                            float (&s)[kVec]) {
    load8<DT>(c.p[base], tile, lane, s);
    if constexpr (NB > 1) add_batch<DT, NB - 1>(c, base + 1, tile, lane, s);
}

template <int DT, int NC>
__device__ __forceinline__ void fold8(const PtrPack& c, int base, int n, int64_t tile, int lane,
                                      float (&s)[kVec]) {
    if constexpr (NC > 0 && NC <= kBatch) {
        first_batch<DT, NC>(c, base, tile, lane, s);
    } else {
        // For bf16 the batch loop keeps a run-time trip count (n, which
        // equals NC when NC is fixed): with the trip count known, the
        // compiler unrolled the single batch after the first at NC = 16 and
        // then issued its loads one at a time, each behind a wait for the one
        // before (16 bf16 contributions: 5.1 TB/s, against 6.2 with the loop
        // kept). fp32 keeps the fixed count, whose unrolled schedule issues
        // the first batches of both tiles together (16 fp32 contributions:
        // 0.7% faster than with the loop kept, same process and buffers).
        const int len = (DT == ZS_BF16 || NC == 0) ? n : NC;
        // The first batch (up to 8) goes out as one batch through a switch
        // over the batch sizes, and for bf16 so does the remainder after the
        // whole batches (up to 7); one load at a time ran bf16 n = 3, 5, 7
        // and 13 6-14% slower (5.3-5.7 against 6.0 TB/s) and fp32 n = 3, 5,
        // 7 1-4% slower. fp32 keeps single loads for the remainder, which
        // measured 0.8% faster at n = 12.
        int q;
        if (NC >= kBatch || len >= kBatch) {
            first_batch<DT, kBatch>(c, base, tile, lane, s);
            q = kBatch;
        } else {
            switch (len) {
                case 7: first_batch<DT, 7>(c, base, tile, lane, s); break;
                case 6: first_batch<DT, 6>(c, base, tile, lane, s); break;
                case 5: first_batch<DT, 5>(c, base, tile, lane, s); break;
                case 4: first_batch<DT, 4>(c, base, tile, lane, s); break;
                case 3: first_batch<DT, 3>(c, base, tile, lane, s); break;
                case 2: first_batch<DT, 2>(c, base, tile, lane, s); break;
                default: first_batch<DT, 1>(c, base, tile, lane, s); break;  // n >= 1
            }
            q = len;
        }
#pragma unroll 1
        for (; q + kBatch <= len; q += kBatch) add_batch<DT, kBatch>(c, base + q, tile, lane, s);
        if constexpr (DT != ZS_BF16) {
#pragma unroll 1
            for (; q < len; ++q) add_batch<DT, 1>(c, base + q, tile, lane, s);
            return;
        }
        switch (len - q) {
            case 7: add_batch<DT, 7>(c, base + q, tile, lane, s); break;
            case 6: add_batch<DT, 6>(c, base + q, tile, lane, s); break;
            case 5: add_batch<DT, 5>(c, base + q, tile, lane, s); break;
            case 4: add_batch<DT, 4>(c, base + q, tile, lane, s); break;
            case 3: add_batch<DT, 3>(c, base + q, tile, lane, s); break;
            case 2: add_batch<DT, 2>(c, base + q, tile, lane, s); break;
            case 1: add_batch<DT, 1>(c, base + q, tile, lane, s); break;
            default: break;
        }
    }
}

template <int DT>
__device__ __forceinline__ float fold1(const PtrPack& c, int base, int n, int64_t i) {
    float s = load1<DT>(c.p[base], i);
    for (int q = 1; q < n; ++q) s = s + load1<DT>(c.p[base + q], i);
    return s;
}

// The value an fp32 partial sum takes once held in the reduce dtype.
template <int DT>
__device__ __forceinline__ float to_reduce_dtype(float x) {
    if constexpr (DT == ZS_BF16) return __uint_as_float(f32_to_bf16(x) << 16);
    return x;
}

// Flat reduce: g = ((c_0 + c_1) + ... + c_{n-1}) * inv_n, in rank order.
// NC > 0 fixes n at compile time, so loads go out in batches of up to 8
// ahead of their adds.
template <int DT, int NC>
struct FlatSum {
    int n;
    float inv_n;
    __device__ __forceinline__ void vec(const PtrPack& c, int64_t tile, int lane,
                                        float (&g)[kVec]) const {
        fold8<DT, NC>(c, 0, n, tile, lane, g);
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = g[e] * inv_n;
    }
    __device__ __forceinline__ float one(const PtrPack& c, int64_t i) const {
        return fold1<DT>(c, 0, n, i) * inv_n;
    }
};

// HYBRID_SHARD reduce: R replica groups of nd contributions each, replica-
// major (c.p[j*nd + k]). Group j folds to s_j; with rnd, s_j is rounded to
// the reduce dtype (a collective's output held in it); the s_j fold left in
// group order to t, rounded again with rnd; g = t * inv_n, inv_n = 1/(R*nd).
template <int DT, int NC>
struct HybridSum {
    int nd;
    int R;
    int rnd;
    float inv_n;
    __device__ __forceinline__ void vec(const PtrPack& c, int64_t tile, int lane,
                                        float (&g)[kVec]) const {
        fold8<DT, NC>(c, 0, nd, tile, lane, g);
        if (rnd) {
#pragma unroll
            for (int e = 0; e < kVec; ++e) g[e] = to_reduce_dtype<DT>(g[e]);
        }
        for (int j = 1; j < R; ++j) {
            float s[kVec];
            fold8<DT, NC>(c, j * nd, nd, tile, lane, s);
#pragma unroll
            for (int e = 0; e < kVec; ++e) g[e] = g[e] + (rnd ? to_reduce_dtype<DT>(s[e]) : s[e]);
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = (rnd ? to_reduce_dtype<DT>(g[e]) : g[e]) * inv_n;
    }
    __device__ __forceinline__ float one(const PtrPack& c, int64_t i) const {
        float t = fold1<DT>(c, 0, nd, i);
        if (rnd) t = to_reduce_dtype<DT>(t);
        for (int j = 1; j < R; ++j) {
            const float s = fold1<DT>(c, j * nd, nd, i);
            t = t + (rnd ? to_reduce_dtype<DT>(s) : s);
        }
        return (rnd ? to_reduce_dtype<DT>(t) : t) * inv_n;
    }
};

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

// Order the wavefront's LDS accesses before and after this point (the LDS
// serves one wavefront's instructions in issue order).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The 8 values of a lane from the run map to the split map, through the
// wavefront's slot of 128 16-byte entries (entry k: tile elements 4k..4k+3).
__device__ __forceinline__ void run_to_split(float (&g)[kVec], f32x4* slot, int lane) {
    slot[2 * lane] = f32x4{g[0], g[1], g[2], g[3]};
    slot[2 * lane + 1] = f32x4{g[4], g[5], g[6], g[7]};
    wave_sync();
    const f32x4 a = slot[lane];
    const f32x4 b = slot[kWave + lane];
    wave_sync();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        g[e] = a[e];
        g[4 + e] = b[e];
    }
}

// AdamW on TP adjacent tiles from tile0, lane `lane`: all state loads, then
// the contributions of every tile, then the arithmetic, then the stores.
template <int DT, int TP, class Sum>
__device__ __forceinline__ void adamw_tiles(f32x4* __restrict__ p4, f32x4* __restrict__ m4,
                                            f32x4* __restrict__ v4, u32x2* __restrict__ w2,
                                            const PtrPack& c, const Sum& sum, const AdamConsts& k,
                                            int64_t tile0, int lane, f32x4* slot) {
    f32x4 pa[TP], pb[TP], ma[TP], mb[TP], va[TP], vb[TP];
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        const int64_t a = (tile0 + u) * (kTile / 4) + lane;  // split map: elements 4a .. 4a+3
        const int64_t b = a + kWave;                          // and 4b .. 4b+3 (256 further)
        pa[u] = ld_once(p4 + a), pb[u] = ld_once(p4 + b);
        ma[u] = ld_once(m4 + a), mb[u] = ld_once(m4 + b);
        va[u] = ld_once(v4 + a), vb[u] = ld_once(v4 + b);
    }
    float g[TP][kVec];
#pragma unroll
    for (int u = 0; u < TP; ++u) sum.vec(c, tile0 + u, lane, g[u]);
    // every tile's exchange (an LDS round trip between wavefront fences) before
    // any tile's arithmetic, so that no fence sits between one tile's stores
    // and the next tile's use of its loads
    if constexpr (DT == ZS_BF16) {
#pragma unroll
        for (int u = 0; u < TP; ++u) run_to_split(g[u], slot, lane);
    }
    // every tile's arithmetic, then the stores stream by stream (p of all
    // tiles, then m, v and w), so that each stream's run of the tile group
    // leaves in consecutive instructions (70B buckets: 0.2-0.3% faster than
    // storing tile by tile, same process and buffers)
    float pp[TP][kVec], mm[TP][kVec], vv[TP][kVec];
    u32x2 wa[TP], wb[TP];
#pragma unroll
    for (int u = 0; u < TP; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pp[u][e] = pa[u][e], pp[u][4 + e] = pb[u][e];
            mm[u][e] = ma[u][e], mm[u][4 + e] = mb[u][e];
            vv[u][e] = va[u][e], vv[u][4 + e] = vb[u][e];
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) adamw1(pp[u][e], mm[u][e], vv[u][e], g[u][e], k);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            wa[u][e] = f32_to_bf16(pp[u][2 * e]) | (f32_to_bf16(pp[u][2 * e + 1]) << 16);
            wb[u][e] = f32_to_bf16(pp[u][4 + 2 * e]) | (f32_to_bf16(pp[u][5 + 2 * e]) << 16);
        }
    }
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        const int64_t a = (tile0 + u) * (kTile / 4) + lane;
        st_once(f32x4{pp[u][0], pp[u][1], pp[u][2], pp[u][3]}, p4 + a);
        st_once(f32x4{pp[u][4], pp[u][5], pp[u][6], pp[u][7]}, p4 + a + kWave);
    }
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        const int64_t a = (tile0 + u) * (kTile / 4) + lane;
        st_once(f32x4{mm[u][0], mm[u][1], mm[u][2], mm[u][3]}, m4 + a);
        st_once(f32x4{mm[u][4], mm[u][5], mm[u][6], mm[u][7]}, m4 + a + kWave);
    }
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        const int64_t a = (tile0 + u) * (kTile / 4) + lane;
        st_once(f32x4{vv[u][0], vv[u][1], vv[u][2], vv[u][3]}, v4 + a);
        st_once(f32x4{vv[u][4], vv[u][5], vv[u][6], vv[u][7]}, v4 + a + kWave);
    }
    // the working shard: non-temporal like the rest, or, when the caller
    // reads it right after (the unit's all-gather), ordinary stores that
    // allocate in L2 and the memory-side Infinity Cache, so that the gather
    // reads it from there (70B step with its unit gather: 97.2 against 99.5
    // ms; with nothing reading it soon, 2.4% slower than non-temporal)
    if (k.keep_w) {
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const int64_t a = (tile0 + u) * (kTile / 4) + lane;
            w2[a] = wa[u];
            w2[a + kWave] = wb[u];
        }
    } else {
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const int64_t a = (tile0 + u) * (kTile / 4) + lane;
            st_once(wa[u], w2 + a);
            st_once(wb[u], w2 + a + kWave);
        }
    }
}

// Fused reduce + AdamW over whole groups of TP adjacent 512-element tiles,
// one group per wavefront and iteration; 16-byte aligned buffers. The last
// workgroup also takes the elements past the last whole group (fewer than
// TP * 512), one per lane.
template <int DT, class Sum, int TP>
__global__ __launch_bounds__(kThreads) ZS_WAVES void adamw_vec_kernel(
    float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
    uint16_t* __restrict__ w, int64_t S, PtrPack c, Sum sum, AdamConsts k) {
    __shared__ f32x4 xpose[kWaves][kTile / 4];
    const int lane = int(threadIdx.x) % kWave;
    const int wave = int(threadIdx.x) / kWave;
    const int64_t stride = int64_t(gridDim.x) * kWaves;
    f32x4* p4 = reinterpret_cast<f32x4*>(p);
    f32x4* m4 = reinterpret_cast<f32x4*>(m);
    f32x4* v4 = reinterpret_cast<f32x4*>(v);
    u32x2* w2 = reinterpret_cast<u32x2*>(w);
    const int64_t ngroups = S / (TP * kTile);
    for (int64_t q = int64_t(blockIdx.x) * kWaves + wave; q < ngroups; q += stride)
        adamw_tiles<DT, TP>(p4, m4, v4, w2, c, sum, k, q * TP, lane, xpose[wave]);
    if (blockIdx.x == gridDim.x - 1) {
        for (int64_t t = ngroups * TP * kTile + threadIdx.x; t < S; t += kThreads) {
            const float g = sum.one(c, t);
            float pp = p[t], mm = m[t], vv = v[t];
            adamw1(pp, mm, vv, g, k);
            p[t] = pp;
            m[t] = mm;
            v[t] = vv;
            w[t] = uint16_t(f32_to_bf16(pp));
        }
    }
}

// Element-at-a-time variant for buffers that are not 16-byte aligned.
template <int DT, class Sum>
__global__ __launch_bounds__(kThreads) void adamw_scalar_kernel(
    float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
    uint16_t* __restrict__ w, int64_t S, PtrPack c, Sum sum, AdamConsts k) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x; t < S; t += stride) {
        const float g = sum.one(c, t);
        float pp = p[t], mm = m[t], vv = v[t];
        adamw1(pp, mm, vv, g, k);
        p[t] = pp;
        m[t] = mm;
        v[t] = vv;
        w[t] = uint16_t(f32_to_bf16(pp));
    }
}

// The reduced gradient of TP adjacent tiles from tile0, stored in the split map.
template <int DT, int TP, class Sum>
__device__ __forceinline__ void reduce_tiles(f32x4* __restrict__ o4, const PtrPack& c,
                                             const Sum& sum, int64_t tile0, int lane,
                                             f32x4* slot) {
    float g[TP][kVec];
#pragma unroll
    for (int u = 0; u < TP; ++u) sum.vec(c, tile0 + u, lane, g[u]);
    if constexpr (DT == ZS_BF16) {
#pragma unroll
        for (int u = 0; u < TP; ++u) run_to_split(g[u], slot, lane);
    }
#pragma unroll
    for (int u = 0; u < TP; ++u) {
        const int64_t a = (tile0 + u) * (kTile / 4) + lane;
        st_once(f32x4{g[u][0], g[u][1], g[u][2], g[u][3]}, o4 + a);
        st_once(f32x4{g[u][4], g[u][5], g[u][6], g[u][7]}, o4 + a + kWave);
    }
}

// Unfused reduce: g written to HBM (fp32), tiles as in adamw_vec_kernel.
template <int DT, class Sum, int TP>
__global__ __launch_bounds__(kThreads) ZS_WAVES void reduce_vec_kernel(float* __restrict__ out,
                                                                       int64_t S, PtrPack c,
                                                                       Sum sum) {
    __shared__ f32x4 xpose[kWaves][kTile / 4];
    const int lane = int(threadIdx.x) % kWave;
    const int wave = int(threadIdx.x) / kWave;
    const int64_t stride = int64_t(gridDim.x) * kWaves;
    f32x4* o4 = reinterpret_cast<f32x4*>(out);
    const int64_t ngroups = S / (TP * kTile);
    for (int64_t q = int64_t(blockIdx.x) * kWaves + wave; q < ngroups; q += stride)
        reduce_tiles<DT, TP>(o4, c, sum, q * TP, lane, xpose[wave]);
    if (blockIdx.x == gridDim.x - 1) {
        for (int64_t t = ngroups * TP * kTile + threadIdx.x; t < S; t += kThreads)
            out[t] = sum.one(c, t);
    }
}

template <int DT, class Sum>
__global__ __launch_bounds__(kThreads) void reduce_scalar_kernel(float* __restrict__ out,
                                                                 int64_t S, PtrPack c, Sum sum) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x; t < S; t += stride)
        out[t] = sum.one(c, t);
}

// ---------------------------------------------------------------- dispatch

// What one launch computes: the AdamW step (out == nullptr) or the reduce
// alone into out.
struct Job {
    float* p;
    float* m;
    float* v;
    uint16_t* w;
    float* out;
    int64_t S;
    AdamConsts k;
    bool aligned;
    hipEvent_t ev_start;  // with ev_stop: recorded at the step kernel's own start and end
    hipEvent_t ev_stop;
};

template <int DT, class Sum>
hipError_t launch_job(const Job& j, const PtrPack& c, const Sum& sum, hipStream_t stream) {
    constexpr int TP = ZS_STEP_TILES;
    static_assert(kThreads == kBlockThreads, "grid arithmetic assumes 256-thread workgroups");
    const unsigned tiled = unsigned(step_tiled_grid(j.S, TP));
    const unsigned scalar = unsigned(step_scalar_grid(j.S));
    if (j.out == nullptr && j.ev_start != nullptr) {
        // timed: the runtime ties the two events to this dispatch's start and
        // end timestamps, with no marker packets around it
        if (j.aligned)
            hipExtLaunchKernelGGL((adamw_vec_kernel<DT, Sum, TP>), dim3(tiled), dim3(kThreads), 0,
                                  stream, j.ev_start, j.ev_stop, 0, j.p, j.m, j.v, j.w, j.S, c,
                                  sum, j.k);
        else
            hipExtLaunchKernelGGL((adamw_scalar_kernel<DT, Sum>), dim3(scalar), dim3(kThreads), 0,
                                  stream, j.ev_start, j.ev_stop, 0, j.p, j.m, j.v, j.w, j.S, c,
                                  sum, j.k);
    } else if (j.out == nullptr) {
        if (j.aligned)
            hipLaunchKernelGGL((adamw_vec_kernel<DT, Sum, TP>), dim3(tiled), dim3(kThreads), 0,
                               stream, j.p, j.m, j.v, j.w, j.S, c, sum, j.k);
        else
            hipLaunchKernelGGL((adamw_scalar_kernel<DT, Sum>), dim3(scalar), dim3(kThreads), 0,
                               stream, j.p, j.m, j.v, j.w, j.S, c, sum, j.k);
    } else {
        if (j.aligned)
            hipLaunchKernelGGL((reduce_vec_kernel<DT, Sum, TP>), dim3(tiled), dim3(kThreads), 0,
                               stream, j.out, j.S, c, sum);
        else
            hipLaunchKernelGGL((reduce_scalar_kernel<DT, Sum>), dim3(scalar), dim3(kThreads), 0,
                               stream, j.out, j.S, c, sum);
    }
    return hipGetLastError();
}

// Compile-time fold length for the common group sizes (all loads of a group
// in flight before its adds); a runtime loop for the others. The scalar
// kernels take the runtime form only.
template <int DT, template <int, int> class SumT, class Make>
hipError_t dispatch_nc(const Job& j, const PtrPack& c, int nc, Make make, hipStream_t stream) {
    if (!j.aligned) return launch_job<DT>(j, c, make(SumT<DT, 0>{}), stream);
    switch (nc) {
        case 1: return launch_job<DT>(j, c, make(SumT<DT, 1>{}), stream);
        case 2: return launch_job<DT>(j, c, make(SumT<DT, 2>{}), stream);
        case 4: return launch_job<DT>(j, c, make(SumT<DT, 4>{}), stream);
        case 8: return launch_job<DT>(j, c, make(SumT<DT, 8>{}), stream);
        case 16: return launch_job<DT>(j, c, make(SumT<DT, 16>{}), stream);
        case 32: return launch_job<DT>(j, c, make(SumT<DT, 32>{}), stream);
        default: return launch_job<DT>(j, c, make(SumT<DT, 0>{}), stream);
    }
}

template <int DT>
hipError_t dispatch(const Job& j, const PtrPack& c, int nd, int R, bool rnd, hipStream_t stream) {
    const float inv_n = j.k.inv_n;
    if (R == 1 && !rnd)
        return dispatch_nc<DT, FlatSum>(j, c, nd, [&](auto s) { s.n = nd; s.inv_n = inv_n; return s; },
                                        stream);
    return dispatch_nc<DT, HybridSum>(
        j, c, nd, [&](auto s) { s.nd = nd; s.R = R; s.rnd = rnd ? 1 : 0; s.inv_n = inv_n; return s; },
        stream);
}

}  // namespace

hipError_t launch_adamw(float* p, float* m, float* v, uint16_t* w, int64_t S,
                        const PtrPack& contribs, int nd, int R, bool rnd, int dtype,
                        const AdamConsts& k, bool aligned, hipStream_t stream,
                        hipEvent_t ev_start, hipEvent_t ev_stop) {
    const Job j{p, m, v, w, nullptr, S, k, aligned, ev_start, ev_stop};
    if (dtype == ZS_BF16) return dispatch<ZS_BF16>(j, contribs, nd, R, rnd, stream);
    return dispatch<ZS_F32>(j, contribs, nd, R, rnd, stream);
}

hipError_t launch_reduce(const PtrPack& contribs, int nd, int R, bool rnd, int dtype, int64_t S,
                         float inv_n, float* out, bool aligned, hipStream_t stream) {
    AdamConsts k{};
    k.inv_n = inv_n;
    const Job j{nullptr, nullptr, nullptr, nullptr, out, S, k, aligned, nullptr, nullptr};
    if (dtype == ZS_BF16) return dispatch<ZS_BF16>(j, contribs, nd, R, rnd, stream);
    return dispatch<ZS_F32>(j, contribs, nd, R, rnd, stream);
}

}  // namespace zs
