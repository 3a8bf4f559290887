// Pack (flat unit -> D shards), gather (D shards -> flat unit) and re-shard
// (D shards -> D' shards of the same unit) for gfx950.
//
// All three are bit copies bound by HBM bandwidth. Work is split into runs
// that are contiguous on both sides (a tensor piece that lands inside one
// shard, or one shard landing in the flat unit). Lanes write whole 16-byte
// destination vectors (dwordx4 stores). The source is read with dwordx4
// loads: 16-byte aligned ones when source and destination share their offset
// within 16 bytes, one load at 4-byte alignment per vector when the source is
// dword aligned, and, for bf16 at an odd element offset, aligned loads whose
// bytes are shifted into place in registers (v_alignbyte), each lane taking
// the second vector it straddles from its neighbour (ds_bpermute). Loads and
// stores of the vector body are non-temporal (each byte is touched once).
// The few elements before the first and after the last aligned destination
// vector of a run are copied one per lane. No lane writes a byte outside the
// run it copies; a shifted load may read up to 15 bytes either side of the
// run's source, always inside an aligned 16-byte vector that holds at least
// one byte of the run (so on a page the run already touches), and never uses
// them.
//
// Grids cover the work (one lane per 16-byte vector in the gather, one
// workgroup per 8 KiB work item in pack and re-shard) rather than
// being persistent: the hardware then hands out workgroups in order and the
// open region of HBM stays compact (70B unit gather per shard: 6.21 TB/s
// against 5.94 with a persistent grid of 4 workgroups per CU, same box).

#include "zs_internal.h"

namespace zs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 16 bytes at 4-byte alignment: gfx950 loads it with one global_load_dwordx4
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
static_assert(sizeof(u32x4_a4) == 16, "a 4-aligned vector keeps 16-byte steps");

// Sources are read through global-address-space pointers. A source address
// that passes through an integer (the alignment tests below) or through
// memory (the pack table) is otherwise a generic pointer, read with flat_load
// instructions, which also count against the LDS/scalar-load counter, so
// that a wait for a table read or a lane exchange waits for the copy loads in
// flight too. Every pointer here is device or pinned memory, never LDS or
// private memory, so the global forms are valid. (Measured on the same
// buffers, the ragged and 70B block units pack and re-shard at the same rate
// either way.) The source vector type for an alignment is a member typedef:
// as a template argument, a typedef loses its 4-byte alignment, and the
// compiler would take a 4-byte aligned source as 16-byte aligned.
#define ZS_GLOBAL __attribute__((address_space(1)))
typedef ZS_GLOBAL const u32x4 g_u32x4;        // 16-byte aligned source vector
typedef ZS_GLOBAL const u32x4_a4 g_u32x4_a4;  // 4-byte aligned source vector
typedef ZS_GLOBAL const uint32_t g_u32;
typedef ZS_GLOBAL const uint16_t g_u16;
template <int A>
struct SrcVec;
template <>
struct SrcVec<16> {
    typedef g_u32x4 T;
};
template <>
struct SrcVec<4> {
    typedef g_u32x4_a4 T;
};

constexpr int kThreads = 256;
// Pack and re-shard work items are 8 KiB of destination: 512 aligned 16-byte
// vectors, two per lane of a 256-thread workgroup, both loads in flight
// before the stores (kUnroll). Measured on a 70B block unit, one launch over
// every shard: 8 KiB items 5.9 (pack) and 6.0-6.2 TB/s (re-shard); 16 KiB
// 5.7 / 5.6-6.2; 4 KiB 4.2-4.7 / 5.2 (the item's table search and index
// arithmetic are no longer hidden); 64 KiB items launched per shard 5.4.
// (kItemBytes is in zs_grid.h, with the rest of the launch geometry.)
static_assert(kThreads == kBlockThreads, "grid arithmetic assumes 256-thread workgroups");
constexpr int kUnroll = 2;  // vectors a lane has in flight in copy_run

template <int ES>
constexpr int64_t kItem = kItemBytes / ES;  // elements per pack / re-shard work item

template <int ES>
struct Elem;
template <>
struct Elem<2> {
    using T = uint16_t;
    typedef g_u16 G;
};
template <>
struct Elem<4> {
    using T = uint32_t;
    typedef g_u32 G;
};

// Body vectors i = tid, tid + nthr, ... < body from 16-byte source vectors
// at address sa, aligned to A (16 or 4) bytes, to 16-byte aligned destination
// vectors, kUnroll loads in flight per lane before their stores.
template <int A>
__device__ __forceinline__ void copy_vecs(u32x4* __restrict__ db, uintptr_t sa, int64_t body,
                                          int64_t tid, int64_t nthr) {
    typedef typename SrcVec<A>::T V;
    const V* __restrict__ s4 = reinterpret_cast<const V*>(sa);
    int64_t i = tid;
    for (; i + (kUnroll - 1) * nthr < body; i += kUnroll * nthr) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x[u] = __builtin_nontemporal_load(s4 + i + u * nthr);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(x[u], db + i + u * nthr);
    }
    for (; i < body; i += nthr)
        __builtin_nontemporal_store(u32x4(__builtin_nontemporal_load(s4 + i)), db + i);
}

// bf16 at an odd element offset: destination vector i is source bytes
// [16 i + 4 W + 2, +16) of the aligned source a4, i.e. the words of the
// aligned vectors a4[i] and a4[i + 1] shifted down by W words and 2 bytes.
// Lane l of a wavefront covers vector i = i0 + l and loads a4[i] only;
// a4[i + 1] is the next lane's load, fetched across lanes (ds_bpermute),
// except for the wavefront's last lane, which loads it itself (the run's
// last vector i = body - 1 takes it from the lane that loads a4[body], which
// holds the run's last bytes). Every lane runs the same trip count (i0 is
// the same for the whole wavefront); tid % 64 is the lane and nthr a
// multiple of 64. On MI355X this replaced eight 2-byte loads per vector
// (re-shard of the ragged 10,000-tensor unit in bf16, 16 -> 12 shards:
// 6.10-6.13 -> 6.26-6.33 TB/s, same process and buffers); two aligned loads
// per lane instead of the cross-lane fetch ran 3-6% slower, and the same
// shift for dword-aligned sources (in place of one unaligned dwordx4 load)
// 5-8% slower.
template <int W>
__device__ __forceinline__ void copy_vecs_odd(u32x4* __restrict__ db,
                                              const g_u32x4* __restrict__ a4, int64_t body,
                                              int64_t tid, int64_t nthr) {
    const int lane = int(tid & 63);
    for (int64_t i0 = tid - lane; i0 < body; i0 += kUnroll * nthr) {
        // every load of the iteration goes out at once, the last lane's
        // extra vector with them (issued after the cross-lane fetch, it came
        // when the neighbouring wavefront's non-temporal load of the same
        // line had left L2 already: 5% more HBM reads)
        u32x4 lo[kUnroll], hi[kUnroll], own[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = i0 + u * nthr + lane;
            lo[u] = i <= body ? __builtin_nontemporal_load(a4 + i) : u32x4{0u, 0u, 0u, 0u};
            own[u] = (lane == 63 && i < body) ? __builtin_nontemporal_load(a4 + i + 1)
                                             : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                hi[u][k] = uint32_t(
                    __builtin_amdgcn_ds_bpermute(((lane + 1) & 63) << 2, int(lo[u][k])));
            if (lane == 63) hi[u] = own[u];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = i0 + u * nthr + lane;
            if (i < body) {
                const uint32_t x[8] = {lo[u][0], lo[u][1], lo[u][2], lo[u][3],
                                       hi[u][0], hi[u][1], hi[u][2], hi[u][3]};
                u32x4 out;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    out[k] = __builtin_amdgcn_alignbyte(x[k + W + 1], x[k + W], 2);
                __builtin_nontemporal_store(out, db + i);
            }
        }
    }
}

// Copy n elements of ES bytes from src to dst. The calling threads are
// numbered tid in [0, nthr), nthr a multiple of 64 with tid % 64 the lane in
// the wavefront; each element is written by exactly one of them.
template <int ES>
__device__ __forceinline__ void copy_run(char* dst, const char* src, int64_t n, int64_t tid,
                                         int64_t nthr) {
    using T = typename Elem<ES>::T;
    typedef typename Elem<ES>::G G;
    constexpr int V = 16 / ES;
    int64_t head = int64_t((16 - (reinterpret_cast<uintptr_t>(dst) & 15)) & 15) / ES;
    if (head > n) head = n;
    const int64_t body = (n - head) / V;
    const int64_t tail = n - head - body * V;
    const G* gs = reinterpret_cast<const G*>(reinterpret_cast<uintptr_t>(src));
    if (tid < head) {
        reinterpret_cast<T*>(dst)[tid] = gs[tid];
    } else if (tid - head < tail) {
        const int64_t e = head + body * V + (tid - head);
        reinterpret_cast<T*>(dst)[e] = gs[e];
    }
    if (body <= 0) return;
    u32x4* db = reinterpret_cast<u32x4*>(dst + head * ES);
    const uintptr_t sa = reinterpret_cast<uintptr_t>(src + head * ES);
    if ((sa & 15) == 0) {
        copy_vecs<16>(db, sa, body, tid, nthr);
    } else if ((sa & 3) == 0) {
        // a dword-aligned source still loads as one dwordx4 per vector
        copy_vecs<4>(db, sa, body, tid, nthr);
    } else {  // 2-byte elements at an odd element offset
        const g_u32x4* a4 = reinterpret_cast<const g_u32x4*>(sa & ~uintptr_t(15));
        switch ((sa & 15) >> 2) {  // the same for every lane of the run
            case 0: copy_vecs_odd<0>(db, a4, body, tid, nthr); break;
            case 1: copy_vecs_odd<1>(db, a4, body, tid, nthr); break;
            case 2: copy_vecs_odd<2>(db, a4, body, tid, nthr); break;
            default: copy_vecs_odd<3>(db, a4, body, tid, nthr); break;
        }
    }
}

// Pack: work item q covers flat[lo, hi) inside shard r = q / per_shard. The
// block finds the first tensor ending after lo (binary search on the table:
// its probes are the same for every lane, so they are scalar loads, mostly
// hits in the scalar cache; a search in which a wavefront's 64 lanes test 64
// entries per round took the ragged 10,000-tensor pack from 5.7 to 6.4 ms),
// copies each tensor piece overlapping [lo, hi), then zero-fills [N, hi).
template <int ES>
__global__ __launch_bounds__(kThreads) void pack_kernel(const zs_tensor_ref* __restrict__ table,
                                                        int T, int64_t N, PtrPack shards,
                                                        int64_t S, int64_t per_shard,
                                                        int64_t q0, int64_t q1) {
    using Tv = typename Elem<ES>::T;
    for (int64_t q = q0 + blockIdx.x; q < q1; q += gridDim.x) {
        const int64_t r = q / per_shard;
        const int64_t base = r * S;
        const int64_t lo = base + (q - r * per_shard) * kItem<ES>;
        const int64_t hi = lo + kItem<ES> < base + S ? lo + kItem<ES> : base + S;
        char* shard = static_cast<char*>(const_cast<void*>(shards.p[r]));
        // smallest j with flat_offset_j + numel_j > lo
        int a = 0, b = T;
        while (a < b) {
            const int mid = (a + b) >> 1;
            if (table[mid].flat_offset + table[mid].numel > lo) b = mid;
            else a = mid + 1;
        }
        for (int j = a; j < T; ++j) {
            const int64_t off = table[j].flat_offset;
            if (off >= hi) break;
            const int64_t s0 = off > lo ? off : lo;
            const int64_t end = off + table[j].numel;
            const int64_t s1 = end < hi ? end : hi;
            if (s1 > s0) {
                copy_run<ES>(shard + (s0 - base) * ES,
                             static_cast<const char*>(table[j].ptr) + (s0 - off) * ES, s1 - s0,
                             threadIdx.x, kThreads);
            }
        }
        if (hi > N) {
            const int64_t z0 = N > lo ? N : lo;
            for (int64_t e = z0 + threadIdx.x; e < hi; e += kThreads)
                reinterpret_cast<Tv*>(shard)[e - base] = Tv(0);
        }
    }
}

// Gather, general case (a shard, or a slot of the unit buffer, not 16-byte
// aligned): one launch per shard, in shard order, the grid copying src[0, n)
// to dst[0, n). When everything is aligned, gather_flat_kernel moves the
// whole unit in one launch whose grid covers it, lane v on destination
// vector v: on the 70B units 6.56 TB/s, against 6.22 for one launch per
// shard (eight short launches, each with its own start and drain), 5.44-5.46
// for a single persistent launch walking the shards in order (whose
// wavefronts drift apart) and 5.43 for one persistent launch giving each
// shard its own slice of the grid.
template <int ES>
__global__ __launch_bounds__(kThreads) void copy_kernel(const char* __restrict__ src, int64_t n,
                                                        char* __restrict__ dst) {
    const int64_t tid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t nthr = int64_t(gridDim.x) * kThreads;
    copy_run<ES>(dst, src, n, tid, nthr);
}

// Gather in one launch when every shard and slot is 16-byte aligned: lane v
// of the grid moves destination vector v, which lies in slot r = v / nv
// (nv vectors per shard); shards marked in place are left alone.
__global__ __launch_bounds__(kThreads) void gather_flat_kernel(PtrPack shards, int64_t nv,
                                                               int64_t total,
                                                               u32x4* __restrict__ flat,
                                                               uint64_t in_place) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t v = int64_t(blockIdx.x) * kThreads + threadIdx.x; v < total; v += stride) {
        const int64_t r = v / nv;
        if ((in_place >> r) & 1) continue;
        const u32x4* src = static_cast<const u32x4*>(shards.p[r]);
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + (v - r * nv)), flat + v);
    }
}

// Re-shard: work item q covers new-flat [lo, hi) inside new shard r2 =
// q / per_shard. Flat position i < N comes from old shard i / S at i % S;
// positions at or past N are the new pad and get +0.
template <int ES>
__global__ __launch_bounds__(kThreads) void reshard_kernel(PtrPack src, int64_t S, PtrPack dst,
                                                           int64_t S2, int64_t N,
                                                           int64_t per_shard, int64_t q0,
                                                           int64_t q1) {
    using Tv = typename Elem<ES>::T;
    for (int64_t q = q0 + blockIdx.x; q < q1; q += gridDim.x) {
        const int64_t r2 = q / per_shard;
        const int64_t base2 = r2 * S2;
        const int64_t lo = base2 + (q - r2 * per_shard) * kItem<ES>;
        const int64_t hi = lo + kItem<ES> < base2 + S2 ? lo + kItem<ES> : base2 + S2;
        char* d = static_cast<char*>(const_cast<void*>(dst.p[r2]));
        const int64_t real_end = hi < N ? hi : N;
        for (int64_t i = lo; i < real_end;) {
            const int64_t r = i / S;
            const int64_t piece_end = (r + 1) * S < real_end ? (r + 1) * S : real_end;
            copy_run<ES>(d + (i - base2) * ES, static_cast<const char*>(src.p[r]) + (i - r * S) * ES,
                         piece_end - i, threadIdx.x, kThreads);
            i = piece_end;
        }
        const int64_t z0 = N > lo ? N : lo;
        for (int64_t e = z0 + threadIdx.x; e < hi; e += kThreads)
            reinterpret_cast<Tv*>(d)[e - base2] = Tv(0);
    }
}

}  // namespace

namespace {

template <int ES>
hipError_t reshard_es(const PtrPack& src, int64_t S, const PtrPack& dst, int D2, int64_t S2,
                      int64_t N, hipStream_t stream) {
    const int64_t per_shard = items_per_shard(S2, ES);
    const int64_t items = per_shard * D2;
    const int64_t blocks = item_grid(S2, ES, D2);
    hipLaunchKernelGGL((reshard_kernel<ES>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       src, S, dst, S2, N, per_shard, int64_t(0), items);
    return hipGetLastError();
}

template <int ES>
hipError_t pack_es(const zs_tensor_ref* d_table, int T, int64_t N, int D, const PtrPack& shards,
                   int64_t S, hipStream_t stream) {
    const int64_t per_shard = items_per_shard(S, ES);
    const int64_t items = per_shard * D;
    const int64_t blocks = item_grid(S, ES, D);
    hipLaunchKernelGGL((pack_kernel<ES>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       d_table, T, N, shards, S, per_shard, int64_t(0), items);
    return hipGetLastError();
}

}  // namespace

// Pack and re-shard: one launch over every destination shard, one workgroup
// per work item (the items of shard r are [r * per_shard, (r + 1) *
// per_shard)), so that, as in the gather, there is no start and drain per
// shard.
hipError_t launch_reshard(const PtrPack& src, int64_t S, const PtrPack& dst, int D2, int64_t S2,
                          int64_t N, int es, hipStream_t stream) {
    return es == 2 ? reshard_es<2>(src, S, dst, D2, S2, N, stream)
                   : reshard_es<4>(src, S, dst, D2, S2, N, stream);
}

hipError_t launch_pack(const zs_tensor_ref* d_table, int T, int64_t N, int es, int D,
                       const PtrPack& shards, int64_t S, hipStream_t stream) {
    return es == 2 ? pack_es<2>(d_table, T, N, D, shards, S, stream)
                   : pack_es<4>(d_table, T, N, D, shards, S, stream);
}

hipError_t launch_gather(const PtrPack& shards, int D, int64_t S, int es, void* flat,
                         uint64_t in_place, hipStream_t stream) {
    bool aligned = (reinterpret_cast<uintptr_t>(flat) & 15) == 0 && (S * es) % 16 == 0;
    for (int r = 0; r < D && aligned; ++r)
        aligned = (reinterpret_cast<uintptr_t>(shards.p[r]) & 15) == 0;
    if (aligned) {
        const int64_t nv = S * es / 16, total = nv * D;
        const int64_t blocks = gather_flat_grid(total);
        hipLaunchKernelGGL(gather_flat_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                           shards, nv, total, reinterpret_cast<u32x4*>(flat), in_place);
        return hipGetLastError();
    }
    const int64_t blocks = gather_copy_grid(S, es);
    char* f = static_cast<char*>(flat);
    for (int r = 0; r < D; ++r) {
        if ((in_place >> r) & 1) continue;
        const char* src = static_cast<const char*>(shards.p[r]);
        char* dst = f + int64_t(r) * S * es;
        if (es == 2)
            hipLaunchKernelGGL((copy_kernel<2>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                               src, S, dst);
        else
            hipLaunchKernelGGL((copy_kernel<4>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                               src, S, dst);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace zs
