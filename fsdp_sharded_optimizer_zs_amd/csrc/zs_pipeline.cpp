// Per-bucket streamed shard step: the arrival of bucket b+1's gradient
// contributions overlaps the fused reduce + AdamW kernel on bucket b.
//
// FSDP prefetches: it issues the collective for the next layer while the
// current one computes, so that communication hides behind compute. On one
// GPU the reduce-scatter's transfer is stood in for by copies from wherever
// the contributions live (pinned host memory over PCIe, or device memory)
// into one of two device staging slots; the fused step kernel of the same
// bucket waits for its slot, and the copies of bucket b+2 wait until the
// step of bucket b has released the slot. Two streams and five pooled events
// order it all; nothing is synchronized on the host, no device memory is
// allocated and no runtime object is created once the pool holds five
// events. The arithmetic is the fused step's, unchanged.

#include <algorithm>
#include <string>
#include <vector>

#include "zs_internal.h"

#define ZS_EXPORT extern "C" __attribute__((visibility("default")))

using namespace zs;

namespace {

struct Tagged {
    Range r;
    int bucket;
    const char* what;
};

}  // namespace

namespace zs {

zs_status pipelined_check(const char* who, const zs_bucket* buckets, int32_t n_buckets,
                          int32_t n_contrib, int32_t dtype, const void* staging0,
                          const void* staging1, int64_t slot_elems, int64_t max_bucket,
                          const zs_adamw_hp* hp) {
    const int es = elem_size(dtype);
    if (es == 0) return fail(ZS_EUNSUPPORTED, "%s: unknown dtype %d", who, dtype);
    if (n_buckets < 0) return fail(ZS_EINVAL, "%s: n_buckets = %d < 0", who, n_buckets);
    if (n_contrib < 1 || n_contrib > ZS_MAX_D)
        return fail(ZS_EINVAL, "%s: n_contrib = %d outside 1..%d", who, n_contrib, ZS_MAX_D);
    zs_status st = check_hp(hp, who);
    if (st != ZS_OK) return st;
    if (n_buckets == 0) return ZS_OK;
    if (buckets == nullptr) return fail(ZS_EINVAL, "%s: buckets is NULL", who);

    // Every output range (p, m, v, w of every bucket, both staging slots)
    // must be disjoint from every other, and no source may overlap one.
    std::vector<Tagged> outs;
    outs.reserve(size_t(n_buckets) * 4 + 2);
    if (slot_elems > 0) {
        outs.push_back({range_of(staging0, slot_elems, es), -1, "staging slot 0"});
        outs.push_back({range_of(staging1, slot_elems, es), -1, "staging slot 1"});
    }
    for (int32_t b = 0; b < n_buckets; ++b) {
        const zs_bucket& k = buckets[b];
        if (!size_ok(k.S, 4)) return fail(ZS_EINVAL, "%s: bucket %d S = %lld out of range", who, b, (long long)k.S);
        if (k.S > max_bucket)
            return fail(ZS_EINVAL, "%s: bucket %d S = %lld exceeds staging_len = %lld", who, b,
                        (long long)k.S, (long long)max_bucket);
        if (k.S == 0) continue;
        if (!k.p || !k.m || !k.v || !k.w_out)
            return fail(ZS_EINVAL, "%s: bucket %d p, m, v or w_out is NULL", who, b);
        if (!aligned(k.p, 4) || !aligned(k.m, 4) || !aligned(k.v, 4) || !aligned(k.w_out, 2))
            return fail(ZS_EINVAL, "%s: bucket %d p, m, v or w_out misaligned", who, b);
        PtrPack src;
        st = take_ptrs(k.sources, n_contrib, es, (std::string(who) + ": bucket sources").c_str(),
                       &src);
        if (st != ZS_OK) return st;
        outs.push_back({range_of(k.p, k.S, 4), b, "p"});
        outs.push_back({range_of(k.m, k.S, 4), b, "m"});
        outs.push_back({range_of(k.v, k.S, 4), b, "v"});
        outs.push_back({range_of(k.w_out, k.S, 2), b, "w_out"});
    }
    std::vector<Tagged> sorted = outs;
    std::sort(sorted.begin(), sorted.end(),
              [](const Tagged& a, const Tagged& b) { return a.r.lo < b.r.lo; });
    for (size_t i = 1; i < sorted.size(); ++i)
        if (overlap(sorted[i - 1].r, sorted[i].r))
            return fail(ZS_EALIAS, "%s: %s (bucket %d) overlaps %s (bucket %d)", who,
                        sorted[i - 1].what, sorted[i - 1].bucket, sorted[i].what, sorted[i].bucket);
    for (int32_t b = 0; b < n_buckets; ++b) {
        const zs_bucket& k = buckets[b];
        if (k.S == 0) continue;
        for (int q = 0; q < n_contrib; ++q) {
            const Range s = range_of(k.sources[q], k.S, es);
            // first output range starting at or after s.lo, and the one before it
            auto it = std::lower_bound(sorted.begin(), sorted.end(), s.lo,
                                       [](const Tagged& t, uintptr_t lo) { return t.r.lo < lo; });
            if ((it != sorted.end() && overlap(it->r, s)) ||
                (it != sorted.begin() && overlap((it - 1)->r, s)))
                return fail(ZS_EALIAS, "%s: bucket %d source %d overlaps an output buffer", who, b, q);
        }
    }
    return ZS_OK;
}

zs_status pipelined_enqueue(const char* who, const zs_bucket* buckets, int32_t n_buckets,
                            int32_t n_contrib, int32_t dtype, void* staging0, void* staging1,
                            int64_t piece, const zs_adamw_hp* hp, hipStream_t compute,
                            hipStream_t transfer, const hipEvent_t ev[5]) {
    const int es = elem_size(dtype);
    const AdamConsts kc = adam_consts(*hp, n_contrib);
    // events: 0 = start, 1 + s = slot s arrived, 3 + s = slot s consumed
    const hipEvent_t start = ev[0], arrived[2] = {ev[1], ev[2]}, consumed[2] = {ev[3], ev[4]};
    // The copies start after everything already enqueued on the compute
    // stream: a previous call's steps may still read the staging slots, and
    // the caller may produce the sources there.
    hipError_t e;
    if ((e = hipEventRecord(start, compute)) != hipSuccess ||
        (e = hipStreamWaitEvent(transfer, start, 0)) != hipSuccess)
        return hip_status(e, "stream ordering");
    char* slot[2] = {static_cast<char*>(staging0), static_cast<char*>(staging1)};
    const size_t stride = size_t(piece) * size_t(es);
    int64_t used = 0;  // pieces enqueued so far; they alternate slots
    for (int32_t b = 0; b < n_buckets; ++b) {
        const zs_bucket& k = buckets[b];
        // a bucket goes in pieces of at most `piece` elements (one piece when
        // the staging slots hold whole buckets); pieces start at multiples of
        // `piece` from the bucket's start, so they keep its alignment
        for (int64_t off = 0; off < k.S; off += piece) {
            const int64_t n = std::min(piece, k.S - off);
            const int s = int(used & 1);
            // transfer: wait until the step two pieces back released this slot
            if (used >= 2 && (e = hipStreamWaitEvent(transfer, consumed[s], 0)) != hipSuccess)
                return hip_status(e, "transfer wait");
            PtrPack staged;
            for (int i = 0; i < ZS_MAX_D; ++i) staged.p[i] = nullptr;
            float* p = k.p + off;
            float* m = k.m + off;
            float* v = k.v + off;
            uint16_t* w = k.w_out + off;
            bool al = aligned(p, 16) && aligned(m, 16) && aligned(v, 16) && aligned(w, 16);
            for (int q = 0; q < n_contrib; ++q) {
                char* dst = slot[s] + size_t(q) * stride;
                e = hipMemcpyAsync(dst, static_cast<const char*>(k.sources[q]) + off * es,
                                   size_t(n) * size_t(es), hipMemcpyDefault, transfer);
                if (e != hipSuccess) return hip_status(e, "contribution copy");
                staged.p[q] = dst;
                al = al && aligned(dst, 16);
            }
            if ((e = hipEventRecord(arrived[s], transfer)) != hipSuccess)
                return hip_status(e, "event record");
            // compute: wait for this piece's contributions, step, release the slot
            if ((e = hipStreamWaitEvent(compute, arrived[s], 0)) != hipSuccess)
                return hip_status(e, "compute wait");
            e = launch_adamw(p, m, v, w, n, staged, n_contrib, 1, false, dtype, kc, al, compute);
            if (e != hipSuccess) return hip_status(e, "step launch");
            if ((e = hipEventRecord(consumed[s], compute)) != hipSuccess)
                return hip_status(e, "event record");
            ++used;
        }
    }
    (void)who;
    return ok();
}

}  // namespace zs

ZS_EXPORT zs_status zs_step_pipelined(const zs_bucket* buckets, int32_t n_buckets,
                                      int32_t n_contrib, int32_t dtype, void* staging0,
                                      void* staging1, int64_t staging_len,
                                      const zs_adamw_hp* hp, hipStream_t compute,
                                      hipStream_t transfer) {
    const char* who = "zs_step_pipelined";
    const int es = elem_size(dtype);
    if (es == 0) return fail(ZS_EUNSUPPORTED, "%s: unknown dtype %d", who, dtype);
    if (n_contrib < 1 || n_contrib > ZS_MAX_D)
        return fail(ZS_EINVAL, "%s: n_contrib = %d outside 1..%d", who, n_contrib, ZS_MAX_D);
    if (n_buckets > 0) {
        if (!size_ok(staging_len, es) || staging_len > INT64_MAX / 16 / n_contrib / es)
            return fail(ZS_EINVAL, "%s: staging_len = %lld out of range", who, (long long)staging_len);
        if (!staging0 || !staging1) return fail(ZS_EINVAL, "%s: a staging slot is NULL", who);
        if (!aligned(staging0, uintptr_t(es)) || !aligned(staging1, uintptr_t(es)))
            return fail(ZS_EINVAL, "%s: a staging slot is not aligned to %d bytes", who, es);
    }
    zs_status st = pipelined_check(who, buckets, n_buckets, n_contrib, dtype, staging0, staging1,
                                   staging_len * n_contrib, staging_len, hp);
    if (st != ZS_OK || n_buckets == 0) return st == ZS_OK ? ok() : st;
    EventLease ev;
    hipError_t e = ev.take(5);
    if (e != hipSuccess) return hip_status(e, "zs_step_pipelined: events");
    const hipEvent_t evs[5] = {ev.ev(0), ev.ev(1), ev.ev(2), ev.ev(3), ev.ev(4)};
    // staging_len >= every bucket's S: each bucket is one piece
    st = pipelined_enqueue(who, buckets, n_buckets, n_contrib, dtype, staging0, staging1,
                           staging_len > 0 ? staging_len : 1, hp, compute, transfer, evs);
    if (st != ZS_OK) return fail(st, "zs_step_pipelined: %s", zs_last_error());
    return ok();
}
