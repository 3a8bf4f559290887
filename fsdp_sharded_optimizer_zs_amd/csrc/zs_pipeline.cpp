// Per-bucket streamed shard step: the arrival of bucket b+1's gradient
// contributions overlaps the fused reduce + AdamW kernel on bucket b.
//
// FSDP prefetches: it issues the collective for the next layer while the
// current one computes, so that communication hides behind compute. On one
// GPU the reduce-scatter's transfer is stood in for by copies from wherever
// the contributions live (pinned host memory over PCIe, or device memory)
// into one of two device staging slots; the fused step kernel of the same
// bucket waits for its slot, and the copies of bucket b+2 wait until the
// step of bucket b has released the slot. Two streams and five events order
// it all; nothing is synchronized on the host and no device memory is
// allocated. The arithmetic is the fused step's, unchanged.

#include <algorithm>
#include <vector>

#include "zs_internal.h"

#define ZS_EXPORT extern "C" __attribute__((visibility("default")))

using namespace zs;

namespace {

struct Events {
    hipEvent_t start = nullptr;
    hipEvent_t arrived[2] = {nullptr, nullptr};
    hipEvent_t consumed[2] = {nullptr, nullptr};
    ~Events() {
        // Destroying an event whose work is still pending is allowed; the
        // runtime releases it once that work completes.
        for (hipEvent_t e : {start, arrived[0], arrived[1], consumed[0], consumed[1]})
            if (e) (void)hipEventDestroy(e);
    }
    hipError_t create() {
        for (hipEvent_t* e : {&start, &arrived[0], &arrived[1], &consumed[0], &consumed[1]}) {
            const hipError_t r = hipEventCreateWithFlags(e, hipEventDisableTiming);
            if (r != hipSuccess) return r;
        }
        return hipSuccess;
    }
};

struct Tagged {
    Range r;
    int bucket;
    const char* what;
};

}  // namespace

ZS_EXPORT zs_status zs_step_pipelined(const zs_bucket* buckets, int32_t n_buckets,
                                      int32_t n_contrib, int32_t dtype, void* staging0,
                                      void* staging1, int64_t staging_len,
                                      const zs_adamw_hp* hp, hipStream_t compute,
                                      hipStream_t transfer) {
    const char* who = "zs_step_pipelined";
    const int es = elem_size(dtype);
    if (es == 0) return fail(ZS_EUNSUPPORTED, "%s: unknown dtype %d", who, dtype);
    if (n_buckets < 0) return fail(ZS_EINVAL, "%s: n_buckets = %d < 0", who, n_buckets);
    if (n_contrib < 1 || n_contrib > ZS_MAX_D)
        return fail(ZS_EINVAL, "%s: n_contrib = %d outside 1..%d", who, n_contrib, ZS_MAX_D);
    zs_status st = check_hp(hp, who);
    if (st != ZS_OK) return st;
    if (n_buckets == 0) return ok();
    if (buckets == nullptr) return fail(ZS_EINVAL, "%s: buckets is NULL", who);
    if (!size_ok(staging_len, es) || staging_len > INT64_MAX / 16 / n_contrib / es)
        return fail(ZS_EINVAL, "%s: staging_len = %lld out of range", who, (long long)staging_len);
    if (!staging0 || !staging1) return fail(ZS_EINVAL, "%s: a staging slot is NULL", who);
    if (!aligned(staging0, uintptr_t(es)) || !aligned(staging1, uintptr_t(es)))
        return fail(ZS_EINVAL, "%s: a staging slot is not aligned to %d bytes", who, es);

    // Every output range (p, m, v, w of every bucket, both staging slots)
    // must be disjoint from every other, and no source may overlap one.
    std::vector<Tagged> outs;
    outs.reserve(size_t(n_buckets) * 4 + 2);
    const int64_t slot_elems = staging_len * n_contrib;
    if (slot_elems > 0) {
        outs.push_back({range_of(staging0, slot_elems, es), -1, "staging slot 0"});
        outs.push_back({range_of(staging1, slot_elems, es), -1, "staging slot 1"});
    }
    for (int32_t b = 0; b < n_buckets; ++b) {
        const zs_bucket& k = buckets[b];
        if (!size_ok(k.S, 4)) return fail(ZS_EINVAL, "%s: bucket %d S = %lld out of range", who, b, (long long)k.S);
        if (k.S > staging_len)
            return fail(ZS_EINVAL, "%s: bucket %d S = %lld exceeds staging_len = %lld", who, b,
                        (long long)k.S, (long long)staging_len);
        if (k.S == 0) continue;
        if (!k.p || !k.m || !k.v || !k.w_out)
            return fail(ZS_EINVAL, "%s: bucket %d p, m, v or w_out is NULL", who, b);
        if (!aligned(k.p, 4) || !aligned(k.m, 4) || !aligned(k.v, 4) || !aligned(k.w_out, 2))
            return fail(ZS_EINVAL, "%s: bucket %d p, m, v or w_out misaligned", who, b);
        PtrPack src;
        st = take_ptrs(k.sources, n_contrib, es, "zs_step_pipelined: bucket sources", &src);
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

    const AdamConsts kc = adam_consts(*hp, n_contrib);
    Events ev;
    hipError_t e = ev.create();
    if (e != hipSuccess) return hip_status(e, "zs_step_pipelined: event creation");
    // The copies start after everything already enqueued on the compute
    // stream: a previous call's steps may still read the staging slots, and
    // the caller may produce the sources there.
    if ((e = hipEventRecord(ev.start, compute)) != hipSuccess ||
        (e = hipStreamWaitEvent(transfer, ev.start, 0)) != hipSuccess)
        return hip_status(e, "zs_step_pipelined: stream ordering");
    char* slot[2] = {static_cast<char*>(staging0), static_cast<char*>(staging1)};
    const size_t stride = size_t(staging_len) * size_t(es);
    int64_t used = 0;  // non-empty buckets enqueued so far; they alternate slots
    for (int32_t b = 0; b < n_buckets; ++b) {
        const zs_bucket& k = buckets[b];
        if (k.S == 0) continue;
        const int s = int(used & 1);
        // transfer: wait until the step two buckets back released this slot
        if (used >= 2 && (e = hipStreamWaitEvent(transfer, ev.consumed[s], 0)) != hipSuccess)
            return hip_status(e, "zs_step_pipelined: transfer wait");
        PtrPack staged;
        for (int i = 0; i < ZS_MAX_D; ++i) staged.p[i] = nullptr;
        bool al = aligned(k.p, 16) && aligned(k.m, 16) && aligned(k.v, 16) && aligned(k.w_out, 16);
        for (int q = 0; q < n_contrib; ++q) {
            char* dst = slot[s] + size_t(q) * stride;
            e = hipMemcpyAsync(dst, k.sources[q], size_t(k.S) * size_t(es), hipMemcpyDefault,
                               transfer);
            if (e != hipSuccess) return hip_status(e, "zs_step_pipelined: contribution copy");
            staged.p[q] = dst;
            al = al && aligned(dst, 16);
        }
        if ((e = hipEventRecord(ev.arrived[s], transfer)) != hipSuccess)
            return hip_status(e, "zs_step_pipelined: event record");
        // compute: wait for this bucket's contributions, step, release the slot
        if ((e = hipStreamWaitEvent(compute, ev.arrived[s], 0)) != hipSuccess)
            return hip_status(e, "zs_step_pipelined: compute wait");
        e = launch_adamw(k.p, k.m, k.v, k.w_out, k.S, staged, n_contrib, 1, false, dtype, kc, al,
                         compute);
        if (e != hipSuccess) return hip_status(e, "zs_step_pipelined: step launch");
        if ((e = hipEventRecord(ev.consumed[s], compute)) != hipSuccess)
            return hip_status(e, "zs_step_pipelined: event record");
        ++used;
    }
    return ok();
}
