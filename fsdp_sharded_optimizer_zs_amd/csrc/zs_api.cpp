// C-ABI entry points of libzs: host-side validation, layout arithmetic and
// the fp32 constants of the AdamW step, then one kernel launch on the
// caller's stream. Nothing here allocates device memory or synchronizes.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "zs_internal.h"

#define ZS_EXPORT extern "C" __attribute__((visibility("default")))

namespace zs {
namespace {
thread_local std::string g_last_error;
}  // namespace

zs_status fail(zs_status code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

zs_status ok() {
    g_last_error.clear();
    return ZS_OK;
}

zs_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(ZS_EHIP, "%s: HIP error %d (%s)", what, int(e), hipGetErrorString(e));
}

int elem_size(int32_t dtype) {
    if (dtype == ZS_BF16) return 2;
    if (dtype == ZS_F32) return 4;
    return 0;
}

Range range_of(const void* p, int64_t count, int es) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + uintptr_t(count) * uintptr_t(es)};
}

bool overlap(const Range& a, const Range& b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Elements S with S * es bytes representable (and addressable) on the host.
bool size_ok(int64_t S, int es) { return S >= 0 && S <= (INT64_MAX / 16) / es; }

// Fill a PtrPack from a host array of n device pointers, checking each.
zs_status take_ptrs(const void* const* src, int n, int es, const char* what, PtrPack* out) {
    if (src == nullptr) return fail(ZS_EINVAL, "%s: pointer array is NULL", what);
    for (int i = 0; i < ZS_MAX_D; ++i) out->p[i] = nullptr;
    for (int i = 0; i < n; ++i) {
        if (src[i] == nullptr) return fail(ZS_EINVAL, "%s[%d] is NULL", what, i);
        if (!aligned(src[i], uintptr_t(es)))
            return fail(ZS_EINVAL, "%s[%d] is not aligned to its %d-byte elements", what, i, es);
        out->p[i] = src[i];
    }
    return ZS_OK;
}

zs_status check_hp(const zs_adamw_hp* hp, const char* who) {
    if (hp == nullptr) return fail(ZS_EINVAL, "%s: hp is NULL", who);
    if (hp->step < 1) return fail(ZS_EINVAL, "%s: step = %lld < 1", who, (long long)hp->step);
    if (!(std::isfinite(hp->lr) && hp->lr >= 0.0))
        return fail(ZS_EINVAL, "%s: lr must be finite and >= 0", who);
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
        return fail(ZS_EINVAL, "%s: betas must lie in [0, 1)", who);
    if (!(std::isfinite(hp->eps) && hp->eps >= 0.0))
        return fail(ZS_EINVAL, "%s: eps must be finite and >= 0", who);
    if (!(std::isfinite(hp->weight_decay) && hp->weight_decay >= 0.0))
        return fail(ZS_EINVAL, "%s: weight_decay must be finite and >= 0", who);
    return ZS_OK;
}

AdamConsts adam_consts(const zs_adamw_hp& hp, int n_contrib) {
    // Double arithmetic, each constant rounded to fp32 once. beta^t is t
    // successive multiplications from 1.0. A training run asks for t, t + 1,
    // ... with the same betas, and every bucket of a step for the same t, so
    // the powers this thread computed last are kept and advanced from (the
    // same products, at O(1) per call instead of O(t)); a change of betas or
    // an earlier t starts again from 1.0.
    struct Powers {
        double beta1, beta2;
        int64_t t;  // b1t = beta1^t, b2t = beta2^t
        double b1t, b2t;
    };
    thread_local Powers pw{-1.0, -1.0, 0, 1.0, 1.0};
    if (pw.beta1 != hp.beta1 || pw.beta2 != hp.beta2 || pw.t > hp.step)
        pw = Powers{hp.beta1, hp.beta2, 0, 1.0, 1.0};
    // Below 2^-54, 1 - b rounds to exactly 1.0 in double, so more factors
    // cannot change any constant derived from b1t or b2t: stop there.
    while (pw.t < hp.step && !(pw.b1t < 0x1p-54 && pw.b2t < 0x1p-54)) {
        pw.b1t = pw.b1t * hp.beta1;
        pw.b2t = pw.b2t * hp.beta2;
        ++pw.t;
    }
    const double b1t = pw.b1t, b2t = pw.b2t;
    AdamConsts k;
    k.dec = float(1.0 - hp.lr * hp.weight_decay);
    k.b1 = float(hp.beta1);
    k.b1c = float(1.0 - hp.beta1);
    k.b2 = float(hp.beta2);
    k.b2c = float(1.0 - hp.beta2);
    k.ss = float(hp.lr / (1.0 - b1t));
    k.bc2s = float(std::sqrt(1.0 - b2t));
    k.eps = float(hp.eps);
    k.inv_n = float(1.0 / double(n_contrib));
    k.keep_w = 0;
    return k;
}

const DeviceInfo& device_info() {
    static std::mutex mu;
    static std::vector<DeviceInfo> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cache.size() <= size_t(dev)) cache.resize(size_t(dev) + 1, DeviceInfo{0});
    DeviceInfo& d = cache[size_t(dev)];
    if (d.cu_count == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cu <= 0)
            cu = 256;
        d.cu_count = cu;
    }
    return d;
}

namespace {
std::mutex g_event_mu;
std::vector<std::vector<hipEvent_t>> g_event_pool;  // per device: events not leased
}  // namespace

hipError_t EventLease::take(int n) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    dev_ = dev;
    {
        std::lock_guard<std::mutex> lock(g_event_mu);
        if (g_event_pool.size() <= size_t(dev)) g_event_pool.resize(size_t(dev) + 1);
        std::vector<hipEvent_t>& pool = g_event_pool[size_t(dev)];
        while (int(ev_.size()) < n && !pool.empty()) {
            ev_.push_back(pool.back());
            pool.pop_back();
        }
    }
    while (int(ev_.size()) < n) {
        hipEvent_t x = nullptr;
        if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess) return e;
        ev_.push_back(x);
    }
    return hipSuccess;
}

EventLease::~EventLease() {
    if (ev_.empty()) return;
    std::lock_guard<std::mutex> lock(g_event_mu);
    std::vector<hipEvent_t>& pool = g_event_pool[size_t(dev_)];
    pool.insert(pool.end(), ev_.begin(), ev_.end());
}

}  // namespace zs

using namespace zs;

ZS_EXPORT const char* zs_last_error(void) { return g_last_error.c_str(); }

ZS_EXPORT int32_t zs_abi_version(void) { return 201; }

ZS_EXPORT zs_status zs_unit_layout(const int64_t* numels, int32_t T, int32_t D,
                                   int64_t* offsets_out, int64_t* n_out, int64_t* n_pad_out,
                                   int64_t* shard_len_out) {
    if (T < 0) return fail(ZS_EINVAL, "zs_unit_layout: T = %d < 0", T);
    if (D < 1 || D > ZS_MAX_D)
        return fail(ZS_EINVAL, "zs_unit_layout: D = %d outside 1..%d", D, ZS_MAX_D);
    if (T > 0 && numels == nullptr) return fail(ZS_EINVAL, "zs_unit_layout: numels is NULL");
    if (!offsets_out || !n_out || !n_pad_out || !shard_len_out)
        return fail(ZS_EINVAL, "zs_unit_layout: an output pointer is NULL");
    int64_t off = 0;
    offsets_out[0] = 0;
    for (int32_t j = 0; j < T; ++j) {
        if (numels[j] < 0)
            return fail(ZS_EINVAL, "zs_unit_layout: numels[%d] = %lld < 0", j, (long long)numels[j]);
        if (numels[j] > INT64_MAX / 16 - off)
            return fail(ZS_EUNSUPPORTED, "zs_unit_layout: unit size overflows");
        off += numels[j];
        offsets_out[j + 1] = off;
    }
    const int64_t S = off / D + (off % D != 0 ? 1 : 0);
    *n_out = off;
    *shard_len_out = S;
    *n_pad_out = S * D;
    return ok();
}

ZS_EXPORT zs_status zs_pack_flat(const zs_tensor_ref* h_table, const zs_tensor_ref* d_table,
                                 int32_t T, int32_t dtype, int32_t D, void* const* shards,
                                 int64_t S, hipStream_t stream) {
    const int es = elem_size(dtype);
    if (es == 0) return fail(ZS_EUNSUPPORTED, "zs_pack_flat: unknown dtype %d", dtype);
    if (T < 0) return fail(ZS_EINVAL, "zs_pack_flat: T = %d < 0", T);
    if (D < 1 || D > ZS_MAX_D)
        return fail(ZS_EINVAL, "zs_pack_flat: D = %d outside 1..%d", D, ZS_MAX_D);
    if (!size_ok(S, es) || S > INT64_MAX / 16 / D)
        return fail(ZS_EINVAL, "zs_pack_flat: S = %lld out of range", (long long)S);
    if (T > 0 && (h_table == nullptr || d_table == nullptr))
        return fail(ZS_EINVAL, "zs_pack_flat: tensor table is NULL");
    int64_t N = 0;
    for (int32_t j = 0; j < T; ++j) {
        const zs_tensor_ref& t = h_table[j];
        if (t.numel < 0)
            return fail(ZS_EINVAL, "zs_pack_flat: tensor %d has numel %lld", j, (long long)t.numel);
        if (t.flat_offset != N)
            return fail(ZS_EINVAL, "zs_pack_flat: tensor %d flat_offset %lld, expected %lld", j,
                        (long long)t.flat_offset, (long long)N);
        if (t.numel > 0 && t.ptr == nullptr)
            return fail(ZS_EINVAL, "zs_pack_flat: tensor %d pointer is NULL", j);
        if (!aligned(t.ptr, uintptr_t(es)))
            return fail(ZS_EINVAL, "zs_pack_flat: tensor %d not aligned to %d bytes", j, es);
        if (t.numel > INT64_MAX / 16 - N) return fail(ZS_EUNSUPPORTED, "zs_pack_flat: N overflows");
        N += t.numel;
    }
    const int64_t want_S = N / D + (N % D != 0 ? 1 : 0);
    if (S != want_S)
        return fail(ZS_EINVAL, "zs_pack_flat: S = %lld but ceil(N/D) = %lld (N = %lld, D = %d)",
                    (long long)S, (long long)want_S, (long long)N, D);
    if (S == 0) return ok();
    PtrPack sp;
    zs_status st = take_ptrs(shards, D, es, "zs_pack_flat: shards", &sp);
    if (st != ZS_OK) return st;
    for (int r = 0; r < D; ++r) {
        const Range a = range_of(sp.p[r], S, es);
        for (int q = r + 1; q < D; ++q)
            if (overlap(a, range_of(sp.p[q], S, es)))
                return fail(ZS_EALIAS, "zs_pack_flat: shards %d and %d overlap", r, q);
        for (int32_t j = 0; j < T; ++j)
            if (overlap(a, range_of(h_table[j].ptr, h_table[j].numel, es)))
                return fail(ZS_EALIAS, "zs_pack_flat: shard %d overlaps tensor %d", r, j);
        if (overlap(a, range_of(d_table, T, int(sizeof(zs_tensor_ref)))))
            return fail(ZS_EALIAS, "zs_pack_flat: shard %d overlaps the device table", r);
    }
    return hip_status(launch_pack(d_table, T, N, es, D, sp, S, stream), "zs_pack_flat launch");
}

namespace {

// Validates a reduce description: nd contributions per group, R groups, and
// the fp32 multiplier of the reduced sum (1 / (R * nd) unless opts->scale is
// set).
zs_status check_groups(const char* who, int32_t nd, const zs_reduce_opts* opts, int* R,
                       bool* rnd, float* mult, int* keep_w) {
    *R = 1;
    *rnd = false;
    *keep_w = 0;
    double scale = 0.0;
    if (opts != nullptr) {
        if (opts->working_shard_hint != ZS_W_STREAM && opts->working_shard_hint != ZS_W_KEEP)
            return fail(ZS_EINVAL, "%s: working_shard_hint = %d is neither ZS_W_STREAM nor ZS_W_KEEP",
                        who, opts->working_shard_hint);
        if (opts->reserved != 0) return fail(ZS_EINVAL, "%s: reserved must be 0", who);
        *keep_w = opts->working_shard_hint == ZS_W_KEEP ? 1 : 0;
        if (opts->replicas < 1)
            return fail(ZS_EINVAL, "%s: replicas = %d < 1", who, opts->replicas);
        if (opts->round_to_reduce_dtype != 0 && opts->round_to_reduce_dtype != 1)
            return fail(ZS_EINVAL, "%s: round_to_reduce_dtype must be 0 or 1", who);
        if (!std::isfinite(opts->scale) || !std::isfinite(float(opts->scale)))
            return fail(ZS_EINVAL, "%s: scale must be finite (in fp32, once rounded)", who);
        *R = opts->replicas;
        *rnd = opts->round_to_reduce_dtype == 1;
        scale = opts->scale;
    }
    if (nd < 1 || nd > ZS_MAX_D)
        return fail(ZS_EINVAL, "%s: D = %d outside 1..%d", who, nd, ZS_MAX_D);
    if (int64_t(*R) * nd > ZS_MAX_D)
        return fail(ZS_EINVAL, "%s: replicas * D = %lld exceeds %d contributions", who,
                    (long long)(int64_t(*R) * nd), ZS_MAX_D);
    *mult = float(scale != 0.0 ? scale : 1.0 / double(int64_t(*R) * nd));
    return ZS_OK;
}

zs_status reduce_common(const char* who, const void* const* contribs, int32_t nd,
                        const zs_reduce_opts* opts, int32_t dtype, int64_t S, float* grad_out,
                        hipStream_t stream) {
    const int es = elem_size(dtype);
    if (es == 0) return fail(ZS_EUNSUPPORTED, "%s: unknown dtype %d", who, dtype);
    int R;
    bool rnd;
    float inv_n;
    int keep_w;  // no working shard here: the hint is ignored
    zs_status st = check_groups(who, nd, opts, &R, &rnd, &inv_n, &keep_w);
    if (st != ZS_OK) return st;
    if (!size_ok(S, 4)) return fail(ZS_EINVAL, "%s: S = %lld out of range", who, (long long)S);
    if (S == 0) return ok();
    if (grad_out == nullptr) return fail(ZS_EINVAL, "%s: grad_out is NULL", who);
    if (!aligned(grad_out, 4)) return fail(ZS_EINVAL, "%s: grad_out not 4-byte aligned", who);
    const int n = R * nd;
    PtrPack cp;
    st = take_ptrs(contribs, n, es, (std::string(who) + ": contribs").c_str(), &cp);
    if (st != ZS_OK) return st;
    const Range out = range_of(grad_out, S, 4);
    bool al = aligned(grad_out, 16);
    for (int k = 0; k < n; ++k) {
        if (overlap(out, range_of(cp.p[k], S, es)))
            return fail(ZS_EALIAS, "%s: grad_out overlaps contribution %d", who, k);
        al = al && aligned(cp.p[k], 16);
    }
    return hip_status(launch_reduce(cp, nd, R, rnd, dtype, S, inv_n, grad_out, al, stream), who);
}

zs_status adamw_common(const char* who, float* p, float* m, float* v, uint16_t* w_out, int64_t S,
                       const void* const* contribs, int32_t nd, const zs_reduce_opts* opts,
                       int32_t dtype, const zs_adamw_hp* hp, hipStream_t stream,
                       hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr) {
    const int es = elem_size(dtype);
    if (es == 0) return fail(ZS_EUNSUPPORTED, "%s: unknown dtype %d", who, dtype);
    int R;
    bool rnd;
    float inv_n;
    int keep_w;
    zs_status st = check_groups(who, nd, opts, &R, &rnd, &inv_n, &keep_w);
    if (st != ZS_OK) return st;
    if (!size_ok(S, 4)) return fail(ZS_EINVAL, "%s: S = %lld out of range", who, (long long)S);
    st = check_hp(hp, who);
    if (st != ZS_OK) return st;
    if (S == 0) return ok();
    if (!p || !m || !v || !w_out) return fail(ZS_EINVAL, "%s: p, m, v or w_out is NULL", who);
    if (!aligned(p, 4) || !aligned(m, 4) || !aligned(v, 4) || !aligned(w_out, 2))
        return fail(ZS_EINVAL, "%s: p, m, v or w_out misaligned for its element type", who);
    const int n = R * nd;
    PtrPack cp;
    st = take_ptrs(contribs, n, es, (std::string(who) + ": contribs").c_str(), &cp);
    if (st != ZS_OK) return st;
    const Range rs[4] = {range_of(p, S, 4), range_of(m, S, 4), range_of(v, S, 4),
                         range_of(w_out, S, 2)};
    const char* names[4] = {"p", "m", "v", "w_out"};
    for (int a = 0; a < 4; ++a)
        for (int b = a + 1; b < 4; ++b)
            if (overlap(rs[a], rs[b]))
                return fail(ZS_EALIAS, "%s: %s overlaps %s", who, names[a], names[b]);
    bool al = aligned(p, 16) && aligned(m, 16) && aligned(v, 16) && aligned(w_out, 16);
    for (int k = 0; k < n; ++k) {
        const Range c = range_of(cp.p[k], S, es);
        for (int a = 0; a < 4; ++a)
            if (overlap(c, rs[a]))
                return fail(ZS_EALIAS, "%s: contribution %d overlaps %s", who, k, names[a]);
        al = al && aligned(cp.p[k], 16);
    }
    AdamConsts k = adam_consts(*hp, n);
    k.inv_n = inv_n;
    k.keep_w = keep_w;
    return hip_status(
        launch_adamw(p, m, v, w_out, S, cp, nd, R, rnd, dtype, k, al, stream, ev_start, ev_stop),
        who);
}

}  // namespace

ZS_EXPORT zs_status zs_reduce_shard(const void* const* contribs, int32_t D, int32_t dtype,
                                    int64_t S, float* grad_out, hipStream_t stream) {
    return reduce_common("zs_reduce_shard", contribs, D, nullptr, dtype, S, grad_out, stream);
}

ZS_EXPORT zs_status zs_reduce_shard_ex(const void* const* contribs, int32_t D,
                                       const zs_reduce_opts* opts, int32_t dtype, int64_t S,
                                       float* grad_out, hipStream_t stream) {
    return reduce_common("zs_reduce_shard_ex", contribs, D, opts, dtype, S, grad_out, stream);
}

ZS_EXPORT zs_status zs_adamw_step(float* p, float* m, float* v, uint16_t* w_out, int64_t S,
                                  const void* const* contribs, int32_t n_contrib, int32_t dtype,
                                  const zs_adamw_hp* hp, hipStream_t stream) {
    return adamw_common("zs_adamw_step", p, m, v, w_out, S, contribs, n_contrib, nullptr, dtype,
                        hp, stream);
}

ZS_EXPORT zs_status zs_adamw_step_ex(float* p, float* m, float* v, uint16_t* w_out, int64_t S,
                                     const void* const* contribs, int32_t D,
                                     const zs_reduce_opts* opts, int32_t dtype,
                                     const zs_adamw_hp* hp, hipStream_t stream) {
    return adamw_common("zs_adamw_step_ex", p, m, v, w_out, S, contribs, D, opts, dtype, hp,
                        stream);
}

ZS_EXPORT zs_status zs_adamw_step_timed(float* p, float* m, float* v, uint16_t* w_out, int64_t S,
                                        const void* const* contribs, int32_t D,
                                        const zs_reduce_opts* opts, int32_t dtype,
                                        const zs_adamw_hp* hp, hipEvent_t start, hipEvent_t stop,
                                        hipStream_t stream) {
    const char* who = "zs_adamw_step_timed";
    if (start == nullptr || stop == nullptr)
        return fail(ZS_EINVAL, "%s: start or stop event is NULL", who);
    if (start == stop) return fail(ZS_EINVAL, "%s: start and stop are the same event", who);
    return adamw_common(who, p, m, v, w_out, S, contribs, D, opts, dtype, hp, stream, start, stop);
}

ZS_EXPORT zs_status zs_gather_unit(const void* const* shards, int32_t D, int64_t S,
                                   int32_t dtype, void* flat_out, hipStream_t stream) {
    const int es = elem_size(dtype);
    if (es == 0) return fail(ZS_EUNSUPPORTED, "zs_gather_unit: unknown dtype %d", dtype);
    if (D < 1 || D > ZS_MAX_D)
        return fail(ZS_EINVAL, "zs_gather_unit: D = %d outside 1..%d", D, ZS_MAX_D);
    if (!size_ok(S, es) || S > INT64_MAX / 16 / D)
        return fail(ZS_EINVAL, "zs_gather_unit: S = %lld out of range", (long long)S);
    if (S == 0) return ok();
    if (flat_out == nullptr) return fail(ZS_EINVAL, "zs_gather_unit: flat_out is NULL");
    if (!aligned(flat_out, uintptr_t(es)))
        return fail(ZS_EINVAL, "zs_gather_unit: flat_out not aligned to %d bytes", es);
    PtrPack sp;
    zs_status st = take_ptrs(shards, D, es, "zs_gather_unit: shards", &sp);
    if (st != ZS_OK) return st;
    // A shard sitting exactly in its own slot (in-place all-gather) is not
    // copied; any other overlap with flat_out would read what a copy writes.
    const Range out = range_of(flat_out, S * D, es);
    char* const f = static_cast<char*>(flat_out);
    uint64_t in_place = 0;
    for (int r = 0; r < D; ++r) {
        if (sp.p[r] == f + int64_t(r) * S * es) {
            in_place |= uint64_t(1) << r;
            continue;
        }
        if (overlap(out, range_of(sp.p[r], S, es)))
            return fail(ZS_EALIAS, "zs_gather_unit: flat_out overlaps shard %d", r);
    }
    return hip_status(launch_gather(sp, D, S, es, flat_out, in_place, stream),
                      "zs_gather_unit launch");
}

ZS_EXPORT zs_status zs_reshard(const void* const* src, int32_t D, int64_t S, int64_t N,
                               int32_t dtype, void* const* dst, int32_t D2, int64_t S2,
                               hipStream_t stream) {
    const char* who = "zs_reshard";
    const int es = elem_size(dtype);
    if (es == 0) return fail(ZS_EUNSUPPORTED, "%s: unknown dtype %d", who, dtype);
    if (D < 1 || D > ZS_MAX_D || D2 < 1 || D2 > ZS_MAX_D)
        return fail(ZS_EINVAL, "%s: D = %d, D2 = %d outside 1..%d", who, D, D2, ZS_MAX_D);
    if (N < 0 || N > INT64_MAX / 16 / es)
        return fail(ZS_EINVAL, "%s: N = %lld out of range", who, (long long)N);
    const int64_t want_S = N / D + (N % D != 0 ? 1 : 0);
    const int64_t want_S2 = N / D2 + (N % D2 != 0 ? 1 : 0);
    if (S != want_S || S2 != want_S2)
        return fail(ZS_EINVAL, "%s: S = %lld, S2 = %lld but ceil(N/D) = %lld, ceil(N/D2) = %lld", who,
                    (long long)S, (long long)S2, (long long)want_S, (long long)want_S2);
    if (N == 0) return ok();
    PtrPack sp, dp;
    zs_status st = take_ptrs(src, D, es, "zs_reshard: src", &sp);
    if (st != ZS_OK) return st;
    st = take_ptrs(const_cast<const void* const*>(dst), D2, es, "zs_reshard: dst", &dp);
    if (st != ZS_OK) return st;
    for (int a = 0; a < D2; ++a) {
        const Range ra = range_of(dp.p[a], S2, es);
        for (int b = a + 1; b < D2; ++b)
            if (overlap(ra, range_of(dp.p[b], S2, es)))
                return fail(ZS_EALIAS, "%s: dst shards %d and %d overlap", who, a, b);
        for (int r = 0; r < D; ++r)
            if (overlap(ra, range_of(sp.p[r], S, es)))
                return fail(ZS_EALIAS, "%s: dst shard %d overlaps src shard %d", who, a, r);
    }
    return hip_status(launch_reshard(sp, S, dp, D2, S2, N, es, stream), "zs_reshard launch");
}

namespace {

zs_status ceiling_common(const char* who, float* p, float* m, float* v, uint16_t* w, int64_t S,
                         const void* const* contribs, int32_t n, int32_t dtype, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop) {
    const int es = elem_size(dtype);
    if (es == 0) return fail(ZS_EUNSUPPORTED, "%s: unknown dtype %d", who, dtype);
    if (n < 1 || n > ZS_MAX_D) return fail(ZS_EINVAL, "%s: n = %d outside 1..%d", who, n, ZS_MAX_D);
    if (!size_ok(S, 4)) return fail(ZS_EINVAL, "%s: S = %lld out of range", who, (long long)S);
    if (S < 1024) return ok();
    if (!p || !m || !v || !w) return fail(ZS_EINVAL, "%s: p, m, v or w is NULL", who);
    if (!aligned(p, 16) || !aligned(m, 16) || !aligned(v, 16) || !aligned(w, 16))
        return fail(ZS_EINVAL, "%s: p, m, v and w must be 16-byte aligned", who);
    PtrPack cp;
    zs_status st = take_ptrs(contribs, n, 16, "zs_stream_ceiling: contribs", &cp);
    if (st != ZS_OK) return st;
    const Range rs[4] = {range_of(p, S, 4), range_of(m, S, 4), range_of(v, S, 4), range_of(w, S, 2)};
    for (int a = 0; a < 4; ++a) {
        for (int b = a + 1; b < 4; ++b)
            if (overlap(rs[a], rs[b])) return fail(ZS_EALIAS, "%s: outputs overlap", who);
        for (int q = 0; q < n; ++q)
            if (overlap(rs[a], range_of(cp.p[q], S, es)))
                return fail(ZS_EALIAS, "%s: contribution %d overlaps an output", who, q);
    }
    return hip_status(launch_streams(p, m, v, w, S, cp, n, dtype, stream, ev_start, ev_stop), who);
}

}  // namespace

ZS_EXPORT zs_status zs_stream_ceiling(float* p, float* m, float* v, uint16_t* w, int64_t S,
                                      const void* const* contribs, int32_t n, int32_t dtype,
                                      hipStream_t stream) {
    return ceiling_common("zs_stream_ceiling", p, m, v, w, S, contribs, n, dtype, stream, nullptr,
                          nullptr);
}

ZS_EXPORT zs_status zs_stream_ceiling_timed(float* p, float* m, float* v, uint16_t* w, int64_t S,
                                            const void* const* contribs, int32_t n,
                                            int32_t dtype, hipEvent_t start, hipEvent_t stop,
                                            hipStream_t stream) {
    const char* who = "zs_stream_ceiling_timed";
    if (start == nullptr || stop == nullptr)
        return fail(ZS_EINVAL, "%s: start or stop event is NULL", who);
    if (start == stop) return fail(ZS_EINVAL, "%s: start and stop are the same event", who);
    return ceiling_common(who, p, m, v, w, S, contribs, n, dtype, stream, start, stop);
}

ZS_EXPORT zs_status zs_hbm_probe(int32_t kind, void* buf, void* buf2, int64_t bytes,
                                 int32_t blocks_per_cu, hipStream_t stream) {
    const char* who = "zs_hbm_probe";
    if (kind != ZS_PROBE_READ && kind != ZS_PROBE_WRITE && kind != ZS_PROBE_COPY &&
        kind != ZS_PROBE_TRIAD)
        return fail(ZS_EINVAL, "%s: unknown kind %d", who, kind);
    if (blocks_per_cu < 0 || blocks_per_cu > 16)
        return fail(ZS_EINVAL, "%s: blocks_per_cu = %d outside 0..16", who, blocks_per_cu);
    if (bytes < 0 || bytes % 16 != 0 || !size_ok(bytes / 16, 32))
        return fail(ZS_EINVAL, "%s: bytes = %lld is not a non-negative multiple of 16", who,
                    (long long)bytes);
    if (bytes == 0) return ok();
    if (buf == nullptr || !aligned(buf, 16))
        return fail(ZS_EINVAL, "%s: buf is NULL or not 16-byte aligned", who);
    const bool two = kind != ZS_PROBE_WRITE;
    if (two) {
        if (buf2 == nullptr || !aligned(buf2, 16))
            return fail(ZS_EINVAL, "%s: buf2 is NULL or not 16-byte aligned", who);
        const int64_t n1 = kind == ZS_PROBE_TRIAD ? 2 * bytes : bytes;
        const int64_t n2 = kind == ZS_PROBE_READ ? 16 : bytes;
        if (overlap(range_of(buf, n1, 1), range_of(buf2, n2, 1)))
            return fail(ZS_EALIAS, "%s: buf and buf2 overlap", who);
    }
    return hip_status(launch_probe(kind, buf, buf2, bytes / 16, blocks_per_cu, stream), who);
}
