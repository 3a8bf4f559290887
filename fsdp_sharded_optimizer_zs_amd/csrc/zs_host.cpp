// The shard step on host cores (ZeRO-Offload): the optimizer state p, m, v
// lives in host memory; each step the reduced gradient comes down from the
// device, the host runs the AdamW update, and the new bf16 working shard goes
// back up.
//
// The host kernel performs the device kernel's arithmetic in the same order:
// fp32, every operation rounded on its own (this file is compiled with
// -ffp-contract=off and the code never calls fma), IEEE sqrt and division,
// denormals kept (each worker clears the SSE flush-to-zero and
// denormals-are-zero modes for its duration), bf16 by integer
// round-to-nearest-even. It is vectorized by the compiler (AVX2 when the CPU
// has it, SSE2 otherwise) and split over persistent worker threads in
// contiguous, 64-element-aligned ranges.

#include <immintrin.h>

#include <algorithm>
#include <condition_variable>
#include <cstdint>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "zs_internal.h"

#define ZS_EXPORT extern "C" __attribute__((visibility("default")))

#pragma clang fp contract(off)

using namespace zs;

namespace {

inline uint16_t to_bf16(float x) {
    uint32_t u;
    __builtin_memcpy(&u, &x, 4);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return uint16_t(((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : rounded);
}

// One AdamW update of elements [lo, hi), in the fixed operation order. The
// constants are copied to locals so that no store can alias them, which
// lets the loop vectorize.
__attribute__((always_inline)) inline void step_body(float* __restrict__ p, float* __restrict__ m,
                                                     float* __restrict__ v,
                                                     uint16_t* __restrict__ w,
                                                     const float* __restrict__ g, int64_t lo,
                                                     int64_t hi, const AdamConsts kc) {
    const float dec = kc.dec, b1 = kc.b1, b1c = kc.b1c, b2 = kc.b2, b2c = kc.b2c, ss = kc.ss,
                bc2s = kc.bc2s, eps = kc.eps;
    for (int64_t i = lo; i < hi; ++i) {
        const float gi = g[i];
        const float p1 = p[i] * dec;
        const float m1 = (b1 * m[i]) + (b1c * gi);
        const float v1 = (b2 * v[i]) + (b2c * (gi * gi));
        // llvm.sqrt: the IEEE square root, without the errno side effect
        // that keeps a libm call from vectorizing
        const float den = (__builtin_elementwise_sqrt(v1) / bc2s) + eps;
        const float p2 = p1 - (ss * (m1 / den));
        p[i] = p2;
        m[i] = m1;
        v[i] = v1;
        w[i] = to_bf16(p2);
    }
}

void run_generic(float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
                 uint16_t* __restrict__ w, const float* __restrict__ g, int64_t lo, int64_t hi,
                 const AdamConsts k) {
    step_body(p, m, v, w, g, lo, hi, k);
}

__attribute__((target("avx2"))) void run_avx2(float* __restrict__ p, float* __restrict__ m,
                                              float* __restrict__ v, uint16_t* __restrict__ w,
                                              const float* __restrict__ g, int64_t lo, int64_t hi,
                                              const AdamConsts k) {
    step_body(p, m, v, w, g, lo, hi, k);
}

void run_range(float* p, float* m, float* v, uint16_t* w, const float* g, int64_t lo, int64_t hi,
               const AdamConsts& k, bool avx2) {
    // exact arithmetic needs denormals kept: clear FTZ (bit 15) and DAZ (bit 6)
    const unsigned int saved = _mm_getcsr();
    _mm_setcsr(saved & ~0x8040u);
    if (avx2)
        run_avx2(p, m, v, w, g, lo, hi, k);
    else
        run_generic(p, m, v, w, g, lo, hi, k);
    _mm_setcsr(saved);
}

// Persistent worker threads: an offload step runs the host update once per
// transfer chunk, and starting fresh threads for every chunk cost a few
// milliseconds per step. Workers are created on first use, grow to the
// largest count asked for, and serve one parallel range at a time (callers
// from several host threads take turns).
class Workers {
public:
    static Workers& get() {
        static Workers w;
        return w;
    }

    // Runs f(t) for t in [0, n): t = 0 on the calling thread, the rest on workers.
    template <class F>
    void run(int n, const F& f) {
        std::lock_guard<std::mutex> turn(call_mu_);
        {
            std::unique_lock<std::mutex> lk(mu_);
            while (int(threads_.size()) < n - 1) {
                const int id = int(threads_.size()) + 1;
                threads_.emplace_back([this, id] { loop(id); });
            }
            task_ = [&f](int t) { f(t); };
            active_ = n;
            remaining_ = n - 1;
            ++generation_;
        }
        cv_.notify_all();
        f(0);
        std::unique_lock<std::mutex> lk(mu_);
        done_cv_.wait(lk, [this] { return remaining_ == 0; });
        task_ = nullptr;
    }

    ~Workers() {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
            ++generation_;
        }
        cv_.notify_all();
        for (auto& t : threads_) t.join();
    }

private:
    void loop(int id) {
        uint64_t seen = 0;
        for (;;) {
            std::function<void(int)> task;
            {
                std::unique_lock<std::mutex> lk(mu_);
                cv_.wait(lk, [&] { return stop_ || generation_ != seen; });
                if (stop_) return;
                seen = generation_;
                if (id >= active_) continue;
                task = task_;
            }
            task(id);
            std::lock_guard<std::mutex> lk(mu_);
            if (--remaining_ == 0) done_cv_.notify_one();
        }
    }

    std::mutex call_mu_, mu_;
    std::condition_variable cv_, done_cv_;
    std::vector<std::thread> threads_;
    std::function<void(int)> task_;
    uint64_t generation_ = 0;
    int active_ = 0;
    int remaining_ = 0;
    bool stop_ = false;
};

void parallel_step(float* p, float* m, float* v, uint16_t* w, const float* g, int64_t S,
                   const AdamConsts& k, int threads) {
    static const bool avx2 = __builtin_cpu_supports("avx2");
    const int64_t per = ((S + threads - 1) / threads + 63) / 64 * 64;
    const int n = int((S + per - 1) / per);
    Workers::get().run(n, [&](int t) {
        const int64_t lo = per * t, hi = std::min(S, lo + per);
        if (lo < hi) run_range(p, m, v, w, g, lo, hi, k, avx2);
    });
}

zs_status check_host_state(const char* who, float* p, float* m, float* v, uint16_t* w,
                           const float* g, int64_t S) {
    if (!p || !m || !v || !w || !g) return fail(ZS_EINVAL, "%s: a buffer is NULL", who);
    if (!aligned(p, 4) || !aligned(m, 4) || !aligned(v, 4) || !aligned(w, 2) || !aligned(g, 4))
        return fail(ZS_EINVAL, "%s: a buffer is misaligned for its element type", who);
    const Range rs[5] = {range_of(p, S, 4), range_of(m, S, 4), range_of(v, S, 4), range_of(w, S, 2),
                         range_of(g, S, 4)};
    const char* names[5] = {"p", "m", "v", "w_out", "grad"};
    for (int a = 0; a < 5; ++a)
        for (int b = a + 1; b < 5; ++b)
            if (overlap(rs[a], rs[b]))
                return fail(ZS_EALIAS, "%s: %s overlaps %s", who, names[a], names[b]);
    return ZS_OK;
}

}  // namespace

ZS_EXPORT zs_status zs_adamw_step_host(float* p, float* m, float* v, uint16_t* w_out, int64_t S,
                                       const float* grad, const zs_adamw_hp* hp,
                                       int32_t threads) {
    const char* who = "zs_adamw_step_host";
    if (!size_ok(S, 4)) return fail(ZS_EINVAL, "%s: S = %lld out of range", who, (long long)S);
    if (threads < 1 || threads > 1024)
        return fail(ZS_EINVAL, "%s: threads = %d outside 1..1024", who, threads);
    zs_status st = check_hp(hp, who);
    if (st != ZS_OK) return st;
    if (S == 0) return ok();
    st = check_host_state(who, p, m, v, w_out, grad, S);
    if (st != ZS_OK) return st;
    // the gradient is the single fp32 contribution: inv_n = 1
    parallel_step(p, m, v, w_out, grad, S, adam_consts(*hp, 1), threads);
    return ok();
}

ZS_EXPORT zs_status zs_offload_step(const void* const* contribs, int32_t D, int32_t dtype,
                                    int64_t S, float* grad_dev, float* grad_host, float* p,
                                    float* m, float* v, uint16_t* w_host, uint16_t* w_dev,
                                    const zs_adamw_hp* hp, int32_t threads, int64_t chunk,
                                    hipStream_t stream, hipStream_t h2d_stream) {
    const char* who = "zs_offload_step";
    const int es = elem_size(dtype);
    if (es == 0) return fail(ZS_EUNSUPPORTED, "%s: unknown dtype %d", who, dtype);
    if (D < 1 || D > ZS_MAX_D) return fail(ZS_EINVAL, "%s: D = %d outside 1..%d", who, D, ZS_MAX_D);
    if (!size_ok(S, 4)) return fail(ZS_EINVAL, "%s: S = %lld out of range", who, (long long)S);
    if (threads < 1 || threads > 1024)
        return fail(ZS_EINVAL, "%s: threads = %d outside 1..1024", who, threads);
    if (chunk < 1) return fail(ZS_EINVAL, "%s: chunk = %lld < 1", who, (long long)chunk);
    zs_status st = check_hp(hp, who);
    if (st != ZS_OK) return st;
    if (S == 0) return ok();
    if (!grad_dev || !w_dev || !aligned(grad_dev, 4) || !aligned(w_dev, 2))
        return fail(ZS_EINVAL, "%s: grad_dev or w_dev NULL or misaligned", who);
    st = check_host_state(who, p, m, v, w_host, grad_host, S);
    if (st != ZS_OK) return st;
    PtrPack cp;
    st = take_ptrs(contribs, D, es, "zs_offload_step: contribs", &cp);
    if (st != ZS_OK) return st;
    const Range gd = range_of(grad_dev, S, 4), wd = range_of(w_dev, S, 2);
    if (overlap(gd, wd)) return fail(ZS_EALIAS, "%s: grad_dev overlaps w_dev", who);
    bool al = aligned(grad_dev, 16);
    for (int q = 0; q < D; ++q) {
        const Range c = range_of(cp.p[q], S, es);
        if (overlap(c, gd) || overlap(c, wd))
            return fail(ZS_EALIAS, "%s: contribution %d overlaps grad_dev or w_dev", who, q);
        al = al && aligned(cp.p[q], 16);
    }

    // 1. device: the reduce-scatter's arithmetic, g in fp32
    hipError_t e = launch_reduce(cp, D, 1, false, dtype, S, float(1.0 / double(D)), grad_dev, al,
                                 stream);
    if (e != hipSuccess) return hip_status(e, "zs_offload_step: reduce launch");
    // 2. g comes down chunk by chunk; 3. the host steps each chunk as soon as
    // it has landed; 4. the chunk's bf16 shard goes back up on h2d_stream.
    // Up to kAhead chunk copies are queued ahead of the host, each followed
    // by a pooled event that the host waits on; chunk c + kAhead is queued
    // (reusing chunk c's event) once the host has waited for chunk c.
    constexpr int64_t kAhead = 8;
    const int64_t nchunks = (S + chunk - 1) / chunk;
    const int64_t ring = std::min(nchunks, kAhead);
    EventLease ev;
    if ((e = ev.take(int(ring))) != hipSuccess) return hip_status(e, "zs_offload_step: events");
    auto queue_down = [&](int64_t c) {
        const int64_t lo = c * chunk, n = std::min(chunk, S - lo);
        hipError_t r = hipMemcpyAsync(grad_host + lo, grad_dev + lo, size_t(n) * 4,
                                      hipMemcpyDeviceToHost, stream);
        if (r == hipSuccess) r = hipEventRecord(ev.ev(int(c % ring)), stream);
        return r;
    };
    for (int64_t c = 0; c < ring; ++c)
        if ((e = queue_down(c)) != hipSuccess) return hip_status(e, "zs_offload_step: gradient copy");
    const AdamConsts k = adam_consts(*hp, 1);
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t lo = c * chunk, n = std::min(chunk, S - lo);
        if ((e = hipEventSynchronize(ev.ev(int(c % ring)))) != hipSuccess)
            return hip_status(e, "zs_offload_step: gradient wait");
        if (c + ring < nchunks && (e = queue_down(c + ring)) != hipSuccess)
            return hip_status(e, "zs_offload_step: gradient copy");
        parallel_step(p + lo, m + lo, v + lo, w_host + lo, grad_host + lo, n, k, threads);
        if ((e = hipMemcpyAsync(w_dev + lo, w_host + lo, size_t(n) * 2, hipMemcpyHostToDevice,
                                h2d_stream)) != hipSuccess)
            return hip_status(e, "zs_offload_step: working shard copy");
    }
    return ok();
}
