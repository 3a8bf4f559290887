// Internal interface between the C-ABI layer (zs_api.cpp) and the kernel
// translation units. Not installed; the public interface is include/zs.h.
#pragma once

#include <stdint.h>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/zs.h"
#include "zs_grid.h"

// Launch shape of the tiled step kernels (workgroups of 256 threads, 4
// wavefronts): ZS_STEP_TILES adjacent 512-element tiles per wavefront, and one
// wavefront per tile group: the grid covers the whole shard (up to
// kMaxGrid workgroups, zs_grid.h; the kernels loop in grid-stride order past
// that).
// Measured on MI355X over the 81 buckets of a 70B rank shard: 6.17 TB/s,
// against 6.05-6.11 for a persistent grid of one workgroup per CU (whose
// wavefronts drift apart over a long launch, so more HBM rows are open at
// once), 6.09 with one tile per wavefront, 5.24 with four; equal or better
// on the 16- and 32-contribution folds too.
#ifndef ZS_STEP_TILES
#define ZS_STEP_TILES 2
#endif

namespace zs {

// Up to ZS_MAX_D device pointers passed by value as a kernel argument.
struct PtrPack {
    const void* p[ZS_MAX_D];
};

// fp32 constants of one AdamW step (rounded once from double on the host).
struct AdamConsts {
    float dec;    // 1 - lr * weight_decay
    float b1;     // beta1
    float b1c;    // 1 - beta1
    float b2;     // beta2
    float b2c;    // 1 - beta2
    float ss;     // lr / (1 - beta1^t)
    float bc2s;   // sqrt(1 - beta2^t)
    float eps;    // eps
    float inv_n;  // 1 / n_contrib
    int keep_w;   // 1: the working shard is stored with cache-allocating stores
};

// Host-side helpers shared by the entry points (zs_api.cpp).
zs_status fail(zs_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
zs_status ok();  // clears the calling thread's error text
zs_status hip_status(hipError_t e, const char* what);
int elem_size(int32_t dtype);  // 2, 4, or 0 for an unknown tag
struct Range {                 // byte range [lo, hi) of a buffer
    uintptr_t lo, hi;
};
Range range_of(const void* p, int64_t count, int es);
bool overlap(const Range& a, const Range& b);
bool aligned(const void* p, uintptr_t a);
bool size_ok(int64_t S, int es);
zs_status take_ptrs(const void* const* src, int n, int es, const char* what, PtrPack* out);
zs_status check_hp(const zs_adamw_hp* hp, const char* who);
AdamConsts adam_consts(const zs_adamw_hp& hp, int n_contrib);

// HIP events that order work between streams, reused across calls so that
// no per-step path creates a runtime object: a lease takes n events from the
// current device's pool (creating them only when the pool runs short) and
// gives them back when it goes out of scope. An event may be recorded again
// once the waits that used it have been enqueued, so a returned event can
// serve the next call at once. Pooled events live until the process ends.
class EventLease {
  public:
    EventLease() = default;
    EventLease(const EventLease&) = delete;
    EventLease& operator=(const EventLease&) = delete;
    ~EventLease();
    hipError_t take(int n);  // ev(0) .. ev(n - 1) valid afterwards
    hipEvent_t ev(int i) const { return ev_[size_t(i)]; }

  private:
    int dev_ = -1;
    std::vector<hipEvent_t> ev_;
};

// The pipelined step (zs_pipeline.cpp), shared by its two entry points:
// argument and aliasing checks (buckets of at most max_bucket elements;
// staging slots of slot_elems elements each), then the enqueue, each
// bucket in pieces of at most `piece` elements that alternate between the
// two slots, ordered by events ev[0..4] (start, arrived[2], consumed[2]).
zs_status pipelined_check(const char* who, const zs_bucket* buckets, int32_t n_buckets,
                          int32_t n_contrib, int32_t dtype, const void* staging0,
                          const void* staging1, int64_t slot_elems, int64_t max_bucket,
                          const zs_adamw_hp* hp);
zs_status pipelined_enqueue(const char* who, const zs_bucket* buckets, int32_t n_buckets,
                            int32_t n_contrib, int32_t dtype, void* staging0, void* staging1,
                            int64_t piece, const zs_adamw_hp* hp, hipStream_t compute,
                            hipStream_t transfer, const hipEvent_t ev[5]);

// Launch geometry of the device the caller's stream runs on.
struct DeviceInfo {
    int cu_count;
};
const DeviceInfo& device_info();

// Kernel launchers (enqueue only; return the launch status). The reduce of
// the step folds R groups of nd contributions (replica-major; R = 1 is the
// flat fold), rounding each level to the reduce dtype when rnd is set. With
// ev_start and ev_stop, the step's one kernel launch records them at its own
// start and end (hipExtLaunchKernel) instead of a plain launch.
hipError_t launch_adamw(float* p, float* m, float* v, uint16_t* w, int64_t S,
                        const PtrPack& contribs, int nd, int R, bool rnd, int dtype,
                        const AdamConsts& k, bool aligned, hipStream_t stream,
                        hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_reduce(const PtrPack& contribs, int nd, int R, bool rnd, int dtype, int64_t S,
                         float inv_n, float* out, bool aligned, hipStream_t stream);
hipError_t launch_pack(const zs_tensor_ref* d_table, int T, int64_t N, int es,
                       int D, const PtrPack& shards, int64_t S, hipStream_t stream);
// in_place: bit r set when shard r already sits in its slot (not copied).
hipError_t launch_gather(const PtrPack& shards, int D, int64_t S, int es, void* flat,
                         uint64_t in_place, hipStream_t stream);
hipError_t launch_streams(float* p, float* m, float* v, uint16_t* w, int64_t S,
                          const PtrPack& contribs, int n, int dtype, hipStream_t stream,
                          hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_probe(int kind, void* buf, void* buf2, int64_t nvec, int per_cu,
                        hipStream_t stream);
hipError_t launch_reshard(const PtrPack& src, int64_t S, const PtrPack& dst, int D2, int64_t S2,
                          int64_t N, int es, hipStream_t stream);

}  // namespace zs
