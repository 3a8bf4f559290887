// The pipelined shard step with its staging in a library-owned device array,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// zs_step_pipelined takes two caller-allocated staging slots that each hold
// a whole bucket's contributions. This variant stages through `scratch`, a
// fixed array in the code object (two slots of kSlotBytes), and moves each
// bucket in pieces that fit a slot; the arithmetic and the results are those
// of zs_step_pipelined, bit for bit (the step is elementwise, so how a bucket
// is cut into launches changes nothing). Each device that runs it holds the
// array until the process ends. Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per
// device, on the first call on that device.

#include <mutex>
#include <vector>

#include "zs_internal.h"

#define ZS_EXPORT extern "C" __attribute__((visibility("default")))

namespace zs {
namespace {

constexpr int64_t kSlotBytes = int64_t(64) << 20;  // each of the two staging slots
constexpr int64_t kScratchBytes = 2 * kSlotBytes;  // 128 MiB per device

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Per-device state, set up on the first call on the device with that device
// current: the array's device address and the five events that order the
// copies and the steps. Never released (it lives as long as the array).
struct StaticState {
    void* ptr = nullptr;
    hipEvent_t ev[5] = {};
};
std::mutex g_mu;
std::vector<StaticState> g_state;

hipError_t static_state(const StaticState** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_state.size() <= size_t(dev)) g_state.resize(size_t(dev) + 1);
    StaticState& st = g_state[size_t(dev)];
    if (st.ptr == nullptr) {
        StaticState fresh;
        if ((e = hipGetSymbolAddress(&fresh.ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        if (fresh.ptr == nullptr || (reinterpret_cast<uintptr_t>(fresh.ptr) & 255) != 0)
            return hipErrorInvalidSymbol;
        for (hipEvent_t& x : fresh.ev) {
            if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess) {
                for (hipEvent_t y : fresh.ev)
                    if (y) (void)hipEventDestroy(y);
                return e;
            }
        }
        st = fresh;
    }
    *out = &st;
    return hipSuccess;
}

}  // namespace
}  // namespace zs

using namespace zs;

ZS_EXPORT zs_status zs_step_pipelined_static(const zs_bucket* buckets, int32_t n_buckets,
                                             int32_t n_contrib, int32_t dtype,
                                             const zs_adamw_hp* hp, hipStream_t compute,
                                             hipStream_t transfer) {
    const char* who = "zs_step_pipelined_static";
    const int es = elem_size(dtype);
    if (es == 0) return fail(ZS_EUNSUPPORTED, "%s: unknown dtype %d", who, dtype);
    if (n_contrib < 1 || n_contrib > ZS_MAX_D)
        return fail(ZS_EINVAL, "%s: n_contrib = %d outside 1..%d", who, n_contrib, ZS_MAX_D);
    // a piece: the most elements whose n_contrib contributions fit one slot,
    // a multiple of 1024 (whole tile pairs, 16-byte aligned staging)
    const int64_t piece = (kSlotBytes / (int64_t(n_contrib) * es)) & ~int64_t(1023);
    static_assert((kSlotBytes / (int64_t(ZS_MAX_D) * 4)) >= 1024, "a slot holds a piece");
    zs_status st = pipelined_check(who, buckets, n_buckets, n_contrib, dtype, nullptr, nullptr, 0,
                                   INT64_MAX, hp);
    if (st != ZS_OK || n_buckets == 0) return st == ZS_OK ? ok() : st;
    const StaticState* ss = nullptr;
    hipError_t e = static_state(&ss);
    if (e != hipSuccess) return hip_status(e, "zs_step_pipelined_static: scratch set-up");
    char* base = static_cast<char*>(ss->ptr);
    st = pipelined_enqueue(who, buckets, n_buckets, n_contrib, dtype, base, base + kSlotBytes,
                           piece, hp, compute, transfer, ss->ev);
    if (st != ZS_OK) return fail(st, "zs_step_pipelined_static: %s", zs_last_error());
    return ok();
}
