// moe_run_noalloc: the layer with its scratch arena in a static device array,
// for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code its name is only a host-side stand-in, so the device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and that
// pointer is what moe_run's kernels receive, exactly as they receive a caller's
// arena.  Nothing in the arena has to start at zero: moe_run's kernels clear
// what they accumulate into (the atomic combine's fp32 accumulator in the route
// launch, the decode down GEMM's per-tile sums and counters in the up/gate
// launch) and write everything else before reading it.  All calls on one GPU
// share its array, so calls that overlap on one GPU (two streams, two host
// threads) race; calls on different GPUs do not.
#include <mutex>

#include "moe.h"
#include "moe_common.h"

namespace {

constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void *g_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

extern "C" int moe_run_noalloc(moe_plan_t plan, const moe_tier *tiers, int n_tiers, const void *x,
                               const int32_t *topk_ids, const float *topk_weights, void *out, int T, int deterministic,
                               void *stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return moe::set_error(MOE_EHIP, "moe_run_noalloc: no current device (or device index above 63)");
  void *p = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
      void *q = nullptr;
      const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !q) return moe::set_error(MOE_EHIP, "moe_run_noalloc: hipGetSymbolAddress failed");
      g_ptr[dev] = q;
    }
    p = g_ptr[dev];
  }
  if (T > 0) {
    const size_t need = moe_scratch_bytes(plan, T, deterministic);
    if (need == 0) return moe::set_error(MOE_EINVAL, "moe_run_noalloc: invalid plan");
    if (need > kStaticScratchBytes) {
      char msg[200];
      snprintf(msg, sizeof msg,
               "moe_run_noalloc: this batch needs %zu bytes of scratch; the static arena holds %zu (64 MiB): "
               "use moe_run with a caller arena",
               need, kStaticScratchBytes);
      return moe::set_error(MOE_ESCRATCH, msg);
    }
  }
  return moe_run(plan, tiers, n_tiers, x, topk_ids, topk_weights, out, T, deterministic, p, kStaticScratchBytes,
                 stream);
}
