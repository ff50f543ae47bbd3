// sfa_run for callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation): the split-K partials that sfa_run keeps in
// the caller's workspace live instead in `scratch`, a file-scope device array of
// kNoAllocScratchBytes that every GPU the library runs on holds until the process ends.
//
// In host code the array's name only stands in for the symbol: its device address is looked up
// once per device with hipGetSymbolAddress (at the first call on that device, with it current)
// and kept per device; only that address reaches the kernels.  Every call on one GPU shares that
// GPU's array, so calls that overlap on one GPU (different streams) race on it.  Nothing in it
// has to start at zero: each split writes its whole partial before the merge reads it.
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/sfa.h"

constexpr size_t kNoAllocScratchBytes = 64ull << 20;  // the MLA decode workload needs 33.7 MB

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up yet)

// Device address of this device's scratch array; null (and *err set) on failure.
void* scratch_address(sfa_status* err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = SFA_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *err = SFA_ERR_HIP;
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t sfa_run_noalloc_max_workspace(void) { return kNoAllocScratchBytes; }

sfa_status sfa_run_noalloc(const sfa_shape* shape, const sfa_strides* strides, sfa_dtype dtype, sfa_layout layout,
                           int causal, float scale, const void* q, const void* k, const void* v,
                           const int32_t* sparse_indices, void* out, float* lse, hipStream_t stream) {
  const size_t need = sfa_workspace_bytes(shape, dtype, causal);
  if (need > kNoAllocScratchBytes) {
    if (getenv("SFA_LOG"))
      fprintf(stderr, "sfa_run_noalloc: the problem needs %zu bytes of split-K scratch, above the %zu available\n",
              need, kNoAllocScratchBytes);
    return SFA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (need > 0) {
    sfa_status err = SFA_OK;
    ws = scratch_address(&err);
    if (!ws) return err;
  }
  return sfa_run(shape, strides, dtype, layout, causal, scale, q, k, v, sparse_indices, out, lse, ws,
                 need > 0 ? kNoAllocScratchBytes : 0, stream);
}

}  // extern "C"
