// cp_attn_bwd_noalloc: the backward of cp_attn_bwd with its scratch (delta =
// rowsum(dO * O), fp32 [H, n_local]) in a device array of this library
// instead of a caller buffer, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable. Each GPU the library runs on
// holds its own copy at its own address until the process ends. In host code
// the variable's name is only a stand-in for the symbol, never an address:
// the device address is looked up once per device, with that device current,
// by hipGetSymbolAddress, and only that address is handed to kernels. Every
// call on a GPU shares that GPU's copy, so calls that overlap on one GPU (two
// streams, two threads) race on it. Nothing in it has to start at zero: the
// dQ launch writes delta for every local row before the dK/dV launch reads it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "internal.h"

namespace {

// 2^21 floats (8 MiB): plans with n_local * H up to 2,097,152 (e.g. 75,600
// local rows x 27 heads, or 262,144 x 8).
constexpr size_t kScratchFloats = size_t(1) << 21;
constexpr size_t kScratchBytes = kScratchFloats * sizeof(float);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kScratchFloats];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of the current GPU's copy of scratch: looked up on the
// first call on that device and kept. nullptr (and *err) on failure.
void* scratch_ptr(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

thdcp_status_t cp_attn_bwd_noalloc(thdcp_plan_t plan, const void* q_local, const void* k,
                                   const void* v, const void* o_local, const float* lse,
                                   const void* d_o, float* dq, float* dk, float* dv,
                                   int32_t zero_untouched, int32_t accumulate_dkv,
                                   void* stream) {
  if (!plan) return thdcp::report_error(THDCP_ERR_ARG, "NULL plan");
  thdcp_plan_info info;
  thdcp_status_t st = thdcp_plan_get_info(plan, &info);
  if (st != THDCP_OK) return st;
  if (info.bwd_scratch_bytes > kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "cp_attn_bwd_noalloc: the plan needs %zu bytes of scratch (n_local x H floats), "
             "above the library's fixed %zu; use cp_attn_bwd with a caller buffer",
             info.bwd_scratch_bytes, kScratchBytes);
    return thdcp::report_error(THDCP_ERR_UNSUPPORTED, msg);
  }
  hipError_t e = hipSuccess;
  void* p = scratch_ptr(&e);
  if (!p) {
    char msg[200];
    snprintf(msg, sizeof(msg), "cp_attn_bwd_noalloc: device address of the scratch: %s",
             hipGetErrorString(e));
    return thdcp::report_error(THDCP_ERR_HIP, msg);
  }
  return cp_attn_bwd(plan, q_local, k, v, o_local, lse, d_o, dq, dk, dv, zero_untouched,
                     accumulate_dkv, p, kScratchBytes, stream);
}

}  // extern "C"
