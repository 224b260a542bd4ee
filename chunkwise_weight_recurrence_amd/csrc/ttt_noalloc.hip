// ttt_chunk_bwd_noalloc: the outer backward of the chunkwise TTT layer without a
// caller workspace, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The backward's scratch (the bf16 dY, G~, dZ round trip between its two kernels,
// the dW_{i+1} checkpoints, the deta / dlambda partial sums and, for vector decay
// without a saved context, the decay preparation) lives in one file-scope device
// array of kScratchBytes.  Each GPU the library runs on holds its own copy until
// the process ends; its address on a device is taken once, with that device
// current, through hipGetSymbolAddress (in host code the array's name is only a
// stand-in, never a device address).  Every call on a device shares that
// device's array, so calls that overlap on one device (different streams, no
// ordering between them) race; calls ordered on one stream do not.  Nothing in
// the scratch needs to start at zero: every region is written before it is read
// within one call.

#include <mutex>

#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr size_t kScratchBytes = size_t{64} << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device (taken once).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace ttt

extern "C" {

TTT_API size_t ttt_noalloc_scratch_bytes(void) { return ttt::kScratchBytes; }

TTT_API int ttt_chunk_bwd_noalloc(const ttt_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                                  const float* gamma, const float* log_decay, const float* w0, const float* w_ckpt,
                                  const void* saved, const void* d_o, const float* d_wfinal, void* dq, void* dk,
                                  void* dv, float* dbeta, float* dgamma, float* dlog_decay, float* dw0,
                                  void* stream) {
  size_t need = 0;
  int st = ttt_workspace_size(desc, TTT_ENTRY_BWD, &need);
  if (st != TTT_OK) return st;
  if (need > ttt::kScratchBytes)
    return ttt::report_error(TTT_ERR_WORKSPACE,
                             "ttt_chunk_bwd_noalloc: this problem needs %zu bytes of scratch, above the library's "
                             "fixed %zu (use ttt_chunk_bwd with a workspace)",
                             need, ttt::kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = ttt::scratch_ptr(&ws);
    if (e != hipSuccess) return ttt::report_hip_error(e, "ttt_chunk_bwd_noalloc: scratch address");
  }
  return ttt_chunk_bwd(desc, q, k, v, beta, gamma, log_decay, w0, w_ckpt, saved, d_o, d_wfinal, dq, dk, dv, dbeta,
                       dgamma, dlog_decay, dw0, ws, need > 0 ? ttt::kScratchBytes : 0, stream);
}

}  // extern "C"
