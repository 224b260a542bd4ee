// Internal (host-side) interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ttt.h"

namespace ttt {

// Validated problem + pointers of one ttt_chunk_fwd call.
struct FwdArgs {
  int B, H, T, dk, dv, C, NC;  // NC = number of chunks = ceil(T / C)
  int dtype, loss, act, decay;
  float b;
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* gamma;
  const float* log_decay;
  const float* w0;
  void* o;
  float* w_final;
  float* w_ckpt;
  char* saved;  // optional saved context for the backward (matrix-core path)
  char* ws;
  size_t ws_bytes;
};

// Validated problem + pointers of one ttt_chunk_bwd call.
struct BwdArgs {
  int B, H, T, dk, dv, C, NC;
  int dtype, loss, act, decay;
  float b;
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* gamma;
  const float* log_decay;
  const float* w0;
  const float* w_ckpt;
  const char* saved;  // optional: the forward's saved context
  const void* d_o;
  const float* d_wfinal;
  void* dq;
  void* dk_out;
  void* dv_out;
  float* dbeta;
  float* dgamma;
  float* dlog_decay;
  float* dw0;
  char* ws;
  size_t ws_bytes;
};

// ---- generic path (VALU fp32 arithmetic; any dtype, dk, dv <= 256, C <= 256) ----
size_t generic_fwd_workspace(const FwdArgs& a);
size_t generic_bwd_workspace(const BwdArgs& a);
hipError_t generic_fwd_launch(const FwdArgs& a, hipStream_t s);
hipError_t generic_bwd_launch(const BwdArgs& a, hipStream_t s);

// ---- matrix-core path (bf16 MFMA; dk, dv in {64, 128}, C % 32 == 0, C <= 256) ----
bool mfma_fwd_supported(const FwdArgs& a);
bool mfma_saved_supported(const FwdArgs& a);  // forward and backward both on the matrix-core path
size_t mfma_fwd_workspace(const FwdArgs& a);
hipError_t mfma_fwd_launch(const FwdArgs& a, hipStream_t s);
// Inner-product loss without an activation: G = -V does not depend on the
// state, and the forward runs chunk-parallel (ttt_linear.hip).
bool linear_fwd_applies(const FwdArgs& a);
size_t linear_fwd_workspace(const FwdArgs& a);
hipError_t linear_fwd_launch(const FwdArgs& a, hipStream_t s);
struct DecayPrep;
bool linear_bwd_applies(const BwdArgs& a);
// dW_{i+1} of every chunk into dWn ([B,H,NC,dk,dv]) and dW_0 into a.dw0
hipError_t linear_bwd_chain(const BwdArgs& a, const DecayPrep& dp, float* dWn, hipStream_t s);
bool mfma_bwd_supported(const BwdArgs& a);
size_t mfma_bwd_workspace(const BwdArgs& a);
hipError_t mfma_bwd_launch(const BwdArgs& a, hipStream_t s);

// ---- vector-decay preparation shared by the matrix-core kernels ----
// Tile-relative Q^m = Q e^{L - M_I}, K^m = K e^{M_I - L} (bf16; M_I the midpoint
// of 32-token tile I's range of L), lambda = e^{L_last} and the prefixes P_I of L
// at the tile boundaries, for every (chain, chunk); L is the in-chunk cumsum of
// log a (ttt_decay_prep.hip).
struct DecayPrep {
  uint16_t* qt;   // [B,H,T,dk] bf16  Q^m
  uint16_t* kt;   // [B,H,T,dk] bf16  K^m
  float* lam;     // [B,H,NC,dk]      e^{L_last}
  float* lpre;    // [B,H,NC,C/32+1,dk]  P_0 = 0 .. P_{C/32} = L_last
};
size_t decay_prep_layout(int B, int H, int T, int dk, int C, int NC, DecayPrep* p, char* base);
hipError_t decay_prep_launch(const float* la, const void* q, const void* k, int B, int H, int T, int dk, int C,
                             int NC, const DecayPrep& p, hipStream_t s);

// ---- saved context: what the matrix-core forward keeps for the backward ----
// Present only for problems the matrix-core kernels run.  Regions a
// configuration does not need (a constant factor) are absent (nullptr).
struct SavedCtx {
  DecayPrep prep;  // vector decay: Q~, K~, lambda, tile prefixes of L
  uint16_t* gh;    // [B,H,T,dv] bf16  eta (.) G
  uint16_t* dfy;   // [B,H,T,dv] bf16  f'(Y)  (with an act)
  uint16_t* z;     // [B,H,T,dv] bf16  Z = K W_i of the train view (with an act)
};
size_t mfma_saved_layout(int B, int H, int T, int dk, int dv, int C, int NC, int act, int decay, SavedCtx* sv,
                         char* base);

// ---- In-Place W_down update ----
// Compute units of the current device (cached per device; 256 if the query fails).
int device_cu_count();

size_t inplace_workspace_bytes(int B, int T, int d_model, int d_ff, int C);
hipError_t inplace_launch(int B, int T, int d_model, int d_ff, int C, float eta, const void* z,
                          const void* vhat, float* w_down, void* o, void* ws, size_t ws_bytes, hipStream_t s);
// The backward of inplace_launch (dz, dvhat, dw0 from d_o and d_wfinal); ws of
// inplace_bwd_workspace_bytes is required.
size_t inplace_bwd_workspace_bytes(int B, int T, int d_model, int d_ff, int C);
hipError_t inplace_bwd_launch(int B, int T, int d_model, int d_ff, int C, float eta, const void* z, const void* vhat,
                              const float* w_final, const void* d_o, const float* d_wfinal, void* dz, void* dvhat,
                              float* dw0, void* ws, hipStream_t s);
// With update clipping (clip_tau finite and > 0) and document resets (doc_starts:
// host, n_docs sorted flat positions b * T + t, 0 < t < T); ws holds the clip
// area first, then optionally the apply's split-K partials.
size_t inplace_guarded_workspace_bytes(int B, int T, int d_model, int d_ff, int C);
hipError_t inplace_launch_guarded(int B, int T, int d_model, int d_ff, int C, float eta, float clip_tau,
                                  const int64_t* doc_starts, int n_docs, const void* z, const void* vhat,
                                  const float* w_init, float* w_down, void* o, void* ws, size_t ws_bytes,
                                  hipStream_t s);
// The backward of inplace_launch_guarded (clip factor differentiated, the
// state's adjoint cut at document starts); the tile path only
// (inplace_bwd_guarded_supported), ws of inplace_bwd_guarded_workspace_bytes.
size_t inplace_bwd_guarded_workspace_bytes(int B, int T, int d_model, int d_ff, int C);
bool inplace_bwd_guarded_supported(int T, int d_model, int d_ff, int C);
hipError_t inplace_bwd_guarded_launch(int B, int T, int d_model, int d_ff, int C, float eta, float clip_tau,
                                      const int64_t* doc_starts, int n_docs, const void* z, const void* vhat,
                                      const float* w0, const float* w_init, const float* w_final, const void* d_o,
                                      const float* d_wfinal, void* dz, void* dvhat, float* dw0, float* dw_init,
                                      void* ws, hipStream_t s);

// ---- the fast net Linear -> Norm (act = TTT_ACT_NORM), one workgroup per chain ----
size_t norm_fwd_workspace(const FwdArgs& a);
size_t norm_bwd_workspace(const BwdArgs& a);
hipError_t norm_fwd_launch(const FwdArgs& a, hipStream_t s);
hipError_t norm_bwd_launch(const BwdArgs& a, hipStream_t s);

// ---- two-layer fast net (TTT-MLP) forward, VALU fp32 ----
size_t mlp_fwd_workspace(const ttt_mlp_desc& d);
hipError_t mlp_fwd_launch(const ttt_mlp_desc& d, const void* q, const void* k, const void* v, const float* beta,
                          const float* gamma, const float* w1_0, const float* w2_0, void* o, float* w1_final,
                          float* w2_final, float* w1_ckpt, float* w2_ckpt, void* saved, void* ws, hipStream_t s);
size_t mlp_saved_bytes(const ttt_mlp_desc& d);
size_t mlp_bwd_workspace(const ttt_mlp_desc& d);
hipError_t mlp_bwd_launch(const ttt_mlp_desc& d, const void* q, const void* k, const void* v, const float* beta,
                          const float* gamma, const float* w1_ckpt, const float* w2_ckpt, const void* saved,
                          const void* d_o, const float* d_w1final, const float* d_w2final, void* dq, void* dk,
                          void* dv, float* dbeta, float* dgamma, float* dw1_0, float* dw2_0, void* ws,
                          hipStream_t s);

// Brackets one kernel launch with HIP events on its stream while per-kernel
// timing is on; does nothing otherwise.
class KernelScope {
 public:
  KernelScope(ttt_kernel kernel, hipStream_t s);
  ~KernelScope();
  KernelScope(const KernelScope&) = delete;
  KernelScope& operator=(const KernelScope&) = delete;

 private:
  hipEvent_t stop_ = nullptr;
  hipStream_t s_;
};

// Set the thread-local message ttt_last_error() returns and return `code`
// (ttt_host.cpp); for entry points defined outside it.
int report_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int report_hip_error(hipError_t e, const char* where);

// Round a byte count up to 256 (workspace sub-buffer alignment).
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace ttt
