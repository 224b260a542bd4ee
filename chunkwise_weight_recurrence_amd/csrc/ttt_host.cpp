// C ABI of libttt.so: host-side validation, workspace sizing and dispatch.
//
// Every check runs on the host before any HIP call, so a rejected call
// launches nothing.  Kernel selection: bf16 problems the matrix-core kernels
// cover (d_k, d_v in {64, 128}, C a multiple of 32 up to 256) run there; all
// other problems, and every fp32 problem, run on the generic VALU kernels.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <utility>

#include "ttt_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return TTT_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(TTT_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

}  // namespace

// The same error reporting for the entry points defined in other files.
int ttt::report_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}
int ttt::report_hip_error(hipError_t e, const char* where) { return hip_fail(e, where); }

namespace {

constexpr int kMaxDim = 256;

// Shape and enum checks shared by forward and backward.
int check_desc(const ttt_desc* d) {
  if (!d) return fail(TTT_ERR_INVALID_ARG, "desc is NULL");
  if (d->B < 0 || d->H < 0 || d->T < 0)
    return fail(TTT_ERR_INVALID_ARG, "B, H, T must be >= 0 (got %d, %d, %d)", d->B, d->H, d->T);
  if (d->dk < 1 || d->dv < 1) return fail(TTT_ERR_INVALID_ARG, "dk, dv must be >= 1 (got %d, %d)", d->dk, d->dv);
  if (d->C < 1) return fail(TTT_ERR_INVALID_ARG, "chunk length C must be >= 1 (got %d)", d->C);
  if (d->dtype != TTT_F32 && d->dtype != TTT_BF16) return fail(TTT_ERR_INVALID_ARG, "invalid dtype %d", d->dtype);
  if (d->loss != TTT_LOSS_MSE && d->loss != TTT_LOSS_IP && d->loss != TTT_LOSS_L1 && d->loss != TTT_LOSS_RMSE)
    return fail(TTT_ERR_INVALID_ARG, "invalid loss %d", d->loss);
  if (d->act != TTT_ACT_NONE && d->act != TTT_ACT_SILU && d->act != TTT_ACT_GELU && d->act != TTT_ACT_NORM)
    return fail(TTT_ERR_INVALID_ARG, "invalid act %d", d->act);
  if (d->decay < TTT_DECAY_NONE || d->decay > TTT_DECAY_VECTOR)
    return fail(TTT_ERR_INVALID_ARG, "invalid decay %d", d->decay);
  if ((d->act == TTT_ACT_NORM || d->loss == TTT_LOSS_RMSE) && d->decay == TTT_DECAY_VECTOR)
    return fail(TTT_ERR_UNSUPPORTED, "the Norm act and the RMSE loss take no vector decay");
  if (!std::isfinite(d->lr_bias)) return fail(TTT_ERR_INVALID_ARG, "lr_bias must be finite");
  if (d->dk > kMaxDim || d->dv > kMaxDim)
    return fail(TTT_ERR_UNSUPPORTED, "dk, dv must be <= %d (got %d, %d)", kMaxDim, d->dk, d->dv);
  if (d->C > kMaxDim) return fail(TTT_ERR_UNSUPPORTED, "chunk length C must be <= %d (got %d)", kMaxDim, d->C);
  // Element counts must stay well inside int64 and the per-chain index math.
  const double elems = static_cast<double>(d->B) * d->H * d->T * (d->dk > d->dv ? d->dk : d->dv);
  if (elems > 4.0e12) return fail(TTT_ERR_UNSUPPORTED, "problem too large (%.3g elements)", elems);
  if (static_cast<double>(d->T) * (d->dk > d->dv ? d->dk : d->dv) > 2.0e9)
    return fail(TTT_ERR_UNSUPPORTED, "T * d too large for one chain");
  return TTT_OK;
}

ttt::FwdArgs make_fwd(const ttt_desc* d) {
  ttt::FwdArgs a{};
  a.B = d->B; a.H = d->H; a.T = d->T; a.dk = d->dk; a.dv = d->dv; a.C = d->C;
  a.NC = (d->T + d->C - 1) / d->C;
  a.dtype = d->dtype; a.loss = d->loss; a.act = d->act; a.decay = d->decay;
  a.b = d->lr_bias;
  return a;
}

ttt::BwdArgs make_bwd(const ttt_desc* d) {
  ttt::BwdArgs a{};
  a.B = d->B; a.H = d->H; a.T = d->T; a.dk = d->dk; a.dv = d->dv; a.C = d->C;
  a.NC = (d->T + d->C - 1) / d->C;
  a.dtype = d->dtype; a.loss = d->loss; a.act = d->act; a.decay = d->decay;
  a.b = d->lr_bias;
  return a;
}

// The row path (one workgroup per chain on the fp32 tile GEMM, ttt_norm.hip)
// takes the Norm act and the RMSE loss (they couple a token's features), and
// every problem without a vector decay that the bf16 matrix-core kernels do
// not take: fp32 inputs and the other widths and chunk lengths.  The VALU path
// keeps vector decay outside the matrix-core kernels.
bool row_fwd(const ttt::FwdArgs& a) {
  return a.act == TTT_ACT_NORM || a.loss == TTT_LOSS_RMSE ||
         (a.decay != TTT_DECAY_VECTOR && !ttt::mfma_fwd_supported(a));
}
bool row_bwd(const ttt::BwdArgs& a) {
  return a.act == TTT_ACT_NORM || a.loss == TTT_LOSS_RMSE ||
         (a.decay != TTT_DECAY_VECTOR && !ttt::mfma_bwd_supported(a));
}

size_t fwd_ws(const ttt::FwdArgs& a) {
  if (row_fwd(a)) return ttt::norm_fwd_workspace(a);
  return ttt::mfma_fwd_supported(a) ? ttt::mfma_fwd_workspace(a) : ttt::generic_fwd_workspace(a);
}
size_t bwd_ws(const ttt::BwdArgs& a) {
  if (row_bwd(a)) return ttt::norm_bwd_workspace(a);
  return ttt::mfma_bwd_supported(a) ? ttt::mfma_bwd_workspace(a) : ttt::generic_bwd_workspace(a);
}
size_t saved_bytes(const ttt::FwdArgs& a) {
  if (a.act == TTT_ACT_NORM || a.loss == TTT_LOSS_RMSE || !ttt::mfma_saved_supported(a)) return 0;
  return ttt::mfma_saved_layout(a.B, a.H, a.T, a.dk, a.dv, a.C, a.NC, a.act, a.decay, nullptr, nullptr);
}

}  // namespace

int ttt::device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

namespace {

// Tensors are moved in 16-byte pieces: every vector-accessed pointer must be
// 16-byte aligned.  Returns the first offending name, or nullptr.
const char* misaligned(std::initializer_list<std::pair<const char*, const void*>> ptrs) {
  for (const auto& p : ptrs)
    if (p.second && (reinterpret_cast<uintptr_t>(p.second) & 15u)) return p.first;
  return nullptr;
}

constexpr int kMaxHidden = 1024;

int check_mlp_desc(const ttt_mlp_desc* d) {
  if (!d) return fail(TTT_ERR_INVALID_ARG, "desc is NULL");
  if (d->B < 0 || d->H < 0 || d->T < 0)
    return fail(TTT_ERR_INVALID_ARG, "B, H, T must be >= 0 (got %d, %d, %d)", d->B, d->H, d->T);
  if (d->dk < 1 || d->dh < 1 || d->dv < 1)
    return fail(TTT_ERR_INVALID_ARG, "dk, dh, dv must be >= 1 (got %d, %d, %d)", d->dk, d->dh, d->dv);
  if (d->C < 1) return fail(TTT_ERR_INVALID_ARG, "chunk length C must be >= 1 (got %d)", d->C);
  if (d->dtype != TTT_F32 && d->dtype != TTT_BF16) return fail(TTT_ERR_INVALID_ARG, "invalid dtype %d", d->dtype);
  if (d->loss != TTT_LOSS_MSE && d->loss != TTT_LOSS_IP && d->loss != TTT_LOSS_L1 && d->loss != TTT_LOSS_RMSE)
    return fail(TTT_ERR_INVALID_ARG, "invalid loss %d", d->loss);
  if (d->act != TTT_ACT_NONE && d->act != TTT_ACT_SILU && d->act != TTT_ACT_GELU)
    return fail(TTT_ERR_INVALID_ARG, "invalid act %d for the two-layer fast net", d->act);
  if (d->decay == TTT_DECAY_VECTOR)
    return fail(TTT_ERR_UNSUPPORTED, "the two-layer fast net takes no vector decay");
  if (d->decay != TTT_DECAY_NONE && d->decay != TTT_DECAY_SCALAR)
    return fail(TTT_ERR_INVALID_ARG, "invalid decay %d", d->decay);
  if (!std::isfinite(d->lr_bias)) return fail(TTT_ERR_INVALID_ARG, "lr_bias must be finite");
  if (d->dk > kMaxDim || d->dv > kMaxDim || d->dh > kMaxHidden)
    return fail(TTT_ERR_UNSUPPORTED, "need dk, dv <= %d and dh <= %d (got %d, %d, %d)", kMaxDim, kMaxHidden, d->dk,
                d->dv, d->dh);
  if (d->C > kMaxDim) return fail(TTT_ERR_UNSUPPORTED, "chunk length C must be <= %d (got %d)", kMaxDim, d->C);
  const int dmax = d->dk > d->dv ? d->dk : d->dv;
  if (static_cast<double>(d->B) * d->H * d->T * dmax > 4.0e12 || static_cast<double>(d->T) * dmax > 2.0e9)
    return fail(TTT_ERR_UNSUPPORTED, "problem too large");
  return TTT_OK;
}

}  // namespace

extern "C" {

const char* ttt_last_error(void) { return g_err; }

const char* ttt_version(void) { return "libttt 0.1 gfx950"; }

int ttt_workspace_size(const ttt_desc* desc, int entry, size_t* bytes) {
  int st = check_desc(desc);
  if (st != TTT_OK) return st;
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  if (entry == TTT_ENTRY_FWD) {
    *bytes = fwd_ws(make_fwd(desc));
  } else if (entry == TTT_ENTRY_BWD) {
    *bytes = bwd_ws(make_bwd(desc));
  } else {
    return fail(TTT_ERR_INVALID_ARG, "invalid entry %d (0 = forward, 1 = backward)", entry);
  }
  return ok();
}

int ttt_saved_size(const ttt_desc* desc, size_t* bytes) {
  int st = check_desc(desc);
  if (st != TTT_OK) return st;
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = saved_bytes(make_fwd(desc));
  return ok();
}

int ttt_chunk_fwd(const ttt_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                  const float* gamma, const float* log_decay, const float* w0, void* o, float* w_final,
                  float* w_ckpt, void* saved, void* ws, size_t ws_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != TTT_OK) return st;
  const bool work = static_cast<int64_t>(desc->B) * desc->H * desc->T > 0;
  if (work && (!q || !k || !v || !beta || !o))
    return fail(TTT_ERR_INVALID_ARG, "q, k, v, beta and o are required");
  if (desc->decay == TTT_DECAY_SCALAR && !gamma) return fail(TTT_ERR_INVALID_ARG, "SCALAR decay needs gamma");
  if (desc->decay == TTT_DECAY_VECTOR && !log_decay && work)
    return fail(TTT_ERR_INVALID_ARG, "VECTOR decay needs log_decay");
  if (const char* bad = misaligned({{"q", q}, {"k", k}, {"v", v}, {"log_decay", log_decay}, {"w0", w0}, {"o", o},
                                    {"w_final", w_final}, {"w_ckpt", w_ckpt}, {"saved", saved}, {"ws", ws}}))
    return fail(TTT_ERR_INVALID_ARG, "%s must be 16-byte aligned", bad);
  ttt::FwdArgs a = make_fwd(desc);
  const size_t need = fwd_ws(a);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu%s", need, ws_bytes,
                ws ? "" : " (NULL)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t BH = static_cast<int64_t>(desc->B) * desc->H;
  if (BH == 0) return ok();
  if (desc->T == 0) {  // no tokens: the state passes through unchanged
    if (w_final) {
      const size_t bytes = sizeof(float) * BH * desc->dk * desc->dv;
      hipError_t e = w0 ? hipMemcpyAsync(w_final, w0, bytes, hipMemcpyDeviceToDevice, s)
                        : hipMemsetAsync(w_final, 0, bytes, s);
      if (e != hipSuccess) return hip_fail(e, "ttt_chunk_fwd (T = 0)");
    }
    return ok();
  }
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.gamma = gamma; a.log_decay = log_decay; a.w0 = w0;
  a.o = o; a.w_final = w_final; a.w_ckpt = w_ckpt; a.ws = static_cast<char*>(ws); a.ws_bytes = ws_bytes;
  a.saved = (saved && saved_bytes(a) > 0) ? static_cast<char*>(saved) : nullptr;
  hipError_t e = row_fwd(a) ? ttt::norm_fwd_launch(a, s)
                 : ttt::mfma_fwd_supported(a) ? ttt::mfma_fwd_launch(a, s)
                                              : ttt::generic_fwd_launch(a, s);
  if (e != hipSuccess) return hip_fail(e, "ttt_chunk_fwd launch");
  return ok();
}

int ttt_chunk_bwd(const ttt_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                  const float* gamma, const float* log_decay, const float* w0, const float* w_ckpt,
                  const void* saved, const void* d_o, const float* d_wfinal, void* dq, void* dk, void* dv,
                  float* dbeta, float* dgamma, float* dlog_decay, float* dw0, void* ws, size_t ws_bytes,
                  void* stream) {
  (void)w0;  // the checkpoints already hold W_0
  int st = check_desc(desc);
  if (st != TTT_OK) return st;
  const bool work = static_cast<int64_t>(desc->B) * desc->H * desc->T > 0;
  if (work && (!q || !k || !v || !beta || !w_ckpt || !d_o || !dq || !dk || !dv || !dbeta))
    return fail(TTT_ERR_INVALID_ARG, "q, k, v, beta, w_ckpt, d_o, dq, dk, dv and dbeta are required");
  if (desc->decay == TTT_DECAY_SCALAR && (!gamma || !dgamma))
    return fail(TTT_ERR_INVALID_ARG, "SCALAR decay needs gamma and dgamma");
  if (desc->decay == TTT_DECAY_VECTOR && work && (!log_decay || !dlog_decay))
    return fail(TTT_ERR_INVALID_ARG, "VECTOR decay needs log_decay and dlog_decay");
  if (const char* bad = misaligned({{"q", q}, {"k", k}, {"v", v}, {"log_decay", log_decay}, {"w_ckpt", w_ckpt},
                                    {"saved", saved}, {"d_o", d_o}, {"d_wfinal", d_wfinal}, {"dq", dq},
                                    {"dk", dk}, {"dv", dv}, {"dlog_decay", dlog_decay}, {"dw0", dw0}, {"ws", ws}}))
    return fail(TTT_ERR_INVALID_ARG, "%s must be 16-byte aligned", bad);
  ttt::BwdArgs a = make_bwd(desc);
  const size_t need = bwd_ws(a);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu%s", need, ws_bytes,
                ws ? "" : " (NULL)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t BH = static_cast<int64_t>(desc->B) * desc->H;
  if (BH == 0) return ok();
  if (desc->T == 0) {  // no tokens: dW0 = dW_T, dgamma = 0
    const size_t bytes = sizeof(float) * BH * desc->dk * desc->dv;
    hipError_t e = hipSuccess;
    if (dw0)
      e = d_wfinal ? hipMemcpyAsync(dw0, d_wfinal, bytes, hipMemcpyDeviceToDevice, s) : hipMemsetAsync(dw0, 0, bytes, s);
    if (e == hipSuccess && desc->decay == TTT_DECAY_SCALAR) e = hipMemsetAsync(dgamma, 0, sizeof(float) * BH, s);
    if (e != hipSuccess) return hip_fail(e, "ttt_chunk_bwd (T = 0)");
    return ok();
  }
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.gamma = gamma; a.log_decay = log_decay; a.w0 = w0;
  a.w_ckpt = w_ckpt; a.d_o = d_o; a.d_wfinal = d_wfinal; a.dq = dq; a.dk_out = dk; a.dv_out = dv;
  a.dbeta = dbeta; a.dgamma = dgamma; a.dlog_decay = dlog_decay; a.dw0 = dw0;
  a.ws = static_cast<char*>(ws); a.ws_bytes = ws_bytes;
  a.saved = (saved && saved_bytes(make_fwd(desc)) > 0) ? static_cast<const char*>(saved) : nullptr;
  hipError_t e = row_bwd(a) ? ttt::norm_bwd_launch(a, s)
                 : ttt::mfma_bwd_supported(a) ? ttt::mfma_bwd_launch(a, s)
                                              : ttt::generic_bwd_launch(a, s);
  if (e != hipSuccess) return hip_fail(e, "ttt_chunk_bwd launch");
  return ok();
}

static int inplace_check(int B, int T, int d_model, int d_ff, int C) {
  if (B < 0 || T < 0) return fail(TTT_ERR_INVALID_ARG, "B, T must be >= 0 (got %d, %d)", B, T);
  if (d_model < 1 || d_ff < 1 || C < 1)
    return fail(TTT_ERR_INVALID_ARG, "d_model, d_ff, C must be >= 1 (got %d, %d, %d)", d_model, d_ff, C);
  if (d_model % 8 != 0 || d_ff % 8 != 0)
    return fail(TTT_ERR_UNSUPPORTED, "d_model and d_ff must be multiples of 8 (got %d, %d)", d_model, d_ff);
  if (static_cast<double>(T) * (d_ff > d_model ? d_ff : d_model) > 4.0e12 ||
      static_cast<double>(d_model) * d_ff > 2.0e9)
    return fail(TTT_ERR_UNSUPPORTED, "problem too large");
  return TTT_OK;
}

// doc_starts: n_docs flat positions b * T + t, 0 < t < T, strictly increasing.
static int check_doc_starts(const int64_t* doc_starts, int n_docs, int B, int T) {
  if (n_docs < 0) return fail(TTT_ERR_INVALID_ARG, "n_docs must be >= 0");
  if (n_docs > 0 && !doc_starts) return fail(TTT_ERR_INVALID_ARG, "doc_starts is NULL with n_docs > 0");
  const int64_t BT = static_cast<int64_t>(B) * T;
  for (int i = 0; i < n_docs; ++i) {
    const int64_t p = doc_starts[i];
    if (p <= 0 || p >= BT || p % T == 0)
      return fail(TTT_ERR_INVALID_ARG, "doc_starts[%d] = %lld is not b*T + t with 0 < t < T", i,
                  static_cast<long long>(p));
    if (i > 0 && p <= doc_starts[i - 1])
      return fail(TTT_ERR_INVALID_ARG, "doc_starts must be strictly increasing (entry %d)", i);
  }
  return TTT_OK;
}

int inplace_ttt_workspace_size(int B, int T, int d_model, int d_ff, int C, size_t* bytes) {
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  const int st = inplace_check(B, T, d_model, d_ff, C);
  if (st != TTT_OK) return st;
  *bytes = ttt::inplace_workspace_bytes(B, T, d_model, d_ff, C);
  return ok();
}

int inplace_ttt_fwd(int B, int T, int d_model, int d_ff, int C, float eta, const void* z, const void* vhat,
                    float* w_down, void* o, void* ws, size_t ws_bytes, void* stream) {
  const int st = inplace_check(B, T, d_model, d_ff, C);
  if (st != TTT_OK) return st;
  if (!std::isfinite(eta)) return fail(TTT_ERR_INVALID_ARG, "eta must be finite");
  if (static_cast<int64_t>(B) * T == 0) return ok();
  if (!z || !vhat || !w_down || !o) return fail(TTT_ERR_INVALID_ARG, "z, vhat, w_down and o are required");
  if (const char* bad = misaligned({{"z", z}, {"vhat", vhat}, {"w_down", w_down}, {"o", o}, {"ws", ws}}))
    return fail(TTT_ERR_INVALID_ARG, "%s must be 16-byte aligned", bad);
  hipError_t e = ttt::inplace_launch(B, T, d_model, d_ff, C, eta, z, vhat, w_down, o, ws, ws ? ws_bytes : 0,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "inplace_ttt_fwd launch");
  return ok();
}

int inplace_ttt_bwd_workspace_size(int B, int T, int d_model, int d_ff, int C, size_t* bytes) {
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  const int st = inplace_check(B, T, d_model, d_ff, C);
  if (st != TTT_OK) return st;
  *bytes = ttt::inplace_bwd_workspace_bytes(B, T, d_model, d_ff, C);
  return ok();
}

int inplace_ttt_bwd(int B, int T, int d_model, int d_ff, int C, float eta, const void* z, const void* vhat,
                    const float* w_final, const void* d_o, const float* d_wfinal, void* dz, void* dvhat, float* dw0,
                    void* ws, size_t ws_bytes, void* stream) {
  const int st = inplace_check(B, T, d_model, d_ff, C);
  if (st != TTT_OK) return st;
  if (!std::isfinite(eta)) return fail(TTT_ERR_INVALID_ARG, "eta must be finite");
  if (static_cast<int64_t>(B) * T == 0) return ok();
  if (!z || !vhat || !w_final || !d_o || !dz || !dvhat || !dw0)
    return fail(TTT_ERR_INVALID_ARG, "z, vhat, w_final, d_o, dz, dvhat and dw0 are required");
  const size_t need = ttt::inplace_bwd_workspace_bytes(B, T, d_model, d_ff, C);
  if (!ws || ws_bytes < need)
    return fail(TTT_ERR_WORKSPACE, "workspace of at least %zu bytes required (got %zu)", need,
                ws ? ws_bytes : static_cast<size_t>(0));
  if (const char* bad = misaligned({{"z", z}, {"vhat", vhat}, {"w_final", w_final}, {"d_o", d_o},
                                    {"d_wfinal", d_wfinal}, {"dz", dz}, {"dvhat", dvhat}, {"dw0", dw0}, {"ws", ws}}))
    return fail(TTT_ERR_INVALID_ARG, "%s must be 16-byte aligned", bad);
  hipError_t e = ttt::inplace_bwd_launch(B, T, d_model, d_ff, C, eta, z, vhat, w_final, d_o, d_wfinal, dz, dvhat, dw0,
                                         ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "inplace_ttt_bwd launch");
  return ok();
}

int inplace_ttt_guarded_workspace_size(int B, int T, int d_model, int d_ff, int C, size_t* bytes) {
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  const int st = inplace_check(B, T, d_model, d_ff, C);
  if (st != TTT_OK) return st;
  *bytes = ttt::inplace_guarded_workspace_bytes(B, T, d_model, d_ff, C);
  return ok();
}

int inplace_ttt_fwd_guarded(int B, int T, int d_model, int d_ff, int C, float eta, float clip_tau,
                            const int64_t* doc_starts, int n_docs, const void* z, const void* vhat,
                            const float* w_init, float* w_down, void* o, void* ws, size_t ws_bytes, void* stream) {
  const int st = inplace_check(B, T, d_model, d_ff, C);
  if (st != TTT_OK) return st;
  if (!std::isfinite(eta)) return fail(TTT_ERR_INVALID_ARG, "eta must be finite");
  if (std::isnan(clip_tau) || clip_tau < 0.0f) return fail(TTT_ERR_INVALID_ARG, "clip_tau must be >= 0 (0 or inf: off)");
  const int dst = check_doc_starts(doc_starts, n_docs, B, T);
  if (dst != TTT_OK) return dst;
  if (static_cast<int64_t>(B) * T == 0) return ok();
  if (!z || !vhat || !w_down || !o) return fail(TTT_ERR_INVALID_ARG, "z, vhat, w_down and o are required");
  if (n_docs > 0 && !w_init) return fail(TTT_ERR_INVALID_ARG, "w_init is required with document starts");
  const bool clip = clip_tau > 0.0f && std::isfinite(clip_tau);
  const size_t need = ttt::inplace_guarded_workspace_bytes(B, T, d_model, d_ff, C) -
                      ttt::inplace_workspace_bytes(B, T, d_model, d_ff, C);
  if (clip && (!ws || ws_bytes < need))
    return fail(TTT_ERR_WORKSPACE, "clipping needs a workspace of at least %zu bytes (got %zu)", need,
                ws ? ws_bytes : static_cast<size_t>(0));
  if (const char* bad = misaligned({{"z", z}, {"vhat", vhat}, {"w_init", w_init}, {"w_down", w_down}, {"o", o},
                                    {"ws", ws}}))
    return fail(TTT_ERR_INVALID_ARG, "%s must be 16-byte aligned", bad);
  hipError_t e = ttt::inplace_launch_guarded(B, T, d_model, d_ff, C, eta, clip_tau, doc_starts, n_docs, z, vhat,
                                             w_init, w_down, o, ws, ws ? ws_bytes : 0,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "inplace_ttt_fwd_guarded launch");
  return ok();
}

int inplace_ttt_bwd_guarded_workspace_size(int B, int T, int d_model, int d_ff, int C, size_t* bytes) {
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  const int st = inplace_check(B, T, d_model, d_ff, C);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(B) * T > 0 && !ttt::inplace_bwd_guarded_supported(T, d_model, d_ff, C))
    return fail(TTT_ERR_UNSUPPORTED, "the guarded backward needs min(T, C) <= 8192 and the tile path's sizes");
  *bytes = ttt::inplace_bwd_guarded_workspace_bytes(B, T, d_model, d_ff, C);
  return ok();
}

int inplace_ttt_bwd_guarded(int B, int T, int d_model, int d_ff, int C, float eta, float clip_tau,
                            const int64_t* doc_starts, int n_docs, const void* z, const void* vhat, const float* w0,
                            const float* w_init, const float* w_final, const void* d_o, const float* d_wfinal,
                            void* dz, void* dvhat, float* dw0, float* dw_init, void* ws, size_t ws_bytes,
                            void* stream) {
  const int st = inplace_check(B, T, d_model, d_ff, C);
  if (st != TTT_OK) return st;
  if (!std::isfinite(eta)) return fail(TTT_ERR_INVALID_ARG, "eta must be finite");
  if (std::isnan(clip_tau) || clip_tau < 0.0f) return fail(TTT_ERR_INVALID_ARG, "clip_tau must be >= 0 (0 or inf: off)");
  const int dst = check_doc_starts(doc_starts, n_docs, B, T);
  if (dst != TTT_OK) return dst;
  if (static_cast<int64_t>(B) * T == 0) return ok();
  if (!ttt::inplace_bwd_guarded_supported(T, d_model, d_ff, C))
    return fail(TTT_ERR_UNSUPPORTED, "the guarded backward needs min(T, C) <= 8192 and the tile path's sizes");
  if (!z || !vhat || !w_final || !d_o || !dz || !dvhat || !dw0)
    return fail(TTT_ERR_INVALID_ARG, "z, vhat, w_final, d_o, dz, dvhat and dw0 are required");
  if (n_docs > 0 && (!w0 || !w_init))
    return fail(TTT_ERR_INVALID_ARG, "w0 and w_init are required with document starts");
  const size_t need = ttt::inplace_bwd_guarded_workspace_bytes(B, T, d_model, d_ff, C);
  if (!ws || ws_bytes < need)
    return fail(TTT_ERR_WORKSPACE, "workspace of at least %zu bytes required (got %zu)", need,
                ws ? ws_bytes : static_cast<size_t>(0));
  if (const char* bad = misaligned({{"z", z}, {"vhat", vhat}, {"w0", w0}, {"w_init", w_init}, {"w_final", w_final},
                                    {"d_o", d_o}, {"d_wfinal", d_wfinal}, {"dz", dz}, {"dvhat", dvhat}, {"dw0", dw0},
                                    {"dw_init", dw_init}, {"ws", ws}}))
    return fail(TTT_ERR_INVALID_ARG, "%s must be 16-byte aligned", bad);
  hipError_t e = ttt::inplace_bwd_guarded_launch(B, T, d_model, d_ff, C, eta, clip_tau, doc_starts, n_docs, z, vhat,
                                                 w0, w_init, w_final, d_o, d_wfinal, dz, dvhat, dw0, dw_init, ws,
                                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "inplace_ttt_bwd_guarded launch");
  return ok();
}

int ttt_mlp_workspace_size(const ttt_mlp_desc* desc, size_t* bytes) {
  const int st = check_mlp_desc(desc);
  if (st != TTT_OK) return st;
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ttt::mlp_fwd_workspace(*desc);
  return ok();
}

int ttt_mlp_chunk_fwd(const ttt_mlp_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                      const float* gamma, const float* w1_0, const float* w2_0, void* o, float* w1_final,
                      float* w2_final, float* w1_ckpt, float* w2_ckpt, void* saved, void* ws, size_t ws_bytes,
                      void* stream) {
  const int st = check_mlp_desc(desc);
  if (st != TTT_OK) return st;
  const int64_t BH = static_cast<int64_t>(desc->B) * desc->H;
  const bool work = BH * desc->T > 0;
  if (work && (!q || !k || !v || !beta || !o))
    return fail(TTT_ERR_INVALID_ARG, "q, k, v, beta and o are required");
  if (desc->decay == TTT_DECAY_SCALAR && !gamma) return fail(TTT_ERR_INVALID_ARG, "SCALAR decay needs gamma");
  if (const char* bad = misaligned({{"q", q}, {"k", k}, {"v", v}, {"w1_0", w1_0}, {"w2_0", w2_0}, {"o", o},
                                    {"w1_final", w1_final}, {"w2_final", w2_final}, {"w1_ckpt", w1_ckpt},
                                    {"w2_ckpt", w2_ckpt}, {"saved", saved}, {"ws", ws}}))
    return fail(TTT_ERR_INVALID_ARG, "%s must be 16-byte aligned", bad);
  const size_t need = ttt::mlp_fwd_workspace(*desc);
  if (work && (!ws || ws_bytes < need))
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu%s", need, ws_bytes,
                ws ? "" : " (NULL)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (BH == 0) return ok();
  if (desc->T == 0) {  // no tokens: the state passes through unchanged
    const std::pair<float*, const float*> w[2] = {{w1_final, w1_0}, {w2_final, w2_0}};
    const size_t n[2] = {static_cast<size_t>(desc->dk) * desc->dh, static_cast<size_t>(desc->dh) * desc->dv};
    for (int i = 0; i < 2; ++i) {
      if (!w[i].first) continue;
      const size_t bytes = sizeof(float) * BH * n[i];
      hipError_t e = w[i].second ? hipMemcpyAsync(w[i].first, w[i].second, bytes, hipMemcpyDeviceToDevice, s)
                                 : hipMemsetAsync(w[i].first, 0, bytes, s);
      if (e != hipSuccess) return hip_fail(e, "ttt_mlp_chunk_fwd (T = 0)");
    }
    return ok();
  }
  hipError_t e = ttt::mlp_fwd_launch(*desc, q, k, v, beta, gamma, w1_0, w2_0, o, w1_final, w2_final, w1_ckpt,
                                     w2_ckpt, saved, ws, s);
  if (e != hipSuccess) return hip_fail(e, "ttt_mlp_chunk_fwd launch");
  return ok();
}

int ttt_mlp_saved_size(const ttt_mlp_desc* desc, size_t* bytes) {
  const int st = check_mlp_desc(desc);
  if (st != TTT_OK) return st;
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ttt::mlp_saved_bytes(*desc);
  return ok();
}

int ttt_mlp_bwd_workspace_size(const ttt_mlp_desc* desc, size_t* bytes) {
  const int st = check_mlp_desc(desc);
  if (st != TTT_OK) return st;
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ttt::mlp_bwd_workspace(*desc);
  return ok();
}

int ttt_mlp_chunk_bwd(const ttt_mlp_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                      const float* gamma, const float* w1_ckpt, const float* w2_ckpt, const void* saved,
                      const void* d_o, const float* d_w1final, const float* d_w2final, void* dq, void* dk, void* dv,
                      float* dbeta, float* dgamma, float* dw1_0, float* dw2_0, void* ws, size_t ws_bytes,
                      void* stream) {
  const int st = check_mlp_desc(desc);
  if (st != TTT_OK) return st;
  const int64_t BH = static_cast<int64_t>(desc->B) * desc->H;
  const bool work = BH * desc->T > 0;
  if (work && (!q || !k || !v || !beta || !w1_ckpt || !w2_ckpt || !d_o || !dq || !dk || !dv || !dbeta))
    return fail(TTT_ERR_INVALID_ARG, "q, k, v, beta, w1_ckpt, w2_ckpt, d_o, dq, dk, dv and dbeta are required");
  if (desc->decay == TTT_DECAY_SCALAR && BH > 0 && (!gamma || !dgamma))
    return fail(TTT_ERR_INVALID_ARG, "SCALAR decay needs gamma and dgamma");
  if (const char* bad = misaligned({{"q", q}, {"k", k}, {"v", v}, {"w1_ckpt", w1_ckpt}, {"w2_ckpt", w2_ckpt},
                                    {"saved", saved}, {"d_o", d_o}, {"d_w1final", d_w1final}, {"d_w2final", d_w2final}, {"dq", dq},
                                    {"dk", dk}, {"dv", dv}, {"dw1_0", dw1_0}, {"dw2_0", dw2_0}, {"ws", ws}}))
    return fail(TTT_ERR_INVALID_ARG, "%s must be 16-byte aligned", bad);
  const size_t need = ttt::mlp_bwd_workspace(*desc);
  if (work && (!ws || ws_bytes < need))
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu%s", need, ws_bytes,
                ws ? "" : " (NULL)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (BH == 0) return ok();
  if (desc->T == 0) {  // no tokens: dW_0 = dW_T and nothing reaches gamma
    const std::pair<float*, const float*> w[2] = {{dw1_0, d_w1final}, {dw2_0, d_w2final}};
    const size_t n[2] = {static_cast<size_t>(desc->dk) * desc->dh, static_cast<size_t>(desc->dh) * desc->dv};
    for (int i = 0; i < 2; ++i) {
      if (!w[i].first) continue;
      const size_t bytes = sizeof(float) * BH * n[i];
      hipError_t e = w[i].second ? hipMemcpyAsync(w[i].first, w[i].second, bytes, hipMemcpyDeviceToDevice, s)
                                 : hipMemsetAsync(w[i].first, 0, bytes, s);
      if (e != hipSuccess) return hip_fail(e, "ttt_mlp_chunk_bwd (T = 0)");
    }
    if (desc->decay == TTT_DECAY_SCALAR) {
      hipError_t e = hipMemsetAsync(dgamma, 0, sizeof(float) * BH, s);
      if (e != hipSuccess) return hip_fail(e, "ttt_mlp_chunk_bwd (T = 0)");
    }
    return ok();
  }
  hipError_t e = ttt::mlp_bwd_launch(*desc, q, k, v, beta, gamma, w1_ckpt, w2_ckpt, saved, d_o, d_w1final,
                                     d_w2final, dq, dk, dv, dbeta, dgamma, dw1_0, dw2_0, ws, s);
  if (e != hipSuccess) return hip_fail(e, "ttt_mlp_chunk_bwd launch");
  return ok();
}

}  // extern "C"
