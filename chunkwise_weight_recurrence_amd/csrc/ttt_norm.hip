// The fast net Linear -> Norm (the Norm primitive) as the act of the chunkwise
// layer (TTT_ACT_NORM), and the other row-coupled or fp32 problems of the row
// path: forward and analytic outer backward on the tile GEMM of tile_gemm.h.
// Only the state (forward) and its adjoint (backward) carry a chain from chunk
// to chunk, so each direction is a sequential kernel with one workgroup per
// chain that does just that carry, beside a kernel with one workgroup per
// (chain, chunk) for everything else (the forward's query view; the backward's
// recomputed forward and its terms free of the carried adjoint).
//
// The Modular TTT summary page composes a fast net's chunk computation from its
// primitives' rules (section "Method step details", Algorithm 1) and names Norm
// among them, with a hand-written backward (sections "Experimental results" and
// "Technical novelty").  Here V_hat = N(K W), N the per-token normalisation over
// the d_v features, and the query view reads O = N(Y).

#include <type_traits>

#include "tile_gemm.h"
#include "ttt_device.h"
#include "ttt_internal.h"

namespace ttt {
namespace {

// ---------------------------------------------------------------------------
// The fast net Linear -> Norm (the Norm primitive): V_hat = N(K W) with the
// per-token normalisation N(z) = (z - mean(z)) / s(z), s(z) = sqrt(var(z) + eps)
// over the d_v features; the query view O = N(Y) with the Linear's dual form Y.
// The normalisation couples a token's features, so a workgroup holds whole
// rows (no column split); the products use the tile GEMM and the per-token
// steps are one wave per row.
// ---------------------------------------------------------------------------

constexpr float kNormEps = 1e-5f;

// The backward sweep's row pass walks a wave's rows t, t + 8, ...; each row's
// values come from global memory, so a row's loads would wait out a full memory
// latency.  prefetch_row loads the first 64 values of the wave's next row
// (clamped into the chunk) from each given array, and keep_live hands them to
// an empty asm statement after the current row's work: the loads are issued
// before that work and waited for after it, so the next row's lines arrive
// meanwhile.
template <int N>
__device__ __forceinline__ void prefetch_row(float (&pf)[N], const float* const (&rows)[N], int t, int c, int w,
                                             int lane) {
  const int tn = min(t + kThreads / 64, c - 1), j = min(lane, w - 1);
#pragma unroll
  for (int i = 0; i < N; ++i) pf[i] = rows[i][static_cast<int64_t>(tn) * w + j];
}
template <int N>
__device__ __forceinline__ void keep_live(const float (&pf)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(pf[i]));
}

// Per-chain scratch of the forward's sequential kernel (floats): the state's two
// buffers, the chunk's staged K and V, and Z.
struct NormScratch {
  int64_t w[2], k, v, z, total;
  __host__ __device__ NormScratch(int C, int dk, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t kv = static_cast<int64_t>(dk) * dv, cv = static_cast<int64_t>(C) * dv,
                  ck = static_cast<int64_t>(C) * dk;
    w[0] = take(kv); w[1] = take(kv);
    k = take(ck); v = take(cv); z = take(cv);
    total = o;
  }
};

// Row t of the train view.  V_hat = N(z) (ACT 3) or f(z) (ACT 0..2); the loss
// signal E (LOSS 3 = RMSE: e / (sqrt(d) ||e||), e = V_hat - v, 0 where e = 0);
// G = J_N^T E = (E - mean E - n <E, n> / d) / s (Norm) or E (.) f'(z).  Returns
// 1/s (Norm) in rs_out and 1 / (sqrt(d) ||e||) (RMSE) in ri_out.
template <int LOSS, int ACT>
__device__ __forceinline__ void train_row(const float* z, const float* vv, float* vh, float* e, float* G, float* Gh,
                                          float& rs_out, float& ri_out, float et, int dv, int lane) {
  float mu = 0.0f, rs = 1.0f;
  if constexpr (ACT == 3) {
    mu = row_sum(dv, lane, [&](int j) { return z[j]; }) / dv;
    const float var = row_sum(dv, lane, [&](int j) { return (z[j] - mu) * (z[j] - mu); });
    rs = rsqrtf(var / dv + kNormEps);
  }
  auto vhat = [&](int j) { return ACT == 3 ? (z[j] - mu) * rs : act_f<ACT>(z[j]); };
  float ri = 0.0f;
  if constexpr (LOSS == 3) {
    const float ne2 = row_sum(dv, lane, [&](int j) { const float d = vhat(j) - vv[j]; return d * d; });
    ri = ne2 > 0.0f ? rsqrtf(ne2 * dv) : 0.0f;
  }
  auto sig = [&](int j) { return LOSS == 3 ? (vhat(j) - vv[j]) * ri : loss_signal<LOSS, 0>(vhat(j), vv[j]); };
  float me = 0.0f, en = 0.0f;
  if constexpr (ACT == 3) {
    me = row_sum(dv, lane, [&](int j) { return sig(j); }) / dv;
    en = row_sum(dv, lane, [&](int j) { return sig(j) * vhat(j); }) / dv;
  }
  for (int j = lane; j < dv; j += 64) {
    const float nj = vhat(j), ej = sig(j);
    const float gj = (ACT == 3) ? (ej - me - nj * en) * rs : ej * act_df<ACT>(z[j]);
    if (vh) vh[j] = nj;
    if (e) e[j] = ej;
    if (G) G[j] = gj;
    Gh[j] = et * gj;
  }
  rs_out = rs;
  ri_out = ri;
}

// Forward workspace of the row path (floats): the per-chain NormScratch of the
// sequential kernel, then eta (.) G of every token ([B,H,T,dv]), the chunk-start
// states ([B,H,NC,dk,dv], used when the caller keeps no checkpoints) and one
// QueryScratch per (chain, chunk) for the query view.
// Few (chain, chunk) items: the query view splits each chunk's rows over
// workgroups of kQueryRows rows (norm_query_kernel<..., true>), each with its
// own copy of the keys.
constexpr int kQueryRows = 64;
__host__ __device__ inline bool row_query_split(const FwdArgs& a) { return a.B * a.H * a.NC < 256; }
struct QueryScratch {
  int64_t q, k, s, y, total;
  __host__ __device__ QueryScratch(int C, int dk, int dv, bool split = false) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    q = take(static_cast<int64_t>(C) * dk);
    k = take(static_cast<int64_t>(split ? (C + kQueryRows - 1) / kQueryRows : 1) * C * dk);  // a key copy per workgroup
    s = take(static_cast<int64_t>(C) * C);
    y = take(static_cast<int64_t>(C) * dv);
    total = o;
  }
};
struct RowFwdWs {
  int64_t gh, ckpt, query, total;
  __host__ __device__ explicit RowFwdWs(const FwdArgs& a) {
    const int64_t BH = static_cast<int64_t>(a.B) * a.H;
    gh = BH * NormScratch(a.C, a.dk, a.dv).total;
    ckpt = gh + BH * a.T * a.dv;
    query = ckpt + BH * a.NC * a.dk * a.dv;
    total = query + BH * a.NC * QueryScratch(a.C, a.dk, a.dv, row_query_split(a)).total;
  }
};

// The chunk-start states of the forward: the caller's checkpoints, or the workspace's.
__host__ __device__ inline float* row_ckpt(const FwdArgs& a, float* ws) {
  return a.w_ckpt ? a.w_ckpt : ws + RowFwdWs(a).ckpt;
}

// Sequential part of the forward, one workgroup per chain: the train view (Z =
// K W_i, the loss signal, eta (.) G to the workspace) and the state transition
// W_{i+1} = g (W_i - K^T (eta (.) G)), with W_i kept as the chunk's checkpoint.
// The query view needs only W_i and eta (.) G, so it runs afterwards for every
// chunk at once (norm_query_kernel).
template <typename T, int LOSS, int ACT>
__global__ __launch_bounds__(kThreads) void norm_fwd_kernel(FwdArgs a, float* scratch) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];
  __shared__ float eta[256];
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  const int bh = blockIdx.x;
  const int dk = a.dk, dv = a.dv, C = a.C;
  const NormScratch L(C, dk, dv);
  float* sc = scratch + static_cast<int64_t>(bh) * L.total;
  float* Z = sc + L.z;
  float* ghall = scratch + RowFwdWs(a).gh + static_cast<int64_t>(bh) * a.T * dv;
  float* ckpt = row_ckpt(a, scratch);
  const bool scalar_decay = a.decay == TTT_DECAY_SCALAR;
  const float g = scalar_decay ? a.gamma[bh % a.H] : 1.0f;
  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk, off_v = static_cast<int64_t>(bh) * a.T * dv;
  const T* k = static_cast<const T*>(a.k) + off_k;
  const T* v = static_cast<const T*>(a.v) + off_v;
  const float* beta = a.beta + static_cast<int64_t>(bh) * a.T;
  const int64_t nw = static_cast<int64_t>(dk) * dv;
  {
    float* W = sc + L.w[0];
    const float* src = a.w0 ? a.w0 + bh * nw : nullptr;
    for (int64_t i = tid; i < nw; i += kThreads) W[i] = src ? src[i] : 0.0f;
  }
  int cur = 0;
  for (int ci = 0; ci < a.NC; ++ci) {
    const int t0 = ci * C, c = min(C, a.T - t0);
    float* W = sc + (cur ? L.w[1] : L.w[0]);
    float* Wn = sc + (cur ? L.w[0] : L.w[1]);
    float* Gh = ghall + static_cast<int64_t>(t0) * dv;
    // fp32 inputs are read in place; other types as fp32 copies in the scratch
    const float *Kc, *Vc;
    if constexpr (std::is_same_v<T, float>) {
      Kc = k + static_cast<int64_t>(t0) * dk;
      Vc = v + static_cast<int64_t>(t0) * dv;
    } else {
      stage_rows<E, 32>(sc + L.k, k + static_cast<int64_t>(t0) * dk, c * dk);
      stage_rows<E, 32>(sc + L.v, v + static_cast<int64_t>(t0) * dv, c * dv);
      Kc = sc + L.k;
      Vc = sc + L.v;
    }
    for (int t = tid; t < c; t += kThreads) eta[t] = lr_gate(beta[t0 + t], a.b);
    stage_rows<Elem<float>>(ckpt + (static_cast<int64_t>(bh) * a.NC + ci) * nw, W, static_cast<int>(nw));
    __syncthreads();
    gemm1<0, 0>(c, dv, Term{Kc, dk, W, dv, dk, 1.0f}, kNoAux, lds,
                [&](int m, int n, float x, float, float, float) { Z[m * dv + n] = x; });
    __syncthreads();
    for (int t = wv; t < c; t += kThreads / 64) {
      float rs, ri;
      train_row<LOSS, ACT>(Z + t * dv, Vc + t * dv, nullptr, nullptr, nullptr, Gh + t * dv, rs, ri, eta[t], dv, lane);
    }
    __syncthreads();
    gemm1<1, 0>(dk, dv, Term{Kc, dk, Gh, dv, c, -1.0f}, Aux{{W, nullptr, nullptr}, dv}, lds,
                [&](int m, int n, float x, float w, float, float) { Wn[m * dv + n] = fmaf(g, w, x); });
    __syncthreads();
    cur ^= 1;
  }
  const float* W = sc + (cur ? L.w[1] : L.w[0]);
  if (a.w_final)
    for (int64_t i = tid; i < nw; i += kThreads) a.w_final[bh * nw + i] = W[i];
}

// Query view of one (chain, chunk): S = Tril(Q K^T), Y = Q W_i - S (eta (.) G),
// O = N(Y) or f(Y), from the chunk-start state and eta (.) G that the
// sequential kernel left; every chunk's workgroup runs at once.  With SPLIT a
// chunk's rows are dealt to kQueryRows-row workgroups (for few chains and
// chunks, where one workgroup per chunk would leave most CUs idle): workgroup
// (chain, chunk, r) forms rows r0 .. r0 + 63 of S (columns up to r0 + 63), Y
// and O.
template <typename T, int ACT, bool SPLIT>
__global__ __launch_bounds__(kThreads, 2) void norm_query_kernel(FwdArgs a, float* scratch) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  const int dk = a.dk, dv = a.dv, C = a.C;
  const int nrt = SPLIT ? (C + kQueryRows - 1) / kQueryRows : 1;
  const int item = blockIdx.x / nrt, rt = blockIdx.x % nrt;
  const int bh = item / a.NC, ci = item % a.NC;
  const int t0 = ci * C, c = min(C, a.T - t0);
  const int r0 = SPLIT ? rt * kQueryRows : 0;
  const int rows = SPLIT ? min(kQueryRows, c - r0) : c;  // this workgroup's rows
  if (rows <= 0) return;                                   // past a short last chunk (whole workgroup)
  const int ncol = r0 + rows;                              // key columns the rows reach
  const QueryScratch L(C, dk, dv, SPLIT);
  const RowFwdWs R(a);
  float* sc = scratch + R.query + static_cast<int64_t>(item) * L.total;
  float *S = sc + L.s + static_cast<int64_t>(r0) * C, *Y = sc + L.y + static_cast<int64_t>(r0) * dv;
  const float* Gh = scratch + R.gh + (static_cast<int64_t>(bh) * a.T + t0) * dv;
  const float* W = row_ckpt(a, scratch) + (static_cast<int64_t>(bh) * a.NC + ci) * dk * dv;
  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk, off_v = static_cast<int64_t>(bh) * a.T * dv;
  const T* q = static_cast<const T*>(a.q) + off_k;
  const T* k = static_cast<const T*>(a.k) + off_k;
  T* o = static_cast<T*>(a.o) + off_v;
  // fp32 inputs are read in place; other types as fp32 copies (a split
  // workgroup stages its rows of Q and its own copy of the keys it reaches)
  const float *Qc, *Kc;
  if constexpr (std::is_same_v<T, float>) {
    Qc = q + static_cast<int64_t>(t0 + r0) * dk;
    Kc = k + static_cast<int64_t>(t0) * dk;
  } else {
    float* qs = sc + L.q + static_cast<int64_t>(r0) * dk;
    float* ks = sc + L.k + static_cast<int64_t>(rt) * C * dk;
    stage_rows<E>(qs, q + static_cast<int64_t>(t0 + r0) * dk, rows * dk);
    stage_rows<E>(ks, k + static_cast<int64_t>(t0) * dk, ncol * dk);
    Qc = qs;
    Kc = ks;
    __syncthreads();
  }
  if constexpr (SPLIT) {
    gemm1<0, 1, false, 1>(rows, ncol, Term{Qc, dk, Kc, dk, dk, 1.0f}, kNoAux, lds,
                [&](int m, int n, float x, float, float, float) { S[m * C + n] = (n <= r0 + m) ? x : 0.0f; });
    __syncthreads();
    gemm<0, 0, 0, 0, false, false, 1>(rows, dv, Term{Qc, dk, W, dv, dk, 1.0f}, Term{S, C, Gh, dv, ncol, -1.0f}, kNoAux, lds,
                     [&](int m, int n, float x, float, float, float) { Y[m * dv + n] = x; });
  } else {
    gemm1<0, 1, true, 1>(c, c, Term{Qc, dk, Kc, dk, dk, 1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { S[m * C + n] = (n <= m) ? x : 0.0f; });
    __syncthreads();
    gemm<0, 0, 0, 0, false, true, 1>(c, dv, Term{Qc, dk, W, dv, dk, 1.0f}, Term{S, C, Gh, dv, c, -1.0f}, kNoAux, lds,
                                  [&](int m, int n, float x, float, float, float) { Y[m * dv + n] = x; });
  }
  __syncthreads();
  for (int t = wv; t < rows; t += kThreads / 64) {  // O = N(Y) or f(Y)
    const float* y = Y + t * dv;
    float mu = 0.0f, rs = 1.0f;
    if constexpr (ACT == 3) {
      mu = row_sum(dv, lane, [&](int j) { return y[j]; }) / dv;
      const float var = row_sum(dv, lane, [&](int j) { return (y[j] - mu) * (y[j] - mu); });
      rs = rsqrtf(var / dv + kNormEps);
    }
    for (int j = lane; j < dv; j += 64)
      E::st(o, static_cast<int64_t>(t0 + r0 + t) * dv + j, ACT == 3 ? (y[j] - mu) * rs : act_f<ACT>(y[j]));
  }
}

// Backward workspace of the row path (floats).  The backward runs in two kernels:
// a chunk-parallel pre-pass that recomputes each chunk's forward and forms every
// term that does not depend on the carried dW' (norm_bwd_pre_kernel), then the
// reverse sweep over the chunks that carries dW' (norm_bwd_kernel).  Per (chain,
// chunk) the pre-pass leaves a BwdChunk for the sweep and uses a BwdPre of its
// own; the sweep uses one BwdSeq per chain.
struct BwdChunk {  // what the sweep reads back
  int64_t k, z, n, e, g, gh, p1, dkp, aq, rs, ri, eta, total;
  __host__ __device__ BwdChunk(int C, int dk, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n_) {
      int64_t r = o;
      o += (n_ + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t cv = static_cast<int64_t>(C) * dv, ck = static_cast<int64_t>(C) * dk;
    k = take(ck); z = take(cv); n = take(cv); e = take(cv); g = take(cv); gh = take(cv); p1 = take(cv);
    dkp = take(ck); aq = take(static_cast<int64_t>(dk) * dv); rs = take(C); ri = take(C); eta = take(C);
    total = o;
  }
};
struct BwdPre {  // the pre-pass's own operands and intermediates
  int64_t q, v, dout, s, y, dy, ds, total;
  __host__ __device__ BwdPre(int C, int dk, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n_) {
      int64_t r = o;
      o += (n_ + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t cv = static_cast<int64_t>(C) * dv, ck = static_cast<int64_t>(C) * dk,
                  cc = static_cast<int64_t>(C) * C;
    q = take(ck); v = take(cv); dout = take(cv); s = take(cc); y = take(cv); dy = take(cv); ds = take(cc);
    total = o;
  }
};
struct BwdSeq {  // the sweep's carried dW' (two buffers), dG~ and dZ
  int64_t dw[2], dgh, dz, total;
  __host__ __device__ BwdSeq(int C, int dk, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n_) {
      int64_t r = o;
      o += (n_ + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t kv = static_cast<int64_t>(dk) * dv, cv = static_cast<int64_t>(C) * dv;
    dw[0] = take(kv); dw[1] = take(kv); dgh = take(cv); dz = take(cv);
    total = o;
  }
};
struct RowBwdWs {
  int64_t chunk, pre, seq, total;
  __host__ __device__ explicit RowBwdWs(const BwdArgs& a) {
    const int64_t items = static_cast<int64_t>(a.B) * a.H * a.NC;
    chunk = 0;
    pre = items * BwdChunk(a.C, a.dk, a.dv).total;
    seq = pre + items * BwdPre(a.C, a.dk, a.dv).total;
    total = seq + static_cast<int64_t>(a.B) * a.H * BwdSeq(a.C, a.dk, a.dv).total;
  }
};

// Pre-pass of the backward for one (chain, chunk), from its checkpoint W_i: the
// chunk's forward again (Z, the train rows, S = Tril(Q K^T), Y) and dY, then
// every term free of dW' = dW_{i+1}:
//   dS = -Tril(dY (eta G)^T);  dq = dY W_i^T + dS K (final);
//   P1 = -S^T dY (dG~ = P1 - K dW');  dKp1 = dS^T Q (dk = dZ W_i^T + dKp1 - (eta G) dW'^T);
//   A_q = Q^T dY (dW_i = g dW' + A_q + K^T dZ).
template <typename T, int LOSS, int ACT>
__global__ __launch_bounds__(kThreads, 2) void norm_bwd_pre_kernel(BwdArgs a, float* scratch) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  const int bh = blockIdx.x / a.NC, ci = blockIdx.x % a.NC;
  const int dk = a.dk, dv = a.dv, C = a.C;
  const int t0 = ci * C, c = min(C, a.T - t0);
  const RowBwdWs R(a);
  const BwdChunk L(C, dk, dv);
  const BwdPre P(C, dk, dv);
  float* ch = scratch + R.chunk + static_cast<int64_t>(blockIdx.x) * L.total;
  float* pr = scratch + R.pre + static_cast<int64_t>(blockIdx.x) * P.total;
  float *Kc = ch + L.k, *Z = ch + L.z, *Nc = ch + L.n, *Ec = ch + L.e, *G = ch + L.g, *Gh = ch + L.gh,
        *P1 = ch + L.p1, *dKp = ch + L.dkp, *Aq = ch + L.aq, *rsv = ch + L.rs, *riv = ch + L.ri, *eta = ch + L.eta;
  float *Qc = pr + P.q, *Vc = pr + P.v, *dOc = pr + P.dout, *S = pr + P.s, *Y = pr + P.y, *dY = pr + P.dy,
        *dS = pr + P.ds;
  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk, off_v = static_cast<int64_t>(bh) * a.T * dv;
  const T* q = static_cast<const T*>(a.q) + off_k;
  const T* k = static_cast<const T*>(a.k) + off_k;
  const T* v = static_cast<const T*>(a.v) + off_v;
  const T* dO = static_cast<const T*>(a.d_o) + off_v;
  T* dq = static_cast<T*>(a.dq) + off_k;
  const float* beta = a.beta + static_cast<int64_t>(bh) * a.T;
  const float* W = a.w_ckpt + (static_cast<int64_t>(bh) * a.NC + ci) * dk * dv;
  stage_rows<E>(Qc, q + static_cast<int64_t>(t0) * dk, c * dk);
  stage_rows<E>(Kc, k + static_cast<int64_t>(t0) * dk, c * dk);
  stage_rows<E>(Vc, v + static_cast<int64_t>(t0) * dv, c * dv);
  stage_rows<E>(dOc, dO + static_cast<int64_t>(t0) * dv, c * dv);
  for (int t = tid; t < c; t += kThreads) eta[t] = lr_gate(beta[t0 + t], a.b);
  __syncthreads();
  // the chunk's forward again
  gemm1<0, 0, false, 1>(c, dv, Term{Kc, dk, W, dv, dk, 1.0f}, kNoAux, lds,
              [&](int m, int n, float x, float, float, float) { Z[m * dv + n] = x; });
  __syncthreads();
  for (int t = wv; t < c; t += kThreads / 64) {
    float rs, ri;
    train_row<LOSS, ACT>(Z + t * dv, Vc + t * dv, Nc + t * dv, Ec + t * dv, G + t * dv, Gh + t * dv, rs, ri, eta[t],
                         dv, lane);
    if (lane == 0) {
      rsv[t] = rs;
      riv[t] = ri;
    }
  }
  gemm1<0, 1, true, 1>(c, c, Term{Qc, dk, Kc, dk, dk, 1.0f}, kNoAux, lds,
                    [&](int m, int n, float x, float, float, float) { S[m * C + n] = (n <= m) ? x : 0.0f; });
  zero_upper_tiles(S, c, C);
  __syncthreads();
  gemm<0, 0, 0, 0, false, true, 1>(c, dv, Term{Qc, dk, W, dv, dk, 1.0f}, Term{S, C, Gh, dv, c, -1.0f}, kNoAux, lds,
                                [&](int m, int n, float x, float, float, float) { Y[m * dv + n] = x; });
  __syncthreads();
  for (int t = wv; t < c; t += kThreads / 64) {  // dY = J_N(Y)^T dO, or dO (.) f'(Y)
    const float* y = Y + t * dv;
    const float* d = dOc + t * dv;
    if constexpr (ACT == 3) {
      const float mu = row_sum(dv, lane, [&](int j) { return y[j]; }) / dv;
      const float var = row_sum(dv, lane, [&](int j) { return (y[j] - mu) * (y[j] - mu); });
      const float rs = rsqrtf(var / dv + kNormEps);
      const float md = row_sum(dv, lane, [&](int j) { return d[j]; }) / dv;
      const float dn = row_sum(dv, lane, [&](int j) { return d[j] * ((y[j] - mu) * rs); }) / dv;
      for (int j = lane; j < dv; j += 64) dY[t * dv + j] = (d[j] - md - (y[j] - mu) * rs * dn) * rs;
    } else {
      for (int j = lane; j < dv; j += 64) dY[t * dv + j] = d[j] * act_df<ACT>(y[j]);
    }
  }
  __syncthreads();
  // the terms without dW'
  gemm1<0, 1, true, 1>(c, c, Term{dY, dv, Gh, dv, dv, -1.0f}, kNoAux, lds,
                    [&](int m, int n, float x, float, float, float) { dS[m * C + n] = (n <= m) ? x : 0.0f; });
  zero_upper_tiles(dS, c, C);
  gemm1<1, 0, false, 1>(c, dv, Term{S, C, dY, dv, c, -1.0f}, kNoAux, lds,
              [&](int m, int n, float x, float, float, float) { P1[m * dv + n] = x; });
  __syncthreads();
  gemm<0, 1, 0, 0, false, true, 1>(c, dk, Term{dY, dv, W, dv, dv, 1.0f}, Term{dS, C, Kc, dk, c, 1.0f}, kNoAux, lds,
                                [&](int m, int n, float x, float, float, float) {
                                  E::st(dq, static_cast<int64_t>(t0 + m) * dk + n, x);
                                });
  gemm1<1, 0, false, 1>(c, dk, Term{dS, C, Qc, dk, c, 1.0f}, kNoAux, lds,
              [&](int m, int n, float x, float, float, float) { dKp[m * dk + n] = x; });
  gemm1<1, 0, false, 1>(dk, dv, Term{Qc, dk, dY, dv, c, 1.0f}, kNoAux, lds,
              [&](int m, int n, float x, float, float, float) { Aq[m * dv + n] = x; });
}

// Reverse sweep of the backward, one workgroup per chain: per chunk, from the
// pre-pass's terms and the carried dW' = dW_{i+1},
//   dG~ = P1 - K dW';  per row dZ, dV, d eta (the act's and the loss's Jacobians);
//   dk = dZ W_i^T + dKp1 - (eta G) dW'^T;  dW_i = g dW' + A_q + K^T dZ.
template <typename T, int LOSS, int ACT>
__global__ __launch_bounds__(kThreads) void norm_bwd_kernel(BwdArgs a, float* scratch) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];
  __shared__ float wsum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  const int bh = blockIdx.x;
  const int dk = a.dk, dv = a.dv, C = a.C;
  const RowBwdWs R(a);
  const BwdChunk L(C, dk, dv);
  const BwdSeq Q(C, dk, dv);
  float* sq = scratch + R.seq + static_cast<int64_t>(bh) * Q.total;
  float *dGh = sq + Q.dgh, *dZ = sq + Q.dz;
  const bool scalar_decay = a.decay == TTT_DECAY_SCALAR;
  const float g = scalar_decay ? a.gamma[bh % a.H] : 1.0f;
  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk, off_v = static_cast<int64_t>(bh) * a.T * dv;
  T* dkk = static_cast<T*>(a.dk_out) + off_k;
  T* dvv = static_cast<T*>(a.dv_out) + off_v;
  float* dbeta = a.dbeta + static_cast<int64_t>(bh) * a.T;
  const int64_t nw = static_cast<int64_t>(dk) * dv;
  {
    float* D = sq + Q.dw[0];
    const float* src = a.d_wfinal ? a.d_wfinal + bh * nw : nullptr;
    for (int64_t i = tid; i < nw; i += kThreads) D[i] = src ? src[i] : 0.0f;
  }
  int cur = 0;
  float dgam = 0.0f;
  __syncthreads();
  for (int ci = a.NC - 1; ci >= 0; --ci) {
    const int t0 = ci * C, c = min(C, a.T - t0);
    const float* W = a.w_ckpt + (static_cast<int64_t>(bh) * a.NC + ci) * nw;
    const float* D = sq + (cur ? Q.dw[1] : Q.dw[0]);  // dW_{i+1}
    float* Do = sq + (cur ? Q.dw[0] : Q.dw[1]);       // dW_i
    const float* ch = scratch + R.chunk + (static_cast<int64_t>(bh) * a.NC + ci) * L.total;
    const float *Kc = ch + L.k, *Z = ch + L.z, *Nc = ch + L.n, *Ec = ch + L.e, *G = ch + L.g, *Gh = ch + L.gh,
                *P1 = ch + L.p1, *dKp = ch + L.dkp, *Aq = ch + L.aq, *rsv = ch + L.rs, *riv = ch + L.ri,
                *eta = ch + L.eta;
    if (scalar_decay)
      dgam = strided_dot(D, W, nw, dgam);
    gemm1<0, 0>(c, dv, Term{Kc, dk, D, dv, dk, -1.0f}, Aux{{P1, nullptr, nullptr}, dv}, lds,
                [&](int m, int n, float x, float p1, float, float) { dGh[m * dv + n] = x + p1; });
    __syncthreads();
    for (int t = wv; t < c; t += kThreads / 64) {  // dZ, dV, d eta of row t
      float pf[5];
      prefetch_row(pf, {dGh, G, Ec, Nc, Z}, t, c, dv, lane);
      const float et = eta[t], rs = rsv[t], ri = riv[t];
      const float *dgh = dGh + t * dv, *gg = G + t * dv, *ee = Ec + t * dv, *nn = Nc + t * dv, *zz = Z + t * dv;
      const float dgg = row_sum(dv, lane, [&](int j) { return dgh[j] * gg[j]; });  // <d(eta G), G>: d eta
      if (lane == 0) dbeta[t0 + t] = dgg * et * (1.0f - 0.5f * et);
      // (dE / dV_hat)^T x of the loss: x (MSE), (x - e_hat <e_hat, x>) / (sqrt(d) ||e||) (RMSE,
      // e_hat = sqrt(d) E), 0 (IP, L1); its derivative in V is the negative (IP: -I)
      auto rt = [&](auto x, float ehx, int j) {
        if constexpr (LOSS == 0) return x(j);
        else if constexpr (LOSS == 3) return (x(j) - sqrtf(static_cast<float>(dv)) * ee[j] * ehx) * ri;
        else return 0.0f;
      };
      if constexpr (ACT == 3) {
        // dG = eta d(eta G);  M x = x - mean x - n <x, n> / d
        const float mdg = row_sum(dv, lane, [&](int j) { return dgh[j]; }) * et / dv;
        const float dgn = row_sum(dv, lane, [&](int j) { return dgh[j] * nn[j]; }) * et / dv;
        const float en = row_sum(dv, lane, [&](int j) { return ee[j] * nn[j]; }) / dv;
        const float dggd = dgg * et / dv;
        auto mdgf = [&](int j) { return et * dgh[j] - mdg - nn[j] * dgn; };
        float ehm = 0.0f;
        if constexpr (LOSS == 3)
          ehm = row_sum(dv, lane, [&](int j) { return sqrtf(static_cast<float>(dv)) * ee[j] * mdgf(j); });
        auto uf = [&](int j) { return rt(mdgf, ehm, j) - en * et * dgh[j] - dgn * ee[j]; };
        const float mu_u = row_sum(dv, lane, [&](int j) { return uf(j); }) / dv;
        const float un = row_sum(dv, lane, [&](int j) { return uf(j) * nn[j]; }) / dv;
        for (int j = lane; j < dv; j += 64) {
          dZ[t * dv + j] = ((uf(j) - mu_u - nn[j] * un) * rs - nn[j] * dggd) * rs;
          const float dvj = (LOSS == 1) ? -mdgf(j) * rs : -rt(mdgf, ehm, j) * rs;
          E::st(dvv, static_cast<int64_t>(t0 + t) * dv + j, dvj);
        }
      } else {
        // dE = dG (.) f'(z);  dZ = dG (.) E (.) f''(z) + f'(z) (.) (dE/dV_hat)^T dE
        auto def = [&](int j) { return et * dgh[j] * act_df<ACT>(zz[j]); };
        float ehd = 0.0f;
        if constexpr (LOSS == 3)
          ehd = row_sum(dv, lane, [&](int j) { return sqrtf(static_cast<float>(dv)) * ee[j] * def(j); });
        for (int j = lane; j < dv; j += 64) {
          const float r = rt(def, ehd, j);
          dZ[t * dv + j] = et * dgh[j] * ee[j] * act_d2f<ACT>(zz[j]) + act_df<ACT>(zz[j]) * r;
          E::st(dvv, static_cast<int64_t>(t0 + t) * dv + j, (LOSS == 1) ? -def(j) : -r);
        }
      }
      keep_live(pf);
    }
    __syncthreads();
    gemm<0, 1, 0, 1>(c, dk, Term{dZ, dv, W, dv, dv, 1.0f}, Term{Gh, dv, D, dv, dv, -1.0f},
                     Aux{{dKp, nullptr, nullptr}, dk}, lds,
                     [&](int m, int n, float x, float dkp, float, float) {
                       E::st(dkk, static_cast<int64_t>(t0 + m) * dk + n, x + dkp);
                     });
    gemm1<1, 0>(dk, dv, Term{Kc, dk, dZ, dv, c, 1.0f}, Aux{{D, Aq, nullptr}, dv}, lds,
                [&](int m, int n, float x, float d, float aq, float) { Do[m * dv + n] = fmaf(g, d, aq + x); });
    __syncthreads();
    cur ^= 1;
  }
  const float* D = sq + (cur ? Q.dw[1] : Q.dw[0]);
  if (a.dw0)
    for (int64_t i = tid; i < nw; i += kThreads) a.dw0[bh * nw + i] = D[i];
  if (scalar_decay) {
    dgam = wave_sum(dgam);
    if (lane == 0) wsum[wv] = dgam;
    __syncthreads();
    if (tid == 0) {
      float t = 0.0f;
      for (int w = 0; w < kThreads / 64; ++w) t += wsum[w];
      a.dgamma[bh] = t;
    }
  }
}

template <class Args, class K>
hipError_t launch_norm(K kern, const Args& a, float* scratch, ttt_kernel id, hipStream_t s, int nblk,
                       size_t lds = kLdsBytes) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  KernelScope timing(id, s);
  hipLaunchKernelGGL(kern, dim3(nblk), dim3(kThreads), lds, s, a, scratch);
  return hipGetLastError();
}

// The row path runs every loss with every act (the host sends it the Norm act,
// the RMSE loss, and the problems the matrix-core kernels do not take); the
// decay is a runtime flag.
template <bool BWD, class Args>
hipError_t norm_dispatch(const Args& a, hipStream_t s) {
  float* sc = reinterpret_cast<float*>(a.ws);
  auto go = [&](auto tt, auto ll, auto aa) -> hipError_t {
    using T = typename decltype(tt)::type;
    constexpr int LS = decltype(ll)::value, AC = decltype(aa)::value;
    const int chains = a.B * a.H;
    if constexpr (BWD) {
      hipError_t e =
          launch_norm(norm_bwd_pre_kernel<T, LS, AC>, a, sc, TTT_KERNEL_NORM_BWD_PRE, s, chains * a.NC, kLdsBytes1);
      if (e != hipSuccess) return e;
      return launch_norm(norm_bwd_kernel<T, LS, AC>, a, sc, TTT_KERNEL_NORM_BWD, s, chains);
    } else {
      hipError_t e = launch_norm(norm_fwd_kernel<T, LS, AC>, a, sc, TTT_KERNEL_NORM_FWD, s, chains);
      if (e != hipSuccess) return e;
      // fewer chunks than CUs: split each chunk's rows over workgroups
      if (row_query_split(a)) {
        const int nrt = (a.C + kQueryRows - 1) / kQueryRows;
        return launch_norm(norm_query_kernel<T, AC, true>, a, sc, TTT_KERNEL_NORM_QUERY, s, chains * a.NC * nrt,
                           kLdsBytes1);
      }
      return launch_norm(norm_query_kernel<T, AC, false>, a, sc, TTT_KERNEL_NORM_QUERY, s, chains * a.NC, kLdsBytes1);
    }
  };
  auto per_act = [&](auto tt, auto ll) -> hipError_t {
    if (a.act == TTT_ACT_NORM) return go(tt, ll, std::integral_constant<int, 3>{});
    if (a.act == TTT_ACT_SILU) return go(tt, ll, std::integral_constant<int, 1>{});
    if (a.act == TTT_ACT_GELU) return go(tt, ll, std::integral_constant<int, 2>{});
    return go(tt, ll, std::integral_constant<int, 0>{});
  };
  auto per_type = [&](auto tt) -> hipError_t {
    if (a.loss == TTT_LOSS_IP) return per_act(tt, std::integral_constant<int, 1>{});
    if (a.loss == TTT_LOSS_L1) return per_act(tt, std::integral_constant<int, 2>{});
    if (a.loss == TTT_LOSS_RMSE) return per_act(tt, std::integral_constant<int, 3>{});
    return per_act(tt, std::integral_constant<int, 0>{});
  };
  if (a.dtype == TTT_BF16) return per_type(std::type_identity<bf16_t>{});
  return per_type(std::type_identity<float>{});
}

}  // namespace

size_t norm_fwd_workspace(const FwdArgs& a) { return align256(sizeof(float) * static_cast<size_t>(RowFwdWs(a).total)); }
size_t norm_bwd_workspace(const BwdArgs& a) { return align256(sizeof(float) * static_cast<size_t>(RowBwdWs(a).total)); }
hipError_t norm_fwd_launch(const FwdArgs& a, hipStream_t s) { return norm_dispatch<false>(a, s); }
hipError_t norm_bwd_launch(const BwdArgs& a, hipStream_t s) { return norm_dispatch<true>(a, s); }

}  // namespace ttt
