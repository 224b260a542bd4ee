// Forward of the two-layer fast net (TTT-MLP): Linear(W1: d_k -> d_h), a
// nonlinearity f, Linear(W2: d_h -> d_v), no biases.  fp32 arithmetic (the
// products on the fp32 matrix cores), any I/O dtype.
//
// The Modular TTT summary page ("Method step details", Algorithm 1) composes a
// layer's TTT computation from per-primitive rules: the train view runs
// forward (Pass 1), the inner loss is differentiated back to the signal at
// each fast Linear (Pass 2), and the query view runs each Linear's chunked dual
// form, O = X W_start - Tril(X X_train^T) diag(eta) dV_hat with the state step
// W_end = W_start - X_train^T diag(eta) dV_hat, on the query-view activations
// (Pass 3).  For this graph, per chunk of c tokens with W1, W2 at its start:
//   Z1 = K W1, A = f(Z1), V_hat = A W2;  G2 = V_hat - V (MSE), -V (IP) or
//   sign(V_hat - V) (L1);
//   G1 = (G2 W2^T) (.) f'(Z1);
//   X1 = Q W1 - Tril(Q K^T) diag(eta) G1;  A_q = f(X1);
//   O  = A_q W2 - Tril(A_q A^T) diag(eta) G2;
//   W1 <- g W1 - K^T diag(eta) G1;  W2 <- g W2 - A^T diag(eta) G2
// with eta_t = 2 Sigmoid(beta_t + b) and g = gamma_h (scalar decay) or 1.
//
// Work split: the two Linears are coupled through G1 = (G2 W2^T) (.) f'(Z1), so a
// chain is not separable over output columns.  Only the train view and the
// state steps carry a chain from chunk to chunk; the query view needs nothing
// but the chunk's start state and the train view's A, eta G1, eta G2.  So one
// kernel (one workgroup per chain) walks the chunks doing the train view and
// the state steps, and a second (one workgroup per (chain, chunk), every chunk
// at once) forms the query view.  Each is a fixed sequence of small GEMMs (64 x
// 64 output tiles on 8 waves: a 32 x 32 fp32 matrix-core block and half of each
// k-slice per wave; operands staged through double-buffered LDS in 64-deep
// k-slices) over fp32 buffers in the caller's workspace.

#include <type_traits>

#include "tile_gemm.h"
#include "ttt_device.h"
#include "ttt_internal.h"
#include "ttt_mlp_common.h"

namespace ttt {
namespace {

// Workspace regions, in floats (each rounded up to 64 floats): per chain the
// sequential kernel's state buffers, staged K, V and the chunk's Z1, G2; per
// (chain, chunk) the train view's A, eta G1, eta G2 for the query view (without
// a saved context, which then holds them) and the query kernel's staged Q, K, a
// score matrix and A_q; the chunk-start states when the caller keeps none.
struct MlpScratch {
  int64_t w1[2], w2[2], k, v, z1, g2, total;
  __host__ __device__ MlpScratch(int C, int dk, int dh, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    w1[0] = take(static_cast<int64_t>(dk) * dh);
    w1[1] = take(static_cast<int64_t>(dk) * dh);
    w2[0] = take(static_cast<int64_t>(dh) * dv);
    w2[1] = take(static_cast<int64_t>(dh) * dv);
    k = take(static_cast<int64_t>(C) * dk);
    v = take(static_cast<int64_t>(C) * dv);
    z1 = take(static_cast<int64_t>(C) * dh);
    g2 = take(static_cast<int64_t>(C) * dv);
    total = o;
  }
};
struct MlpChunk {
  int64_t a, g1e, g2e, q, k, s, aq, total;
  __host__ __device__ MlpChunk(int C, int dk, int dh, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    a = take(static_cast<int64_t>(C) * dh);
    g1e = take(static_cast<int64_t>(C) * dh);
    g2e = take(static_cast<int64_t>(C) * dv);
    q = take(static_cast<int64_t>(C) * dk);
    k = take(static_cast<int64_t>(C) * dk);
    s = take(static_cast<int64_t>(C) * C);  // Tril(Q K^T), then Tril(A_q A^T)
    aq = take(static_cast<int64_t>(C) * dh);
    total = o;
  }
};
struct MlpWs {
  int64_t chunk, ck1, ck2, total;
  __host__ __device__ MlpWs(int B, int H, int T, int C, int dk, int dh, int dv) {
    const int64_t BH = static_cast<int64_t>(B) * H, NC = (T + C - 1) / C;
    chunk = BH * MlpScratch(C, dk, dh, dv).total;
    ck1 = chunk + BH * NC * MlpChunk(C, dk, dh, dv).total;
    ck2 = ck1 + BH * NC * dk * dh;
    total = ck2 + BH * NC * dh * dv;
  }
};

// Staging of one 64 x 64 k-slice of A and of B: thread tid moves the
// elements tid + 512 i, i < 8, walking the operand's contiguous index so that
// neighbouring threads read neighbouring addresses.  Along a contiguous k the
// thread keeps one k and steps the row by 8; along a contiguous m or n it
// keeps one column and steps k by 8.
struct MlpArgs {
  int B, H, T, dk, dh, dv, C, NC, decay;
  float b;
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* gamma;
  const float* w1_0;
  const float* w2_0;
  void* o;
  float* w1_final;
  float* w2_final;
  float* w1_ckpt;  // [B,H,NC,dk,dh] or null: W1 at each chunk's start
  float* w2_ckpt;  // [B,H,NC,dh,dv] or null
  float* saved;    // MlpSaved per (chain, chunk), or null
  float* scratch;
};

// Where chunk ci of chain bh keeps what the query view reads: the train view's
// A, eta G1, eta G2 (the saved context, or the workspace) and its start states
// (the caller's checkpoints, or the workspace).
struct MlpChunkPtrs {
  float *a, *g1e, *g2e, *w1, *w2;
};
__device__ __forceinline__ MlpChunkPtrs mlp_chunk_ptrs(const MlpArgs& a, int bh, int ci) {
  const MlpWs W(a.B, a.H, a.T, a.C, a.dk, a.dh, a.dv);
  const int64_t item = static_cast<int64_t>(bh) * a.NC + ci;
  MlpChunkPtrs p;
  if (a.saved) {
    const MlpSaved SV(a.C, a.dh, a.dv);
    float* sb = a.saved + item * SV.per_chunk;
    p.a = sb + SV.a; p.g1e = sb + SV.gh1; p.g2e = sb + SV.gh2;
  } else {
    const MlpChunk L(a.C, a.dk, a.dh, a.dv);
    float* cb = a.scratch + W.chunk + item * L.total;
    p.a = cb + L.a; p.g1e = cb + L.g1e; p.g2e = cb + L.g2e;
  }
  p.w1 = (a.w1_ckpt ? a.w1_ckpt : a.scratch + W.ck1) + item * a.dk * a.dh;
  p.w2 = (a.w2_ckpt ? a.w2_ckpt : a.scratch + W.ck2) + item * a.dh * a.dv;
  return p;
}

// Sequential part, one workgroup per chain: per chunk the train view (Z1, A,
// the loss signal G2, eta G1) and the state steps, with the chunk's start states
// copied out for the query view.
template <typename T, int LOSS, int ACT>
__global__ __launch_bounds__(kThreads) void mlp_fwd_kernel(MlpArgs a) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];  // two slice buffers, then the k-half sums (kLdsBytes)
  __shared__ float eta[256];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int dk = a.dk, dh = a.dh, dv = a.dv, C = a.C;
  const MlpScratch L(C, dk, dh, dv);
  float* sc = a.scratch + static_cast<int64_t>(bh) * L.total;
  float* Kc = sc + L.k;
  float* Vc = sc + L.v;
  const bool scalar_decay = a.decay == TTT_DECAY_SCALAR;
  const float g = scalar_decay ? a.gamma[bh % a.H] : 1.0f;

  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk;
  const int64_t off_v = static_cast<int64_t>(bh) * a.T * dv;
  const T* k = static_cast<const T*>(a.k) + off_k;
  const T* v = static_cast<const T*>(a.v) + off_v;
  const float* beta = a.beta + static_cast<int64_t>(bh) * a.T;
  const int64_t n1 = static_cast<int64_t>(dk) * dh, n2 = static_cast<int64_t>(dh) * dv;

  int cur = 0;
  {
    float* W1 = sc + L.w1[0];
    float* W2 = sc + L.w2[0];
    const float* w1src = a.w1_0 ? a.w1_0 + bh * n1 : nullptr;
    const float* w2src = a.w2_0 ? a.w2_0 + bh * n2 : nullptr;
    for (int64_t i = tid; i < n1; i += kThreads) W1[i] = w1src ? w1src[i] : 0.0f;
    for (int64_t i = tid; i < n2; i += kThreads) W2[i] = w2src ? w2src[i] : 0.0f;
  }

  for (int ci = 0; ci < a.NC; ++ci) {
    const int t0 = ci * C;
    const int c = min(C, a.T - t0);
    float* W1 = sc + (cur ? L.w1[1] : L.w1[0]);
    float* W2 = sc + (cur ? L.w2[1] : L.w2[0]);
    float* W1n = sc + (cur ? L.w1[0] : L.w1[1]);
    float* W2n = sc + (cur ? L.w2[0] : L.w2[1]);
    const MlpChunkPtrs cp = mlp_chunk_ptrs(a, bh, ci);
    // Where this chunk's intermediates go: A, eta G1, eta G2 per chunk (above); Z1
    // and G2 per chain, or the saved context (then also P and the RMSE row scales).
    float *Z1c = sc + L.z1, *Acc = cp.a, *G2c = sc + L.g2, *G2ec = cp.g2e, *G1ec = cp.g1e;
    float *Pc = nullptr, *RIc = nullptr;
    if (a.saved) {
      const MlpSaved SV(C, dh, dv);
      float* sb = a.saved + (static_cast<int64_t>(bh) * a.NC + ci) * SV.per_chunk;
      Z1c = sb + SV.z1; Pc = sb + SV.p; G2c = sb + SV.g2; RIc = sb + SV.ri;
    }

    // The chunk's inputs as fp32 rows, eta, and the start states for the query view.
    stage_rows<E, 32>(Kc, k + static_cast<int64_t>(t0) * dk, c * dk);
    stage_rows<E, 32>(Vc, v + static_cast<int64_t>(t0) * dv, c * dv);
    for (int t = tid; t < c; t += kThreads) eta[t] = lr_gate(beta[t0 + t], a.b);
    stage_rows<Elem<float>, 32>(cp.w1, W1, static_cast<int>(n1));
    stage_rows<Elem<float>, 32>(cp.w2, W2, static_cast<int>(n2));
    __syncthreads();

    // Pass 1, first Linear and f:  Z1 = K W1,  A = f(Z1).
    gemm1<0, 0>(c, dh, Term{Kc, dk, W1, dh, dk, 1.0f}, kNoAux, lds, [&](int m, int n, float x, float, float, float) {
      Z1c[m * dh + n] = x;
      Acc[m * dh + n] = act_f<ACT>(x);
    });
    if constexpr (LOSS == 1) {  // IP: the signal at the output does not depend on the state
      for (int i = tid; i < c * dv; i += kThreads) {
        G2c[i] = -Vc[i];
        G2ec[i] = -eta[i / dv] * Vc[i];
      }
    }
    __syncthreads();
    if constexpr (LOSS != 1) {  // Pass 1, second Linear, and the signal G2 = A W2 - V (MSE), its sign (L1)
      gemm1<0, 0>(c, dv, Term{Acc, dh, W2, dv, dh, 1.0f}, Aux{{Vc, nullptr, nullptr}, dv}, lds,  // or e (RMSE)
                  [&](int m, int n, float x, float vv, float, float) {
        const float e = loss_signal<(LOSS == 3 ? 0 : LOSS), 0>(x, vv);
        G2c[m * dv + n] = e;
        G2ec[m * dv + n] = eta[m] * e;
      });
      __syncthreads();
    }

    if constexpr (LOSS == 3) {  // RMSE: G2 = e / (sqrt(d_v) ||e||) per token (0 where e = 0)
      for (int t = tid / 64; t < c; t += kThreads / 64) {
        const int lane = tid % 64;
        float ss = 0.0f;
        for (int j = lane; j < dv; j += 64) ss = fmaf(G2c[t * dv + j], G2c[t * dv + j], ss);
        ss = wave_sum(ss);
        const float ri = ss > 0.0f ? rsqrtf(ss * dv) : 0.0f;
        for (int j = lane; j < dv; j += 64) {
          const float e = G2c[t * dv + j] * ri;
          G2c[t * dv + j] = e;
          G2ec[t * dv + j] = eta[t] * e;
        }
        if (RIc && lane == 0) RIc[t] = ri;
      }
      __syncthreads();
    }

    // Pass 2 through the first Linear: eta G1 = eta (G2 W2^T) (.) f'(Z1).
    gemm1<0, 1>(c, dh, Term{G2c, dv, W2, dv, dv, 1.0f}, Aux{{Z1c, nullptr, nullptr}, dh}, lds,
                [&](int m, int n, float x, float z, float, float) {
                  G1ec[m * dh + n] = eta[m] * x * act_df<ACT>(z);
                  if (Pc) Pc[m * dh + n] = x;
                });
    __syncthreads();

    // Both state steps.
    gemm1<1, 0>(dk, dh, Term{Kc, dk, G1ec, dh, c, -1.0f}, Aux{{W1, nullptr, nullptr}, dh}, lds,
                [&](int m, int n, float x, float w, float, float) { W1n[m * dh + n] = fmaf(g, w, x); });
    gemm1<1, 0>(dh, dv, Term{Acc, dh, G2ec, dv, c, -1.0f}, Aux{{W2, nullptr, nullptr}, dv}, lds,
                [&](int m, int n, float x, float w, float, float) { W2n[m * dv + n] = fmaf(g, w, x); });
    __syncthreads();
    cur ^= 1;
  }

  const float* W1 = sc + (cur ? L.w1[1] : L.w1[0]);
  const float* W2 = sc + (cur ? L.w2[1] : L.w2[0]);
  if (a.w1_final)
    for (int64_t i = tid; i < n1; i += kThreads) a.w1_final[bh * n1 + i] = W1[i];
  if (a.w2_final)
    for (int64_t i = tid; i < n2; i += kThreads) a.w2_final[bh * n2 + i] = W2[i];
}

// Query view of one (chain, chunk), from the sequential kernel's start states
// and A, eta G1, eta G2:
//   X1 = Q W1 - Tril(Q K^T) eta G1;  A_q = f(X1);  O = A_q W2 - Tril(A_q A^T) eta G2.
// With a saved context X1, A_q and both score matrices (strictly upper tiles
// zeroed) go there for the backward.
template <typename T, int ACT>
__global__ __launch_bounds__(kThreads, 2) void mlp_query_kernel(MlpArgs a) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];
  const int bh = blockIdx.x / a.NC, ci = blockIdx.x % a.NC;
  const int dk = a.dk, dh = a.dh, dv = a.dv, C = a.C;
  const int t0 = ci * C;
  const int c = min(C, a.T - t0);
  const MlpWs W(a.B, a.H, a.T, C, dk, dh, dv);
  const MlpChunk L(C, dk, dh, dv);
  float* cb = a.scratch + W.chunk + static_cast<int64_t>(blockIdx.x) * L.total;
  float *Qc = cb + L.q, *Kc = cb + L.k;
  const MlpChunkPtrs cp = mlp_chunk_ptrs(a, bh, ci);
  float *S1c = cb + L.s, *S2c = cb + L.s, *Aqc = cb + L.aq, *X1c = nullptr;
  if (a.saved) {
    const MlpSaved SV(C, dh, dv);
    float* sb = a.saved + (static_cast<int64_t>(bh) * a.NC + ci) * SV.per_chunk;
    S1c = sb + SV.s1; S2c = sb + SV.s2; Aqc = sb + SV.aq; X1c = sb + SV.x1;
  }
  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk;
  const int64_t off_v = static_cast<int64_t>(bh) * a.T * dv;
  const T* q = static_cast<const T*>(a.q) + off_k;
  const T* k = static_cast<const T*>(a.k) + off_k;
  T* o = static_cast<T*>(a.o) + off_v;
  stage_rows<E>(Qc, q + static_cast<int64_t>(t0) * dk, c * dk);
  stage_rows<E>(Kc, k + static_cast<int64_t>(t0) * dk, c * dk);
  __syncthreads();

  // Tril(Q K^T); Pass 3, first Linear: A_q = f(Q W1 - Tril(Q K^T) eta G1).
  gemm1<0, 1, true, 1>(c, c, Term{Qc, dk, Kc, dk, dk, 1.0f}, kNoAux, lds,
                    [&](int m, int n, float x, float, float, float) { S1c[m * C + n] = (n <= m) ? x : 0.0f; });
  if (a.saved) zero_upper_tiles(S1c, c, C);
  __syncthreads();
  gemm<0, 0, 0, 0, false, true, 1>(c, dh, Term{Qc, dk, cp.w1, dh, dk, 1.0f}, Term{S1c, C, cp.g1e, dh, c, -1.0f}, kNoAux,
                                lds, [&](int m, int n, float x, float, float, float) {
                                  Aqc[m * dh + n] = act_f<ACT>(x);
                                  if (X1c) X1c[m * dh + n] = x;
                                });
  __syncthreads();
  gemm1<0, 1, true, 1>(c, c, Term{Aqc, dh, cp.a, dh, dh, 1.0f}, kNoAux, lds,
                    [&](int m, int n, float x, float, float, float) { S2c[m * C + n] = (n <= m) ? x : 0.0f; });
  if (a.saved) zero_upper_tiles(S2c, c, C);
  __syncthreads();

  // Pass 3, second Linear: O = A_q W2 - Tril(A_q A^T) eta G2.
  gemm<0, 0, 0, 0, false, true, 1>(c, dv, Term{Aqc, dh, cp.w2, dv, dh, 1.0f}, Term{S2c, C, cp.g2e, dv, c, -1.0f}, kNoAux,
                                lds, [&](int m, int n, float x, float, float, float) {
                                  E::st(o, static_cast<int64_t>(t0 + m) * dv + n, x);
                                });
}

template <class K>
hipError_t launch_mlp(K kern, const MlpArgs& a, ttt_kernel id, int nblk, hipStream_t s, size_t lds = kLdsBytes) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  KernelScope timing(id, s);
  hipLaunchKernelGGL(kern, dim3(nblk), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <typename T, int LOSS, int ACT>
hipError_t launch_t(const MlpArgs& a, hipStream_t s) {
  hipError_t e = launch_mlp(mlp_fwd_kernel<T, LOSS, ACT>, a, TTT_KERNEL_MLP_FWD, a.B * a.H, s);
  if (e != hipSuccess) return e;
  return launch_mlp(mlp_query_kernel<T, ACT>, a, TTT_KERNEL_MLP_QUERY, a.B * a.H * a.NC, s, kLdsBytes1);
}

struct FwdL {
  template <typename T, int LOSS, int ACT>
  static hipError_t run(const MlpArgs& a, hipStream_t s) { return launch_t<T, LOSS, ACT>(a, s); }
};
}  // namespace

size_t mlp_fwd_workspace(const ttt_mlp_desc& d) {
  return align256(sizeof(float) * static_cast<size_t>(MlpWs(d.B, d.H, d.T, d.C, d.dk, d.dh, d.dv).total));
}

hipError_t mlp_fwd_launch(const ttt_mlp_desc& d, const void* q, const void* k, const void* v, const float* beta,
                          const float* gamma, const float* w1_0, const float* w2_0, void* o, float* w1_final,
                          float* w2_final, float* w1_ckpt, float* w2_ckpt, void* saved, void* ws, hipStream_t s) {
  MlpArgs a{};
  a.B = d.B; a.H = d.H; a.T = d.T; a.dk = d.dk; a.dh = d.dh; a.dv = d.dv; a.C = d.C;
  a.NC = (d.T + d.C - 1) / d.C;
  a.decay = d.decay;
  a.b = d.lr_bias;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.gamma = gamma; a.w1_0 = w1_0; a.w2_0 = w2_0;
  a.o = o; a.w1_final = w1_final; a.w2_final = w2_final; a.w1_ckpt = w1_ckpt; a.w2_ckpt = w2_ckpt;
  a.saved = static_cast<float*>(saved);
  a.scratch = static_cast<float*>(ws);
  return by_enums<FwdL>(a, d, s);
}

}  // namespace ttt
