// Generic HIP path of the chunkwise TTT layer: fp32 VALU arithmetic, any I/O
// dtype, d_k, d_v <= 256, 1 <= C <= 256, ragged last chunk allowed.
//
// This path serves fp32 inputs (MI355X's fp32 vector and fp32 matrix peaks are
// the same, 157 TFLOP/s, so plain FMAs are the natural fp32 engine) and shapes
// outside the bf16 matrix-core kernels.  It evaluates the chunk equations of
// the Modular TTT summary page ("Method step details": Algorithm 1's passes and
// the chunked dual form; "Prerequisites": eta = 2 Sigmoid(beta + b), scalar and
// vector decay) directly, term by term.
//
// Forward: one workgroup per (chain, 32-column block of d_v).  The forward is
// separable over the columns of W (Z, G, Y, O and the W update act column by
// column; only the C x C scores are shared), so each workgroup carries its
// dk x 32 slice of W in LDS across the chunk loop.
// Backward: one workgroup per chain, with per-chain scratch in the workspace;
// the reverse chunk sweep carries dW_{i+1}.

#include "ttt_device.h"
#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr int kNB = 32;        // d_v columns per forward workgroup
constexpr int kTQ = 8;         // query rows per score block (forward)
constexpr int kFwdThreads = 256;
constexpr int kBwdThreads = 512;

// L[b,h,t,:] = inclusive cumulative sum of log_decay over the tokens of t's chunk.
__global__ void decay_cumsum_kernel(const float* __restrict__ la, float* __restrict__ L, int BH,
                                    int T, int C, int NC, int dk) {
  int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t total = static_cast<int64_t>(BH) * NC * dk;
  if (idx >= total) return;
  int d = static_cast<int>(idx % dk);
  int64_t r = idx / dk;
  int ci = static_cast<int>(r % NC);
  int64_t bh = r / NC;
  int t0 = ci * C;
  int t1 = min(T, t0 + C);
  const float* src = la + bh * T * dk;
  float* dst = L + bh * T * dk;
  float acc = 0.0f;
  for (int t = t0; t < t1; ++t) {
    acc += src[static_cast<int64_t>(t) * dk + d];
    dst[static_cast<int64_t>(t) * dk + d] = acc;
  }
}

// STAGE: the chunk's keys [C][dk + 1] and each block of kTQ query rows [kTQ][dk + 1]
// are staged in LDS (fp32, rows padded by one word so that threads on consecutive
// rows hit different banks) and every product reads them there; without it
// (widths whose chunk does not fit) they are read from global memory.
template <typename T, int LOSS, int ACT, int DECAY, bool STAGE>
__global__ __launch_bounds__(kFwdThreads) void fwd_generic_kernel(FwdArgs a, const float* __restrict__ Lbuf) {
  using E = Elem<T>;
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int h = bh % a.H;
  const int col0 = blockIdx.y * kNB;
  const int ncol = min(kNB, a.dv - col0);
  const int dk = a.dk, dv = a.dv, C = a.C;
  float* Ws = smem;                  // [dk][kNB]
  float* Gh = Ws + dk * kNB;         // [C][kNB]   eta (.) G
  float* eta = Gh + C * kNB;         // [C]
  float* Sb = eta + C;               // [kTQ][C]   causal scores of one query block
  float* lam = Sb + kTQ * C;         // [dk]       row scale of the transition
  const int kp = dk + 1;             // padded row of the staged keys / queries
  float* Ks = lam + dk;              // [C][dk + 1]    keys of the chunk (STAGE)
  float* Qb = Ks + (STAGE ? C * kp : 0);  // [kTQ][dk + 1] one query block (STAGE)

  const T* q = static_cast<const T*>(a.q) + static_cast<int64_t>(bh) * a.T * dk;
  const T* k = static_cast<const T*>(a.k) + static_cast<int64_t>(bh) * a.T * dk;
  const T* v = static_cast<const T*>(a.v) + static_cast<int64_t>(bh) * a.T * dv;
  T* o = static_cast<T*>(a.o) + static_cast<int64_t>(bh) * a.T * dv;
  const float* beta = a.beta + static_cast<int64_t>(bh) * a.T;
  const float* L = (DECAY == 2) ? Lbuf + static_cast<int64_t>(bh) * a.T * dk : nullptr;

  for (int i = tid; i < dk * kNB; i += blockDim.x) {
    int d = i / kNB, n = i % kNB;
    Ws[i] = (n < ncol && a.w0) ? a.w0[(static_cast<int64_t>(bh) * dk + d) * dv + col0 + n] : 0.0f;
  }
  __syncthreads();

  for (int ci = 0; ci < a.NC; ++ci) {
    const int t0 = ci * C;
    const int c = min(C, a.T - t0);
    if (a.w_ckpt) {
      float* ck = a.w_ckpt + (static_cast<int64_t>(bh) * a.NC + ci) * dk * dv;
      for (int i = tid; i < dk * kNB; i += blockDim.x) {
        int d = i / kNB, n = i % kNB;
        if (n < ncol) ck[static_cast<int64_t>(d) * dv + col0 + n] = Ws[i];
      }
    }
    for (int t = tid; t < c; t += blockDim.x) eta[t] = lr_gate(beta[t0 + t], a.b);
    for (int d = tid; d < dk; d += blockDim.x) {
      if constexpr (DECAY == 2) lam[d] = expf(L[static_cast<int64_t>(t0 + c - 1) * dk + d]);
      else if constexpr (DECAY == 1) lam[d] = a.gamma[h];
      else lam[d] = 1.0f;
    }
    if constexpr (STAGE) {
      for (int i = tid; i < c * dk; i += blockDim.x) {
        const int t = i / dk, d = i % dk;
        Ks[t * kp + d] = E::ld(k, static_cast<int64_t>(t0) * dk + i);
      }
    }
    __syncthreads();
    auto kval = [&](int t, int d) -> float {
      if constexpr (STAGE) return Ks[t * kp + d];
      else return E::ld(k, static_cast<int64_t>(t0 + t) * dk + d);
    };

    // Pass 1 + 2 (train view at W_i): Z = K W, G = dL/dZ, stored as eta (.) G.
    for (int i = tid; i < c * kNB; i += blockDim.x) {
      int t = i / kNB, n = i % kNB;
      float g = 0.0f;
      if (n < ncol) {
        float z = 0.0f;
        for (int d = 0; d < dk; ++d) z = fmaf(kval(t, d), Ws[d * kNB + n], z);
        float vv = E::ld(v, static_cast<int64_t>(t0 + t) * dv + col0 + n);
        float e = loss_signal<LOSS, ACT>(z, vv);
        g = e * act_df<ACT>(z);
      }
      Gh[i] = eta[t] * g;
    }
    __syncthreads();

    // Pass 3 (query view): Y = Q~ W_i - Tril(S) (eta (.) G), O = f(Y).
    for (int tb = 0; tb < c; tb += kTQ) {
      if constexpr (STAGE) {
        for (int i = tid; i < kTQ * dk; i += blockDim.x) {
          const int r = i / dk, d = i % dk;
          Qb[r * kp + d] = (tb + r < c) ? E::ld(q, static_cast<int64_t>(t0 + tb) * dk + i) : 0.0f;
        }
        __syncthreads();
      }
      auto qval = [&](int r, int d) -> float {
        if constexpr (STAGE) return Qb[r * kp + d];
        else return E::ld(q, static_cast<int64_t>(t0 + tb + r) * dk + d);
      };
      for (int i = tid; i < kTQ * c; i += blockDim.x) {
        int r = i / c, s = i % c, t = tb + r;
        float val = 0.0f;
        if (t < c && s <= t) {
          const int64_t rt = static_cast<int64_t>(t0 + t) * dk, rs = static_cast<int64_t>(t0 + s) * dk;
          for (int d = 0; d < dk; ++d) {
            float p = qval(r, d) * kval(s, d);
            if constexpr (DECAY == 2) p *= expf(L[rt + d] - L[rs + d]);
            val += p;
          }
        }
        Sb[r * C + s] = val;
      }
      __syncthreads();
      for (int i = tid; i < kTQ * kNB; i += blockDim.x) {
        int r = i / kNB, n = i % kNB, t = tb + r;
        if (t >= c || n >= ncol) continue;
        const int64_t rt = static_cast<int64_t>(t0 + t) * dk;
        float y = 0.0f;
        for (int d = 0; d < dk; ++d) {
          float qq = qval(r, d);
          if constexpr (DECAY == 2) qq *= expf(L[rt + d]);
          y = fmaf(qq, Ws[d * kNB + n], y);
        }
        for (int s = 0; s <= t; ++s) y -= Sb[r * C + s] * Gh[s * kNB + n];
        E::st(o, static_cast<int64_t>(t0 + t) * dv + col0 + n, act_f<ACT>(y));
      }
      __syncthreads();
    }

    // State transition: W <- diag(lam) W - K_bar^T (eta (.) G).
    for (int i = tid; i < dk * kNB; i += blockDim.x) {
      int d = i / kNB, n = i % kNB;
      float acc = 0.0f;
      for (int s = 0; s < c; ++s) {
        float kb = kval(s, d);
        if constexpr (DECAY == 2)
          kb *= expf(L[static_cast<int64_t>(t0 + c - 1) * dk + d] - L[static_cast<int64_t>(t0 + s) * dk + d]);
        acc = fmaf(kb, Gh[s * kNB + n], acc);
      }
      Ws[i] = lam[d] * Ws[i] - acc;
    }
    __syncthreads();
  }
  if (a.w_final) {
    for (int i = tid; i < dk * kNB; i += blockDim.x) {
      int d = i / kNB, n = i % kNB;
      if (n < ncol) a.w_final[(static_cast<int64_t>(bh) * dk + d) * dv + col0 + n] = Ws[i];
    }
  }
}

// Per-chain scratch of the generic backward, in floats.
struct BwdScratch {
  int64_t dW, Z, Ev, G, dY, dGh, dZ, S, dS, dL, dKK, total;
  __host__ __device__ BwdScratch(int C, int dk, int dv) {
    int64_t o = 0;
    dW = o; o += static_cast<int64_t>(dk) * dv;
    Z = o; o += static_cast<int64_t>(C) * dv;
    Ev = o; o += static_cast<int64_t>(C) * dv;
    G = o; o += static_cast<int64_t>(C) * dv;
    dY = o; o += static_cast<int64_t>(C) * dv;
    dGh = o; o += static_cast<int64_t>(C) * dv;
    dZ = o; o += static_cast<int64_t>(C) * dv;
    S = o; o += static_cast<int64_t>(C) * C;
    dS = o; o += static_cast<int64_t>(C) * C;
    dL = o; o += static_cast<int64_t>(C) * dk;
    dKK = o; o += static_cast<int64_t>(C) * dk;
    total = (o + 63) & ~static_cast<int64_t>(63);
  }
};

template <typename T, int LOSS, int ACT, int DECAY>
__global__ __launch_bounds__(kBwdThreads) void bwd_generic_kernel(BwdArgs a, const float* __restrict__ Lbuf,
                                                                  float* __restrict__ scratch) {
  using E = Elem<T>;
  __shared__ float eta[256];
  __shared__ float lam[256];
  __shared__ float red[kBwdThreads];
  const int tid = threadIdx.x, nth = blockDim.x;
  const int bh = blockIdx.x;
  const int h = bh % a.H;
  const int dk = a.dk, dv = a.dv, C = a.C;
  const BwdScratch L_(C, dk, dv);
  float* sc = scratch + static_cast<int64_t>(bh) * L_.total;
  float* dW = sc + L_.dW;
  float* Zs = sc + L_.Z;
  float* Es = sc + L_.Ev;
  float* Gs = sc + L_.G;
  float* dYs = sc + L_.dY;
  float* dGhs = sc + L_.dGh;
  float* dZs = sc + L_.dZ;
  float* Ss = sc + L_.S;
  float* dSs = sc + L_.dS;
  float* dLs = sc + L_.dL;
  float* dKKs = sc + L_.dKK;

  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk;
  const int64_t off_v = static_cast<int64_t>(bh) * a.T * dv;
  const T* q = static_cast<const T*>(a.q) + off_k;
  const T* k = static_cast<const T*>(a.k) + off_k;
  const T* v = static_cast<const T*>(a.v) + off_v;
  const T* dO = static_cast<const T*>(a.d_o) + off_v;
  T* dq = static_cast<T*>(a.dq) + off_k;
  T* dkk = static_cast<T*>(a.dk_out) + off_k;
  T* dvv = static_cast<T*>(a.dv_out) + off_v;
  const float* beta = a.beta + static_cast<int64_t>(bh) * a.T;
  float* dbeta = a.dbeta + static_cast<int64_t>(bh) * a.T;
  const float* L = (DECAY == 2) ? Lbuf + off_k : nullptr;
  float* dla = (DECAY == 2) ? a.dlog_decay + off_k : nullptr;

  for (int i = tid; i < dk * dv; i += nth)
    dW[i] = a.d_wfinal ? a.d_wfinal[static_cast<int64_t>(bh) * dk * dv + i] : 0.0f;
  float dgamma_acc = 0.0f;  // meaningful in thread 0 only
  __syncthreads();

  for (int ci = a.NC - 1; ci >= 0; --ci) {
    const int t0 = ci * C;
    const int c = min(C, a.T - t0);
    const float* W = a.w_ckpt + (static_cast<int64_t>(bh) * a.NC + ci) * dk * dv;
    const int64_t Lc = static_cast<int64_t>(t0 + c - 1) * dk;
    for (int t = tid; t < c; t += nth) eta[t] = lr_gate(beta[t0 + t], a.b);
    for (int d = tid; d < dk; d += nth) {
      if constexpr (DECAY == 2) lam[d] = expf(L[Lc + d]);
      else if constexpr (DECAY == 1) lam[d] = a.gamma[h];
      else lam[d] = 1.0f;
    }
    __syncthreads();

    // Recompute the train view: Z = K W_i, E, G.
    for (int i = tid; i < c * dv; i += nth) {
      int t = i / dv, n = i % dv;
      const int64_t rt = static_cast<int64_t>(t0 + t) * dk;
      float z = 0.0f;
      for (int d = 0; d < dk; ++d) z = fmaf(E::ld(k, rt + d), W[d * dv + n], z);
      float vv = E::ld(v, static_cast<int64_t>(t0 + t) * dv + n);
      float e = loss_signal<LOSS, ACT>(z, vv);
      Zs[i] = z;
      Es[i] = e;
      Gs[i] = e * act_df<ACT>(z);
    }
    // Scores S_ts (s <= t).
    for (int i = tid; i < c * c; i += nth) {
      int t = i / c, s = i % c;
      float val = 0.0f;
      if (s <= t) {
        const int64_t rt = static_cast<int64_t>(t0 + t) * dk, rs = static_cast<int64_t>(t0 + s) * dk;
        for (int d = 0; d < dk; ++d) {
          float p = E::ld(q, rt + d) * E::ld(k, rs + d);
          if constexpr (DECAY == 2) p *= expf(L[rt + d] - L[rs + d]);
          val += p;
        }
      }
      Ss[t * C + s] = val;
    }
    __syncthreads();

    // Query view again: Y = Q~ W_i - S (eta G); dY = dO (.) f'(Y).
    for (int i = tid; i < c * dv; i += nth) {
      int t = i / dv, n = i % dv;
      const int64_t rt = static_cast<int64_t>(t0 + t) * dk;
      float y = 0.0f;
      for (int d = 0; d < dk; ++d) {
        float qq = E::ld(q, rt + d);
        if constexpr (DECAY == 2) qq *= expf(L[rt + d]);
        y = fmaf(qq, W[d * dv + n], y);
      }
      for (int s = 0; s <= t; ++s) y -= Ss[t * C + s] * eta[s] * Gs[s * dv + n];
      dYs[i] = E::ld(dO, static_cast<int64_t>(t0 + t) * dv + n) * act_df<ACT>(y);
    }
    __syncthreads();

    // dGh = -S^T dY - K_bar dW_{i+1};  dG = eta dGh;  dZ;  dV = -dE.
    for (int i = tid; i < c * dv; i += nth) {
      int s = i / dv, n = i % dv;
      float acc = 0.0f;
      for (int t = s; t < c; ++t) acc += Ss[t * C + s] * dYs[t * dv + n];
      const int64_t rs = static_cast<int64_t>(t0 + s) * dk;
      float acc2 = 0.0f;
      for (int d = 0; d < dk; ++d) {
        float kb = E::ld(k, rs + d);
        if constexpr (DECAY == 2) kb *= expf(L[Lc + d] - L[rs + d]);
        acc2 = fmaf(kb, dW[d * dv + n], acc2);
      }
      float dgh = -acc - acc2;
      dGhs[i] = dgh;
      float dg = eta[s] * dgh;
      float z = Zs[i];
      float f1 = act_df<ACT>(z);
      float de = dg * f1;
      float dz = dg * Es[i] * act_d2f<ACT>(z);
      if (LOSS == 0) dz += de * f1;
      dZs[i] = dz;
      E::st(dvv, static_cast<int64_t>(t0 + s) * dv + n, loss_dsignal_dv<LOSS>() * de);
    }
    // dS_ts = -(dY_t . eta_s G_s) for s <= t.
    for (int i = tid; i < c * c; i += nth) {
      int t = i / c, s = i % c;
      float val = 0.0f;
      if (s <= t) {
        for (int n = 0; n < dv; ++n) val += dYs[t * dv + n] * Gs[s * dv + n];
        val = -val * eta[s];
      }
      dSs[t * C + s] = val;
    }
    __syncthreads();

    // dQ (and the query-side share of dL).
    for (int i = tid; i < c * dk; i += nth) {
      int t = i / dk, d = i % dk;
      const int64_t rt = static_cast<int64_t>(t0 + t) * dk;
      float dqt = 0.0f;
      for (int n = 0; n < dv; ++n) dqt = fmaf(dYs[t * dv + n], W[d * dv + n], dqt);
      float dqs = 0.0f;
      for (int s = 0; s <= t; ++s) {
        float kk = E::ld(k, static_cast<int64_t>(t0 + s) * dk + d);
        if constexpr (DECAY == 2) kk *= expf(L[rt + d] - L[static_cast<int64_t>(t0 + s) * dk + d]);
        dqs = fmaf(dSs[t * C + s], kk, dqs);
      }
      float qq = E::ld(q, rt + d);
      if constexpr (DECAY == 2) {
        float eL = expf(L[rt + d]);
        E::st(dq, rt + d, dqt * eL + dqs);
        dLs[t * dk + d] = qq * dqs + dqt * qq * eL;
      } else {
        E::st(dq, rt + d, dqt + dqs);
      }
    }
    __syncthreads();

    // dK (and the key-side share of dL).
    for (int i = tid; i < c * dk; i += nth) {
      int s = i / dk, d = i % dk;
      const int64_t rs = static_cast<int64_t>(t0 + s) * dk;
      float dkz = 0.0f, dkb = 0.0f;
      for (int n = 0; n < dv; ++n) {
        dkz = fmaf(dZs[s * dv + n], W[d * dv + n], dkz);
        dkb = fmaf(Gs[s * dv + n], dW[d * dv + n], dkb);
      }
      dkb = -eta[s] * dkb;
      float dks = 0.0f;
      for (int t = s; t < c; ++t) {
        float qq = E::ld(q, static_cast<int64_t>(t0 + t) * dk + d);
        if constexpr (DECAY == 2) qq *= expf(L[static_cast<int64_t>(t0 + t) * dk + d] - L[rs + d]);
        dks = fmaf(dSs[t * C + s], qq, dks);
      }
      float kk = E::ld(k, rs + d);
      if constexpr (DECAY == 2) {
        float sc2 = expf(L[Lc + d] - L[rs + d]);
        E::st(dkk, rs + d, dkz + dkb * sc2 + dks);
        float kbar = kk * sc2;
        dLs[s * dk + d] += -kk * dks - dkb * kbar;
        dKKs[s * dk + d] = dkb * kbar;
      } else {
        E::st(dkk, rs + d, dkz + dkb + dks);
      }
    }
    // deta and dbeta.
    for (int s = tid; s < c; s += nth) {
      float acc = 0.0f;
      for (int n = 0; n < dv; ++n) acc += dGhs[s * dv + n] * Gs[s * dv + n];
      float e = eta[s];
      dbeta[t0 + s] = acc * e * (1.0f - 0.5f * e);
    }
    __syncthreads();

    // dlambda: scalar decay accumulates d gamma; vector decay feeds dL at the last token.
    if constexpr (DECAY == 1) {
      float part = 0.0f;
      for (int i = tid; i < dk * dv; i += nth) part += dW[i] * W[i];
      red[tid] = part;
      __syncthreads();
      if (tid == 0) {
        float s = 0.0f;
        for (int j = 0; j < nth; ++j) s += red[j];
        dgamma_acc += s;
      }
      __syncthreads();
    }
    if constexpr (DECAY == 2) {
      for (int d = tid; d < dk; d += nth) {
        float dl = 0.0f;
        for (int n = 0; n < dv; ++n) dl += dW[d * dv + n] * W[d * dv + n];
        float dlc = dl * lam[d];
        for (int s = 0; s < c; ++s) dlc += dKKs[s * dk + d];
        dLs[(c - 1) * dk + d] += dlc;
        // d log a_r = sum_{t >= r} dL_t  (L is the inclusive in-chunk cumsum)
        float acc = 0.0f;
        for (int t = c - 1; t >= 0; --t) {
          acc += dLs[t * dk + d];
          dla[static_cast<int64_t>(t0 + t) * dk + d] = acc;
        }
      }
    }
    __syncthreads();

    // dW_i = diag(lam) dW_{i+1} + Q~^T dY + K^T dZ.
    for (int i = tid; i < dk * dv; i += nth) {
      int d = i / dv, n = i % dv;
      float acc = lam[d] * dW[i];
      for (int t = 0; t < c; ++t) {
        const int64_t rt = static_cast<int64_t>(t0 + t) * dk + d;
        float qq = E::ld(q, rt);
        if constexpr (DECAY == 2) qq *= expf(L[rt]);
        acc = fmaf(qq, dYs[t * dv + n], acc);
        acc = fmaf(E::ld(k, rt), dZs[t * dv + n], acc);
      }
      dW[i] = acc;
    }
    __syncthreads();
  }
  if (a.dw0)
    for (int i = tid; i < dk * dv; i += nth) a.dw0[static_cast<int64_t>(bh) * dk * dv + i] = dW[i];
  if (DECAY == 1 && tid == 0 && a.dgamma) a.dgamma[bh] = dgamma_acc;
}

size_t fwd_lds_bytes(int dk, int C, bool stage) {
  const size_t staged = stage ? static_cast<size_t>(C + kTQ) * (dk + 1) : 0;
  return sizeof(float) * (static_cast<size_t>(dk) * kNB + static_cast<size_t>(C) * kNB + C +
                          static_cast<size_t>(kTQ) * C + dk + staged);
}
constexpr size_t kLdsMax = 160 * 1024;

template <typename T, int LOSS, int ACT, int DECAY>
hipError_t fwd_launch_t(const FwdArgs& a, hipStream_t s, const float* L) {
  dim3 grid(a.B * a.H, (a.dv + kNB - 1) / kNB);
  const bool stage = fwd_lds_bytes(a.dk, a.C, true) <= kLdsMax;
  size_t lds = fwd_lds_bytes(a.dk, a.C, stage);
  auto kern = stage ? fwd_generic_kernel<T, LOSS, ACT, DECAY, true> : fwd_generic_kernel<T, LOSS, ACT, DECAY, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  KernelScope timing(TTT_KERNEL_GENERIC_FWD, s);
  hipLaunchKernelGGL(kern, grid, dim3(kFwdThreads), lds, s, a, L);
  return hipGetLastError();
}

template <typename T, int LOSS, int ACT, int DECAY>
hipError_t bwd_launch_t(const BwdArgs& a, hipStream_t s, const float* L, float* scratch) {
  KernelScope timing(TTT_KERNEL_GENERIC_BWD, s);
  hipLaunchKernelGGL((bwd_generic_kernel<T, LOSS, ACT, DECAY>), dim3(a.B * a.H), dim3(kBwdThreads), 0, s,
                     a, L, scratch);
  return hipGetLastError();
}

// Expand the runtime enums into template instantiations.
template <template <typename, int, int, int> class F, typename Args, typename... X>
hipError_t dispatch(const Args& a, X... x) {
  auto by_decay = [&](auto tt, auto ll, auto aa) -> hipError_t {
    using TT = typename decltype(tt)::type;
    constexpr int LL = decltype(ll)::value, AA = decltype(aa)::value;
    switch (a.decay) {
      case 0: return F<TT, LL, AA, 0>::run(a, x...);
      case 1: return F<TT, LL, AA, 1>::run(a, x...);
      default: return F<TT, LL, AA, 2>::run(a, x...);
    }
  };
  auto by_act = [&](auto tt, auto ll) -> hipError_t {
    if (a.act == 1) return by_decay(tt, ll, std::integral_constant<int, 1>{});
    if (a.act == 2) return by_decay(tt, ll, std::integral_constant<int, 2>{});
    return by_decay(tt, ll, std::integral_constant<int, 0>{});
  };
  auto by_loss = [&](auto tt) -> hipError_t {
    if (a.loss == 1) return by_act(tt, std::integral_constant<int, 1>{});
    if (a.loss == 2) return by_act(tt, std::integral_constant<int, 2>{});
    return by_act(tt, std::integral_constant<int, 0>{});
  };
  if (a.dtype == TTT_BF16) return by_loss(std::type_identity<bf16_t>{});
  return by_loss(std::type_identity<float>{});
}

template <typename T, int LOSS, int ACT, int DECAY> struct FwdRun {
  static hipError_t run(const FwdArgs& a, hipStream_t s, const float* L) {
    return fwd_launch_t<T, LOSS, ACT, DECAY>(a, s, L);
  }
};
template <typename T, int LOSS, int ACT, int DECAY> struct BwdRun {
  static hipError_t run(const BwdArgs& a, hipStream_t s, const float* L, float* sc) {
    return bwd_launch_t<T, LOSS, ACT, DECAY>(a, s, L, sc);
  }
};

hipError_t launch_cumsum(const float* la, float* L, int BH, int T, int C, int NC, int dk, hipStream_t s) {
  int64_t total = static_cast<int64_t>(BH) * NC * dk;
  int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  KernelScope timing(TTT_KERNEL_DECAY_CUMSUM, s);
  hipLaunchKernelGGL(decay_cumsum_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, s, la, L,
                     BH, T, C, NC, dk);
  return hipGetLastError();
}

}  // namespace

size_t generic_fwd_workspace(const FwdArgs& a) {
  if (a.decay != TTT_DECAY_VECTOR) return 0;
  return align256(sizeof(float) * static_cast<size_t>(a.B) * a.H * a.T * a.dk);
}

size_t generic_bwd_workspace(const BwdArgs& a) {
  size_t L = (a.decay == TTT_DECAY_VECTOR) ? align256(sizeof(float) * static_cast<size_t>(a.B) * a.H * a.T * a.dk)
                                            : 0;
  BwdScratch sc(a.C, a.dk, a.dv);
  return L + align256(sizeof(float) * static_cast<size_t>(a.B) * a.H * sc.total);
}

hipError_t generic_fwd_launch(const FwdArgs& a, hipStream_t s) {
  float* L = nullptr;
  if (a.decay == TTT_DECAY_VECTOR) {
    L = reinterpret_cast<float*>(a.ws);
    hipError_t e = launch_cumsum(a.log_decay, L, a.B * a.H, a.T, a.C, a.NC, a.dk, s);
    if (e != hipSuccess) return e;
  }
  return dispatch<FwdRun>(a, s, static_cast<const float*>(L));
}

hipError_t generic_bwd_launch(const BwdArgs& a, hipStream_t s) {
  char* p = a.ws;
  float* L = nullptr;
  if (a.decay == TTT_DECAY_VECTOR) {
    L = reinterpret_cast<float*>(p);
    p += align256(sizeof(float) * static_cast<size_t>(a.B) * a.H * a.T * a.dk);
    hipError_t e = launch_cumsum(a.log_decay, L, a.B * a.H, a.T, a.C, a.NC, a.dk, s);
    if (e != hipSuccess) return e;
  }
  return dispatch<BwdRun>(a, s, static_cast<const float*>(L), reinterpret_cast<float*>(p));
}

}  // namespace ttt
