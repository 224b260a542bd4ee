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
// chain is not separable over output columns; one workgroup carries one
// chain through its chunks.  Each chunk is a fixed sequence of small GEMMs
// (64 x 64 output tiles on 8 waves: a 32 x 32 fp32 matrix-core block and half
// of each k-slice per wave; operands staged through double-buffered LDS in
// 64-deep k-slices) over fp32 per-chain buffers in the caller's workspace; the state
// W1, W2 is double-buffered there so the update of chunk i can run beside its
// output.

#include "ttt_device.h"
#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr int kThreads = 512;     // 8 waves: two per output quadrant, one per half of each k-slice
constexpr int kTile = 64;          // output tile (rows and columns)
constexpr int kKS = 64;            // k-slice staged per LDS round
constexpr int kPitch = kTile + 4;  // LDS row pitch (floats): 16-byte aligned rows
constexpr int kPerThr = kTile * kKS / kThreads;  // staged elements per operand and thread
constexpr int kBuf = 2 * kKS * kPitch;           // floats of one staged slice: A, then B
constexpr size_t kLdsBytes = sizeof(float) * (2 * kBuf + 4 * 16 * 64);

// One product term alpha * op(A) op(B) of a GEMM over fp32 memory, op(A)
// [M x K], op(B) [K x N].  Element (m, k) of op(A) is a[m * lda + k], or
// a[k * lda + m] when A is taken transposed (AT); likewise (k, n) of op(B) is
// b[k * ldb + n], or b[n * ldb + k] (BT).
struct Term {
  const float* a;
  int lda;
  const float* b;
  int ldb;
  int K;
  float alpha;
};

// Per-chain workspace regions, in floats (each rounded up to 64 floats).
struct MlpScratch {
  int64_t w1[2], w2[2], q, k, v, z1, a, g2, g2e, g1e, s, total;
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
    q = take(static_cast<int64_t>(C) * dk);
    k = take(static_cast<int64_t>(C) * dk);
    v = take(static_cast<int64_t>(C) * dv);
    z1 = take(static_cast<int64_t>(C) * dh);  // Z1, then A_q (Z1 is dead once G1 is formed)
    a = take(static_cast<int64_t>(C) * dh);
    g2 = take(static_cast<int64_t>(C) * dv);
    g2e = take(static_cast<int64_t>(C) * dv);
    g1e = take(static_cast<int64_t>(C) * dh);
    s = take(static_cast<int64_t>(C) * C);  // Tril(Q K^T), then Tril(A_q A^T)
    total = o;
  }
};

// Staging of one 64 x 64 k-slice of A and of B: thread tid moves the
// elements tid + 512 i, i < 8, walking the operand's contiguous index so that
// neighbouring threads read neighbouring addresses.  Along a contiguous k the
// thread keeps one k and steps the row by 8; along a contiguous m or n it
// keeps one column and steps k by 8.
// The thread index as a value the compiler cannot see through.  The staging
// offsets derive from it; taking it anew at every slice keeps them from being
// hoisted out of the chunk loop for each of the chunk's GEMMs at once (which
// would hold hundreds of registers for the whole kernel).
__device__ __forceinline__ int opaque_tid() {
  int t = static_cast<int>(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

template <int TR> struct SliceMap;
template <> struct SliceMap<0> {  // contiguous along k: (row, k) = (tid / 64 + 8 i, tid % 64)
  static __device__ __forceinline__ int row(int tid, int i) { return tid / kKS + (kThreads / kKS) * i; }
  static __device__ __forceinline__ int kk(int tid, int) { return tid % kKS; }
};
template <> struct SliceMap<1> {  // contiguous along the row index: (row, k) = (tid % 64, tid / 64 + 8 i)
  static __device__ __forceinline__ int row(int tid, int) { return tid % kTile; }
  static __device__ __forceinline__ int kk(int tid, int i) { return tid / kTile + (kThreads / kTile) * i; }
};

// The registers of one staged k-slice.  A row-major A and a transposed B are
// contiguous along k (map 0); a transposed A and a row-major B along the row
// or column index (map 1).
struct Slice {
  float a[kPerThr], b[kPerThr];
  unsigned ma, mb;  // bit i: element i lies inside the operand (else it stages as zero)
};

// The loads are unconditional (an element outside the operand reads offset 0,
// which every operand has) and the bounds are applied when the slice is
// written to LDS: a load under a branch makes the compiler wait for it on the
// spot, which would serialise the prefetch.
template <int AT, int BT>
__device__ __forceinline__ void load_slice(Slice& r, const Term& t, int M, int N, int m0, int n0, int k0) {
  using MA = SliceMap<AT>;
  using MB = SliceMap<BT ? 0 : 1>;
  const int tid = opaque_tid();
  r.ma = 0;
  r.mb = 0;
#pragma unroll
  for (int i = 0; i < kPerThr; ++i) {
    const int gm = m0 + MA::row(tid, i), gk = k0 + MA::kk(tid, i);
    const bool in = gm < M && gk < t.K;
    const int off = AT ? gk * t.lda + gm : gm * t.lda + gk;  // per-chain buffers: < 2^31 elements
    r.a[i] = t.a[in ? off : 0];
    r.ma |= static_cast<unsigned>(in) << i;
  }
#pragma unroll
  for (int i = 0; i < kPerThr; ++i) {
    const int gn = n0 + MB::row(tid, i), gk = k0 + MB::kk(tid, i);
    const bool in = gk < t.K && gn < N;
    const int off = BT ? gn * t.ldb + gk : gk * t.ldb + gn;
    r.b[i] = t.b[in ? off : 0];
    r.mb |= static_cast<unsigned>(in) << i;
  }
}

template <int AT, int BT>
__device__ __forceinline__ void store_slice(const Slice& r, float alpha, float* buf) {
  using MA = SliceMap<AT>;
  using MB = SliceMap<BT ? 0 : 1>;
  const int tid = opaque_tid();
  float* As = buf;
  float* Bs = buf + kKS * kPitch;
#pragma unroll
  for (int i = 0; i < kPerThr; ++i)
    As[MA::kk(tid, i) * kPitch + MA::row(tid, i)] = ((r.ma >> i) & 1u) ? alpha * r.a[i] : 0.0f;
#pragma unroll
  for (int i = 0; i < kPerThr; ++i)
    Bs[MB::kk(tid, i) * kPitch + MB::row(tid, i)] = ((r.mb >> i) & 1u) ? r.b[i] : 0.0f;
}

typedef float floatx16 __attribute__((ext_vector_type(16)));

// Wave w of the workgroup owns the 32 x 32 quadrant q = w % 4, at (32 (q % 2),
// 32 (q / 2)), of a 64 x 64 output tile, for the half g = w / 4 of every
// k-slice (k = 32 g ... 32 g + 31), and accumulates it with
// v_mfma_f32_32x32x2_f32 (fp32 operands, fp32 accumulation): per step lane l
// feeds op(A)[l % 32][k + l / 32] and op(B)[k + l / 32][l % 32], and after it
// holds element r of the quadrant at row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.  The two halves are added at the end of the tile.
__device__ __forceinline__ int quad_row(int r) { return 8 * (r / 4) + 4 * (static_cast<int>(threadIdx.x) % 64 / 32) + r % 4; }

// This wave's products of one staged slice: acc += its k-half of A_s B_s.
__device__ __forceinline__ void slice_products(floatx16& acc, const float* buf) {
  const int lane = threadIdx.x % 64, w = threadIdx.x / 64, q = w % 4, g = w / 4;
  const int a_off = (kKS / 2 * g + lane / 32) * kPitch + 32 * (q % 2) + lane % 32;
  const int b_off = kKS * kPitch + (kKS / 2 * g + lane / 32) * kPitch + 32 * (q / 2) + lane % 32;
  float av[kKS / 4], bv[kKS / 4];  // all LDS reads of the half-slice first, then the products
#pragma unroll
  for (int j = 0; j < kKS / 4; ++j) {
    av[j] = buf[2 * j * kPitch + a_off];
    bv[j] = buf[2 * j * kPitch + b_off];
  }
#pragma unroll
  for (int j = 0; j < kKS / 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[j], bv[j], acc, 0, 0, 0);
}

// out(m, n) = epi(m, n, op(A1) op(B1) [+ op(A2) op(B2)]) for m < M, n < N, in
// 64 x 64 tiles.  The second term is used when K2 = t2.K > 0.
// Causal shortcuts: LOWER computes only the tiles that reach the diagonal or
// below (n0 < m0 + 64; a causal score matrix, whose strictly upper tiles are
// never read), and TRI2 ends the second term's k range at the row tile's last
// row (its A is such a score matrix, zero right of the diagonal).
//
// The GEMM is one flat sequence of steps (tile, term, k-slice).  Slices are
// double-buffered in LDS: the next step's slice -- in the same tile or the
// next -- is fetched into registers before this step's products and written to
// the other buffer after them, so one barrier per step suffices and a tile's
// first slice is not waited for.  At a tile's end the two k-halves are added
// through a separate LDS area: group 0 finishes elements 0..7 of its quadrant,
// group 1 elements 8..15.
template <int AT1, int BT1, int AT2, int BT2, bool LOWER = false, bool TRI2 = false, class Epi>
__device__ __forceinline__ void gemm(int M, int N, const Term& t1, const Term& t2, const float* aux, int ldaux,
                                     float* lds, Epi epi) {
  const int lane = threadIdx.x % 64, w = threadIdx.x / 64, q = w % 4, g = w / 4;
  float* red = lds + 2 * kBuf + q * 16 * 64;  // [quadrant][element][lane]
  const int ntm = (M + kTile - 1) / kTile, ntn = (N + kTile - 1) / kTile;
  auto k2_of = [&](int mt) { return TRI2 ? min(t2.K, (mt + 1) * kTile) : t2.K; };
  auto ntn_of = [&](int mt) { return LOWER ? min(ntn, mt + 1) : ntn; };
  // step state: row tile, column tile, term (0 / 1), slice
  int mt = 0, nt = 0, tm = 0, sl = 0;
  auto fetch = [&](Slice& r, int mt_, int nt_, int tm_, int sl_) {
    if (tm_ == 0) {
      load_slice<AT1, BT1>(r, t1, M, N, mt_ * kTile, nt_ * kTile, sl_ * kKS);
    } else {
      Term u = t2;
      u.K = k2_of(mt_);
      load_slice<AT2, BT2>(r, u, M, N, mt_ * kTile, nt_ * kTile, sl_ * kKS);
    }
  };
  auto put = [&](const Slice& r, int tm_, float* buf) {
    if (tm_ == 0) store_slice<AT1, BT1>(r, t1.alpha, buf);
    else store_slice<AT2, BT2>(r, t2.alpha, buf);
  };
  Slice r;
  fetch(r, 0, 0, 0, 0);
  put(r, 0, lds);
  __syncthreads();
  floatx16 acc = {};
  int b = 0;
  for (;;) {
    // the step after (mt, nt, tm, sl)
    int mt2 = mt, nt2 = nt, tm2 = tm, sl2 = sl + 1;
    const int nsl = ((tm == 0 ? t1.K : k2_of(mt)) + kKS - 1) / kKS;
    if (sl2 >= nsl) {
      sl2 = 0;
      if (tm == 0 && k2_of(mt) > 0) {
        tm2 = 1;
      } else {
        tm2 = 0;
        if (++nt2 >= ntn_of(mt)) {
          nt2 = 0;
          ++mt2;
        }
      }
    }
    const bool more = mt2 < ntm;
    if (more) fetch(r, mt2, nt2, tm2, sl2);
    slice_products(acc, lds + b * kBuf);
    if (more) put(r, tm2, lds + (b ^ 1) * kBuf);
    __syncthreads();
    if (!more || mt2 != mt || nt2 != nt) {  // the tile (mt, nt) is complete
      const int n = nt * kTile + 32 * (q / 2) + lane % 32;
      const int mq = mt * kTile + 32 * (q % 2);
      // The epilogue's own operand (aux at the output position) is loaded for all
      // eight elements at once, before the exchange, so its latency overlaps it.
      float ax[8];
      const int nc = min(n, N - 1);
      if (g == 0) {
        if (aux) {
#pragma unroll
          for (int e = 0; e < 8; ++e) ax[e] = aux[min(mq + quad_row(e), M - 1) * ldaux + nc];
        }
#pragma unroll
        for (int e = 8; e < 16; ++e) red[e * 64 + lane] = acc[e];
      } else {
        if (aux) {
#pragma unroll
          for (int e = 0; e < 8; ++e) ax[e] = aux[min(mq + quad_row(e + 8), M - 1) * ldaux + nc];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) red[e * 64 + lane] = acc[e];
      }
      __syncthreads();
      if (g == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = mq + quad_row(e);
          if (m < M && n < N) epi(m, n, acc[e] + red[e * 64 + lane], aux ? ax[e] : 0.0f);
        }
      } else {
#pragma unroll
        for (int e = 8; e < 16; ++e) {
          const int m = mq + quad_row(e);
          if (m < M && n < N) epi(m, n, acc[e] + red[e * 64 + lane], aux ? ax[e - 8] : 0.0f);
        }
      }
      acc = floatx16{};
      // red is next written at the following tile's end, after at least one more step barrier
    }
    if (!more) break;
    mt = mt2; nt = nt2; tm = tm2; sl = sl2;
    b ^= 1;
  }
  __syncthreads();  // the caller's next GEMM restages slice buffer 0 and red
}

template <int AT, int BT, bool LOWER = false, class Epi>
__device__ __forceinline__ void gemm1(int M, int N, const Term& t, const float* aux, int ldaux, float* lds, Epi epi) {
  gemm<AT, BT, 0, 0, LOWER>(M, N, t, Term{nullptr, 0, nullptr, 0, 0, 0.0f}, aux, ldaux, lds, epi);
}

// dst[i] = src[i] as fp32 for i < n: each thread issues eight loads (clamped
// to the last element) before it stores, so their latencies overlap.
template <class E, typename T>
__device__ __forceinline__ void stage_rows(float* __restrict__ dst, const T* __restrict__ src, int n) {
  constexpr int kU = 8;
  for (int i0 = threadIdx.x; i0 < n; i0 += kThreads * kU) {
    float x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) x[u] = E::ld(src, min(i0 + u * kThreads, n - 1));
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (i0 + u * kThreads < n) dst[i0 + u * kThreads] = x[u];
  }
}

struct MlpArgs {
  int B, H, T, dk, dh, dv, C, NC;
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
  float* scratch;
};

template <typename T, int LOSS, int ACT, int DECAY>
__global__ __launch_bounds__(kThreads) void mlp_fwd_kernel(MlpArgs a) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];  // two slice buffers, then the k-half sums (kLdsBytes)
  __shared__ float eta[256];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int dk = a.dk, dh = a.dh, dv = a.dv, C = a.C;
  const MlpScratch L(C, dk, dh, dv);
  float* sc = a.scratch + static_cast<int64_t>(bh) * L.total;
  float* Qc = sc + L.q;
  float* Kc = sc + L.k;
  float* Vc = sc + L.v;
  float* Z1 = sc + L.z1;
  float* Aq = sc + L.z1;
  float* Ac = sc + L.a;
  float* G2 = sc + L.g2;
  float* G2e = sc + L.g2e;
  float* G1e = sc + L.g1e;
  float* S = sc + L.s;
  const float g = (DECAY == 1) ? a.gamma[bh % a.H] : 1.0f;

  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk;
  const int64_t off_v = static_cast<int64_t>(bh) * a.T * dv;
  const T* q = static_cast<const T*>(a.q) + off_k;
  const T* k = static_cast<const T*>(a.k) + off_k;
  const T* v = static_cast<const T*>(a.v) + off_v;
  T* o = static_cast<T*>(a.o) + off_v;
  const float* beta = a.beta + static_cast<int64_t>(bh) * a.T;

  int cur = 0;
  {
    const int64_t n1 = static_cast<int64_t>(dk) * dh, n2 = static_cast<int64_t>(dh) * dv;
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

    // The chunk's inputs as fp32 rows, and eta.
    stage_rows<E>(Qc, q + static_cast<int64_t>(t0) * dk, c * dk);
    stage_rows<E>(Kc, k + static_cast<int64_t>(t0) * dk, c * dk);
    stage_rows<E>(Vc, v + static_cast<int64_t>(t0) * dv, c * dv);
    for (int t = tid; t < c; t += kThreads) eta[t] = lr_gate(beta[t0 + t], a.b);
    __syncthreads();

    // Pass 1, first Linear and f:  Z1 = K W1,  A = f(Z1).
    gemm1<0, 0>(c, dh, Term{Kc, dk, W1, dh, dk, 1.0f}, nullptr, 0, lds, [&](int m, int n, float x, float) {
      Z1[m * dh + n] = x;
      Ac[m * dh + n] = act_f<ACT>(x);
    });
    if constexpr (LOSS == 1) {  // IP: the signal at the output does not depend on the state
      for (int i = tid; i < c * dv; i += kThreads) {
        G2[i] = -Vc[i];
        G2e[i] = -eta[i / dv] * Vc[i];
      }
    }
    __syncthreads();
    if constexpr (LOSS != 1) {  // Pass 1, second Linear, and the signal G2 = A W2 - V (MSE) or its sign (L1).
      gemm1<0, 0>(c, dv, Term{Ac, dh, W2, dv, dh, 1.0f}, Vc, dv, lds, [&](int m, int n, float x, float vv) {
        const float e = loss_signal<LOSS, 0>(x, vv);
        G2[m * dv + n] = e;
        G2e[m * dv + n] = eta[m] * e;
      });
      __syncthreads();
    }

    // Pass 2 through the first Linear: eta G1 = eta (G2 W2^T) (.) f'(Z1).  And Tril(Q K^T).
    gemm1<0, 1>(c, dh, Term{G2, dv, W2, dv, dv, 1.0f}, Z1, dh, lds,
                [&](int m, int n, float x, float z) { G1e[m * dh + n] = eta[m] * x * act_df<ACT>(z); });
    gemm1<0, 1, true>(c, c, Term{Qc, dk, Kc, dk, dk, 1.0f}, nullptr, 0, lds,
                      [&](int m, int n, float x, float) { S[m * C + n] = (n <= m) ? x : 0.0f; });
    __syncthreads();

    // Pass 3, first Linear: A_q = f(Q W1 - Tril(Q K^T) eta G1).
    gemm<0, 0, 0, 0, false, true>(c, dh, Term{Qc, dk, W1, dh, dk, 1.0f}, Term{S, C, G1e, dh, c, -1.0f}, nullptr, 0,
                                  lds, [&](int m, int n, float x, float) { Aq[m * dh + n] = act_f<ACT>(x); });
    __syncthreads();
    gemm1<0, 1, true>(c, c, Term{Aq, dh, Ac, dh, dh, 1.0f}, nullptr, 0, lds,
                      [&](int m, int n, float x, float) { S[m * C + n] = (n <= m) ? x : 0.0f; });
    __syncthreads();

    // Pass 3, second Linear: O = A_q W2 - Tril(A_q A^T) eta G2; and both state steps.
    gemm<0, 0, 0, 0, false, true>(c, dv, Term{Aq, dh, W2, dv, dh, 1.0f}, Term{S, C, G2e, dv, c, -1.0f}, nullptr, 0,
                                  lds, [&](int m, int n, float x, float) {
                                    E::st(o, static_cast<int64_t>(t0 + m) * dv + n, x);
                                  });
    gemm1<1, 0>(dk, dh, Term{Kc, dk, G1e, dh, c, -1.0f}, W1, dh, lds,
                [&](int m, int n, float x, float w) { W1n[m * dh + n] = fmaf(g, w, x); });
    gemm1<1, 0>(dh, dv, Term{Ac, dh, G2e, dv, c, -1.0f}, W2, dv, lds,
                [&](int m, int n, float x, float w) { W2n[m * dv + n] = fmaf(g, w, x); });
    __syncthreads();
    cur ^= 1;
  }

  const int64_t n1 = static_cast<int64_t>(dk) * dh, n2 = static_cast<int64_t>(dh) * dv;
  const float* W1 = sc + (cur ? L.w1[1] : L.w1[0]);
  const float* W2 = sc + (cur ? L.w2[1] : L.w2[0]);
  if (a.w1_final)
    for (int64_t i = tid; i < n1; i += kThreads) a.w1_final[bh * n1 + i] = W1[i];
  if (a.w2_final)
    for (int64_t i = tid; i < n2; i += kThreads) a.w2_final[bh * n2 + i] = W2[i];
}

template <typename T, int LOSS, int ACT, int DECAY>
hipError_t launch_t(const MlpArgs& a, hipStream_t s) {
  auto kern = mlp_fwd_kernel<T, LOSS, ACT, DECAY>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
  if (e != hipSuccess) return e;
  KernelScope timing(TTT_KERNEL_MLP_FWD, s);
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(kThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

template <typename T, int LOSS, int ACT>
hipError_t by_decay(const MlpArgs& a, int decay, hipStream_t s) {
  return decay == TTT_DECAY_SCALAR ? launch_t<T, LOSS, ACT, 1>(a, s) : launch_t<T, LOSS, ACT, 0>(a, s);
}

template <typename T, int LOSS>
hipError_t by_act(const MlpArgs& a, int act, int decay, hipStream_t s) {
  if (act == TTT_ACT_SILU) return by_decay<T, LOSS, 1>(a, decay, s);
  if (act == TTT_ACT_GELU) return by_decay<T, LOSS, 2>(a, decay, s);
  return by_decay<T, LOSS, 0>(a, decay, s);
}

template <typename T>
hipError_t by_loss(const MlpArgs& a, int loss, int act, int decay, hipStream_t s) {
  if (loss == TTT_LOSS_IP) return by_act<T, 1>(a, act, decay, s);
  if (loss == TTT_LOSS_L1) return by_act<T, 2>(a, act, decay, s);
  return by_act<T, 0>(a, act, decay, s);
}

}  // namespace

size_t mlp_fwd_workspace(const ttt_mlp_desc& d) {
  const MlpScratch L(d.C, d.dk, d.dh, d.dv);
  return align256(sizeof(float) * static_cast<size_t>(d.B) * d.H * L.total);
}

hipError_t mlp_fwd_launch(const ttt_mlp_desc& d, const void* q, const void* k, const void* v, const float* beta,
                          const float* gamma, const float* w1_0, const float* w2_0, void* o, float* w1_final,
                          float* w2_final, void* ws, hipStream_t s) {
  MlpArgs a{};
  a.B = d.B; a.H = d.H; a.T = d.T; a.dk = d.dk; a.dh = d.dh; a.dv = d.dv; a.C = d.C;
  a.NC = (d.T + d.C - 1) / d.C;
  a.b = d.lr_bias;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.gamma = gamma; a.w1_0 = w1_0; a.w2_0 = w2_0;
  a.o = o; a.w1_final = w1_final; a.w2_final = w2_final;
  a.scratch = static_cast<float*>(ws);
  if (d.dtype == TTT_BF16) return by_loss<bf16_t>(a, d.loss, d.act, d.decay, s);
  return by_loss<float>(a, d.loss, d.act, d.decay, s);
}

}  // namespace ttt
