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

#include <type_traits>

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
// Saved context of the forward for its backward, per (chain, chunk), in floats:
// the train view's Z1, A, G2, eta G2, P = G2 W2^T and eta G1, the query view's X1
// and A_q, and both causal score matrices (strictly upper tiles zeroed).
struct MlpSaved {
  int64_t z1, a, x1, aq, p, gh1, g2, gh2, s1, s2, per_chunk;
  __host__ __device__ MlpSaved(int C, int dh, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t ch = static_cast<int64_t>(C) * dh, cv = static_cast<int64_t>(C) * dv,
                  cc = static_cast<int64_t>(C) * C;
    z1 = take(ch);
    a = take(ch);
    x1 = take(ch);
    aq = take(ch);
    p = take(ch);
    gh1 = take(ch);
    g2 = take(cv);
    gh2 = take(cv);
    s1 = take(cc);
    s2 = take(cc);
    per_chunk = o;
  }
};

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
// Up to three operands of the epilogue, each read at the output position (m, n)
// as p[j][m * ld + n]; a null p[j] reads as 0.
struct Aux {
  const float* p[3];
  int ld;
};

template <int AT1, int BT1, int AT2, int BT2, bool LOWER = false, bool TRI2 = false, class Epi>
__device__ __forceinline__ void gemm(int M, int N, const Term& t1, const Term& t2, const Aux& aux, float* lds,
                                     Epi epi) {
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
      // The epilogue's own operands (aux at the output position) are loaded for all
      // eight elements at once, before the exchange, so their latency overlaps it.
      float ax[3][8];
      const int nc = min(n, N - 1);
      const int eb = 8 * g;  // this group finishes elements eb .. eb + 7
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (aux.p[j]) {
#pragma unroll
          for (int e = 0; e < 8; ++e) ax[j][e] = aux.p[j][min(mq + quad_row(e + eb), M - 1) * aux.ld + nc];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) ax[j][e] = 0.0f;
        }
      }
      if (g == 0) {
#pragma unroll
        for (int e = 8; e < 16; ++e) red[e * 64 + lane] = acc[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[e * 64 + lane] = acc[e];
      }
      __syncthreads();
      if (g == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = mq + quad_row(e);
          if (m < M && n < N) epi(m, n, acc[e] + red[e * 64 + lane], ax[0][e], ax[1][e], ax[2][e]);
        }
      } else {
#pragma unroll
        for (int e = 8; e < 16; ++e) {
          const int m = mq + quad_row(e);
          if (m < M && n < N) epi(m, n, acc[e] + red[e * 64 + lane], ax[0][e - 8], ax[1][e - 8], ax[2][e - 8]);
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

constexpr Aux kNoAux{{nullptr, nullptr, nullptr}, 0};

template <int AT, int BT, bool LOWER = false, class Epi>
__device__ __forceinline__ void gemm1(int M, int N, const Term& t, const Aux& aux, float* lds, Epi epi) {
  gemm<AT, BT, 0, 0, LOWER>(M, N, t, Term{nullptr, 0, nullptr, 0, 0, 0.0f}, aux, lds, epi);
}

// Zero the strictly upper 64 x 64 tiles of a c x c causal score matrix (row
// pitch ld), which a LOWER GEMM leaves unwritten: the backward also reads these
// matrices transposed over their full width.
__device__ __forceinline__ void zero_upper_tiles(float* S, int c, int ld) {
  for (int i = threadIdx.x; i < c * c; i += kThreads) {
    const int m = i / c, n = i % c;
    if (n >= (m / kTile + 1) * kTile) S[m * ld + n] = 0.0f;
  }
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
  float* w1_ckpt;  // [B,H,NC,dk,dh] or null: W1 at each chunk's start
  float* w2_ckpt;  // [B,H,NC,dh,dv] or null
  float* saved;    // MlpSaved per (chain, chunk), or null
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
    // Where this chunk's intermediates go: the workspace, or the saved context (then
    // also P and X1, with A_q and the second score matrix kept apart).
    float *Z1c = Z1, *Acc = Ac, *Aqc = Aq, *G2c = G2, *G2ec = G2e, *G1ec = G1e, *S1c = S, *S2c = S;
    float *Pc = nullptr, *X1c = nullptr;
    if (a.saved) {
      const MlpSaved SV(C, dh, dv);
      float* sb = a.saved + (static_cast<int64_t>(bh) * a.NC + ci) * SV.per_chunk;
      Z1c = sb + SV.z1; Acc = sb + SV.a; X1c = sb + SV.x1; Aqc = sb + SV.aq; Pc = sb + SV.p; G1ec = sb + SV.gh1;
      G2c = sb + SV.g2; G2ec = sb + SV.gh2; S1c = sb + SV.s1; S2c = sb + SV.s2;
    }

    // The chunk's inputs as fp32 rows, and eta.
    stage_rows<E>(Qc, q + static_cast<int64_t>(t0) * dk, c * dk);
    stage_rows<E>(Kc, k + static_cast<int64_t>(t0) * dk, c * dk);
    stage_rows<E>(Vc, v + static_cast<int64_t>(t0) * dv, c * dv);
    for (int t = tid; t < c; t += kThreads) eta[t] = lr_gate(beta[t0 + t], a.b);
    {
      const int64_t n1 = static_cast<int64_t>(dk) * dh, n2 = static_cast<int64_t>(dh) * dv;
      const int64_t ck = static_cast<int64_t>(bh) * a.NC + ci;
      if (a.w1_ckpt) stage_rows<Elem<float>>(a.w1_ckpt + ck * n1, W1, static_cast<int>(n1));
      if (a.w2_ckpt) stage_rows<Elem<float>>(a.w2_ckpt + ck * n2, W2, static_cast<int>(n2));
    }
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
    if constexpr (LOSS != 1) {  // Pass 1, second Linear, and the signal G2 = A W2 - V (MSE) or its sign (L1).
      gemm1<0, 0>(c, dv, Term{Acc, dh, W2, dv, dh, 1.0f}, Aux{{Vc, nullptr, nullptr}, dv}, lds,
                  [&](int m, int n, float x, float vv, float, float) {
        const float e = loss_signal<LOSS, 0>(x, vv);
        G2c[m * dv + n] = e;
        G2ec[m * dv + n] = eta[m] * e;
      });
      __syncthreads();
    }

    // Pass 2 through the first Linear: eta G1 = eta (G2 W2^T) (.) f'(Z1).  And Tril(Q K^T).
    gemm1<0, 1>(c, dh, Term{G2c, dv, W2, dv, dv, 1.0f}, Aux{{Z1c, nullptr, nullptr}, dh}, lds,
                [&](int m, int n, float x, float z, float, float) {
                  G1ec[m * dh + n] = eta[m] * x * act_df<ACT>(z);
                  if (Pc) Pc[m * dh + n] = x;
                });
    gemm1<0, 1, true>(c, c, Term{Qc, dk, Kc, dk, dk, 1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { S1c[m * C + n] = (n <= m) ? x : 0.0f; });
    if (a.saved) zero_upper_tiles(S1c, c, C);
    __syncthreads();

    // Pass 3, first Linear: A_q = f(Q W1 - Tril(Q K^T) eta G1).
    gemm<0, 0, 0, 0, false, true>(c, dh, Term{Qc, dk, W1, dh, dk, 1.0f}, Term{S1c, C, G1ec, dh, c, -1.0f}, kNoAux,
                                  lds, [&](int m, int n, float x, float, float, float) {
                                    Aqc[m * dh + n] = act_f<ACT>(x);
                                    if (X1c) X1c[m * dh + n] = x;
                                  });
    __syncthreads();
    gemm1<0, 1, true>(c, c, Term{Aqc, dh, Acc, dh, dh, 1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { S2c[m * C + n] = (n <= m) ? x : 0.0f; });
    if (a.saved) zero_upper_tiles(S2c, c, C);
    __syncthreads();

    // Pass 3, second Linear: O = A_q W2 - Tril(A_q A^T) eta G2; and both state steps.
    gemm<0, 0, 0, 0, false, true>(c, dv, Term{Aqc, dh, W2, dv, dh, 1.0f}, Term{S2c, C, G2ec, dv, c, -1.0f}, kNoAux,
                                  lds, [&](int m, int n, float x, float, float, float) {
                                    E::st(o, static_cast<int64_t>(t0 + m) * dv + n, x);
                                  });
    gemm1<1, 0>(dk, dh, Term{Kc, dk, G1ec, dh, c, -1.0f}, Aux{{W1, nullptr, nullptr}, dh}, lds,
                [&](int m, int n, float x, float w, float, float) { W1n[m * dh + n] = fmaf(g, w, x); });
    gemm1<1, 0>(dh, dv, Term{Acc, dh, G2ec, dv, c, -1.0f}, Aux{{W2, nullptr, nullptr}, dv}, lds,
                [&](int m, int n, float x, float w, float, float) { W2n[m * dv + n] = fmaf(g, w, x); });
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

// ---------------------------------------------------------------------------
// Outer backward: the reverse chunk sweep.  For the outer loss
// <dO, O> + <dW1_T, W1_T> + <dW2_T, W2_T>, chunk i (from the last to the first)
// recomputes its forward from the checkpoints W1_i, W2_i and differentiates its
// steps in reverse order, carrying dW1_{i+1}, dW2_{i+1} (written D1, D2 below):
//   dS2 = -Tril(dO (eta G2)^T);  d(eta G2) = -S2^T dO - A D2
//   dX1 = (dO W2^T + dS2 A) (.) f'(X1);  dA = dS2^T A_q - (eta G2) D2^T
//   dS1 = -Tril(dX1 (eta G1)^T);  dQ = dX1 W1^T + dS1 K
//   d(eta G1) = -S1^T dX1 - K D1;  dG1 = eta d(eta G1);  dP = dG1 (.) f'(Z1)
//   dZ1 = dG1 (.) P (.) f''(Z1) + (dA + dV_hat W2^T) (.) f'(Z1)
//   dG2 = eta d(eta G2) + dP W2;  dV_hat = dG2 (MSE, else 0);  dV = -dG2 (MSE, IP) or 0 (L1)
//   dK = dS1^T Q - (eta G1) D1^T + dZ1 W1^T
//   dW1_i = g D1 + Q^T dX1 + K^T dZ1;  dW2_i = g D2 + A_q^T dO + dP^T G2 + A^T dV_hat
//   d eta_t = <d(eta G1)_t, G1_t> + <d(eta G2)_t, G2_t>;  d beta = d eta eta (1 - eta / 2)
//   d gamma += <D1, W1_i> + <D2, W2_i>
// with P = G2 W2^T and G1 = P (.) f'(Z1) as in the forward.  Every product is a
// GEMM of the same tile machinery; the chunk's intermediates live in the
// workspace.
// ---------------------------------------------------------------------------

struct MlpBwdScratch {
  int64_t dw1[2], dw2[2], q, k, v, dout, z1, a, x1, aq, p, gh1, dx1, dgh1, da, dp, dz1, g2, gh2, dgh2, dg2, dkp,
      s1, s2, ds, total;
  __host__ __device__ MlpBwdScratch(int C, int dk, int dh, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t ch = static_cast<int64_t>(C) * dh, cv = static_cast<int64_t>(C) * dv,
                  ckk = static_cast<int64_t>(C) * dk, cc = static_cast<int64_t>(C) * C;
    dw1[0] = take(static_cast<int64_t>(dk) * dh);
    dw1[1] = take(static_cast<int64_t>(dk) * dh);
    dw2[0] = take(static_cast<int64_t>(dh) * dv);
    dw2[1] = take(static_cast<int64_t>(dh) * dv);
    q = take(ckk);
    k = take(ckk);
    v = take(cv);
    dout = take(cv);
    z1 = take(ch);
    a = take(ch);
    x1 = take(ch);
    aq = take(ch);
    p = take(ch);
    gh1 = take(ch);
    dx1 = take(ch);
    dgh1 = take(ch);
    da = take(ch);
    dp = take(ch);
    dz1 = take(ch);
    g2 = take(cv);
    gh2 = take(cv);
    dgh2 = take(cv);
    dg2 = take(cv);
    dkp = take(ckk);
    s1 = take(cc);
    s2 = take(cc);
    ds = take(cc);
    total = o;
  }
};

struct MlpBwdArgs {
  int B, H, T, dk, dh, dv, C, NC;
  float b;
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* gamma;
  const float* w1_ckpt;
  const float* w2_ckpt;
  const float* saved;  // the forward's MlpSaved per (chain, chunk), or null: recompute
  const void* d_o;
  const float* d_w1final;
  const float* d_w2final;
  void* dq;
  void* dk_out;
  void* dv_out;
  float* dbeta;
  float* dgamma;
  float* dw1_0;
  float* dw2_0;
  float* scratch;
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <typename T, int LOSS, int ACT, int DECAY>
__global__ __launch_bounds__(kThreads) void mlp_bwd_kernel(MlpBwdArgs a) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];
  __shared__ float eta[256];
  __shared__ float wsum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  const int bh = blockIdx.x;
  const int dk = a.dk, dh = a.dh, dv = a.dv, C = a.C;
  const MlpBwdScratch L(C, dk, dh, dv);
  float* sc = a.scratch + static_cast<int64_t>(bh) * L.total;
  float* Qc = sc + L.q;
  float* Kc = sc + L.k;
  float* Vc = sc + L.v;
  float* dOc = sc + L.dout;
  float* const Z1_ws = sc + L.z1;
  float* const Ac_ws = sc + L.a;
  float* const X1_ws = sc + L.x1;
  float* const Aq_ws = sc + L.aq;
  float* const P_ws = sc + L.p;
  float* const Gh1_ws = sc + L.gh1;
  float* dX1 = sc + L.dx1;
  float* dGh1 = sc + L.dgh1;
  float* dA = sc + L.da;
  float* dP = sc + L.dp;
  float* dZ1 = sc + L.dz1;
  float* const G2_ws = sc + L.g2;
  float* const Gh2_ws = sc + L.gh2;
  float* dGh2 = sc + L.dgh2;
  float* dG2 = sc + L.dg2;
  float* dKp = sc + L.dkp;
  float* const S1_ws = sc + L.s1;
  float* const S2_ws = sc + L.s2;
  float* dS = sc + L.ds;
  const float g = (DECAY == 1) ? a.gamma[bh % a.H] : 1.0f;

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
  const int64_t n1 = static_cast<int64_t>(dk) * dh, n2 = static_cast<int64_t>(dh) * dv;

  {  // dW_T: the final states' gradients (zero when not given)
    float* D1 = sc + L.dw1[0];
    float* D2 = sc + L.dw2[0];
    const float* s1 = a.d_w1final ? a.d_w1final + bh * n1 : nullptr;
    const float* s2 = a.d_w2final ? a.d_w2final + bh * n2 : nullptr;
    for (int64_t i = tid; i < n1; i += kThreads) D1[i] = s1 ? s1[i] : 0.0f;
    for (int64_t i = tid; i < n2; i += kThreads) D2[i] = s2 ? s2[i] : 0.0f;
  }
  int cur = 0;
  float dgam = 0.0f;  // this thread's share of d gamma, summed in a fixed order
  __syncthreads();

  for (int ci = a.NC - 1; ci >= 0; --ci) {
    const int t0 = ci * C;
    const int c = min(C, a.T - t0);
    const int64_t ck = static_cast<int64_t>(bh) * a.NC + ci;
    const float* W1 = a.w1_ckpt + ck * n1;
    const float* W2 = a.w2_ckpt + ck * n2;
    const float* D1 = sc + (cur ? L.dw1[1] : L.dw1[0]);  // dW1_{i+1}
    const float* D2 = sc + (cur ? L.dw2[1] : L.dw2[0]);
    float* D1o = sc + (cur ? L.dw1[0] : L.dw1[1]);  // dW1_i (written)
    float* D2o = sc + (cur ? L.dw2[0] : L.dw2[1]);

    // The chunk's forward intermediates: recomputed into the workspace, or read from the
    // forward's saved context.
    float *Z1 = Z1_ws, *Ac = Ac_ws, *X1 = X1_ws, *Aq = Aq_ws, *P = P_ws, *Gh1 = Gh1_ws, *G2 = G2_ws, *Gh2 = Gh2_ws,
          *S1 = S1_ws, *S2 = S2_ws;
    const bool have = a.saved != nullptr;
    if (have) {
      const MlpSaved SV(C, dh, dv);
      float* sb = const_cast<float*>(a.saved) + ck * SV.per_chunk;
      Z1 = sb + SV.z1; Ac = sb + SV.a; X1 = sb + SV.x1; Aq = sb + SV.aq; P = sb + SV.p; Gh1 = sb + SV.gh1;
      G2 = sb + SV.g2; Gh2 = sb + SV.gh2; S1 = sb + SV.s1; S2 = sb + SV.s2;
    }
    stage_rows<E>(Qc, q + static_cast<int64_t>(t0) * dk, c * dk);
    stage_rows<E>(Kc, k + static_cast<int64_t>(t0) * dk, c * dk);
    if (!have) stage_rows<E>(Vc, v + static_cast<int64_t>(t0) * dv, c * dv);
    stage_rows<E>(dOc, dO + static_cast<int64_t>(t0) * dv, c * dv);
    for (int t = tid; t < c; t += kThreads) eta[t] = lr_gate(beta[t0 + t], a.b);
    if constexpr (DECAY == 1) {
      for (int64_t i = tid; i < n1; i += kThreads) dgam = fmaf(D1[i], W1[i], dgam);
      for (int64_t i = tid; i < n2; i += kThreads) dgam = fmaf(D2[i], W2[i], dgam);
    }
    __syncthreads();

    if (!have) {  // ---- the chunk's forward again ----
      gemm1<0, 0>(c, dh, Term{Kc, dk, W1, dh, dk, 1.0f}, kNoAux, lds, [&](int m, int n, float x, float, float, float) {
        Z1[m * dh + n] = x;
        Ac[m * dh + n] = act_f<ACT>(x);
      });
      if constexpr (LOSS == 1) {
        for (int i = tid; i < c * dv; i += kThreads) {
          G2[i] = -Vc[i];
          Gh2[i] = -eta[i / dv] * Vc[i];
        }
      }
      __syncthreads();
      if constexpr (LOSS != 1) {
        gemm1<0, 0>(c, dv, Term{Ac, dh, W2, dv, dh, 1.0f}, Aux{{Vc, nullptr, nullptr}, dv}, lds,
                    [&](int m, int n, float x, float vv, float, float) {
                      const float e = loss_signal<LOSS, 0>(x, vv);
                      G2[m * dv + n] = e;
                      Gh2[m * dv + n] = eta[m] * e;
                    });
        __syncthreads();
      }
      gemm1<0, 1>(c, dh, Term{G2, dv, W2, dv, dv, 1.0f}, Aux{{Z1, nullptr, nullptr}, dh}, lds,
                  [&](int m, int n, float x, float z, float, float) {
                    P[m * dh + n] = x;
                    Gh1[m * dh + n] = eta[m] * x * act_df<ACT>(z);
                  });
      gemm1<0, 1, true>(c, c, Term{Qc, dk, Kc, dk, dk, 1.0f}, kNoAux, lds,
                        [&](int m, int n, float x, float, float, float) { S1[m * C + n] = (n <= m) ? x : 0.0f; });
      zero_upper_tiles(S1, c, C);
      __syncthreads();
      gemm<0, 0, 0, 0, false, true>(c, dh, Term{Qc, dk, W1, dh, dk, 1.0f}, Term{S1, C, Gh1, dh, c, -1.0f}, kNoAux,
                                    lds, [&](int m, int n, float x, float, float, float) {
                                      X1[m * dh + n] = x;
                                      Aq[m * dh + n] = act_f<ACT>(x);
                                    });
      __syncthreads();
      gemm1<0, 1, true>(c, c, Term{Aq, dh, Ac, dh, dh, 1.0f}, kNoAux, lds,
                        [&](int m, int n, float x, float, float, float) { S2[m * C + n] = (n <= m) ? x : 0.0f; });
      zero_upper_tiles(S2, c, C);
      __syncthreads();
    }

    // ---- its backward ----
    gemm1<0, 1, true>(c, c, Term{dOc, dv, Gh2, dv, dv, -1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { dS[m * C + n] = (n <= m) ? x : 0.0f; });
    zero_upper_tiles(dS, c, C);
    gemm<1, 0, 0, 0>(c, dv, Term{S2, C, dOc, dv, c, -1.0f}, Term{Ac, dh, D2, dv, dh, -1.0f}, kNoAux, lds,
                     [&](int m, int n, float x, float, float, float) { dGh2[m * dv + n] = x; });
    __syncthreads();
    gemm<0, 1, 0, 0, false, true>(c, dh, Term{dOc, dv, W2, dv, dv, 1.0f}, Term{dS, C, Ac, dh, c, 1.0f},
                                  Aux{{X1, nullptr, nullptr}, dh}, lds,
                                  [&](int m, int n, float x, float x1, float, float) {
                                    dX1[m * dh + n] = x * act_df<ACT>(x1);
                                  });
    gemm<1, 0, 0, 1>(c, dh, Term{dS, C, Aq, dh, c, 1.0f}, Term{Gh2, dv, D2, dv, dv, -1.0f}, kNoAux, lds,
                     [&](int m, int n, float x, float, float, float) { dA[m * dh + n] = x; });
    __syncthreads();
    gemm1<0, 1, true>(c, c, Term{dX1, dh, Gh1, dh, dh, -1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { dS[m * C + n] = (n <= m) ? x : 0.0f; });
    zero_upper_tiles(dS, c, C);
    __syncthreads();
    gemm<0, 1, 0, 0, false, true>(c, dk, Term{dX1, dh, W1, dh, dh, 1.0f}, Term{dS, C, Kc, dk, c, 1.0f}, kNoAux, lds,
                                  [&](int m, int n, float x, float, float, float) {
                                    E::st(dq, static_cast<int64_t>(t0 + m) * dk + n, x);
                                  });
    gemm<1, 0, 0, 0>(c, dh, Term{S1, C, dX1, dh, c, -1.0f}, Term{Kc, dk, D1, dh, dk, -1.0f},
                     Aux{{P, Z1, nullptr}, dh}, lds, [&](int m, int n, float x, float pp, float z, float) {
                       dGh1[m * dh + n] = x;
                       const float dg1 = eta[m] * x;
                       dP[m * dh + n] = dg1 * act_df<ACT>(z);
                       dZ1[m * dh + n] = dg1 * pp * act_d2f<ACT>(z);
                     });
    gemm<1, 0, 0, 1>(c, dk, Term{dS, C, Qc, dk, c, 1.0f}, Term{Gh1, dh, D1, dh, dh, -1.0f}, kNoAux, lds,
                     [&](int m, int n, float x, float, float, float) { dKp[m * dk + n] = x; });
    __syncthreads();
    gemm1<0, 0>(c, dv, Term{dP, dh, W2, dv, dh, 1.0f}, Aux{{dGh2, nullptr, nullptr}, dv}, lds,
                [&](int m, int n, float x, float dgh, float, float) {
                  const float d = fmaf(eta[m], dgh, x);
                  dG2[m * dv + n] = d;
                  E::st(dvv, static_cast<int64_t>(t0 + m) * dv + n, loss_dsignal_dv<LOSS>() * d);
                });
    // d eta per token, one wave per row
    for (int t = wv; t < c; t += kThreads / 64) {
      float sum = 0.0f;
      for (int j = lane; j < dh; j += 64) sum += dGh1[t * dh + j] * P[t * dh + j] * act_df<ACT>(Z1[t * dh + j]);
      for (int j = lane; j < dv; j += 64) sum += dGh2[t * dv + j] * G2[t * dv + j];
      sum = wave_sum(sum);
      if (lane == 0) {
        const float et = eta[t];
        dbeta[t0 + t] = sum * et * (1.0f - 0.5f * et);
      }
    }
    __syncthreads();
    if constexpr (LOSS == 0) {  // dZ1 += (dA + dG2 W2^T) (.) f'(Z1)
      gemm1<0, 1>(c, dh, Term{dG2, dv, W2, dv, dv, 1.0f}, Aux{{dA, dZ1, Z1}, dh}, lds,
                  [&](int m, int n, float x, float da, float dz, float z) {
                    dZ1[m * dh + n] = fmaf(da + x, act_df<ACT>(z), dz);
                  });
    } else {  // dZ1 += dA (.) f'(Z1)
      constexpr int kU = 4;
      const int nz = c * dh;
      for (int i0 = tid; i0 < nz; i0 += kThreads * kU) {
        float da[kU], dz[kU], z[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = min(i0 + u * kThreads, nz - 1);
          da[u] = dA[i];
          dz[u] = dZ1[i];
          z[u] = Z1[i];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (i0 + u * kThreads < nz) dZ1[i0 + u * kThreads] = fmaf(da[u], act_df<ACT>(z[u]), dz[u]);
      }
    }
    __syncthreads();
    gemm1<0, 1>(c, dk, Term{dZ1, dh, W1, dh, dh, 1.0f}, Aux{{dKp, nullptr, nullptr}, dk}, lds,
                [&](int m, int n, float x, float dkp, float, float) {
                  E::st(dkk, static_cast<int64_t>(t0 + m) * dk + n, dkp + x);
                });
    gemm<1, 0, 1, 0>(dk, dh, Term{Qc, dk, dX1, dh, c, 1.0f}, Term{Kc, dk, dZ1, dh, c, 1.0f},
                     Aux{{D1, nullptr, nullptr}, dh}, lds,
                     [&](int m, int n, float x, float d1, float, float) { D1o[m * dh + n] = fmaf(g, d1, x); });
    gemm<1, 0, 1, 0>(dh, dv, Term{Aq, dh, dOc, dv, c, 1.0f}, Term{dP, dh, G2, dv, c, 1.0f},
                     Aux{{D2, nullptr, nullptr}, dv}, lds,
                     [&](int m, int n, float x, float d2, float, float) { D2o[m * dv + n] = fmaf(g, d2, x); });
    if constexpr (LOSS == 0) {  // + A^T dV_hat, dV_hat = dG2
      __syncthreads();
      gemm1<1, 0>(dh, dv, Term{Ac, dh, dG2, dv, c, 1.0f}, Aux{{D2o, nullptr, nullptr}, dv}, lds,
                  [&](int m, int n, float x, float d2, float, float) { D2o[m * dv + n] = d2 + x; });
    }
    __syncthreads();
    cur ^= 1;
  }

  const float* D1 = sc + (cur ? L.dw1[1] : L.dw1[0]);
  const float* D2 = sc + (cur ? L.dw2[1] : L.dw2[0]);
  if (a.dw1_0)
    for (int64_t i = tid; i < n1; i += kThreads) a.dw1_0[bh * n1 + i] = D1[i];
  if (a.dw2_0)
    for (int64_t i = tid; i < n2; i += kThreads) a.dw2_0[bh * n2 + i] = D2[i];
  if constexpr (DECAY == 1) {
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

template <typename T, int LOSS, int ACT, int DECAY>
hipError_t launch_bwd_t(const MlpBwdArgs& a, hipStream_t s) {
  auto kern = mlp_bwd_kernel<T, LOSS, ACT, DECAY>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
  if (e != hipSuccess) return e;
  KernelScope timing(TTT_KERNEL_MLP_BWD, s);
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(kThreads), kLdsBytes, s, a);
  return hipGetLastError();
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

// Runtime enums to template instantiations; F is the forward or the backward launcher.
struct FwdL {
  template <typename T, int LOSS, int ACT, int DECAY>
  static hipError_t run(const MlpArgs& a, hipStream_t s) { return launch_t<T, LOSS, ACT, DECAY>(a, s); }
};
struct BwdL {
  template <typename T, int LOSS, int ACT, int DECAY>
  static hipError_t run(const MlpBwdArgs& a, hipStream_t s) { return launch_bwd_t<T, LOSS, ACT, DECAY>(a, s); }
};

template <class F, typename T, int LOSS, int ACT, class A>
hipError_t by_decay(const A& a, int decay, hipStream_t s) {
  return decay == TTT_DECAY_SCALAR ? F::template run<T, LOSS, ACT, 1>(a, s) : F::template run<T, LOSS, ACT, 0>(a, s);
}

template <class F, typename T, int LOSS, class A>
hipError_t by_act(const A& a, int act, int decay, hipStream_t s) {
  if (act == TTT_ACT_SILU) return by_decay<F, T, LOSS, 1>(a, decay, s);
  if (act == TTT_ACT_GELU) return by_decay<F, T, LOSS, 2>(a, decay, s);
  return by_decay<F, T, LOSS, 0>(a, decay, s);
}

template <class F, class A>
hipError_t by_enums(const A& a, const ttt_mlp_desc& d, hipStream_t s) {
  auto per_loss = [&](auto tt) -> hipError_t {
    using T = typename decltype(tt)::type;
    if (d.loss == TTT_LOSS_IP) return by_act<F, T, 1>(a, d.act, d.decay, s);
    if (d.loss == TTT_LOSS_L1) return by_act<F, T, 2>(a, d.act, d.decay, s);
    return by_act<F, T, 0>(a, d.act, d.decay, s);
  };
  if (d.dtype == TTT_BF16) return per_loss(std::type_identity<bf16_t>{});
  return per_loss(std::type_identity<float>{});
}

}  // namespace

size_t mlp_fwd_workspace(const ttt_mlp_desc& d) {
  const MlpScratch L(d.C, d.dk, d.dh, d.dv);
  return align256(sizeof(float) * static_cast<size_t>(d.B) * d.H * L.total);
}

hipError_t mlp_fwd_launch(const ttt_mlp_desc& d, const void* q, const void* k, const void* v, const float* beta,
                          const float* gamma, const float* w1_0, const float* w2_0, void* o, float* w1_final,
                          float* w2_final, float* w1_ckpt, float* w2_ckpt, void* saved, void* ws, hipStream_t s) {
  MlpArgs a{};
  a.B = d.B; a.H = d.H; a.T = d.T; a.dk = d.dk; a.dh = d.dh; a.dv = d.dv; a.C = d.C;
  a.NC = (d.T + d.C - 1) / d.C;
  a.b = d.lr_bias;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.gamma = gamma; a.w1_0 = w1_0; a.w2_0 = w2_0;
  a.o = o; a.w1_final = w1_final; a.w2_final = w2_final; a.w1_ckpt = w1_ckpt; a.w2_ckpt = w2_ckpt;
  a.saved = static_cast<float*>(saved);
  a.scratch = static_cast<float*>(ws);
  return by_enums<FwdL>(a, d, s);
}

size_t mlp_saved_bytes(const ttt_mlp_desc& d) {
  const MlpSaved SV(d.C, d.dh, d.dv);
  const int64_t nc = (static_cast<int64_t>(d.T) + d.C - 1) / d.C;
  return align256(sizeof(float) * static_cast<size_t>(d.B) * d.H * nc * SV.per_chunk);
}

size_t mlp_bwd_workspace(const ttt_mlp_desc& d) {
  const MlpBwdScratch L(d.C, d.dk, d.dh, d.dv);
  return align256(sizeof(float) * static_cast<size_t>(d.B) * d.H * L.total);
}

hipError_t mlp_bwd_launch(const ttt_mlp_desc& d, const void* q, const void* k, const void* v, const float* beta,
                          const float* gamma, const float* w1_ckpt, const float* w2_ckpt, const void* saved,
                          const void* d_o, const float* d_w1final, const float* d_w2final, void* dq, void* dk,
                          void* dv, float* dbeta, float* dgamma, float* dw1_0, float* dw2_0, void* ws,
                          hipStream_t s) {
  MlpBwdArgs a{};
  a.B = d.B; a.H = d.H; a.T = d.T; a.dk = d.dk; a.dh = d.dh; a.dv = d.dv; a.C = d.C;
  a.NC = (d.T + d.C - 1) / d.C;
  a.b = d.lr_bias;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.gamma = gamma; a.w1_ckpt = w1_ckpt; a.w2_ckpt = w2_ckpt;
  a.saved = static_cast<const float*>(saved);
  a.d_o = d_o; a.d_w1final = d_w1final; a.d_w2final = d_w2final;
  a.dq = dq; a.dk_out = dk; a.dv_out = dv; a.dbeta = dbeta; a.dgamma = dgamma; a.dw1_0 = dw1_0; a.dw2_0 = dw2_0;
  a.scratch = static_cast<float*>(ws);
  return by_enums<BwdL>(a, d, s);
}

}  // namespace ttt
