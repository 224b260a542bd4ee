// In-Place TTT W_down chunk update on gfx950 matrix cores.
//
// "In-Place Test-Time Training" (summary page, "Core method and technical
// details"): the MLP's down projection W_down is the fast weight; each chunk i
// first applies O_[i] = Z_[i] W_down^(i)T, then updates
// W_down^(i+1) = W_down^(i) + eta V_hat_[i]^T Z_[i].
//
// Both steps are dense GEMMs (1024 x 9728 x 2560 at chunk 1024), so they run
// on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation:
//   apply : O[t][m]  = sum_f Z[t][f] * bf16(W[m][f])     (W read as fp32, rounded)
//   update: W[m][f] += eta * sum_t V_hat[t][m] * Z[t][f]  (fp32 state, RMW)
// One templated tile kernel serves both; operands whose contraction index is
// not contiguous in memory (V_hat^T and Z in the update) are staged k-major and
// read column-wise from LDS.
//
// The guarded variant adds the page's long-context safeguards (section
// "Practical advice", the stability item): the update dW = eta V_hat^T Z of a
// chunk is scaled to Frobenius norm tau when it is larger -- a third GEMM of
// the update's shape reduces sum(dW^2) per tile and a one-workgroup kernel turns
// the tile sums into the scale -- and at a document start the state restarts
// from the pretrained W_down: that chunk's apply reads w_init and its update
// writes w_init + dW, so a reset costs no copy.

#include <cstddef>
#include <type_traits>
#include <vector>

#include "ttt_device.h"
#include "ttt_internal.h"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 128, kBN = 128;  // output tile per workgroup
constexpr int kBK = 64;              // k per LDS stage (four k16 MFMA steps)
constexpr int kPad = 8;              // bf16 elements of row padding in LDS
constexpr int kLdsRow = kBK + kPad;  // 144-byte rows: consecutive rows start 4 banks apart
constexpr int kThreads = 512;        // 8 waves, 4 x 2 over the tile, 32 x 64 each; two
                                     // workgroups per CU (4 waves per SIMD, 128 VGPRs)
                                     // give each SIMD four waves to overlap stage loads

// Epilogues.
constexpr int kEpiStoreBf16 = 0;  // C[m][n] = bf16(acc)
constexpr int kEpiAxpyF32 = 1;    // C[m][n] += alpha * acc (fp32)
constexpr int kEpiPartialF32 = 2; // C[split][m][n] = acc (fp32 split-K partial sums)
constexpr int kEpiSumSqF32 = 3;   // C[workgroup] = sum over the tile of acc^2

struct GemmArgs {
  int M, N, K;
  const void* A;   // A(m, k): A_T ? A[k*lda + m] : A[m*lda + k]
  const void* Bm;  // B(k, n): B_T ? B[k*ldb + n] : B[n*ldb + k]
  void* Cm;        // C[m*ldc + n]
  int64_t lda, ldb, ldc;
  float alpha;
  int k_split;  // contraction length per blockIdx.z (a multiple of kBK, or K)
  const float* Csrc = nullptr;   // kEpiAxpyF32: old values read from here (NULL: from C)
  const float* scale = nullptr;  // kEpiAxpyF32: alpha is multiplied by *scale (NULL: by 1)
  // Two-term products: with A_alt set, blockIdx.z = 1 forms A_alt * B_alt over the
  // whole K (blockIdx.z = 0 forms A * B) and scales its partial sums by alt_scale.
  const void* A_alt = nullptr;
  const void* B_alt = nullptr;
  float alt_scale = 1.0f;
};

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t pack_bf16x8(const f32x4_t& a, const f32x4_t& b) {
  return u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
}

// One operand tile of a stage, ROWS x kBK, contiguous in k (piece = 8 consecutive
// k of a row), held in registers between its global loads and its LDS writes.
// The loaded values are kept raw (fp32 operands are rounded to bf16, and pieces
// past the matrix zeroed, only when written to LDS): an operation on a loaded
// value right after its load would make the load complete there, before the
// current stage's products.
template <int ROWS, typename X>
struct Stage {
  static constexpr int kPieces = ROWS * kBK / 8 / kThreads;
  static constexpr int kVec = sizeof(X) == 4 ? 2 : 1;  // 16-byte loads per piece
  using V = std::conditional_t<sizeof(X) == 4, f32x4_t, u32x4_t>;
  V v[kPieces][kVec];
  uint32_t ok_bits;

  __device__ __forceinline__ void load(const X* g, int64_t ld, int row0, int nrows, int k0, int K) {
    ok_bits = 0;
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const int r = idx / (kBK / 8), kk = (idx % (kBK / 8)) * 8;
      const int gr = row0 + r, gk = k0 + kk;
      // rows are multiples of 8 long in k, so a piece is wholly inside or outside
      const bool ok = gr < nrows && gk < K;
      ok_bits |= ok ? (1u << i) : 0u;
      const int64_t off = ok ? static_cast<int64_t>(gr) * ld + gk : 0;
#pragma unroll
      for (int h = 0; h < kVec; ++h) v[i][h] = *reinterpret_cast<const V*>(g + off + 4 * h);
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds) const {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const int r = idx / (kBK / 8), kk = (idx % (kBK / 8)) * 8;
      u32x4_t x;
      if constexpr (sizeof(X) == 4) x = pack_bf16x8(v[i][0], v[i][1]);
      else x = v[i][0];
      const uint32_t m = (ok_bits >> i) & 1u ? 0xffffffffu : 0u;
      *reinterpret_cast<u32x4_t*>(lds + r * kLdsRow + kk) = x & m;
    }
  }
};

// A bf16 operand that is contiguous in the row index (k-major in memory: the
// update's V_hat^T and Z) is staged as it lies, [kBK][ROWS] with a 16-byte
// granule XOR swizzle: 16-byte pieces of 8 rows at one k, raw until written,
// every thread taking two.  The MFMA reads it column-wise with
// ds_read_b64_tr_b16 (tr_frag).  gfx950's LDS has 64 four-byte banks and serves
// such a read 32 lanes (256 bytes) a cycle: those lanes name four consecutive k
// rows and four adjacent granules in each, and the key 4 (k % 4) + 2 ((k / 2) % 2)
// over 16 granules sends the 16 pieces to 16 different bank groups (measured:
// no bank-conflict cycles; the key 2 (k % 4) + (k / 4) % 2, conflict-free for 32
// banks, left two pieces on each group).  (Transposing into a [row][k] layout on
// the way in, one bf16 per LDS write, hit the same banks from most lanes of a
// wave and cost the update GEMM about three quarters of its time.)
template <int NCOL>
__device__ __forceinline__ int swzk(int k, int col) {
  return k * NCOL + (((col >> 3) ^ (4 * (k & 3) + 2 * ((k >> 1) & 1))) << 3) + (col & 7);
}

template <int ROWS>
struct StageK {
  static constexpr int kPieces = ROWS * kBK / 8 / kThreads;
  u32x4_t v[kPieces];
  uint32_t ok_bits;

  __device__ __forceinline__ void load(const bf16_t* g, int64_t ld, int row0, int nrows, int k0, int K) {
    ok_bits = 0;
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const int kk = idx / (ROWS / 8), r = (idx % (ROWS / 8)) * 8;
      const bool ok = k0 + kk < K && row0 + r < nrows;  // rows come in whole pieces of 8
      ok_bits |= ok ? (1u << i) : 0u;
      v[i] = *reinterpret_cast<const u32x4_t*>(g + (ok ? static_cast<int64_t>(k0 + kk) * ld + row0 + r : 0));
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds) const {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const int kk = idx / (ROWS / 8), r = (idx % (ROWS / 8)) * 8;
      *reinterpret_cast<u32x4_t*>(lds + swzk<ROWS>(kk, r)) = v[i] & ((ok_bits >> i) & 1u ? 0xffffffffu : 0u);
    }
  }
};

// A k-major fp32 operand (the backward's W_down and its gradient), rounded to
// bf16 when written to LDS and otherwise staged like StageK: 8 rows at one k
// per piece, two 16-byte loads each, raw until written.
template <int ROWS>
struct StageKF {
  static constexpr int kPieces = ROWS * kBK / 8 / kThreads;
  f32x4_t v[kPieces][2];
  uint32_t ok_bits;

  __device__ __forceinline__ void load(const float* g, int64_t ld, int row0, int nrows, int k0, int K) {
    ok_bits = 0;
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const int kk = idx / (ROWS / 8), r = (idx % (ROWS / 8)) * 8;
      const bool ok = k0 + kk < K && row0 + r < nrows;
      ok_bits |= ok ? (1u << i) : 0u;
      const float* p = g + (ok ? static_cast<int64_t>(k0 + kk) * ld + row0 + r : 0);
      v[i][0] = *reinterpret_cast<const f32x4_t*>(p);
      v[i][1] = *reinterpret_cast<const f32x4_t*>(p + 4);
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds) const {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const int kk = idx / (ROWS / 8), r = (idx % (ROWS / 8)) * 8;
      *reinterpret_cast<u32x4_t*>(lds + swzk<ROWS>(kk, r)) =
          pack_bf16x8(v[i][0], v[i][1]) & ((ok_bits >> i) & 1u ? 0xffffffffu : 0u);
    }
  }
};

// MFMA operand (A or B of v_mfma_f32_32x32x16_bf16) from a k-major [kBK][NCOL]
// tile: lane (l32, hi) gets k = 16 kb + 8 hi .. +7 of column col_block + l32.  In
// each 16-lane group of ds_read_b64_tr_b16, lane 4a + b receives element b of the
// 8-byte pieces named by lanes a, a + 4, a + 8, a + 12; so lane l32 names k row
// 8 hi + 4 h + (l32 % 16) / 4 (h = 0, 1) and columns 16 (l32 / 16) + 4 (l32 % 4)
// .. +3 of the block, and gets back four consecutive k of column l32.
template <int NCOL>
__device__ __forceinline__ bf16x8_t tr_frag(const bf16_t* lds, int kb, int col_block, int l32, int hi) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const int col = col_block + 16 * (l32 >> 4) + 4 * (l32 & 3);
  const int r0 = 16 * kb + 8 * hi + ((l32 & 15) >> 2);
  const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lds + swzk<NCOL>(r0, col)));
  const v4s y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lds + swzk<NCOL>(r0 + 4, col)));
  bf16x8_t f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(x[j]));
    f[4 + j] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(y[j]));
  }
  return f;
}

// C(m, n) = sum_k A(m, k) B(k, n) on v_mfma_f32_32x32x16_bf16, fp32 accumulate.
// Double-buffered LDS: the global loads of stage s + 1 are in flight while stage
// s is multiplied, and one barrier per stage separates the buffers' uses.
template <bool A_T, bool B_T, typename AX, typename BX, int EPI>
__global__ __launch_bounds__(kThreads, 4) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][kBN * kLdsRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave rows wm * 32 .. +31, columns wn * 64 .. +63
  // Tile order: the hardware deals workgroup L to XCD L % 8.  Tiles are numbered
  // n-major (all M tiles of an N tile consecutive) and tile j goes to workgroup
  // L with j = (L % 8) * (count / 8) + L / 8, so the M tiles that read the same B
  // columns (the fp32 W_down rows of the apply step) run on one XCD and share
  // its L2 instead of each fetching them from HBM.
  const int mt = gridDim.y, tiles = gridDim.x * gridDim.y, nblk = tiles * gridDim.z;
  const int L = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
  const int j = (nblk % 8 == 0) ? (L % 8) * (nblk / 8) + L / 8 : L;
  const int split = j / tiles, jt = j % tiles;
  const int m0 = (jt % mt) * kBM, n0 = (jt / mt) * kBN;
  // split-K: this workgroup's share [k_lo, k_hi) of the contraction
  const bool alt = g.A_alt != nullptr && split == 1;  // the second term of a two-term product
  const int k_lo = g.A_alt ? 0 : split * g.k_split, k_hi = g.A_alt ? g.K : min(g.K, k_lo + g.k_split);
  const int l32 = lane & 31, hi = lane >> 5;

  f32x16_t acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

  const AX* Ag = static_cast<const AX*>(alt ? g.A_alt : g.A);
  const BX* Bg = static_cast<const BX*>(alt ? g.B_alt : g.Bm);
  static_assert(!A_T || sizeof(AX) == 2, "a k-major A operand is bf16");
  static_assert(kBK * kBM <= kBM * kLdsRow && kBK * kBN <= kBN * kLdsRow, "k-major tiles fit the buffers");
  using SA = std::conditional_t<A_T, StageK<kBM>, Stage<kBM, AX>>;
  using SB = std::conditional_t<B_T, std::conditional_t<sizeof(BX) == 4, StageKF<kBN>, StageK<kBN>>, Stage<kBN, BX>>;
  SA sa;
  SB sb;
  auto load_stage = [&](int k0) {
    sa.load(Ag, g.lda, m0, g.M, k0, k_hi);
    sb.load(Bg, g.ldb, n0, g.N, k0, k_hi);
  };
  auto store_stage = [&](int buf) {
    sa.store(As[buf]);
    sb.store(Bs[buf]);
  };
  const int nst = (k_hi - k_lo + kBK - 1) / kBK;
  auto compute = [&](int buf) {
    const bf16_t* Ac = As[buf];
    const bf16_t* Bc = Bs[buf];
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
      bf16x8_t af, bfr[2];
      if constexpr (A_T) af = tr_frag<kBM>(Ac, ks / 16, wm * 32, l32, hi);
      else af = *reinterpret_cast<const bf16x8_t*>(Ac + (wm * 32 + l32) * kLdsRow + ks + hi * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (B_T) bfr[j] = tr_frag<kBN>(Bc, ks / 16, wn * 64 + j * 32, l32, hi);
        else bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bc + (wn * 64 + j * 32 + l32) * kLdsRow + ks + hi * 8);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[j], acc[j], 0, 0, 0);
    }
  };
  load_stage(k_lo);
  store_stage(0);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int cur = s & 1;
    if (s + 1 < nst) load_stage(k_lo + (s + 1) * kBK);
    compute(cur);
    if (s + 1 < nst) store_stage(cur ^ 1);
    __syncthreads();
  }
  // 32x32 MFMA output layout: lane (n = l32, hi) holds rows 8*(r/4) + 4*hi + (r%4).
  // The fp32 read-modify-write first loads every element this lane updates, then
  // stores them all: element by element, each store would have to wait for its
  // load, and each load for the stores before it that might alias it.
  const int mb = m0 + wm * 32 + 4 * hi;
  if constexpr (EPI == kEpiStoreBf16 || EPI == kEpiPartialF32) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r / 4) + (r % 4);
        if (n < g.N && m < g.M) {
          if constexpr (EPI == kEpiStoreBf16)
            static_cast<bf16_t*>(g.Cm)[static_cast<int64_t>(m) * g.ldc + n] = f32_to_bf16(g.alpha * acc[j][r]);
          else
            static_cast<float*>(g.Cm)[(static_cast<int64_t>(split) * g.M + m) * g.ldc + n] =
                (alt ? g.alt_scale : 1.0f) * acc[j][r];
        }
      }
    }
  } else if constexpr (EPI == kEpiSumSqF32) {
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r / 4) + (r % 4);
        ss += (n < g.N && m < g.M) ? acc[j][r] * acc[j][r] : 0.0f;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    float* red = reinterpret_cast<float*>(&As[0][0]);  // free: the k loop ended with a barrier
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = 0.0f;
      for (int i = 0; i < kThreads / 64; ++i) t += red[i];
      static_cast<float*>(g.Cm)[j] = t;  // j: this workgroup's tile, unique in the launch
    }
  } else {
    float* c = static_cast<float*>(g.Cm);
    const float* src = g.Csrc ? g.Csrc : c;
    const float alpha = g.scale ? g.alpha * *g.scale : g.alpha;
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // one accumulator at a time keeps 16 loaded values live, not 32
      const int n = n0 + wn * 64 + j * 32 + l32;
      float old[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r / 4) + (r % 4);
        const bool ok = n < g.N && m < g.M;
        old[r] = src[ok ? static_cast<int64_t>(m) * g.ldc + n : 0];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r / 4) + (r % 4);
        if (n < g.N && m < g.M) c[static_cast<int64_t>(m) * g.ldc + n] = old[r] + alpha * acc[j][r];
      }
    }
  }
}

// Clip scale of one chunk's update from the per-tile sums of squares of
// V_hat^T Z: ||dW||_F = |eta| sqrt(sum); scale = tau / ||dW||_F when that is
// below 1, else 1.  The sums are added in a fixed order (fp64).
__global__ __launch_bounds__(256) void clip_scale_kernel(const float* __restrict__ part, int n, float eta, float tau,
                                                         float* __restrict__ scale) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) s += static_cast<double>(part[i]);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double norm = fabs(static_cast<double>(eta)) * sqrt(red[0]);
    scale[0] = norm > static_cast<double>(tau) ? static_cast<float>(static_cast<double>(tau) / norm) : 1.0f;
  }
}

// O = bf16(scale * sum of the split-K partials); 4 elements per thread (M N % 8 == 0).
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int ks, int64_t mn,
                                                           bf16_t* __restrict__ out, float scale) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= mn) return;
  float4 acc = *reinterpret_cast<const float4*>(part + i);
  for (int s = 1; s < ks; ++s) {
    const float4 x = *reinterpret_cast<const float4*>(part + s * mn + i);
    acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
  }
  acc.x *= scale; acc.y *= scale; acc.z *= scale; acc.w *= scale;
  const uint32_t lo = pack_bf16x2(acc.x, acc.y);
  const uint32_t hi = pack_bf16x2(acc.z, acc.w);
  *reinterpret_cast<uint2*>(out + i) = make_uint2(lo, hi);
}

// Split of the apply GEMM's contraction (d_ff) for a c x d_model output: enough
// workgroups for two per CU, at most 8 splits and at least 8 stages each.
int apply_splits(int c, int d_model, int d_ff) {
  const int tiles = ((c + kBM - 1) / kBM) * ((d_model + kBN - 1) / kBN);
  const int stages = (d_ff + kBK - 1) / kBK;
  int ks = 2 * device_cu_count() / tiles;
  ks = ks < 8 ? ks : 8;
  ks = ks < stages / 8 ? ks : stages / 8;
  return ks > 1 ? ks : 1;
}

// ---------------------------------------------------------------------------
// The forward's tile GEMMs when a workspace is given.
//
// Output tiles of 256 x 128 (one workgroup per CU, 8 waves of 64 x 64), a ring
// of three 64-deep LDS stages filled by direct buffer -> LDS loads (each lane's
// 16 bytes land at LDS base + 16 lane of its wave's 1 KB window, so the lane
// chooses which global piece to fetch to build the swizzled layout), no
// registers or VALU spent on staging.  Two products:
//   apply  : O[t][m] (+)= sum_f Z[t][f] Wb[m][f]           (both operands k-contiguous)
//   update : W[m][f] = W_src[m][f] + alpha sum_t Z[t][f] V_hat[t][m]
// The update's tile rows are f and its columns m, so each lane's four
// consecutive accumulator rows are four consecutive floats of W[m][.]: the fp32
// read-modify-write moves 16 bytes per lane per access.  It also writes Wb =
// bf16(W), the next chunk's apply operand: the apply rounds W_down to bf16
// anyway, so the copy is exact and the apply streams 2 bytes per weight.
// ---------------------------------------------------------------------------
constexpr int kTM = 256, kTN = 128, kTK = 64, kTStages = 3, kTThreads = 512;
constexpr int kTDma = (kTM + kTN) / 64;  // direct loads per wave per stage
constexpr uint32_t kOob = 0x7ffffff0u;   // every resource's size: a load at this offset returns zeros
constexpr int kGuardedBwdMaxC = 8192;    // the guarded backward's chunk bound (its Gram matrices are C x C)

typedef __attribute__((address_space(3))) void lds_void_t;

typedef int rsrc_t __attribute__((ext_vector_type(4)));  // buffer resource (4 SGPRs)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return rsrc_t{static_cast<int>(a & 0xffffffffu), static_cast<int>(a >> 32), static_cast<int>(kOob), 0x00020000};
}
// One wave-wide direct load: lane i's 16 bytes at byte voff of the resource go
// to LDS address lds + 16 i (lds uniform over the wave; M0 holds it).  Written
// as asm so that the compiler's wait insertion, which cannot tell the ring's
// slots apart, does not hold every later LDS read until the newest such load
// has landed; the ring waits for its loads explicitly instead.  m0 is used by
// nothing else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // the m0 clobber (a reserved register)
__device__ __forceinline__ void dma16(rsrc_t rs, const bf16_t* lds, uint32_t voff) {
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)(lds)));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(a), "v"(voff), "s"(rs)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// Wait until at most N of this wave's vector memory operations are in flight
// and its LDS reads are done.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// Workgroup barrier that leaves vector memory in flight (the ring's direct
// loads are waited for explicitly, stage by stage); the empty asm statements
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup L runs on XCD L % 8; tiles j are dealt so that each XCD receives a
// contiguous range of j (neighbouring tiles share operands in its L2).
__device__ __forceinline__ int xcd_tile(int L, int n) {
  const int q = n / 8, r = n % 8, x = L % 8, i = L / 8;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// A k-contiguous operand, ROWS x kTK per stage at [row][k] (128-byte rows) with
// the 16-byte granule g of row r stored at slot g ^ (r % 8) ^ ((r / 8) % 2).  A
// ds_read_b128 of an MFMA operand names one granule in each of 32 consecutive
// rows and is served 16 lanes (256 bytes, all 64 banks) a cycle: rows r and
// r + 8 sit in the same half of the banks, and the second term keeps their
// pieces apart (with g ^ (r % 8) alone they collided, measured).  Window w
// (8 rows) is filled by one wave-wide load: lane i takes row 8 w + i / 8, granule
// (i % 8) ^ (i / 8) ^ (w % 2).
template <int ROWS>
struct KRing {
  static constexpr int kPer = ROWS / 64;  // windows per wave
  uint32_t off[kPer];  // byte offset of the lane's piece at k = 0 (kOob: row outside)
  int g8;              // 8 * granule: the piece's first k
  __device__ __forceinline__ void init(int wave, int lane, int nrows, int64_t ld) {
    const int g = (lane & 7) ^ (lane >> 3) ^ (wave & 1);  // windows wave + 8 i: w % 2 == wave % 2
    g8 = 8 * g;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = 8 * (wave + 8 * i) + (lane >> 3);
      off[i] = r < nrows ? static_cast<uint32_t>((static_cast<int64_t>(r) * ld + g8) * 2) : kOob;
    }
  }
  // windows I0 .. I1 - 1 of this wave
  template <int I0, int I1>
  __device__ __forceinline__ void issue(rsrc_t rs, bf16_t* tile, int wave, int k0, int k_hi) const {
    const bool kok = k0 + g8 < k_hi;
#pragma unroll
    for (int i = I0; i < I1; ++i)
      dma16(rs, tile + (wave + 8 * i) * 512, kok && off[i] != kOob ? off[i] + 2u * k0 : kOob);
  }
  // MFMA operand: row R, k = 16 kb + 8 hi .. +7
  static __device__ __forceinline__ bf16x8_t frag(const bf16_t* tile, int R, int kb, int hi) {
    return *reinterpret_cast<const bf16x8_t*>(tile + R * kTK + (((2 * kb + hi) ^ (R & 7) ^ ((R >> 3) & 1)) << 3));
  }
};

// A row-contiguous operand (the contraction index t strides by ld), kTK x NCOL
// per stage at [t][col] in the swzk layout read by tr_frag.  Window w holds
// 512 / NCOL consecutive t: lane i takes t = (512 w + 8 i) / NCOL and the logical
// granule stored at slot ((512 w + 8 i) % NCOL) / 8.  The offsets are those of
// the tile at column 0 and t = 0; a load adds the tile's own.
template <int NCOL>
struct TRing {
  static constexpr int kPer = NCOL / 64;
  uint32_t off[kPer];  // byte offset of the lane's piece relative to the tile's origin
  int kk[kPer];        // the piece's t within the stage
  int col[kPer];       // the piece's first column within the tile
  __device__ __forceinline__ void init(int wave, int lane, int64_t ld) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = (wave + 8 * i) * 512 + 8 * lane;
      const int t = e / NCOL, slot = (e % NCOL) >> 3;
      kk[i] = t;
      col[i] = (slot ^ (4 * (t & 3) + 2 * ((t >> 1) & 1))) << 3;
      off[i] = static_cast<uint32_t>((static_cast<int64_t>(t) * ld + col[i]) * 2);
    }
  }
  // windows I0 .. I1 - 1 of this wave for the tile at (t0, col0) of a matrix
  // with t_hi rows and ncols columns; origin: its byte offset in the resource
  template <int I0, int I1>
  __device__ __forceinline__ void issue(rsrc_t rs, bf16_t* tile, int wave, int t0, int t_hi, int col0, int ncols,
                                        uint32_t origin) const {
#pragma unroll
    for (int i = I0; i < I1; ++i)
      dma16(rs, tile + (wave + 8 * i) * 512, t0 + kk[i] < t_hi && col0 + col[i] < ncols ? off[i] + origin : kOob);
  }
};

struct TileArgs {
  int M, N, K;       // output rows, columns, contraction length
  const bf16_t* A;   // apply: Z [M][lda] (k-contiguous); update: Z [K][lda] (rows f)
  const bf16_t* B;   // apply: Wb [N][ldb];                update: V_hat [K][ldb] (columns m)
  int64_t lda, ldb;
  int k_split;       // apply: contraction per split (a multiple of kTK)
  const bf16_t* A2;  // apply, two-term form: split 1 multiplies A2 by B2 over the whole K
  const bf16_t* B2;
  // apply outputs
  bf16_t* o;         // ks == 1: O[t][m] (ldo)
  float* part;       // ks > 1: part[split][t][m] (ldo)
  int64_t ldo;
  // update: W[m][f] = W_src[m][f] + alpha * (*scale) * acc, Wb = bf16(W)  (ldw)
  const float* w_src;
  float* w;
  bf16_t* wb;
  int64_t ldw;
  float alpha;
  const float* scale;
  float wb_scale;    // update: Wb = bf16(wb_scale * W)
};

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;
}

// The apply, O = Z Wb^T, split over d_ff: one 256 x 128 output tile and one
// contraction range per workgroup.  With B_TR, B is stored [k][n] (n
// contiguous: the backward's dZ = dO W_i + V_hat (eta dW)) and read with the
// transpose read; with A2 set, split 1 is the second term A2 B2 over the whole K.
template <bool B_TR>
__global__ __launch_bounds__(kTThreads, 1) void apply_kernel(TileArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t As[kTStages][kTM * kTK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[kTStages][kTN * kTK];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // wave rows wm * 64 .. +63, columns wn * 64 .. +63
  const int l32 = lane & 31, hi = lane >> 5;
  const int mt = (g.M + kTM - 1) / kTM, nt = (g.N + kTN - 1) / kTN;
  // row tiles fastest, then column tiles, then splits
  const int j = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (j % mt) * kTM, n0 = ((j / mt) % nt) * kTN, split = j / (mt * nt);
  const bool two = g.A2 != nullptr;
  const int k_lo = two ? 0 : split * g.k_split;
  const int k_hi = two ? g.K : min(g.K, k_lo + g.k_split);
  const int nst = (k_hi - k_lo + kTK - 1) / kTK;
  const bf16_t* Ag = two && split == 1 ? g.A2 : g.A;
  const bf16_t* Bg = two && split == 1 ? g.B2 : g.B;

  f32x16_t acc[2][2];
  zero_acc(acc);
  KRing<kTM> ra;
  std::conditional_t<B_TR, TRing<kTN>, KRing<kTN>> rb;
  ra.init(wave, lane, g.M - m0, g.lda);
  if constexpr (B_TR) rb.init(wave, lane, g.ldb);
  else rb.init(wave, lane, g.N - n0, g.ldb);
  const rsrc_t rsa = make_rsrc(Ag + static_cast<int64_t>(m0) * g.lda);
  const rsrc_t rsb = B_TR ? make_rsrc(Bg) : make_rsrc(Bg + static_cast<int64_t>(n0) * g.ldb);
  // Stage s's direct loads in three parts of two per wave (A windows 0-1, A
  // windows 2-3, B windows 0-1), issued between the k-steps of the products
  // rather than in one burst.
  auto issue_part = [&](int s, int part) {
    if (s < nst) {
      const int k0 = k_lo + s * kTK;
      bf16_t* at = As[s % kTStages];
      bf16_t* bt = Bs[s % kTStages];
      if (part == 0) ra.issue<0, 2>(rsa, at, wave, k0, k_hi);
      else if (part == 1) ra.issue<2, 4>(rsa, at, wave, k0, k_hi);
      else if constexpr (B_TR)
        rb.template issue<0, 2>(rsb, bt, wave, k0, k_hi, n0, g.N,
                                static_cast<uint32_t>((static_cast<int64_t>(k0) * g.ldb + n0) * 2));
      else rb.template issue<0, 2>(rsb, bt, wave, k0, k_hi);
    }
  };
  auto issue = [&](int s) {
    issue_part(s, 0);
    issue_part(s, 1);
    issue_part(s, 2);
  };

  // A whole stage's MFMA operands are read into registers one stage ahead:
  // stage s is multiplied from registers while stage s + 1's reads are in
  // flight, and the barrier that releases stage s + 1 comes before stage s's
  // products, so no wave waits on LDS with the matrix unit idle.  A slot is
  // free once its fragments are in registers: stage s + 3 is loaded into
  // stage s's slot, three stages ahead.
  struct Frags {
    bf16x8_t a[kTK / 16][2], b[kTK / 16][2];
  };
  auto read = [&](Frags& F, int s) {
    const bf16_t* Ac = As[s % kTStages];
    const bf16_t* Bc = Bs[s % kTStages];
#pragma unroll
    for (int kb = 0; kb < kTK / 16; ++kb)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        F.a[kb][i] = KRing<kTM>::frag(Ac, wm * 64 + 32 * i + l32, kb, hi);
        if constexpr (B_TR) F.b[kb][i] = tr_frag<kTN>(Bc, kb, wn * 64 + 32 * i, l32, hi);
        else F.b[kb][i] = KRing<kTN>::frag(Bc, wn * 64 + 32 * i + l32, kb, hi);
      }
  };
  auto mma = [&](const Frags& F, int kb) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.a[kb][i], F.b[kb][jj], acc[i][jj], 0, 0, 0);
  };
  // An empty asm statement reading every fragment of a stage: the compiler
  // must have their LDS reads complete here, before the next stage's reads
  // are issued (left to itself it waits at the first product, by which time
  // it can only wait for all reads in flight, the next stage's included).
  auto touch = [&](Frags& F) {
#pragma unroll
    for (int kb = 0; kb < kTK / 16; ++kb)
#pragma unroll
      for (int i = 0; i < 2; ++i) asm volatile("" ::"v"(F.a[kb][i]), "v"(F.b[kb][i]));
  };
  auto step = [&](int s, Frags& cur, Frags& nxt) {
    if (s >= nst) return;
    // stage s's fragments are in registers and stage s + 1 has landed (stage
    // s + 2's loads may be in flight); one wait on every path, so that the
    // products below need none
    if (s + 2 < nst) wait_vm<kTDma>();
    else wait_vm<0>();
    touch(cur);
    const bool more = s + 1 < nst;
    if (more) {
      ring_barrier();  // every wave holds stage s: its slot takes stage s + 3
      read(nxt, s + 1);
    }
#pragma unroll
    for (int kb = 0; kb < kTK / 16; ++kb) {
      mma(cur, kb);
      __builtin_amdgcn_sched_barrier(0);
      if (kb < 3 && more) issue_part(s + 3, kb);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  Frags f0, f1;
  issue(0);
  issue(1);
  issue(2);
  if (nst >= 3) wait_vm<2 * kTDma>();
  else if (nst == 2) wait_vm<kTDma>();
  else wait_vm<0>();
  ring_barrier();
  if (nst > 0) read(f0, 0);
  for (int s = 0; s < nst; s += 2) {
    step(s, f0, f1);
    step(s + 1, f1, f0);
  }

  // 32x32 MFMA output: lane (l32, hi) holds column l32 and rows 8 (r / 4) + 4 hi + r % 4
  const int tb = m0 + wm * 64 + 4 * hi;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int n = n0 + wn * 64 + 32 * jj + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = tb + 32 * i + 8 * (r / 4) + (r % 4);
        if (t < g.M && n < g.N) {
          if (g.part)
            g.part[(static_cast<int64_t>(split) * g.M + t) * g.ldo + n] = acc[i][jj][r];
          else
            g.o[static_cast<int64_t>(t) * g.ldo + n] = f32_to_bf16(acc[i][jj][r]);
        }
      }
    }
}

// wait_vm<n'> for the largest listed n' <= n (waiting for more than needed is safe)
__device__ __forceinline__ void wait_vm_at_most(int n) {
  if (n >= 48) wait_vm<48>();
  else if (n >= 38) wait_vm<38>();
  else if (n >= 32) wait_vm<32>();
  else if (n >= 26) wait_vm<26>();
  else if (n >= 22) wait_vm<22>();
  else if (n >= 20) wait_vm<20>();
  else if (n >= 16) wait_vm<16>();
  else if (n >= 14) wait_vm<14>();
  else if (n >= 10) wait_vm<10>();
  else if (n >= 8) wait_vm<8>();
  else if (n >= 6) wait_vm<6>();
  else if (n >= 4) wait_vm<4>();
  else wait_vm<0>();
}

// The update, W[m][f] = W_src[m][f] + alpha sum_t Z[t][f] V_hat[t][m] with
// Wb = bf16(W): tile rows f (Z read column-wise with tr_frag), columns m.
//
// Persistent: one workgroup per CU walks its tiles (every gridDim.x-th tile of
// its XCD's range) and the ring of stages runs on across tile boundaries, so a
// tile starts with its first stages already in LDS.  A tile's results are
// written during the next tile's first four stages, one slice (i, jj) after
// each stage's products: for every row m of a wave's block a slice is 32
// consecutive floats of W (128 bytes, two lanes) and their 64 bytes of Wb, so
// no cache line leaves L2 half written.  (Written at the end of a one-tile
// workgroup, the 150 MB of writes per 1024-token chunk held each CU until they
// drained: 104 us a launch against 69 us without them, measured at d_model
// 2560, d_ff 9728; this schedule takes 99 us.)  The old W of a tile is loaded
// two stages before its end, into the registers the previous tile's results
// have left.
//
// NORM: the same products for the clip norm of the guarded update: no W is
// read or written; each tile's sum of acc^2 goes to g.w[j] (j the tile's index).
template <bool NORM>
__global__ __launch_bounds__(kTThreads, 1) void update_kernel(TileArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t As[kTStages][kTM * kTK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[kTStages][kTN * kTK];
  __shared__ float red[kTThreads / 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const int mt = (g.M + kTM - 1) / kTM, nt = (g.N + kTN - 1) / kTN, ntile = mt * nt;
  const int G = gridDim.x, L = blockIdx.x;
  const int mine = L < ntile ? (ntile - L + G - 1) / G : 0;  // tiles of this workgroup
  const int nst = (g.K + kTK - 1) / kTK;                      // stages per tile
  const int total = mine * nst;                               // steps of this workgroup
  const int s_old = nst >= 2 ? nst - 2 : 0;                   // the step that loads a tile's old W
  // tile r of this workgroup: rows f0.., columns m0.. (columns fastest within an XCD's range)
  auto origin = [&](int r, int& f0, int& m0) {
    const int j = xcd_tile(L + r * G, ntile);
    f0 = (j / nt) * kTM;
    m0 = (j % nt) * kTN;
  };

  TRing<kTM> ra;
  TRing<kTN> rb;
  ra.init(wave, lane, g.lda);
  rb.init(wave, lane, g.ldb);
  const rsrc_t rsa = make_rsrc(g.A), rsb = make_rsrc(g.B);
  // The stream of direct loads runs two stages ahead of the products and on
  // across tile boundaries.  Its position is kept incrementally: positions
  // recomputed from the step index (integer divisions) cost every wave more
  // scalar work per stage than the stage's products take.
  int dg = 0, dp = 0, dr = 0, dslot = 0, df0 = 0, dm0 = 0;
  if (total > 0) origin(0, df0, dm0);
  auto stream_part = [&](int part) {
    if (dg < total) {
      const int t0 = dp * kTK;
      bf16_t* at = As[dslot];
      bf16_t* bt = Bs[dslot];
      if (part == 0 || part == 1) {
        const uint32_t o = static_cast<uint32_t>((static_cast<int64_t>(t0) * g.lda + df0) * 2);
        if (part == 0) ra.issue<0, 2>(rsa, at, wave, t0, g.K, df0, g.M, o);
        else ra.issue<2, 4>(rsa, at, wave, t0, g.K, df0, g.M, o);
      } else {
        const uint32_t o = static_cast<uint32_t>((static_cast<int64_t>(t0) * g.ldb + dm0) * 2);
        rb.issue<0, 2>(rsb, bt, wave, t0, g.K, dm0, g.N, o);
      }
    }
  };
  auto stream_advance = [&]() {
    ++dg;
    dslot = dslot == kTStages - 1 ? 0 : dslot + 1;
    if (++dp == nst) {
      dp = 0;
      ++dr;
      if (dg < total) origin(dr, df0, dm0);
    }
  };

  const float alpha = g.scale ? g.alpha * *g.scale : g.alpha;
  f32x16_t acc[2][2];
  zero_acc(acc);
  // w: the old W of the current tile (from its step s_old), then its results
  // until they are written, four slices w[i][jj] of 16 floats
  f32x4_t w[2][2][4];
  int pf0 = 0, pm0 = 0;  // origin of the tile whose results w holds
  auto elem = [&](int f0, int m0, int i, int jj, int q4, int& f, int& m) {
    f = f0 + wm * 64 + 32 * i + 8 * q4 + 4 * hi;
    m = m0 + wn * 64 + 32 * jj + l32;
  };
  auto load_old = [&](int f0, int m0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          int f, m;
          elem(f0, m0, i, jj, q4, f, m);
          const bool ok = f < g.M && m < g.N;
          w[i][jj][q4] = *reinterpret_cast<const f32x4_t*>(g.w_src + (ok ? static_cast<int64_t>(m) * g.ldw + f : 0));
        }
  };
  auto finish = [&]() {  // w = old W + alpha acc; acc = 0
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
          for (int e = 0; e < 4; ++e) w[i][jj][q4][e] += alpha * acc[i][jj][4 * q4 + e];
    zero_acc(acc);
  };
  // The writes are buffer stores whose out-of-range lanes the hardware drops:
  // with no branch around them every slice issues exactly four memory
  // operations, which the explicit waits count (a skipped store would make a
  // wait too weak).
  const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(g.w, 0, static_cast<int>(kOob), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_wb = __builtin_amdgcn_make_buffer_rsrc(g.wb, 0, static_cast<int>(kOob), 0x00020000);
  // slice q = (i, jj): the lane's four float4 of one row of W, 128 whole bytes
  // (and 64 of Wb), written together so that no cache line leaves L2 half
  // written: 8 memory operations
  auto store_slice = [&](auto Q) {
    constexpr int q = decltype(Q)::value;
    constexpr int i = q / 2, jj = q % 2;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      int f, m;
      elem(pf0, pm0, i, jj, q4, f, m);
      const bool ok = f < g.M && m < g.N;
      const uint32_t o = static_cast<uint32_t>(static_cast<int64_t>(m) * g.ldw + f);
      const f32x4_t x = w[i][jj][q4];
      const float cs = g.wb_scale;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), rs_w, ok ? 4 * o : kOob, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(cs * x[0], cs * x[1]), pack_bf16x2(cs * x[2], cs * x[3])},
                                            rs_wb, ok ? 2 * o : kOob, 0, 0);
    }
  };
  // slices of the previous tile written at step position p, and the vector
  // memory operations a step of tile r at position p adds after its loads
  // (the waits count them)
  auto slices_at = [&](int p) { return p < s_old ? (p < 4 ? 1 : 0) : (p == s_old ? (p < 4 ? 4 - p : 0) : 0); };
  auto extra_ops = [&](int r, int p) {
    return NORM ? 0 : (r >= 1 ? 8 * slices_at(p) : 0) + (p == s_old ? 16 : 0);
  };
  int gcur = 0, cslot = 0;  // the step about to run and its ring slot
  int e1 = 0, e2 = 0;       // extra operations of the previous step and of the one before it
  // one stage of the ring: wait for its loads, release it, multiply, and issue
  // stage gcur + 2's loads between the k-steps; e: the operations the caller
  // issues after it
  auto step = [&](int e) {
    // this wave's loads of stage gcur have landed; in flight after them may be
    // step gcur - 2's extra operations, stage gcur + 1's loads and step gcur - 1's
    wait_vm_at_most(e2 + (gcur + 1 < total ? kTDma : 0) + e1);
    ring_barrier();  // every wave's stage gcur is in LDS; stage gcur - 1's slot is free
    const bf16_t* Ac = As[cslot];
    const bf16_t* Bc = Bs[cslot];
    // k-step kb + 1's operands are read before k-step kb's products, so that
    // the products do not wait on their own reads
    bf16x8_t af[2][2], bfr[2][2];
    auto read = [&](int kb, bf16x8_t(&a)[2], bf16x8_t(&b)[2]) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = tr_frag<kTM>(Ac, kb, wm * 64 + 32 * i, l32, hi);
        b[i] = tr_frag<kTN>(Bc, kb, wn * 64 + 32 * i, l32, hi);
      }
    };
    read(0, af[0], bfr[0]);
#pragma unroll
    for (int kb = 0; kb < kTK / 16; ++kb) {
      if (kb + 1 < kTK / 16) read(kb + 1, af[(kb + 1) & 1], bfr[(kb + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kb & 1][i], bfr[kb & 1][jj], acc[i][jj], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (kb < 3) stream_part(kb);
      if (kb == 2) stream_advance();
      __builtin_amdgcn_sched_barrier(0);
    }
    ++gcur;
    cslot = cslot == kTStages - 1 ? 0 : cslot + 1;
    e2 = e1;
    e1 = e;
  };

  for (int i = 0; i < 2; ++i) {  // the loads of stages 0 and 1
    stream_part(0), stream_part(1), stream_part(2);
    stream_advance();
  }
  if constexpr (NORM) {
    // a tile's sum of squares: lanes, then waves (fixed order); the products of
    // rows and columns outside the matrix are zero (their operands load as zeros)
    for (int r = 0; r < mine; ++r) {
      for (int p = 0; p < nst; ++p) step(0);
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) ss += acc[i][jj][e] * acc[i][jj][e];
      zero_acc(acc);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
      if (lane == 0) red[wave] = ss;
      // lgkmcnt(0) and a barrier that leaves the ring's loads in flight (a
      // fenced __syncthreads would wait for the next tile's first stages);
      // thread 0's store counts as one more operation after those loads,
      // which only makes the next waits stricter
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
      ring_barrier();
      if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int i = 0; i < kTThreads / 64; ++i) t += red[i];
        g.w[xcd_tile(L + r * G, ntile)] = t;
      }
      // red is written again only after the next tile's first step's barrier
    }
    return;
  }
  // A tile's steps in fixed phases (slice writes, plain steps, the old W, the
  // rest, the results), so that every path from the old W's loads to the
  // slice writes visibly passes through the results: the compiler then holds
  // no write for a load.
  const int nA = s_old < 4 ? s_old : 4;  // steps that write one slice each
  for (int r = 0; r < mine; ++r) {
    [&]<int... Q>(std::integer_sequence<int, Q...>) {
      (
          [&] {
            if (Q < nA) {
              step(extra_ops(r, Q));
              if (r >= 1) store_slice(std::integral_constant<int, Q>{});
            }
          }(),
          ...);
    }(std::make_integer_sequence<int, 4>{});
    for (int p = nA; p < s_old; ++p) step(extra_ops(r, p));
    step(extra_ops(r, s_old));
    if (r >= 1) {  // the slices still unwritten (s_old < 4)
      [&]<int... Q>(std::integer_sequence<int, Q...>) {
        ((Q >= nA ? store_slice(std::integral_constant<int, Q>{}) : void()), ...);
      }(std::make_integer_sequence<int, 4>{});
    }
    {
      int f0, m0;
      origin(r, f0, m0);
      load_old(f0, m0);
    }
    for (int p = s_old + 1; p < nst; ++p) step(extra_ops(r, p));
    finish();
    origin(r, pf0, pm0);
  }
  // the last tile's results
  if (total > 0) {
    [&]<int... Q>(std::integer_sequence<int, Q...>) {
      (store_slice(std::integral_constant<int, Q>{}), ...);
    }(std::make_integer_sequence<int, 4>{});
  }
}

// Wb = bf16(scale W), 8 weights per thread (count % 8 == 0).
__global__ __launch_bounds__(256) void round_bf16_kernel(const float* __restrict__ w, bf16_t* __restrict__ wb,
                                                         int64_t n8, float scale) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4_t a = reinterpret_cast<const f32x4_t*>(w)[2 * i];
  const f32x4_t b = reinterpret_cast<const f32x4_t*>(w)[2 * i + 1];
  reinterpret_cast<u32x4_t*>(wb)[i] = pack_bf16x8(scale * a, scale * b);
}

// Splits of the apply's contraction for the 256 x 128 tiles: about one
// workgroup per CU, at most 8 splits and at least 8 stages each.
int tile_apply_splits(int c, int d_model, int d_ff) {
  const int tiles = ((c + kTM - 1) / kTM) * ((d_model + kTN - 1) / kTN);
  const int stages = (d_ff + kTK - 1) / kTK;
  int ks = device_cu_count() / tiles;
  ks = ks < 8 ? ks : 8;
  ks = ks < stages / 8 ? ks : stages / 8;
  return ks > 1 ? ks : 1;
}

// The most rows of split partial sums, ks(c) * c, over the chunk lengths
// 1 <= c <= cmax (ks_of returns 0 where the apply is not split).  A short
// last chunk has fewer row tiles and may split further than a full one; ks
// depends on c only through the row tiles, so the longest c of each count of
// tiles is enough.
template <typename F>
int64_t split_rows_max(int cmax, int tile_rows, F ks_of) {
  int64_t best = 0;
  for (int q = 1; static_cast<int64_t>(q - 1) * tile_rows < cmax; ++q) {
    const int c = static_cast<int64_t>(q) * tile_rows < cmax ? q * tile_rows : cmax;
    const int64_t v = static_cast<int64_t>(ks_of(c)) * c;
    best = v > best ? v : best;
  }
  return best;
}

// Rows of the tile path's apply partials, at most, for chunks of up to cmax tokens.
int64_t tile_split_rows(int cmax, int n, int k) {
  return split_rows_max(cmax, kTM, [&](int c) {
    const int ks = tile_apply_splits(c, n, k);
    return ks > 1 ? ks : 0;
  });
}

// Workspace of the tile path: Wb, then the apply's split partials.
size_t tile_ws_bytes(int c, int d_model, int d_ff) {
  const int64_t rows = tile_split_rows(c, d_model, d_ff);
  return align256(static_cast<size_t>(d_model) * d_ff * 2) +
         (rows > 0 ? align256(static_cast<size_t>(rows) * d_model * sizeof(float)) : 0);
}

// The tile path's byte offsets must stay below the buffer range: a tile's rows
// of Z or dO, a chunk's rows of Z, V_hat and dO, and W_down and its bf16 copies.
bool tile_path_fits(int c, int d_model, int d_ff) {
  const double lim = static_cast<double>(kOob) - (1 << 20);
  return static_cast<double>(kTM) * d_ff * 2 < lim && static_cast<double>(c) * d_ff * 2 < lim &&
         static_cast<double>(c) * d_model * 2 < lim && static_cast<double>(kTN) * d_ff * 2 < lim &&
         static_cast<double>(kTM) * d_model * 2 < lim &&  // a tile's rows of dO (the backward's dZ)
         static_cast<double>(d_model) * d_ff * 4 < lim;   // the update's writes of W
}

}  // namespace

size_t inplace_workspace_bytes(int B, int T, int d_model, int d_ff, int C) {
  if (static_cast<int64_t>(B) * T == 0) return 0;
  const int c = T < C ? T : C;
  if (tile_path_fits(c, d_model, d_ff)) return tile_ws_bytes(c, d_model, d_ff);
  const int64_t rows = split_rows_max(c, kBM, [&](int cc) {
    const int ks = apply_splits(cc, d_model, d_ff);
    return ks > 1 ? ks : 0;
  });
  return static_cast<size_t>(rows) * d_model * sizeof(float);
}

namespace {

// Update tiles per chunk: one sum of squares each in the clip area.
size_t clip_area_bytes(int d_model, int d_ff) {
  const size_t tiles = static_cast<size_t>((d_model + kBM - 1) / kBM) * ((d_ff + kBN - 1) / kBN);
  return align256(tiles * sizeof(float)) + 256;  // the partial sums, then the scale
}

struct ChunkIO {
  const bf16_t* z;     // [c, d_ff]
  const bf16_t* v;     // [c, d_model]
  const float* w_src;  // W_down the chunk starts from
  float* w_dst;        // W_down after the update (may equal w_src)
  bf16_t* o;           // [c, d_model]
};

// Clip factor of one chunk's update: per-tile sums of squares of V_hat^T Z into
// clip_ws, then min(1, tau / (|eta| sqrt(sum))) on the device at *scale.
hipError_t clip_norm(const ChunkIO& io, int c, int d_model, int d_ff, float eta, float tau, float* clip_ws,
                     const float** scale, hipStream_t s) {
  const dim3 gu((d_ff + kBN - 1) / kBN, (d_model + kBM - 1) / kBM, 1);
  const size_t tiles = static_cast<size_t>(gu.x) * gu.y;
  float* sc = reinterpret_cast<float*>(reinterpret_cast<char*>(clip_ws) + align256(tiles * sizeof(float)));
  GemmArgs np{d_model, d_ff, c, io.v, io.z, clip_ws, d_model, d_ff, d_ff, 1.0f, c};
  KernelScope timing(TTT_KERNEL_INPLACE_NORM, s);
  hipLaunchKernelGGL((gemm_kernel<true, true, bf16_t, bf16_t, kEpiSumSqF32>), gu, dim3(kThreads), 0, s, np);
  hipLaunchKernelGGL(clip_scale_kernel, dim3(1), dim3(256), 0, s, static_cast<const float*>(clip_ws),
                     static_cast<int>(tiles), eta, tau, sc);
  *scale = sc;
  return hipGetLastError();
}

// Apply, [clip scale], update for one chunk of c tokens.
hipError_t chunk_step(const ChunkIO& io, int c, int d_model, int d_ff, float eta, bool clip, float tau,
                      float* clip_ws, void* split_ws, size_t split_bytes, hipStream_t s) {
  // split-K partials in the workspace when it is large enough, else one pass
  const size_t per_split = static_cast<size_t>(c) * d_model * sizeof(float);
  int ks = split_ws ? apply_splits(c, d_model, d_ff) : 1;
  while (ks > 1 && static_cast<size_t>(ks) * per_split > split_bytes) --ks;
  const int stages = (d_ff + kBK - 1) / kBK;
  const int k_split = ks > 1 ? ((stages + ks - 1) / ks) * kBK : d_ff;
  GemmArgs ap{c, d_model, d_ff, io.z, io.w_src, ks > 1 ? split_ws : static_cast<void*>(io.o), d_ff, d_ff, d_model,
              1.0f, k_split};
  dim3 ga((d_model + kBN - 1) / kBN, (c + kBM - 1) / kBM, ks);
  hipError_t e;
  {
    KernelScope timing(TTT_KERNEL_INPLACE_APPLY, s);
    if (ks > 1) {
      hipLaunchKernelGGL((gemm_kernel<false, false, bf16_t, float, kEpiPartialF32>), ga, dim3(kThreads), 0, s, ap);
      const int64_t mn = static_cast<int64_t>(c) * d_model;
      const unsigned nb = static_cast<unsigned>((mn / 4 + 255) / 256);
      hipLaunchKernelGGL(split_reduce_kernel, dim3(nb), dim3(256), 0, s, static_cast<const float*>(split_ws), ks, mn,
                         io.o, 1.0f);
    } else {
      hipLaunchKernelGGL((gemm_kernel<false, false, bf16_t, float, kEpiStoreBf16>), ga, dim3(kThreads), 0, s, ap);
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  dim3 gu((d_ff + kBN - 1) / kBN, (d_model + kBM - 1) / kBM, 1);
  const float* scale = nullptr;
  if (clip) {
    e = clip_norm(io, c, d_model, d_ff, eta, tau, clip_ws, &scale, s);
    if (e != hipSuccess) return e;
  }
  GemmArgs up{d_model, d_ff, c, io.v, io.z, io.w_dst, d_model, d_ff, d_ff, eta, c, io.w_src, scale};
  {
    KernelScope timing(TTT_KERNEL_INPLACE_UPDATE, s);
    hipLaunchKernelGGL((gemm_kernel<true, true, bf16_t, bf16_t, kEpiAxpyF32>), gu, dim3(kThreads), 0, s, up);
    e = hipGetLastError();
  }
  return e;
}

// Bytes of Wb at the start of the tile path's workspace.
size_t wb_bytes(int d_model, int d_ff) { return align256(static_cast<size_t>(d_model) * d_ff * 2); }

// Whether inplace_launch / inplace_launch_guarded take the tile path: the
// workspace holds Wb and the apply's partials, and every offset fits.
bool use_tile_path(int T, int d_model, int d_ff, int C, void* ws, size_t ws_bytes) {
  const int c = T < C ? T : C;
  return ws && tile_path_fits(c, d_model, d_ff) && ws_bytes >= tile_ws_bytes(c, d_model, d_ff);
}

hipError_t round_bf16(const float* w, bf16_t* wb, int64_t n, hipStream_t s, float scale = 1.0f) {
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(round_bf16_kernel, dim3(static_cast<unsigned>((n8 + 255) / 256)), dim3(256), 0, s, w, wb, n8,
                     scale);
  return hipGetLastError();
}

// The clip factor on the tile path: the per-tile sums of squares of V_hat^T Z
// from update_kernel<true> (one per 256 x 128 tile, fewer than the clip area's
// slots for 128 x 128 tiles), then the factor at the area's scale slot.
hipError_t clip_norm_tile(const ChunkIO& io, int c, int d_model, int d_ff, float eta, float tau, float* clip_ws,
                          const float** scale, hipStream_t s) {
  const size_t slots = static_cast<size_t>((d_ff + kBN - 1) / kBN) * ((d_model + kBM - 1) / kBM);
  float* sc = reinterpret_cast<float*>(reinterpret_cast<char*>(clip_ws) + align256(slots * sizeof(float)));
  TileArgs np{};
  np.M = d_ff;
  np.N = d_model;
  np.K = c;
  np.A = io.z;
  np.B = io.v;
  np.lda = d_ff;
  np.ldb = d_model;
  np.w = clip_ws;
  const int utiles = ((d_ff + kTM - 1) / kTM) * ((d_model + kTN - 1) / kTN);
  const int grid = utiles < device_cu_count() ? utiles : device_cu_count();
  KernelScope timing(TTT_KERNEL_INPLACE_NORM, s);
  hipLaunchKernelGGL(update_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(kTThreads), 0, s, np);
  hipLaunchKernelGGL(clip_scale_kernel, dim3(1), dim3(256), 0, s, static_cast<const float*>(clip_ws), utiles, eta, tau,
                     sc);
  *scale = sc;
  return hipGetLastError();
}

// Apply and update of one chunk on the tile path.  wb holds bf16 of the
// chunk's starting W_down (io.w_src) and receives bf16 of the updated one;
// scale: the clip factor on the device, or NULL.
hipError_t tile_chunk_step(const ChunkIO& io, int c, int d_model, int d_ff, float eta, const float* scale,
                           bf16_t* wb, float* part, hipStream_t s) {
  const int ks = tile_apply_splits(c, d_model, d_ff);
  const int stages = (d_ff + kTK - 1) / kTK;
  TileArgs ap{};
  ap.M = c;
  ap.N = d_model;
  ap.K = d_ff;
  ap.A = io.z;
  ap.B = wb;
  ap.lda = d_ff;
  ap.ldb = d_ff;
  ap.k_split = ks > 1 ? ((stages + ks - 1) / ks) * kTK : d_ff;
  ap.o = io.o;
  ap.part = ks > 1 ? part : nullptr;
  ap.ldo = d_model;
  const int tiles = ((c + kTM - 1) / kTM) * ((d_model + kTN - 1) / kTN);
  hipError_t e;
  {
    KernelScope timing(TTT_KERNEL_INPLACE_APPLY, s);
    hipLaunchKernelGGL(apply_kernel<false>, dim3(static_cast<unsigned>(tiles * ks)), dim3(kTThreads), 0, s, ap);
    if (ks > 1) {
      const int64_t mn = static_cast<int64_t>(c) * d_model;
      hipLaunchKernelGGL(split_reduce_kernel, dim3(static_cast<unsigned>((mn / 4 + 255) / 256)), dim3(256), 0, s,
                         static_cast<const float*>(part), ks, mn, io.o, 1.0f);
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  TileArgs up{};
  up.M = d_ff;
  up.N = d_model;
  up.K = c;
  up.A = io.z;
  up.B = io.v;
  up.lda = d_ff;
  up.ldb = d_model;
  up.w_src = io.w_src;
  up.w = io.w_dst;
  up.wb = wb;
  up.ldw = d_ff;
  up.alpha = eta;
  up.scale = scale;
  up.wb_scale = 1.0f;
  const int utiles = ((d_ff + kTM - 1) / kTM) * ((d_model + kTN - 1) / kTN);
  const int grid = utiles < device_cu_count() ? utiles : device_cu_count();  // persistent: one per CU
  KernelScope timing(TTT_KERNEL_INPLACE_UPDATE, s);
  hipLaunchKernelGGL(update_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(kTThreads), 0, s, up);
  return hipGetLastError();
}

}  // namespace

size_t inplace_guarded_workspace_bytes(int B, int T, int d_model, int d_ff, int C) {
  if (static_cast<int64_t>(B) * T == 0) return 0;
  return clip_area_bytes(d_model, d_ff) + inplace_workspace_bytes(B, T, d_model, d_ff, C);
}

hipError_t inplace_launch(int B, int T, int d_model, int d_ff, int C, float eta, const void* z,
                          const void* vhat, float* w_down, void* o, void* ws, size_t ws_bytes, hipStream_t s) {
  if (use_tile_path(T, d_model, d_ff, C, ws, ws_bytes)) {
    bf16_t* wbuf = static_cast<bf16_t*>(ws);
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + wb_bytes(d_model, d_ff));
    const int64_t wsz = static_cast<int64_t>(d_model) * d_ff;
    for (int b = 0; b < B; ++b) {
      const bf16_t* zb = static_cast<const bf16_t*>(z) + static_cast<int64_t>(b) * T * d_ff;
      const bf16_t* vb = static_cast<const bf16_t*>(vhat) + static_cast<int64_t>(b) * T * d_model;
      bf16_t* ob = static_cast<bf16_t*>(o) + static_cast<int64_t>(b) * T * d_model;
      float* wb = w_down + b * wsz;
      hipError_t e = round_bf16(wb, wbuf, wsz, s);
      for (int t0 = 0; t0 < T && e == hipSuccess; t0 += C) {
        const int c = (T - t0 < C) ? T - t0 : C;
        const ChunkIO io{zb + static_cast<int64_t>(t0) * d_ff, vb + static_cast<int64_t>(t0) * d_model, wb, wb,
                         ob + static_cast<int64_t>(t0) * d_model};
        e = tile_chunk_step(io, c, d_model, d_ff, eta, nullptr, wbuf, part, s);
      }
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  for (int b = 0; b < B; ++b) {
    const bf16_t* zb = static_cast<const bf16_t*>(z) + static_cast<int64_t>(b) * T * d_ff;
    const bf16_t* vb = static_cast<const bf16_t*>(vhat) + static_cast<int64_t>(b) * T * d_model;
    bf16_t* ob = static_cast<bf16_t*>(o) + static_cast<int64_t>(b) * T * d_model;
    float* wb = w_down + static_cast<int64_t>(b) * d_model * d_ff;
    for (int t0 = 0; t0 < T; t0 += C) {
      const int c = (T - t0 < C) ? T - t0 : C;
      const ChunkIO io{zb + static_cast<int64_t>(t0) * d_ff, vb + static_cast<int64_t>(t0) * d_model, wb, wb,
                       ob + static_cast<int64_t>(t0) * d_model};
      hipError_t e = chunk_step(io, c, d_model, d_ff, eta, false, 0.0f, nullptr, ws, ws_bytes, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

namespace {

// dst = src, or 0 where src is NULL; four floats per thread (n4 = count / 4).
__global__ __launch_bounds__(256) void copy_or_zero_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                           int64_t n4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  reinterpret_cast<float4*>(dst)[i] = src ? reinterpret_cast<const float4*>(src)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, s, dst, src, n4);
  return hipGetLastError();
}

}  // namespace

// Backward workspace: the rewound W_i (one sequence at a time), the two partial
// sums of dZ, and the split-K partials of dV_hat.
size_t inplace_bwd_workspace_bytes(int B, int T, int d_model, int d_ff, int C) {
  if (static_cast<int64_t>(B) * T == 0) return 0;
  const int c = T < C ? T : C;
  if (tile_path_fits(c, d_model, d_ff)) {  // + bf16 W_i and bf16 eta dW
    const int64_t rows = tile_split_rows(c, d_model, d_ff);
    return align256(static_cast<size_t>(d_model) * d_ff * 4) + 2 * wb_bytes(d_model, d_ff) +
           align256(static_cast<size_t>(2) * c * d_ff * 4) +
           (rows > 0 ? align256(static_cast<size_t>(rows) * d_model * 4) : 0);
  }
  const int64_t rows = split_rows_max(c, kBM, [&](int cc) {
    const int ks = apply_splits(cc, d_model, d_ff);
    return ks > 1 ? ks : 0;
  });
  return align256(static_cast<size_t>(d_model) * d_ff * 4) + align256(static_cast<size_t>(2) * c * d_ff * 4) +
         (rows > 0 ? align256(static_cast<size_t>(rows) * d_model * 4) : 0);
}

namespace {

// The backward on the tile path, one chunk of c tokens at zc, vc, oc:
//   rewind  W_i = W_{i+1} - eta V_hat_i^T Z_i     update_kernel, writes bf16(W_i)
//   dZ_i    = dO_i W_i + V_hat_i (eta dW)          apply_kernel<true>, the two terms as two splits
//   dV_hat_i = Z_i (eta dW)^T                      apply_kernel<false>, split over d_ff
//   dW     += dO_i^T Z_i                           update_kernel, writes bf16(eta dW)
// W holds W_{i+1} on entry and W_i on return; dW holds dL/dW_{i+1} on entry
// (dW16 its bf16(eta dW), from the previous accumulation) and dL/dW_i on return.
hipError_t tile_bwd_chunk(const bf16_t* zc, const bf16_t* vc, const bf16_t* oc, bf16_t* dzc, bf16_t* dvc, int c,
                          int d_model, int d_ff, float eta, float* W, float* dW, bf16_t* W16, bf16_t* dW16, float* pz,
                          float* pv, hipStream_t s) {
  const int cus = device_cu_count();
  const int ut = ((d_ff + kTM - 1) / kTM) * ((d_model + kTN - 1) / kTN);
  const int ugrid = ut < cus ? ut : cus;
  hipError_t e;
  {  // W_i = W_{i+1} - eta V_hat_i^T Z_i, and bf16(W_i)
    KernelScope timing(TTT_KERNEL_INPLACE_BWD_W, s);
    TileArgs u{};
    u.M = d_ff, u.N = d_model, u.K = c, u.A = zc, u.B = vc, u.lda = d_ff, u.ldb = d_model;
    u.w_src = W, u.w = W, u.wb = W16, u.ldw = d_ff, u.alpha = -eta, u.wb_scale = 1.0f;
    hipLaunchKernelGGL(update_kernel<false>, dim3(static_cast<unsigned>(ugrid)), dim3(kTThreads), 0, s, u);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  {  // dZ_i = dO_i W_i + V_hat_i (eta dW_{i+1})
    KernelScope timing(TTT_KERNEL_INPLACE_BWD_DZ, s);
    TileArgs a{};
    a.M = c, a.N = d_ff, a.K = d_model, a.A = oc, a.B = W16, a.A2 = vc, a.B2 = dW16;
    a.lda = d_model, a.ldb = d_ff, a.k_split = d_model, a.part = pz, a.ldo = d_ff;
    const int tiles = ((c + kTM - 1) / kTM) * ((d_ff + kTN - 1) / kTN);
    hipLaunchKernelGGL(apply_kernel<true>, dim3(static_cast<unsigned>(2 * tiles)), dim3(kTThreads), 0, s, a);
    const int64_t mn = static_cast<int64_t>(c) * d_ff;
    hipLaunchKernelGGL(split_reduce_kernel, dim3(static_cast<unsigned>((mn / 4 + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(pz), 2, mn, dzc, 1.0f);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  {  // dV_hat_i = Z_i (eta dW_{i+1})^T
    KernelScope timing(TTT_KERNEL_INPLACE_BWD_DV, s);
    const int ks = tile_apply_splits(c, d_model, d_ff);
    const int stages = (d_ff + kTK - 1) / kTK;
    TileArgs a{};
    a.M = c, a.N = d_model, a.K = d_ff, a.A = zc, a.B = dW16, a.lda = d_ff, a.ldb = d_ff;
    a.k_split = ks > 1 ? ((stages + ks - 1) / ks) * kTK : d_ff;
    bf16_t* out = dvc;
    a.o = out, a.part = ks > 1 ? pv : nullptr, a.ldo = d_model;
    const int tiles = ((c + kTM - 1) / kTM) * ((d_model + kTN - 1) / kTN);
    hipLaunchKernelGGL(apply_kernel<false>, dim3(static_cast<unsigned>(tiles * ks)), dim3(kTThreads), 0, s, a);
    if (ks > 1) {
      const int64_t mn = static_cast<int64_t>(c) * d_model;
      hipLaunchKernelGGL(split_reduce_kernel, dim3(static_cast<unsigned>((mn / 4 + 255) / 256)), dim3(256), 0, s,
                         static_cast<const float*>(pv), ks, mn, out, 1.0f);
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  {  // dW += dO_i^T Z_i, and bf16(eta dW)
    KernelScope timing(TTT_KERNEL_INPLACE_BWD_DW, s);
    TileArgs u{};
    u.M = d_ff, u.N = d_model, u.K = c, u.A = zc, u.B = oc, u.lda = d_ff, u.ldb = d_model;
    u.w_src = dW, u.w = dW, u.wb = dW16, u.ldw = d_ff, u.alpha = 1.0f, u.wb_scale = eta;
    hipLaunchKernelGGL(update_kernel<false>, dim3(static_cast<unsigned>(ugrid)), dim3(kTThreads), 0, s, u);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  return hipSuccess;
}

// The backward on the tile path, one sequence, chunk by chunk from the last.
hipError_t tile_bwd_sequence(int T, int d_model, int d_ff, int C, float eta, const bf16_t* zb, const bf16_t* vb,
                             const bf16_t* ob, bf16_t* dzb, bf16_t* dvb, float* W, float* dW, bf16_t* W16,
                             bf16_t* dW16, float* pz, float* pv, hipStream_t s) {
  const int64_t wsz = static_cast<int64_t>(d_model) * d_ff;
  hipError_t e = round_bf16(dW, dW16, wsz, s, eta);
  const int nch = (T + C - 1) / C;
  for (int ci = nch - 1; ci >= 0 && e == hipSuccess; --ci) {
    const int t0 = ci * C;
    const int c = (T - t0 < C) ? T - t0 : C;
    e = tile_bwd_chunk(zb + static_cast<int64_t>(t0) * d_ff, vb + static_cast<int64_t>(t0) * d_model,
                       ob + static_cast<int64_t>(t0) * d_model, dzb + static_cast<int64_t>(t0) * d_ff,
                       dvb + static_cast<int64_t>(t0) * d_model, c, d_model, d_ff, eta, W, dW, W16, dW16, pz, pv, s);
  }
  return e;
}

// ---------------------------------------------------------------------------
// Backward of the guarded forward (update clipping and document resets).
//
// With D_i = eta V_hat_i^T Z_i, n = ||D_i||_F and the applied update s D_i,
// s = min(1, tau / n): past the threshold s = tau / n depends on D_i, and the
// adjoint of D_i is G = s A - kappa D_i with A = dL/dW_{i+1} and
// kappa = s <D_i, A> / n^2 (kappa = 0 where the update is not clipped).  The
// terms of D_i are formed through the chunk's Gram matrices, which keeps every
// product the size of a chunk:
//   <D_i, A>  = <V_hat_i, P>, P = Z_i (eta A)^T            (the dV_hat product)
//   dV_hat_i  = s P - kappa eta^2 (Z_i Z_i^T) V_hat_i
//   dZ_i      = dO_i W_i + s V_hat_i (eta A) - kappa eta^2 (V_hat_i V_hat_i^T) Z_i

// The per-chunk scalars, on the device.
struct ClipStats {
  double norm;  // ||D_i||_F
  float scale;  // s
  float kappa;  // s <D_i, A> / n^2 where clipped, else 0
};

// Sum of one double per thread of a 256-thread block, in a fixed order; the
// result is valid in thread 0.
__device__ double block_sum256(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  return red[0];
}

// norm and s of one chunk from the per-tile sums of squares of V_hat^T Z.
__global__ __launch_bounds__(256) void clip_stats_kernel(const float* __restrict__ part, int n, float eta, float tau,
                                                         ClipStats* __restrict__ st) {
  __shared__ double red[256];
  double v = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) v += static_cast<double>(part[i]);
  const double sum = block_sum256(v, red);
  if (threadIdx.x == 0) {
    const double norm = fabs(static_cast<double>(eta)) * sqrt(sum);
    st->norm = norm;
    st->scale = norm > static_cast<double>(tau) ? static_cast<float>(static_cast<double>(tau) / norm) : 1.0f;
    st->kappa = 0.0f;
  }
}

// P = the sum of the ks split partials (written over split 0), and per block
// the sum of V_hat (.) P; 4 elements per thread (mn % 4 == 0).
__global__ __launch_bounds__(256) void pdot_kernel(float* __restrict__ part, int ks, int64_t mn,
                                                   const bf16_t* __restrict__ vhat, double* __restrict__ bsum) {
  __shared__ double red[256];
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  double v = 0.0;
  if (i < mn) {
    f32x4_t acc = *reinterpret_cast<const f32x4_t*>(part + i);
    for (int k = 1; k < ks; ++k) acc += *reinterpret_cast<const f32x4_t*>(part + k * mn + i);
    *reinterpret_cast<f32x4_t*>(part + i) = acc;
    const u32x2_t h = *reinterpret_cast<const u32x2_t*>(vhat + i);
    v = static_cast<double>(bf16_to_f32(static_cast<uint16_t>(h[0] & 0xffffu)) * acc[0]) +
        static_cast<double>(bf16_to_f32(static_cast<uint16_t>(h[0] >> 16)) * acc[1]) +
        static_cast<double>(bf16_to_f32(static_cast<uint16_t>(h[1] & 0xffffu)) * acc[2]) +
        static_cast<double>(bf16_to_f32(static_cast<uint16_t>(h[1] >> 16)) * acc[3]);
  }
  const double sum = block_sum256(v, red);
  if (threadIdx.x == 0) bsum[blockIdx.x] = sum;
}

// kappa of one chunk from pdot's block sums.
__global__ __launch_bounds__(256) void kappa_kernel(const double* __restrict__ bsum, int nb, float tau,
                                                    ClipStats* __restrict__ st) {
  __shared__ double red[256];
  double v = 0.0;
  for (int i = threadIdx.x; i < nb; i += 256) v += bsum[i];
  const double dot = block_sum256(v, red);
  if (threadIdx.x == 0) {
    const double n = st->norm;
    st->kappa = n > static_cast<double>(tau) ? static_cast<float>(st->scale * dot / (n * n)) : 0.0f;
  }
}

// dV_hat = bf16(s P - kappa eta^2 R), R = (Z Z^T) V_hat; 4 elements per thread.
__global__ __launch_bounds__(256) void dv_combine_kernel(const float* __restrict__ p, const float* __restrict__ r,
                                                         int64_t mn, const ClipStats* __restrict__ st, float eta2,
                                                         bf16_t* __restrict__ out) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= mn) return;
  const float sc = st->scale, kc = -st->kappa * eta2;
  const f32x4_t x = sc * *reinterpret_cast<const f32x4_t*>(p + i) + kc * *reinterpret_cast<const f32x4_t*>(r + i);
  *reinterpret_cast<u32x2_t*>(out + i) = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
}

// dZ = bf16(p0 + s p1 - kappa eta^2 p2) over the three partial products.
__global__ __launch_bounds__(256) void dz_combine_kernel(const float* __restrict__ p, int64_t mn,
                                                         const ClipStats* __restrict__ st, float eta2,
                                                         bf16_t* __restrict__ out) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= mn) return;
  const float sc = st->scale, kc = -st->kappa * eta2;
  const f32x4_t x = *reinterpret_cast<const f32x4_t*>(p + i) + sc * *reinterpret_cast<const f32x4_t*>(p + mn + i) +
                    kc * *reinterpret_cast<const f32x4_t*>(p + 2 * mn + i);
  *reinterpret_cast<u32x2_t*>(out + i) = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
}

// The Gram matrix in bf16 from its split partials ([ks][c][c] fp32), as rows
// of ldg >= c elements whose tail (columns c .. ldg - 1) is zero: the apply
// reads its contraction in 8-element pieces, and the piece that straddles c
// must read zeros past it.
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ part, int ks, int c, int ldg,
                                                          bf16_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(c) * ldg) return;
  const int t = static_cast<int>(i / ldg), k = static_cast<int>(i % ldg);
  float v = 0.0f;
  if (k < c) {
    const int64_t mn = static_cast<int64_t>(c) * c;
    for (int q = 0; q < ks; ++q) v += part[q * mn + static_cast<int64_t>(t) * c + k];
  }
  out[i] = f32_to_bf16(v);
}

// dst += src; four floats per thread (n4 = count / 4).
__global__ __launch_bounds__(256) void accumulate_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                         int64_t n4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  reinterpret_cast<f32x4_t*>(dst)[i] += reinterpret_cast<const f32x4_t*>(src)[i];
}

int round_up8(int x) { return (x + 7) / 8 * 8; }

// The device address of a ClipStats's s (host code never dereferences st).
const float* scale_ptr(const ClipStats* st) {
  return reinterpret_cast<const float*>(reinterpret_cast<const char*>(st) + offsetof(ClipStats, scale));
}

// Buffers of the guarded backward (one sequence at a time).
struct GuardedBufs {
  float* W;          // the state, fp32 [d_model][d_ff]
  bf16_t* W16;       // bf16(W_i)
  bf16_t* dW16;      // bf16(eta A)
  float* pz;         // dZ's three partial products [3][c][d_ff]
  float* pv;         // P's split partials [ks][c][d_model]
  float* rv;         // (Z Z^T) V_hat [c][d_model]
  bf16_t* gram;      // a Gram matrix [c][round_up8(c)]
  float* gpart;      // its split partials [ks][c][c]
  float* clip_part;  // the norm's per-tile sums
  double* bsum;      // pdot's block sums
  ClipStats* st;
};

size_t guarded_bwd_bytes_parts(int cmax, int d_model, int d_ff, size_t* off) {
  const int64_t wsz = static_cast<int64_t>(d_model) * d_ff;
  const int64_t pv_rows = split_rows_max(cmax, kTM, [&](int c) { return tile_apply_splits(c, d_model, d_ff); });
  const int utiles = ((d_ff + kTM - 1) / kTM) * ((d_model + kTN - 1) / kTN);
  const int64_t nb = (static_cast<int64_t>(cmax) * d_model / 4 + 255) / 256;
  const size_t sz[11] = {align256(static_cast<size_t>(wsz) * 4),
                         wb_bytes(d_model, d_ff),
                         wb_bytes(d_model, d_ff),
                         align256(static_cast<size_t>(3) * cmax * d_ff * 4),
                         align256(static_cast<size_t>(pv_rows) * d_model * 4),
                         align256(static_cast<size_t>(cmax) * d_model * 4),
                         align256(static_cast<size_t>(cmax) * round_up8(cmax) * 2),
                         align256(static_cast<size_t>(8) * cmax * cmax * 4),  // ks <= 8
                         align256(static_cast<size_t>(utiles) * 4),
                         align256(static_cast<size_t>(nb) * 8),
                         align256(sizeof(ClipStats))};
  size_t total = 0;
  for (int i = 0; i < 11; ++i) {
    if (off) off[i] = total;
    total += sz[i];
  }
  return total;
}

GuardedBufs guarded_bufs(void* ws, int cmax, int d_model, int d_ff) {
  size_t off[11];
  guarded_bwd_bytes_parts(cmax, d_model, d_ff, off);
  char* p = static_cast<char*>(ws);
  return GuardedBufs{reinterpret_cast<float*>(p + off[0]),  reinterpret_cast<bf16_t*>(p + off[1]),
                     reinterpret_cast<bf16_t*>(p + off[2]), reinterpret_cast<float*>(p + off[3]),
                     reinterpret_cast<float*>(p + off[4]),  reinterpret_cast<float*>(p + off[5]),
                     reinterpret_cast<bf16_t*>(p + off[6]), reinterpret_cast<float*>(p + off[7]),
                     reinterpret_cast<float*>(p + off[8]),  reinterpret_cast<double*>(p + off[9]),
                     reinterpret_cast<ClipStats*>(p + off[10])};
}

// The update's products for one chunk (update_kernel on Z, V_hat): W = W_src +
// alpha (*scale) V_hat^T Z with bf16(W) into wb.
hipError_t tile_update(const bf16_t* zc, const bf16_t* vc, int c, int d_model, int d_ff, float* W, bf16_t* wb,
                       float alpha, const float* scale, float wb_scale, hipStream_t s) {
  const int ut = ((d_ff + kTM - 1) / kTM) * ((d_model + kTN - 1) / kTN);
  const int cus = device_cu_count();
  TileArgs u{};
  u.M = d_ff, u.N = d_model, u.K = c, u.A = zc, u.B = vc, u.lda = d_ff, u.ldb = d_model;
  u.w_src = W, u.w = W, u.wb = wb, u.ldw = d_ff, u.alpha = alpha, u.scale = scale, u.wb_scale = wb_scale;
  hipLaunchKernelGGL(update_kernel<false>, dim3(static_cast<unsigned>(ut < cus ? ut : cus)), dim3(kTThreads), 0, s, u);
  return hipGetLastError();
}

// norm and s of the update of one chunk into g.st.
hipError_t tile_clip_stats(const bf16_t* zc, const bf16_t* vc, int c, int d_model, int d_ff, float eta, float tau,
                           const GuardedBufs& g, hipStream_t s) {
  TileArgs np{};
  np.M = d_ff, np.N = d_model, np.K = c, np.A = zc, np.B = vc, np.lda = d_ff, np.ldb = d_model, np.w = g.clip_part;
  const int ut = ((d_ff + kTM - 1) / kTM) * ((d_model + kTN - 1) / kTN);
  const int cus = device_cu_count();
  KernelScope timing(TTT_KERNEL_INPLACE_NORM, s);
  hipLaunchKernelGGL(update_kernel<true>, dim3(static_cast<unsigned>(ut < cus ? ut : cus)), dim3(kTThreads), 0, s, np);
  hipLaunchKernelGGL(clip_stats_kernel, dim3(1), dim3(256), 0, s, static_cast<const float*>(g.clip_part), ut, eta, tau,
                     g.st);
  return hipGetLastError();
}

// O-shaped product X Y^T (X [m][k], Y [n][k], both k-contiguous) as ks split
// partials [ks][m][n] fp32 into part; returns ks.
int tile_apply_partials(const bf16_t* X, int64_t ldx, const bf16_t* Y, int64_t ldy, int m, int n, int k, float* part,
                        hipStream_t s) {
  const int ks = tile_apply_splits(m, n, k);
  const int stages = (k + kTK - 1) / kTK;
  TileArgs a{};
  a.M = m, a.N = n, a.K = k, a.A = X, a.B = Y, a.lda = ldx, a.ldb = ldy;
  a.k_split = ks > 1 ? ((stages + ks - 1) / ks) * kTK : k;
  a.part = part, a.ldo = n;
  const int tiles = ((m + kTM - 1) / kTM) * ((n + kTN - 1) / kTN);
  hipLaunchKernelGGL(apply_kernel<false>, dim3(static_cast<unsigned>(tiles * ks)), dim3(kTThreads), 0, s, a);
  return ks;
}

// The Gram matrix X X^T of a chunk (X [c][k]) into g.gram (bf16, rows of round_up8(c)).
hipError_t tile_gram(const bf16_t* X, int c, int k, const GuardedBufs& g, hipStream_t s) {
  const int ks = tile_apply_partials(X, k, X, k, c, c, k, g.gpart, s);
  const int ldg = round_up8(c);
  const int64_t n = static_cast<int64_t>(c) * ldg;
  hipLaunchKernelGGL(gram_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const float*>(g.gpart), ks, c, ldg, g.gram);
  return hipGetLastError();
}

// (Gram) Y for Y [c][n] (n contiguous), fp32 into out [c][n] (one split).
hipError_t tile_gram_times(const bf16_t* Y, int c, int n, const GuardedBufs& g, float* out, hipStream_t s) {
  TileArgs a{};
  a.M = c, a.N = n, a.K = c, a.A = g.gram, a.B = Y, a.lda = round_up8(c), a.ldb = n, a.k_split = c;
  a.part = out, a.ldo = n;
  const int tiles = ((c + kTM - 1) / kTM) * ((n + kTN - 1) / kTN);
  hipLaunchKernelGGL(apply_kernel<true>, dim3(static_cast<unsigned>(tiles)), dim3(kTThreads), 0, s, a);
  return hipGetLastError();
}

// One chunk of the guarded backward with clipping (c tokens at zc, vc, oc):
// on entry g.W = W_{i+1} and g.dW16 = bf16(eta A), A = dL/dW_{i+1} (fp32 in
// dW); on return g.W = W_i, dW = dL/dW_i and g.dW16 its bf16(eta .).
hipError_t tile_bwd_clipped_chunk(const bf16_t* zc, const bf16_t* vc, const bf16_t* oc, bf16_t* dzc, bf16_t* dvc,
                                  int c, int d_model, int d_ff, float eta, float tau, float* dW,
                                  const GuardedBufs& g, hipStream_t s) {
  hipError_t e = tile_clip_stats(zc, vc, c, d_model, d_ff, eta, tau, g, s);
  if (e != hipSuccess) return e;
  {  // W_i = W_{i+1} - s eta V_hat_i^T Z_i, and bf16(W_i)
    KernelScope timing(TTT_KERNEL_INPLACE_BWD_W, s);
    e = tile_update(zc, vc, c, d_model, d_ff, g.W, g.W16, -eta, scale_ptr(g.st), 1.0f, s);
  }
  if (e != hipSuccess) return e;
  const float eta2 = eta * eta;
  {  // dV_hat_i = s P - kappa eta^2 (Z Z^T) V_hat, and kappa from <V_hat, P>
    KernelScope timing(TTT_KERNEL_INPLACE_BWD_DV, s);
    e = tile_gram(zc, c, d_ff, g, s);
    if (e == hipSuccess) e = tile_gram_times(vc, c, d_model, g, g.rv, s);
    const int ks = tile_apply_partials(zc, d_ff, g.dW16, d_ff, c, d_model, d_ff, g.pv, s);
    const int64_t mn = static_cast<int64_t>(c) * d_model;
    const int nb = static_cast<int>((mn / 4 + 255) / 256);
    hipLaunchKernelGGL(pdot_kernel, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s, g.pv, ks, mn, vc, g.bsum);
    hipLaunchKernelGGL(kappa_kernel, dim3(1), dim3(256), 0, s, static_cast<const double*>(g.bsum), nb, tau, g.st);
    hipLaunchKernelGGL(dv_combine_kernel, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s,
                       static_cast<const float*>(g.pv), static_cast<const float*>(g.rv), mn,
                       static_cast<const ClipStats*>(g.st), eta2, dvc);
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  {  // dZ_i = dO_i W_i + s V_hat_i (eta A) - kappa eta^2 (V_hat V_hat^T) Z_i
    KernelScope timing(TTT_KERNEL_INPLACE_BWD_DZ, s);
    TileArgs a{};
    a.M = c, a.N = d_ff, a.K = d_model, a.A = oc, a.B = g.W16, a.A2 = vc, a.B2 = g.dW16;
    a.lda = d_model, a.ldb = d_ff, a.k_split = d_model, a.part = g.pz, a.ldo = d_ff;
    const int tiles = ((c + kTM - 1) / kTM) * ((d_ff + kTN - 1) / kTN);
    hipLaunchKernelGGL(apply_kernel<true>, dim3(static_cast<unsigned>(2 * tiles)), dim3(kTThreads), 0, s, a);
    const int64_t mn = static_cast<int64_t>(c) * d_ff;
    e = tile_gram(vc, c, d_model, g, s);
    if (e == hipSuccess) e = tile_gram_times(zc, c, d_ff, g, g.pz + 2 * mn, s);
    hipLaunchKernelGGL(dz_combine_kernel, dim3(static_cast<unsigned>((mn / 4 + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(g.pz), mn, static_cast<const ClipStats*>(g.st), eta2, dzc);
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  {  // dW += dO_i^T Z_i, and bf16(eta dW)
    KernelScope timing(TTT_KERNEL_INPLACE_BWD_DW, s);
    e = tile_update(zc, oc, c, d_model, d_ff, dW, g.dW16, 1.0f, nullptr, eta, s);
  }
  return e;
}

}  // namespace

size_t inplace_bwd_guarded_workspace_bytes(int B, int T, int d_model, int d_ff, int C) {
  if (static_cast<int64_t>(B) * T == 0) return 0;
  const int c = T < C ? T : C;
  return guarded_bwd_bytes_parts(c, d_model, d_ff, nullptr);
}

bool inplace_bwd_guarded_supported(int T, int d_model, int d_ff, int C) {
  const int c = T < C ? T : C;
  return tile_path_fits(c, d_model, d_ff) && c <= kGuardedBwdMaxC;
}

// The backward of inplace_launch_guarded, sequence by sequence and, within a
// sequence, document by document from the last.  The last document starts
// from w_final and dL/dW_final; every other document's final state is first
// recomputed by its forward updates from its starting state (w0 for the first
// document, w_init for the others), and its final adjoint is zero (the reset
// discards that state).  Each document is then walked back chunk by chunk; its
// adjoint at the first token is dL/dw0 (first document) or is added to
// dL/dw_init (the others).
hipError_t inplace_bwd_guarded_launch(int B, int T, int d_model, int d_ff, int C, float eta, float clip_tau,
                                      const int64_t* doc_starts, int n_docs, const void* z, const void* vhat,
                                      const float* w0, const float* w_init, const float* w_final, const void* d_o,
                                      const float* d_wfinal, void* dz, void* dvhat, float* dw0, float* dw_init,
                                      void* ws, hipStream_t s) {
  const bool clip = clip_tau > 0.0f && clip_tau < INFINITY;
  const int64_t wsz = static_cast<int64_t>(d_model) * d_ff;
  const int cmax = T < C ? T : C;
  const GuardedBufs g = guarded_bufs(ws, cmax, d_model, d_ff);
  int d = 0;  // next entry of doc_starts
  for (int b = 0; b < B; ++b) {
    const bf16_t* zb = static_cast<const bf16_t*>(z) + static_cast<int64_t>(b) * T * d_ff;
    const bf16_t* vb = static_cast<const bf16_t*>(vhat) + static_cast<int64_t>(b) * T * d_model;
    const bf16_t* ob = static_cast<const bf16_t*>(d_o) + static_cast<int64_t>(b) * T * d_model;
    bf16_t* dzb = static_cast<bf16_t*>(dz) + static_cast<int64_t>(b) * T * d_ff;
    bf16_t* dvb = static_cast<bf16_t*>(dvhat) + static_cast<int64_t>(b) * T * d_model;
    float* dW = dw0 + b * wsz;
    std::vector<int> bounds{0};
    while (d < n_docs && doc_starts[d] < static_cast<int64_t>(b + 1) * T)
      bounds.push_back(static_cast<int>(doc_starts[d++] - static_cast<int64_t>(b) * T));
    bounds.push_back(T);
    const int nd = static_cast<int>(bounds.size()) - 1;
    hipError_t e = hipSuccess;
    if (dw_init) e = copy_or_zero(dw_init + b * wsz, nullptr, wsz, s);
    for (int j = nd - 1; j >= 0 && e == hipSuccess; --j) {
      const int a = bounds[j], end = bounds[j + 1];
      if (j == nd - 1) {
        e = copy_or_zero(g.W, w_final + b * wsz, wsz, s);
        if (e == hipSuccess) e = copy_or_zero(dW, d_wfinal ? d_wfinal + b * wsz : nullptr, wsz, s);
      } else {  // the document's final state, from its start
        e = copy_or_zero(g.W, (j == 0 ? w0 : w_init) + b * wsz, wsz, s);
        for (int t0 = a; t0 < end && e == hipSuccess; t0 += C) {
          const int c = (end - t0 < C) ? end - t0 : C;
          const bf16_t* zc = zb + static_cast<int64_t>(t0) * d_ff;
          const bf16_t* vc = vb + static_cast<int64_t>(t0) * d_model;
          if (clip) e = tile_clip_stats(zc, vc, c, d_model, d_ff, eta, clip_tau, g, s);
          if (e == hipSuccess) {
            KernelScope timing(TTT_KERNEL_INPLACE_UPDATE, s);
            e = tile_update(zc, vc, c, d_model, d_ff, g.W, g.W16, eta, clip ? scale_ptr(g.st) : nullptr, 1.0f, s);
          }
        }
        if (e == hipSuccess) e = copy_or_zero(dW, nullptr, wsz, s);
      }
      if (e == hipSuccess) e = round_bf16(dW, g.dW16, wsz, s, eta);
      const int nch = (end - a + C - 1) / C;
      for (int k = nch - 1; k >= 0 && e == hipSuccess; --k) {
        const int t0 = a + k * C;
        const int c = (end - t0 < C) ? end - t0 : C;
        const bf16_t* zc = zb + static_cast<int64_t>(t0) * d_ff;
        const bf16_t* vc = vb + static_cast<int64_t>(t0) * d_model;
        const bf16_t* oc = ob + static_cast<int64_t>(t0) * d_model;
        bf16_t* dzc = dzb + static_cast<int64_t>(t0) * d_ff;
        bf16_t* dvc = dvb + static_cast<int64_t>(t0) * d_model;
        if (clip)
          e = tile_bwd_clipped_chunk(zc, vc, oc, dzc, dvc, c, d_model, d_ff, eta, clip_tau, dW, g, s);
        else
          e = tile_bwd_chunk(zc, vc, oc, dzc, dvc, c, d_model, d_ff, eta, g.W, dW, g.W16, g.dW16, g.pz, g.pv, s);
      }
      if (e == hipSuccess && j > 0 && dw_init) {
        const int64_t n4 = wsz / 4;
        hipLaunchKernelGGL(accumulate_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, s,
                           dw_init + b * wsz, static_cast<const float*>(dW), n4);
        e = hipGetLastError();
      }
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The reverse-mode derivative of the apply-then-update chain, chunk by chunk from
// the last: with dW = dL/dW_{i+1} (starting from d_wfinal, or 0),
//   W_i       = W_{i+1} - eta V_hat_i^T Z_i     (the state rewound from W_final)
//   dZ_i      = dO_i W_i + eta V_hat_i dW        (one launch, the two products as two splits)
//   dV_hat_i  = eta Z_i dW^T                     (the apply GEMM with dW for W)
//   dW       += dO_i^T Z_i                       (the update GEMM with dO for V_hat)
// and dw0 receives dW after the first chunk.
hipError_t inplace_bwd_launch(int B, int T, int d_model, int d_ff, int C, float eta, const void* z, const void* vhat,
                              const float* w_final, const void* d_o, const float* d_wfinal, void* dz, void* dvhat,
                              float* dw0, void* ws, hipStream_t s) {
  const int64_t wsz = static_cast<int64_t>(d_model) * d_ff;
  const int cmax = T < C ? T : C;
  if (tile_path_fits(cmax, d_model, d_ff)) {
    char* p = static_cast<char*>(ws);
    float* W = reinterpret_cast<float*>(p);
    p += align256(static_cast<size_t>(wsz) * 4);
    bf16_t* W16 = reinterpret_cast<bf16_t*>(p);
    p += wb_bytes(d_model, d_ff);
    bf16_t* dW16 = reinterpret_cast<bf16_t*>(p);
    p += wb_bytes(d_model, d_ff);
    float* pz = reinterpret_cast<float*>(p);
    p += align256(static_cast<size_t>(2) * cmax * d_ff * 4);
    float* pv = reinterpret_cast<float*>(p);
    for (int b = 0; b < B; ++b) {
      float* dW = dw0 + b * wsz;
      hipError_t e = copy_or_zero(W, w_final + b * wsz, wsz, s);
      if (e == hipSuccess) e = copy_or_zero(dW, d_wfinal ? d_wfinal + b * wsz : nullptr, wsz, s);
      if (e == hipSuccess)
        e = tile_bwd_sequence(T, d_model, d_ff, C, eta, static_cast<const bf16_t*>(z) + static_cast<int64_t>(b) * T * d_ff,
                              static_cast<const bf16_t*>(vhat) + static_cast<int64_t>(b) * T * d_model,
                              static_cast<const bf16_t*>(d_o) + static_cast<int64_t>(b) * T * d_model,
                              static_cast<bf16_t*>(dz) + static_cast<int64_t>(b) * T * d_ff,
                              static_cast<bf16_t*>(dvhat) + static_cast<int64_t>(b) * T * d_model, W, dW, W16, dW16, pz,
                              pv, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  float* Wb = static_cast<float*>(ws);
  float* pz = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(static_cast<size_t>(wsz) * 4));
  float* pv = reinterpret_cast<float*>(reinterpret_cast<char*>(pz) + align256(static_cast<size_t>(2) * cmax * d_ff * 4));
  for (int b = 0; b < B; ++b) {
    const bf16_t* zb = static_cast<const bf16_t*>(z) + static_cast<int64_t>(b) * T * d_ff;
    const bf16_t* vb = static_cast<const bf16_t*>(vhat) + static_cast<int64_t>(b) * T * d_model;
    const bf16_t* ob = static_cast<const bf16_t*>(d_o) + static_cast<int64_t>(b) * T * d_model;
    bf16_t* dzb = static_cast<bf16_t*>(dz) + static_cast<int64_t>(b) * T * d_ff;
    bf16_t* dvb = static_cast<bf16_t*>(dvhat) + static_cast<int64_t>(b) * T * d_model;
    float* dW = dw0 + b * wsz;
    hipError_t e = copy_or_zero(Wb, w_final + b * wsz, wsz, s);
    if (e == hipSuccess) e = copy_or_zero(dW, d_wfinal ? d_wfinal + b * wsz : nullptr, wsz, s);
    if (e != hipSuccess) return e;
    const int nch = (T + C - 1) / C;
    for (int ci = nch - 1; ci >= 0; --ci) {
      const int t0 = ci * C;
      const int c = (T - t0 < C) ? T - t0 : C;
      const bf16_t* zc = zb + static_cast<int64_t>(t0) * d_ff;
      const bf16_t* vc = vb + static_cast<int64_t>(t0) * d_model;
      const bf16_t* oc = ob + static_cast<int64_t>(t0) * d_model;
      const dim3 gu((d_ff + kBN - 1) / kBN, (d_model + kBM - 1) / kBM, 1);
      {  // W_i = W_{i+1} - eta V_hat_i^T Z_i
        KernelScope timing(TTT_KERNEL_INPLACE_BWD_W, s);
        const GemmArgs rw{d_model, d_ff, c, vc, zc, Wb, d_model, d_ff, d_ff, -eta, c};
        hipLaunchKernelGGL((gemm_kernel<true, true, bf16_t, bf16_t, kEpiAxpyF32>), gu, dim3(kThreads), 0, s, rw);
        e = hipGetLastError();
      }
      if (e != hipSuccess) return e;
      {  // dZ_i = dO_i W_i + eta V_hat_i dW
        KernelScope timing(TTT_KERNEL_INPLACE_BWD_DZ, s);
        GemmArgs gz{c, d_ff, d_model, oc, Wb, pz, d_model, d_ff, d_ff, 1.0f, d_model};
        gz.A_alt = vc;
        gz.B_alt = dW;
        gz.alt_scale = eta;
        const dim3 grid((d_ff + kBN - 1) / kBN, (c + kBM - 1) / kBM, 2);
        hipLaunchKernelGGL((gemm_kernel<false, true, bf16_t, float, kEpiPartialF32>), grid, dim3(kThreads), 0, s, gz);
        const int64_t mn = static_cast<int64_t>(c) * d_ff;
        hipLaunchKernelGGL(split_reduce_kernel, dim3(static_cast<unsigned>((mn / 4 + 255) / 256)), dim3(256), 0, s,
                           static_cast<const float*>(pz), 2, mn, dzb + static_cast<int64_t>(t0) * d_ff, 1.0f);
        e = hipGetLastError();
      }
      if (e != hipSuccess) return e;
      {  // dV_hat_i = eta Z_i dW^T
        KernelScope timing(TTT_KERNEL_INPLACE_BWD_DV, s);
        const int ks = apply_splits(c, d_model, d_ff);
        const int stages = (d_ff + kBK - 1) / kBK;
        const int k_split = ks > 1 ? ((stages + ks - 1) / ks) * kBK : d_ff;
        bf16_t* out = dvb + static_cast<int64_t>(t0) * d_model;
        const GemmArgs gv{c, d_model, d_ff, zc, dW, ks > 1 ? static_cast<void*>(pv) : static_cast<void*>(out), d_ff,
                          d_ff, d_model, eta, k_split};
        const dim3 grid((d_model + kBN - 1) / kBN, (c + kBM - 1) / kBM, ks);
        if (ks > 1) {
          hipLaunchKernelGGL((gemm_kernel<false, false, bf16_t, float, kEpiPartialF32>), grid, dim3(kThreads), 0, s, gv);
          const int64_t mn = static_cast<int64_t>(c) * d_model;
          hipLaunchKernelGGL(split_reduce_kernel, dim3(static_cast<unsigned>((mn / 4 + 255) / 256)), dim3(256), 0, s,
                             static_cast<const float*>(pv), ks, mn, out, eta);
        } else {
          hipLaunchKernelGGL((gemm_kernel<false, false, bf16_t, float, kEpiStoreBf16>), grid, dim3(kThreads), 0, s, gv);
        }
        e = hipGetLastError();
      }
      if (e != hipSuccess) return e;
      {  // dW += dO_i^T Z_i
        KernelScope timing(TTT_KERNEL_INPLACE_BWD_DW, s);
        const GemmArgs gw{d_model, d_ff, c, oc, zc, dW, d_model, d_ff, d_ff, 1.0f, c};
        hipLaunchKernelGGL((gemm_kernel<true, true, bf16_t, bf16_t, kEpiAxpyF32>), gu, dim3(kThreads), 0, s, gw);
        e = hipGetLastError();
      }
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t inplace_launch_guarded(int B, int T, int d_model, int d_ff, int C, float eta, float clip_tau,
                                  const int64_t* doc_starts, int n_docs, const void* z, const void* vhat,
                                  const float* w_init, float* w_down, void* o, void* ws, size_t ws_bytes,
                                  hipStream_t s) {
  const bool clip = clip_tau > 0.0f && clip_tau < INFINITY;
  const size_t clip_bytes = clip_area_bytes(d_model, d_ff);
  float* clip_ws = static_cast<float*>(ws);
  void* split_ws = ws_bytes > clip_bytes ? static_cast<char*>(ws) + clip_bytes : nullptr;
  const size_t split_bytes = ws_bytes > clip_bytes ? ws_bytes - clip_bytes : 0;
  // tile path: Wb and the partials after the clip area
  const bool tile = use_tile_path(T, d_model, d_ff, C, split_ws, split_bytes);
  bf16_t* wbuf = tile ? static_cast<bf16_t*>(split_ws) : nullptr;
  float* part = tile ? reinterpret_cast<float*>(static_cast<char*>(split_ws) + wb_bytes(d_model, d_ff)) : nullptr;
  const int64_t wsz = static_cast<int64_t>(d_model) * d_ff;
  int d = 0;  // next entry of doc_starts (sorted over b * T + t)
  for (int b = 0; b < B; ++b) {
    const bf16_t* zb = static_cast<const bf16_t*>(z) + static_cast<int64_t>(b) * T * d_ff;
    const bf16_t* vb = static_cast<const bf16_t*>(vhat) + static_cast<int64_t>(b) * T * d_model;
    bf16_t* ob = static_cast<bf16_t*>(o) + static_cast<int64_t>(b) * T * d_model;
    float* wb = w_down + b * wsz;
    const float* wib = w_init ? w_init + b * wsz : nullptr;
    if (tile) {
      hipError_t err = round_bf16(wb, wbuf, wsz, s);
      if (err != hipSuccess) return err;
    }
    int a = 0;  // first token of the current document
    bool reset = false;
    while (a < T) {
      int e = T;
      if (d < n_docs && doc_starts[d] < static_cast<int64_t>(b + 1) * T)
        e = static_cast<int>(doc_starts[d++] - static_cast<int64_t>(b) * T);
      for (int t0 = a; t0 < e; t0 += C) {
        const int c = (e - t0 < C) ? e - t0 : C;
        const bool restart = reset && t0 == a;
        const ChunkIO io{zb + static_cast<int64_t>(t0) * d_ff, vb + static_cast<int64_t>(t0) * d_model,
                         restart ? wib : wb, wb, ob + static_cast<int64_t>(t0) * d_model};
        hipError_t err = hipSuccess;
        if (tile) {
          const float* scale = nullptr;
          if (restart) err = round_bf16(wib, wbuf, wsz, s);  // the apply reads the restarted state
          if (err == hipSuccess && clip) err = clip_norm_tile(io, c, d_model, d_ff, eta, clip_tau, clip_ws, &scale, s);
          if (err == hipSuccess) err = tile_chunk_step(io, c, d_model, d_ff, eta, scale, wbuf, part, s);
        } else {
          err = chunk_step(io, c, d_model, d_ff, eta, clip, clip_tau, clip_ws, split_ws, split_bytes, s);
        }
        if (err != hipSuccess) return err;
      }
      a = e;
      reset = true;
    }
  }
  return hipSuccess;
}

}  // namespace ttt
