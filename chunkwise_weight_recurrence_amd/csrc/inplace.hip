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

#include <type_traits>

#include "ttt_device.h"
#include "ttt_internal.h"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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
  auto two = [](float x, float y) {
    return static_cast<uint32_t>(f32_to_bf16(x)) | (static_cast<uint32_t>(f32_to_bf16(y)) << 16);
  };
  return u32x4_t{two(a[0], a[1]), two(a[2], a[3]), two(b[0], b[1]), two(b[2], b[3])};
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
// ds_read_b64_tr_b16 (tr_frag), whose 16-lane groups name two adjacent granules
// in each of four consecutive k rows; the key 2 (k % 4) + (k / 4) % 2 puts those
// eight pieces in eight different bank groups (the key k % 8 put them in four,
// a two-way conflict on every read).  (Transposing into a [row][k] layout on the
// way in, one bf16 per LDS write, hit the same banks from most lanes of a wave
// and cost the update GEMM about three quarters of its time.)
template <int NCOL>
__device__ __forceinline__ int swzk(int k, int col) {
  return k * NCOL + (((col >> 3) ^ (((k & 3) << 1) | ((k >> 2) & 1))) << 3) + (col & 7);
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
  const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(acc.x)) | (static_cast<uint32_t>(f32_to_bf16(acc.y)) << 16);
  const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(acc.z)) | (static_cast<uint32_t>(f32_to_bf16(acc.w)) << 16);
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

}  // namespace

size_t inplace_workspace_bytes(int B, int T, int d_model, int d_ff, int C) {
  if (static_cast<int64_t>(B) * T == 0) return 0;
  const int c = T < C ? T : C;
  const int ks = apply_splits(c, d_model, d_ff);
  return ks > 1 ? static_cast<size_t>(ks) * c * d_model * sizeof(float) : 0;
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
    const size_t tiles = static_cast<size_t>(gu.x) * gu.y;
    float* sc = reinterpret_cast<float*>(reinterpret_cast<char*>(clip_ws) + align256(tiles * sizeof(float)));
    GemmArgs np{d_model, d_ff, c, io.v, io.z, clip_ws, d_model, d_ff, d_ff, 1.0f, c};
    KernelScope timing(TTT_KERNEL_INPLACE_NORM, s);
    hipLaunchKernelGGL((gemm_kernel<true, true, bf16_t, bf16_t, kEpiSumSqF32>), gu, dim3(kThreads), 0, s, np);
    hipLaunchKernelGGL(clip_scale_kernel, dim3(1), dim3(256), 0, s, static_cast<const float*>(clip_ws),
                       static_cast<int>(tiles), eta, tau, sc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    scale = sc;
  }
  GemmArgs up{d_model, d_ff, c, io.v, io.z, io.w_dst, d_model, d_ff, d_ff, eta, c, io.w_src, scale};
  {
    KernelScope timing(TTT_KERNEL_INPLACE_UPDATE, s);
    hipLaunchKernelGGL((gemm_kernel<true, true, bf16_t, bf16_t, kEpiAxpyF32>), gu, dim3(kThreads), 0, s, up);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

size_t inplace_guarded_workspace_bytes(int B, int T, int d_model, int d_ff, int C) {
  if (static_cast<int64_t>(B) * T == 0) return 0;
  return clip_area_bytes(d_model, d_ff) + inplace_workspace_bytes(B, T, d_model, d_ff, C);
}

hipError_t inplace_launch(int B, int T, int d_model, int d_ff, int C, float eta, const void* z,
                          const void* vhat, float* w_down, void* o, void* ws, size_t ws_bytes, hipStream_t s) {
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
  const int ks = apply_splits(c, d_model, d_ff);
  return align256(static_cast<size_t>(d_model) * d_ff * 4) + align256(static_cast<size_t>(2) * c * d_ff * 4) +
         (ks > 1 ? align256(static_cast<size_t>(ks) * c * d_model * 4) : 0);
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
  int d = 0;  // next entry of doc_starts (sorted over b * T + t)
  for (int b = 0; b < B; ++b) {
    const bf16_t* zb = static_cast<const bf16_t*>(z) + static_cast<int64_t>(b) * T * d_ff;
    const bf16_t* vb = static_cast<const bf16_t*>(vhat) + static_cast<int64_t>(b) * T * d_model;
    bf16_t* ob = static_cast<bf16_t*>(o) + static_cast<int64_t>(b) * T * d_model;
    float* wb = w_down + static_cast<int64_t>(b) * d_model * d_ff;
    const float* wib = w_init ? w_init + static_cast<int64_t>(b) * d_model * d_ff : nullptr;
    int a = 0;  // first token of the current document
    bool reset = false;
    while (a < T) {
      int e = T;
      if (d < n_docs && doc_starts[d] < static_cast<int64_t>(b + 1) * T)
        e = static_cast<int>(doc_starts[d++] - static_cast<int64_t>(b) * T);
      for (int t0 = a; t0 < e; t0 += C) {
        const int c = (e - t0 < C) ? e - t0 : C;
        const ChunkIO io{zb + static_cast<int64_t>(t0) * d_ff, vb + static_cast<int64_t>(t0) * d_model,
                         (reset && t0 == a) ? wib : wb, wb, ob + static_cast<int64_t>(t0) * d_model};
        hipError_t err = chunk_step(io, c, d_model, d_ff, eta, clip, clip_tau, clip_ws, split_ws, split_bytes, s);
        if (err != hipSuccess) return err;
      }
      a = e;
      reset = true;
    }
  }
  return hipSuccess;
}

}  // namespace ttt
