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
// not contiguous in memory (V_hat^T and Z in the update) are transposed while
// being staged into LDS.

#include "ttt_device.h"
#include "ttt_internal.h"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 32;          // k per LDS stage (two k16 MFMA steps)
constexpr int kPad = 8;          // bf16 elements of row padding in LDS
constexpr int kLdsRow = kBK + kPad;
constexpr int kThreads = 256;    // 4 waves, 2 x 2 over the output tile

// Epilogues.
constexpr int kEpiStoreBf16 = 0;  // C[m][n] = bf16(acc)
constexpr int kEpiAxpyF32 = 1;    // C[m][n] += alpha * acc (fp32)

struct GemmArgs {
  int M, N, K;
  const void* A;   // A(m, k): A_T ? A[k*lda + m] : A[m*lda + k]
  const void* Bm;  // B(k, n): B_T ? B[k*ldb + n] : B[n*ldb + k]
  void* Cm;        // C[m*ldc + n]
  int64_t lda, ldb, ldc;
  float alpha;
};

template <typename X> __device__ __forceinline__ void load8(const X* p, float (&f)[8]);
template <> __device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float (&f)[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float (&f)[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Stage one BROWS x kBK operand tile into LDS as [row][k] bf16.
//   TRANS = false: global is row-major in k (8 consecutive k per thread load)
//   TRANS = true : global is row-major in the row index (8 consecutive rows per load)
template <int BROWS, bool TRANS, typename X>
struct Stager {
  static constexpr int kLoads = BROWS * kBK / 8 / kThreads;  // 8-element loads per thread
  float buf[kLoads][8];

  __device__ __forceinline__ void fetch(const X* g, int64_t ld, int row0, int nrows, int k0, int K) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      int idx = threadIdx.x + i * kThreads;
      int r, kk;
      if (!TRANS) { r = idx / (kBK / 8); kk = (idx % (kBK / 8)) * 8; }
      else { kk = idx / (BROWS / 8); r = (idx % (BROWS / 8)) * 8; }
      int gr = row0 + r, gk = k0 + kk;
      bool ok = !TRANS ? (gr < nrows && gk < K) : (gk < K && gr < nrows);
      if (ok) {
        const X* p = !TRANS ? g + static_cast<int64_t>(gr) * ld + gk : g + static_cast<int64_t>(gk) * ld + gr;
        load8<X>(p, buf[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) buf[i][j] = 0.0f;
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      int idx = threadIdx.x + i * kThreads;
      if (!TRANS) {
        int r = idx / (kBK / 8), kk = (idx % (kBK / 8)) * 8;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = static_cast<uint32_t>(f32_to_bf16(buf[i][2 * j])) |
                 (static_cast<uint32_t>(f32_to_bf16(buf[i][2 * j + 1])) << 16);
        *reinterpret_cast<uint4*>(lds + r * kLdsRow + kk) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        int kk = idx / (BROWS / 8), r = (idx % (BROWS / 8)) * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) lds[(r + j) * kLdsRow + kk] = f32_to_bf16(buf[i][j]);
      }
    }
  }
};

// Output tile BM x BN per workgroup; each of the 4 waves owns (BM/2) x (BN/2)
// as (BM/64) x (BN/64) MFMA tiles of 32 x 32.
template <int BM, int BN, bool A_T, bool B_T, typename AX, typename BX, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[BN * kLdsRow];
  constexpr int TM = BM / 64, TN = BN / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int l32 = lane & 31, hi = lane >> 5;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  Stager<BM, A_T, AX> sa;
  Stager<BN, B_T, BX> sb;  // B(k, n): B_T means n is contiguous, i.e. transposed staging
  const AX* Ag = static_cast<const AX*>(g.A);
  const BX* Bg = static_cast<const BX*>(g.Bm);
  sa.fetch(Ag, g.lda, m0, g.M, 0, g.K);
  sb.fetch(Bg, g.ldb, n0, g.N, 0, g.K);
  for (int k0 = 0; k0 < g.K; k0 += kBK) {
    __syncthreads();
    sa.store(As);
    sb.store(Bs);
    __syncthreads();
    if (k0 + kBK < g.K) {
      sa.fetch(Ag, g.lda, m0, g.M, k0 + kBK, g.K);
      sb.fetch(Bg, g.ldb, n0, g.N, k0 + kBK, g.K);
    }
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * (BM / 2) + i * 32 + l32) * kLdsRow + ks + hi * 8);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * (BN / 2) + j * 32 + l32) * kLdsRow + ks + hi * 8);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  // 32x32 MFMA output layout: lane (n = l32, hi) holds rows 8*(r/4) + 4*hi + (r%4).
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int n = n0 + wn * (BN / 2) + j * 32 + l32;
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int m = m0 + wm * (BM / 2) + i * 32 + 8 * (r / 4) + 4 * hi + (r % 4);
        if (m >= g.M) continue;
        int64_t off = static_cast<int64_t>(m) * g.ldc + n;
        if constexpr (EPI == kEpiStoreBf16) {
          static_cast<bf16_t*>(g.Cm)[off] = f32_to_bf16(acc[i][j][r]);
        } else {
          float* c = static_cast<float*>(g.Cm);
          c[off] = c[off] + g.alpha * acc[i][j][r];
        }
      }
    }
}

}  // namespace

hipError_t inplace_launch(int B, int T, int d_model, int d_ff, int C, float eta, const void* z,
                          const void* vhat, float* w_down, void* o, hipStream_t s) {
  constexpr int AM = 64, AN = 128;    // apply tile: tokens x d_model
  constexpr int UM = 128, UN = 128;   // update tile: d_model x d_ff
  for (int b = 0; b < B; ++b) {
    const bf16_t* zb = static_cast<const bf16_t*>(z) + static_cast<int64_t>(b) * T * d_ff;
    const bf16_t* vb = static_cast<const bf16_t*>(vhat) + static_cast<int64_t>(b) * T * d_model;
    bf16_t* ob = static_cast<bf16_t*>(o) + static_cast<int64_t>(b) * T * d_model;
    float* wb = w_down + static_cast<int64_t>(b) * d_model * d_ff;
    for (int t0 = 0; t0 < T; t0 += C) {
      int c = (T - t0 < C) ? T - t0 : C;
      GemmArgs ap{c, d_model, d_ff, zb + static_cast<int64_t>(t0) * d_ff, wb, ob + static_cast<int64_t>(t0) * d_model,
                  d_ff, d_ff, d_model, 1.0f};
      dim3 ga((d_model + AN - 1) / AN, (c + AM - 1) / AM);
      hipError_t e;
      {
        KernelScope timing(TTT_KERNEL_INPLACE_APPLY, s);
        hipLaunchKernelGGL((gemm_kernel<AM, AN, false, false, bf16_t, float, kEpiStoreBf16>), ga, dim3(kThreads),
                           0, s, ap);
        e = hipGetLastError();
      }
      if (e != hipSuccess) return e;
      GemmArgs up{d_model, d_ff, c, vb + static_cast<int64_t>(t0) * d_model, zb + static_cast<int64_t>(t0) * d_ff,
                  wb, d_model, d_ff, d_ff, eta};
      dim3 gu((d_ff + UN - 1) / UN, (d_model + UM - 1) / UM);
      {
        KernelScope timing(TTT_KERNEL_INPLACE_UPDATE, s);
        hipLaunchKernelGGL((gemm_kernel<UM, UN, true, true, bf16_t, bf16_t, kEpiAxpyF32>), gu, dim3(kThreads), 0,
                           s, up);
        e = hipGetLastError();
      }
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace ttt
