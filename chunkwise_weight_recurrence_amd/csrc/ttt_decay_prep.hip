// Vector-decay preparation for the matrix-core kernels (gfx950).
//
// Modular TTT summary page, "Prerequisites" (weight decay): with a per-token,
// per-feature decay a_t, the chunk's dual form scales queries and keys by the
// decay accumulated inside the chunk.  For chunk i and feature d, with L the
// inclusive cumulative sum of log a over the chunk's tokens:
//   Q~ = Q e^{L},  K~ = K e^{-L},  lambda = e^{L_last}
// (K_bar = K~ lambda and the state transition W <- lambda (.) (W - K~^T G~)
// follow from these).  These depend on the inputs only, not on the state, so
// they are formed once per (chain, chunk) here, fully in parallel, instead of in
// every column-block workgroup of the sequential kernels.
//
// Outputs (the caller's workspace):
//   qt, kt [B,H,T,dk] bf16            Q~, K~ rounded to bf16 (the MFMA operands)
//   lam    [B,H,NC,dk] f32            e^{L_last} of each chunk
//   lpre   [B,H,NC,C/32,dk] f32       L just before each 32-token tile of the
//                                     chunk (0 for the first tile; L_last for
//                                     tiles past the end of a short last chunk)
//
// Work split: one workgroup per (chain, chunk) of (d_k / 8) x 32 threads; thread =
// (group of 8 features, segment of C/32 consecutive tokens).  A thread loads
// its segment's log a once, all loads issued together, and keeps it in
// registers; segment totals are combined through LDS; then q and k are read,
// scaled and written back as bf16 rows (16-byte accesses; the threads of a
// wave cover whole rows).

#include "ttt_device.h"
#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr int kPrepSeg = 32;     // token segments per chunk
constexpr int kPrepSegMax = 8;   // tokens per segment at C = 256

__device__ __forceinline__ void bf16x8_unpack(uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 bf16x8_pack(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = static_cast<uint32_t>(f32_to_bf16(f[2 * j])) | (static_cast<uint32_t>(f32_to_bf16(f[2 * j + 1])) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int DK>
__global__ __launch_bounds__(DK / 8 * kPrepSeg) void decay_prep_kernel(const float* __restrict__ la,
                                                                   const bf16_t* __restrict__ q,
                                                                   const bf16_t* __restrict__ k, DecayPrep out,
                                                                   int T, int C, int NC) {
  constexpr int NG = DK / 8;                 // feature groups of 8
  constexpr int NSEG = kPrepSeg;
  __shared__ float segtot[NSEG][DK];

  const int tid = threadIdx.x;
  const int g = tid % NG, sg = tid / NG;
  const int ci = blockIdx.x % NC;
  const int64_t bh = blockIdx.x / NC;
  const int t0 = ci * C;
  const int c = min(C, T - t0);
  const int seglen = C / NSEG;               // C in {32, 64, 128, 256}: 1..8 tokens
  const int s0 = sg * seglen;
  const int64_t row0 = bh * T + t0;
  const float* lap = la + row0 * DK + 8 * g;

  // log a of this thread's tokens (rows >= c read as zero, addresses clamped)
  float x[kPrepSegMax][8];
#pragma unroll
  for (int u = 0; u < kPrepSegMax; ++u) {
    const int t = s0 + u;
    const bool ok = u < seglen && t < c;
    const float* p = lap + static_cast<int64_t>(ok ? t : 0) * DK;
    const float4 a0 = *reinterpret_cast<const float4*>(p);
    const float4 a1 = *reinterpret_cast<const float4*>(p + 4);
    x[u][0] = ok ? a0.x : 0.0f; x[u][1] = ok ? a0.y : 0.0f; x[u][2] = ok ? a0.z : 0.0f; x[u][3] = ok ? a0.w : 0.0f;
    x[u][4] = ok ? a1.x : 0.0f; x[u][5] = ok ? a1.y : 0.0f; x[u][6] = ok ? a1.z : 0.0f; x[u][7] = ok ? a1.w : 0.0f;
  }
  float run[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kPrepSegMax; ++u) s += x[u][j];
    segtot[sg][8 * g + j] = s;
    run[j] = 0.0f;
  }
  __syncthreads();
  for (int s = 0; s < sg; ++s) {
#pragma unroll
    for (int j = 0; j < 8; ++j) run[j] += segtot[s][8 * g + j];
  }

  // scaled rows and the tile prefixes
  const int ntile = C / 32;
  float* lpre = out.lpre + ((bh * NC + ci) * ntile) * DK + 8 * g;
  const bf16_t* qp = q + row0 * DK + 8 * g;
  const bf16_t* kp = k + row0 * DK + 8 * g;
  bf16_t* qtp = out.qt + row0 * DK + 8 * g;
  bf16_t* ktp = out.kt + row0 * DK + 8 * g;
  constexpr int UB = 4;  // rows per batch of q / k loads
#pragma unroll
  for (int u0 = 0; u0 < kPrepSegMax; u0 += UB) {
    uint4 qq[UB], kk[UB];
#pragma unroll
    for (int u = u0; u < u0 + UB; ++u) {
      const int t = s0 + u;
      const bool ok = u < seglen && t < c;
      const int64_t o = static_cast<int64_t>(ok ? t : 0) * DK;
      qq[u - u0] = *reinterpret_cast<const uint4*>(qp + o);
      kk[u - u0] = *reinterpret_cast<const uint4*>(kp + o);
    }
#pragma unroll
    for (int u = u0; u < u0 + UB; ++u) {
      const int t = s0 + u;
      if (u < seglen && t < c) {
        if ((t & 31) == 0) {  // L before this tile
#pragma unroll
          for (int j = 0; j < 8; ++j) lpre[(t >> 5) * DK + j] = run[j];
        }
        float qf[8], kf[8], qo[8], ko[8];
        bf16x8_unpack(qq[u - u0], qf);
        bf16x8_unpack(kk[u - u0], kf);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          run[j] += x[u][j];
          qo[j] = qf[j] * __expf(run[j]);
          ko[j] = kf[j] * __expf(-run[j]);
        }
        const int64_t o = static_cast<int64_t>(t) * DK;
        *reinterpret_cast<uint4*>(qtp + o) = bf16x8_pack(qo);
        *reinterpret_cast<uint4*>(ktp + o) = bf16x8_pack(ko);
      }
    }
  }
  // The last segment ends with L_last (a segment past the chunk's end holds the
  // prefix of all earlier ones, which is then L_last too).
  if (sg == NSEG - 1) {
    float* lam = out.lam + (bh * NC + ci) * DK + 8 * g;
#pragma unroll
    for (int j = 0; j < 8; ++j) lam[j] = __expf(run[j]);
    for (int X = (c + 31) / 32; X < ntile; ++X) {
#pragma unroll
      for (int j = 0; j < 8; ++j) lpre[X * DK + j] = run[j];
    }
  }
}

}  // namespace

size_t decay_prep_layout(int B, int H, int T, int dk, int C, int NC, DecayPrep* p, char* base) {
  const size_t BH = static_cast<size_t>(B) * H;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return base ? base + o : nullptr;
  };
  char* a = take(BH * T * dk * 2);
  char* b = take(BH * T * dk * 2);
  char* c = take(BH * NC * dk * 4);
  char* d = take(BH * NC * (C / 32) * dk * 4);
  if (p) {
    p->qt = reinterpret_cast<bf16_t*>(a);
    p->kt = reinterpret_cast<bf16_t*>(b);
    p->lam = reinterpret_cast<float*>(c);
    p->lpre = reinterpret_cast<float*>(d);
  }
  return off;
}

hipError_t decay_prep_launch(const float* la, const void* q, const void* k, int B, int H, int T, int dk, int C,
                             int NC, const DecayPrep& p, hipStream_t s) {
  const int64_t nblk = static_cast<int64_t>(B) * H * NC;
  if (nblk == 0) return hipSuccess;
  KernelScope timing(TTT_KERNEL_DECAY_PREP, s);
  const auto* qb = static_cast<const bf16_t*>(q);
  const auto* kb = static_cast<const bf16_t*>(k);
  if (dk == 128)
    hipLaunchKernelGGL(decay_prep_kernel<128>, dim3(static_cast<unsigned>(nblk)), dim3(128 / 8 * kPrepSeg), 0, s, la,
                       qb, kb, p, T, C, NC);
  else
    hipLaunchKernelGGL(decay_prep_kernel<64>, dim3(static_cast<unsigned>(nblk)), dim3(64 / 8 * kPrepSeg), 0, s, la,
                       qb, kb, p, T, C, NC);
  return hipGetLastError();
}

}  // namespace ttt
