// Vector-decay preparation for the matrix-core kernels (gfx950).
//
// Modular TTT summary page, "Prerequisites" (weight decay): with a per-token,
// per-feature decay a_t, query t of a chunk sees key s <= t through the factor
// exp(L_t - L_s), L the inclusive cumulative sum of log a over the chunk's
// tokens (the decay accumulated between the two tokens).  The kernels split
// that factor at 32-token tiles so that every number they form stays in range
// whatever the decay: for tile I with P_I = L just before the tile and
// P_{I+1} = L at its last token, the reference M_I = (P_I + P_{I+1}) / 2 is the
// midpoint of the tile's range of L, and
//   Q^m_t = Q_t e^{L_t - M_I},  K^m_s = K_s e^{M_I - L_s}    (t, s in tile I)
// grow by at most e^{(P_I - P_{I+1}) / 2}, half the tile's own decay.  Pairs
// inside one tile multiply Q^m K^m directly; across tiles the kernels carry
// tile-start states scaled by factors e^{M_I - M_J} <= 1 formed from the
// prefixes below.  These depend on the inputs only, so they are formed once
// per (chain, chunk) here, fully in parallel.
//
// Outputs (the caller's workspace or the forward's saved context):
//   qt, kt [B,H,T,dk] bf16               Q^m, K^m rounded to bf16 (MFMA operands)
//   lam    [B,H,NC,dk] f32               e^{L_last} of each chunk
//   lpre   [B,H,NC,C/32+1,dk] f32        P_0 = 0, P_1, ..., P_{C/32} = L_last: L
//                                        before each 32-token tile and after the
//                                        last (tiles past the end of a short
//                                        last chunk hold L_last)
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
    w[j] = pack_bf16x2(f[2 * j], f[2 * j + 1]);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int DK>
__global__ __launch_bounds__(DK / 8 * kPrepSeg) void decay_prep_kernel(const float* __restrict__ la,
                                                                   const bf16_t* __restrict__ q,
                                                                   const bf16_t* __restrict__ k, DecayPrep out,
                                                                   int T, int C, int NC) {
  constexpr int NG = DK / 8;                 // feature groups of 8
  constexpr int NSEG = kPrepSeg;
  __shared__ __attribute__((aligned(16))) float segtot[NSEG][DK];

  const int tid = threadIdx.x;
  const int g = tid % NG, sg = tid / NG;
  const int ci = blockIdx.x % NC;
  const int64_t bh = blockIdx.x / NC;
  const int t0 = ci * C;
  const int c = min(C, T - t0);
  const int seglen = C / NSEG;               // C in {32, 64, 128, 256}: 1..8 tokens
  const int spt = NSEG * 32 / C;             // segments per 32-token tile
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
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kPrepSegMax; ++u) s += x[u][j];
    segtot[sg][8 * g + j] = s;
  }
  __syncthreads();
  // in-tile run at the segment start (relative to P_I), half the tile's total
  // decay, and the prefixes P_I (before the tile) and L_last
  const int I = sg / spt;
  const int sfirst = I * spt;
  // (three runs over the segment totals: before the tile, inside it up to this
  // segment, and to the tile's end; the thread of the last segment ends with L_last)
  float pI[8], inrun[8], half[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { pI[j] = 0.0f; inrun[j] = 0.0f; half[j] = 0.0f; }
  for (int s = 0; s < sfirst; ++s) {
    const float4 a0 = *reinterpret_cast<const float4*>(&segtot[s][8 * g]);
    const float4 a1 = *reinterpret_cast<const float4*>(&segtot[s][8 * g + 4]);
    pI[0] += a0.x; pI[1] += a0.y; pI[2] += a0.z; pI[3] += a0.w;
    pI[4] += a1.x; pI[5] += a1.y; pI[6] += a1.z; pI[7] += a1.w;
  }
  for (int s = sfirst; s < sfirst + spt; ++s) {
    const float4 a0 = *reinterpret_cast<const float4*>(&segtot[s][8 * g]);
    const float4 a1 = *reinterpret_cast<const float4*>(&segtot[s][8 * g + 4]);
    const float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      half[j] += v[j];
      if (s < sg) inrun[j] += v[j];
    }
  }
  float last[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    last[j] = pI[j] + half[j];  // L at the tile's end (L_last for the last tile)
    half[j] *= 0.5f;
  }

  const int ntile = C / 32;
  float* lpre = out.lpre + ((bh * NC + ci) * (ntile + 1)) * DK + 8 * g;
  if (sg == sfirst) {
#pragma unroll
    for (int j = 0; j < 8; ++j) lpre[I * DK + j] = pI[j];
  }
  if (sg == NSEG - 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) lpre[ntile * DK + j] = last[j];
    float* lam = out.lam + (bh * NC + ci) * DK + 8 * g;
#pragma unroll
    for (int j = 0; j < 8; ++j) lam[j] = __expf(last[j]);
  }

  // scaled rows: e = L_t - M_I = (in-tile inclusive run) - half
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
        float qf[8], kf[8], qo[8], ko[8];
        bf16x8_unpack(qq[u - u0], qf);
        bf16x8_unpack(kk[u - u0], kf);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          inrun[j] += x[u][j];
          const float e = inrun[j] - half[j];
          qo[j] = qf[j] * __expf(e);
          ko[j] = kf[j] * __expf(-e);
        }
        const int64_t o = static_cast<int64_t>(t) * DK;
        *reinterpret_cast<uint4*>(qtp + o) = bf16x8_pack(qo);
        *reinterpret_cast<uint4*>(ktp + o) = bf16x8_pack(ko);
      }
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
  char* d = take(BH * NC * (C / 32 + 1) * dk * 4);
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
