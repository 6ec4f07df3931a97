// Chunkwise backward of the Muir gated delta rule (gfx950).
//
// The pages (arXiv 2611.08376, Methodology and fig:kernel) say only that a
// custom backward pass is used.  This file is the adjoint of the chunkwise
// forward in fwd.hip, in two parts.
//
// 1. bwd_scan walks the chunks of one (b, h) in reverse and carries the
//    gradient of the state.  With the chunk summary (W, Q', Kbar, Gamma_C)
//    the forward update S_next = diag(Gamma_C) S + Kbar^T (U~ - W S),
//    o = O~ + Q' S has the adjoint
//        dS = diag(Gamma_C) dS_next + Q'^T dO - W^T (Kbar dS_next).
//    It stores dS_next for every chunk (the gradient at the chunk's end).
//
// 2. bwd_chunk, one workgroup per chunk, gets the chunk's initial state S0
//    and end gradient dS_C and forms every input gradient with three sweeps
//    over the chunk's 16-token blocks (boundary pivots as in the forward):
//      F1 (forward): deltas Delta_I = T_II (U_I - X_I S_I) and the state S_I
//         at each block boundary;  d(qt)_r = S_r dO_r   (S_r: state after r)
//      R  (reverse): the state gradient D at block boundaries, pivoted at
//         B_{J+1}; dR_J = T_JJ^T (Ke_J D + P_JJ^T dO_J)  (gradient of the
//         deltas' right-hand side, i.e. of write*v);  d(k)_i = E_i Delta_i
//         with E_i the state gradient at token i;  then
//         D <- diag(exp(B_{J+1} - B_J)) D + Y_J^T dO_J - X_J^T dR_J
//      F2 (forward): d(ek)_r = -S'_r dR_r  (S'_r: decayed state before r's write)
//    and finally, with ek = erase*k and qt = gamma*q,
//      dLam_r = ek_r * d(ek)_r + qt_r * d(qt)_r - k_r * d(k)_r
//               (+ rowsum(S_C * dS_C) on the chunk's last token)
//      dlog_a_i = sum_{r >= i in the chunk} dLam_r
//      derase = k * d(ek), dk = d(k) + erase * d(ek), dq = gamma * d(qt),
//      dgamma = q * d(qt), dv = write * dR, dwrite = v * dR.
//    Each per-token product splits into a boundary part (a tile product with
//    S_I, D or the deltas, times a factor exp(.) <= 1) and a 16 x 16 leaf part
//    formed from per-pair factors exp(Lam_r - Lam_i), r >= i.
#include "chunk_common.h"
#include "kernels.h"
#include "mma.h"

namespace muir {

namespace {

constexpr int BSCAN_SB = 64;

// Summary layout written by the prep kernel for the backward:
//   W [DK][C], Qp [DK][C], Kb [C][DK] (compute type), gC [DK] fp32 at the end.
template <typename Tin, int DK, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_scan_kernel(
    int T, int H, int C, const char* __restrict__ summ, size_t summ_bytes,
    const Tin* __restrict__ dO, const float* __restrict__ dS_T, float* __restrict__ dS_chunks,
    float* __restrict__ dS0) {
  typedef Tin TC;
  typedef MM<TC> M;
  typedef typename M::frag frag;
  constexpr int DV = DK;
  constexpr int RT = DK / 16;
  constexpr int NV = 16 * NW;
  constexpr int PK = BSCAN_SB + 4;
  constexpr int PW = DK + 4;

  const int NC = T / C;
  const int nvb = DV / NV;
  const int bh = blockIdx.x / nvb;
  const int vb = blockIdx.x - bh * nvb;
  const int b = bh / H;
  const int h = bh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int colg = vb * NV + 16 * wave + c16;

  __shared__ __attribute__((aligned(16))) TC sWt[DK][PK];
  __shared__ __attribute__((aligned(16))) TC sQt[DK][PK];
  __shared__ __attribute__((aligned(16))) TC sKr[BSCAN_SB][PW];
  __shared__ float sgC[DK];

  const size_t sbase = static_cast<size_t>(bh) * DK * DV;
  f32x4 dS[RT];
#pragma unroll
  for (int s = 0; s < RT; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dS[s][i] = dS_T ? dS_T[sbase + static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] : 0.f;

  for (int c = NC - 1; c >= 0; --c) {
    const char* base = summ + (static_cast<size_t>(bh) * NC + c) * summ_bytes;
    const TC* Wt = reinterpret_cast<const TC*>(base);
    const TC* Qt = Wt + static_cast<size_t>(C) * DK;
    const TC* Kb = Qt + static_cast<size_t>(C) * DK;
    const float* gC = reinterpret_cast<const float*>(Kb + static_cast<size_t>(C) * (DK + 2 * DV));
    {
      float* dst = dS_chunks + (static_cast<size_t>(bh) * NC + c) * DK * DV;
#pragma unroll
      for (int s = 0; s < RT; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] = dS[s][i];
    }
    frag dSf[RT];
#pragma unroll
    for (int s = 0; s < RT; ++s) dSf[s] = M::from_f32(dS[s]);
    f32x4 Z[RT];
#pragma unroll
    for (int s = 0; s < RT; ++s) Z[s] = zero4();

    for (int sb = 0; sb < C; sb += BSCAN_SB) {
      __syncthreads();
      for (int idx = tid; idx < DK * BSCAN_SB / 4; idx += 64 * NW) {
        const int j = idx / (BSCAN_SB / 4);
        const int r4 = (idx - j * (BSCAN_SB / 4)) * 4;
        const f32x4 wv = load4(Wt + static_cast<size_t>(j) * C + sb + r4);
        const f32x4 qv = load4(Qt + static_cast<size_t>(j) * C + sb + r4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sWt[j][r4 + i] = M::cvt(wv[i]);
          sQt[j][r4 + i] = M::cvt(qv[i]);
        }
      }
      for (int idx = tid; idx < BSCAN_SB * DK / 4; idx += 64 * NW) {
        const int r = idx / (DK / 4);
        const int j4 = (idx - r * (DK / 4)) * 4;
        const f32x4 kv = load4(Kb + static_cast<size_t>(sb + r) * DK + j4);
#pragma unroll
        for (int i = 0; i < 4; ++i) sKr[r][j4 + i] = M::cvt(kv[i]);
      }
      if (sb == 0)
        for (int j = tid; j < DK; j += 64 * NW) sgC[j] = gC[j];
      __syncthreads();
#pragma unroll 1
      for (int m = 0; m < BSCAN_SB / 16; ++m) {
        // X = Kbar_m dS_next  (16 tokens x this wave's 16 columns)
        f32x4 X = zero4();
#pragma unroll
        for (int s = 0; s < RT; ++s) X = M::mma(M::load(&sKr[16 * m + c16][16 * s + 4 * g]), dSf[s], X);
        f32x4 dov;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = c * C + sb + 16 * m + 4 * g + i;
          dov[i] = Elem<Tin>::load(dO, ((static_cast<size_t>(b) * T + t) * H + h) * DV + colg);
        }
        const frag dof = M::from_f32(dov);
        const frag xf = M::from_f32(-X);
#pragma unroll
        for (int s = 0; s < RT; ++s) {
          Z[s] = M::mma(M::load(&sQt[16 * s + c16][16 * m + 4 * g]), dof, Z[s]);
          Z[s] = M::mma(M::load(&sWt[16 * s + c16][16 * m + 4 * g]), xf, Z[s]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) dS[s][i] = sgC[16 * s + 4 * g + i] * dS[s][i] + Z[s][i];
  }
  if (dS0) {
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) dS0[sbase + static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] = dS[s][i];
  }
}

}  // namespace

hipError_t launch_bwd_scan(const ChunkShape& s, const void* summ, const void* dO, const float* dS_T,
                           float* dS_chunks, float* dS0, hipStream_t stream) {
  const int heads = s.B * s.H;
  if (heads == 0) return hipSuccess;
  const bool wide = static_cast<long long>(heads) * (s.DV / 64) >= 256;
#define MUIR_BSCAN(TT, DD, NW)                                                                     \
  hipLaunchKernelGGL((bwd_scan_kernel<TT, DD, NW>), dim3(heads * (s.DV / (16 * NW))),              \
                     dim3(64 * NW), 0, stream, s.T, s.H, s.C, (const char*)summ, s.summary_bytes(), \
                     (const TT*)dO, dS_T, dS_chunks, dS0)
  if (s.bf16) {
    if (s.DK == 128) {
      if (wide) MUIR_BSCAN(uint16_t, 128, 4); else MUIR_BSCAN(uint16_t, 128, 1);
    } else {
      if (wide) MUIR_BSCAN(uint16_t, 64, 4); else MUIR_BSCAN(uint16_t, 64, 1);
    }
  } else {
    if (s.DK == 128) {
      if (wide) MUIR_BSCAN(float, 128, 4); else MUIR_BSCAN(float, 128, 1);
    } else {
      if (wide) MUIR_BSCAN(float, 64, 4); else MUIR_BSCAN(float, 64, 1);
    }
  }
#undef MUIR_BSCAN
  return hipGetLastError();
}

}  // namespace muir
