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

constexpr int BCH_THREADS = 256;

template <typename Tin, int DK>
__global__ __launch_bounds__(BCH_THREADS) void bwd_chunk_kernel(
    int T, int H, int C, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ log_a, const Tin* __restrict__ erase,
    const Tin* __restrict__ write, const Tin* __restrict__ gamma,
    const float* __restrict__ S_chunks, const float* __restrict__ dS_chunks,
    const Tin* __restrict__ dO, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dlog_a, float* __restrict__ derase,
    float* __restrict__ dwrite, float* __restrict__ dgamma, float* __restrict__ scratch) {
  typedef Tin TC;
  typedef MM<TC> M;
  typedef typename M::frag frag;
  constexpr int DV = DK;
  constexpr int RT = DK / 16;          // row tiles of a state
  constexpr int CWv = DV / 4;          // state columns per wave
  constexpr int NTv = CWv / 16;
  constexpr int CWk = DK / 4;          // gradient channels per wave
  constexpr int NTk = CWk / 16;
  constexpr int SPLIT = (sizeof(TC) == 4 && DK == 128) ? 2 : 1;  // staged state in column passes
  constexpr int SW = DV / SPLIT;       // staged columns per pass
  constexpr int PAD = DK + 1;
  constexpr int PT = DK + 4;
  constexpr int PS = SW + 4;

  const int NC = T / C;
  const int NB = C / 16;
  const int chunk = blockIdx.x;
  const int bh = chunk / NC;
  const int c = chunk - bh * NC;
  const int b = bh / H;
  const int h = bh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;

  const size_t rowbase = (static_cast<size_t>(b) * T + static_cast<size_t>(c) * C) * H + h;
  auto gidx = [&](int t, int j) -> size_t { return (rowbase + static_cast<size_t>(t) * H) * DK + j; };
  float* gDel = scratch + static_cast<size_t>(chunk) * 2 * C * DV;  // deltas [C][DV]
  float* gdR = gDel + static_cast<size_t>(C) * DV;                  // their gradients [C][DV]
  const float* S0c = S_chunks + static_cast<size_t>(chunk) * DK * DV;
  const float* dSC = dS_chunks + static_cast<size_t>(chunk) * DK * DV;

  __shared__ __attribute__((aligned(16))) float sB[17][DK];
  __shared__ float sL[16][PAD];
  __shared__ float sEK[16][PAD];
  __shared__ float sQT[16][PAD];
  __shared__ float sK[16][PAD];
  __shared__ __attribute__((aligned(16))) TC sRowOp[16][PT];   // X rows (F1) / Ke rows (R)
  __shared__ __attribute__((aligned(16))) TC sColOp[DK][20];   // Ke^T (F1, F2) / X^T (R)
  __shared__ __attribute__((aligned(16))) TC sYt[DK][20];      // Y^T (R)
  __shared__ float sU[DV][17];                                 // (write*v)^T (F1)
  __shared__ float sWa[16][17];
  __shared__ float sWt[16][17];
  __shared__ __attribute__((aligned(16))) TC sT[16][20];
  __shared__ __attribute__((aligned(16))) TC sP[16][20];
  __shared__ __attribute__((aligned(16))) TC sSD[DK][PS];      // staged S or D, [dk][dv]
  __shared__ float sLf[2][16][17];                             // leaf gradient matrices
  __shared__ float sG[DK];
  __shared__ float sRow[4][DK];
  __shared__ float sTot[DK];

  // ---- block boundaries of the cumulative log-decay ----
  if (tid < DK) {
    float L = 0.f;
    sB[0][tid] = 0.f;
    for (int t = 0; t < C; ++t) {
      L += Elem<Tin>::load(log_a, gidx(t, tid));
      if ((t & 15) == 15) sB[(t >> 4) + 1][tid] = L;
    }
  }
  __syncthreads();

  // Per-block tiles.  mode 0: F1 (X rows, Ke^T, U^T);  mode 1: R (Ke rows, X^T, Y^T);
  // mode 2: F2 (Ke^T).  Always: Lam, ek, qt, k of the block and exp(B_{I+1} - B_I).
  auto stage = [&](int I, int mode) {
    const int r0 = 16 * I;
    if (tid < DK) {
      float L = sB[I][tid];
#pragma unroll 4
      for (int r = 0; r < 16; ++r) {
        L += Elem<Tin>::load(log_a, gidx(r0 + r, tid));
        sL[r][tid] = L;
      }
      sG[tid] = __expf(sB[I + 1][tid] - sB[I][tid]);
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * DK; idx += BCH_THREADS) {
      const int r = idx / DK;
      const int j = idx - r * DK;
      const size_t gi = gidx(r0 + r, j);
      const float kj = Elem<Tin>::load(k, gi);
      const float ek = Elem<Tin>::load(erase, gi) * kj;
      const float qt = Elem<Tin>::load(gamma, gi) * Elem<Tin>::load(q, gi);
      const float L = sL[r][j];
      sEK[r][j] = ek;
      sQT[r][j] = qt;
      sK[r][j] = kj;
      const float fs = __expf(L - sB[I][j]);      // exp(Lam_r - B_I)
      const float fe = __expf(sB[I + 1][j] - L);  // exp(B_{I+1} - Lam_r)
      if (mode == 0) {
        sRowOp[r][j] = M::cvt(ek * fs);
        sColOp[j][r] = M::cvt(kj * fe);
        sU[j][r] = Elem<Tin>::load(write, gi) * Elem<Tin>::load(v, gi);
      } else if (mode == 1) {
        sRowOp[r][j] = M::cvt(kj * fe);
        sColOp[j][r] = M::cvt(ek * fs);
        sYt[j][r] = M::cvt(qt * fs);
      } else {
        sColOp[j][r] = M::cvt(kj * fe);
      }
    }
    __syncthreads();
  };

  // A_II, P_II and T_II = (I + A_II)^-1 of the staged block (as in the forward).
  auto leaf = [&]() {
    const int r = tid >> 4;
    const int i = tid & 15;
    float a = 0.f, p = 0.f;
    if (i <= r) {
      for (int j = 0; j < DK; ++j) {
        const float kk = sK[i][j] * __expf(sL[r][j] - sL[i][j]);
        a += sEK[r][j] * kk;
        p += sQT[r][j] * kk;
      }
    }
    if (i >= r) a = 0.f;
    sP[r][i] = M::cvt(p);
    sWa[r][i] = a;
    sWt[r][i] = (r == i ? 1.f : 0.f) - a;
    __syncthreads();
#pragma unroll 1
    for (int step = 0; step < 3; ++step) {
      float sq = 0.f;
#pragma unroll
      for (int x = 0; x < 16; ++x) sq += sWa[r][x] * sWa[x][i];
      __syncthreads();
      sWa[r][i] = sq;
      __syncthreads();
      float t2 = sWt[r][i];
#pragma unroll
      for (int x = 0; x < 16; ++x) t2 += sWt[r][x] * sWa[x][i];
      __syncthreads();
      sWt[r][i] = t2;
      __syncthreads();
    }
    sT[r][i] = M::cvt(sWt[r][i]);
    __syncthreads();
  };

  // 16 x 16 product  out[r][i] = sum_m A[r0+r][m] * Bm[r0+i][m] over the DV columns
  // of two [C][DV] fp32 scratch arrays (or dO for A), masked by `lower` (i <= r or i < r).
  auto leaf_dot = [&](int r0, const float* Arow, bool a_is_dO, const float* Brow, bool strict,
                      float (*dst)[17]) {
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < DV / 16; ++kk) {
      f32x4 av;
      if (a_is_dO) {
        const Tin* p = dO + gidx(r0 + c16, 16 * kk + 4 * g);
        av = load4(p);
      } else {
        av = load4(Arow + static_cast<size_t>(r0 + c16) * DV + 16 * kk + 4 * g);
      }
      const f32x4 bv = load4(Brow + static_cast<size_t>(r0 + c16) * DV + 16 * kk + 4 * g);
      acc = M::mma(M::from_f32(av), M::from_f32(bv), acc);
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int r = 4 * g + ii;
      const bool keep = strict ? (c16 < r) : (c16 <= r);
      dst[r][c16] = keep ? acc[ii] : 0.f;
    }
  };

  // Stage columns [p*SW, (p+1)*SW) of a state held as accumulators st[s][n]
  // (rows 16s+4g+i, column wave*CWv + 16n + c16) into sSD as [dk][col].
  auto stage_state = [&](const f32x4 (*st)[NTv], int p) {
#pragma unroll
    for (int n = 0; n < NTv; ++n) {
      const int col = wave * CWv + 16 * n + c16 - p * SW;
      if (col >= 0 && col < SW) {
#pragma unroll
        for (int s = 0; s < RT; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) sSD[16 * s + 4 * g + i][col] = M::cvt(st[s][n][i]);
      }
    }
  };

  // acc[n] += sum over staged columns: Arow[token r0+c16][col] * sSD[wave's dk col][col]
  auto dv_contract = [&](f32x4* acc, int r0, const float* Arow, bool a_is_dO, int p) {
#pragma unroll
    for (int kk = 0; kk < SW / 16; ++kk) {
      const int col = p * SW + 16 * kk + 4 * g;
      f32x4 av;
      if (a_is_dO)
        av = load4(dO + gidx(r0 + c16, col));
      else
        av = load4(Arow + static_cast<size_t>(r0 + c16) * DV + col);
      const frag af = M::from_f32(av);
#pragma unroll
      for (int n = 0; n < NTk; ++n)
        acc[n] = M::mma(af, M::load(&sSD[wave * CWk + 16 * n + c16][16 * kk + 4 * g]), acc[n]);
    }
  };

  // ================= F1: forward sweep ==================
  f32x4 S[RT][NTv];
#pragma unroll
  for (int s = 0; s < RT; ++s)
#pragma unroll
    for (int n = 0; n < NTv; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[s][n][i] = S0c[static_cast<size_t>(16 * s + 4 * g + i) * DV + wave * CWv + 16 * n + c16];

#pragma unroll 1
  for (int I = 0; I < NB; ++I) {
    const int r0 = 16 * I;
    stage(I, 0);
    leaf();
    // Delta_I = T_II (U_I - X_I S_I)
    f32x4 Dl[NTv];
    {
      f32x4 XS[NTv];
#pragma unroll
      for (int n = 0; n < NTv; ++n) XS[n] = zero4();
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        const frag xa = M::load(&sRowOp[c16][16 * s + 4 * g]);
#pragma unroll
        for (int n = 0; n < NTv; ++n) XS[n] = M::mma(xa, M::from_f32(S[s][n]), XS[n]);
      }
      const frag ta = M::load(&sT[c16][4 * g]);
#pragma unroll
      for (int n = 0; n < NTv; ++n) {
        const int colv = wave * CWv + 16 * n + c16;
        f32x4 rhs;
#pragma unroll
        for (int i = 0; i < 4; ++i) rhs[i] = sU[colv][4 * g + i] - XS[n][i];
        Dl[n] = M::mma(ta, M::from_f32(rhs), zero4());
#pragma unroll
        for (int i = 0; i < 4; ++i) gDel[static_cast<size_t>(r0 + 4 * g + i) * DV + colv] = Dl[n][i];
      }
    }
    __syncthreads();
    if (wave == 0) leaf_dot(r0, nullptr, true, gDel, false, sLf[0]);  // dO_r . Delta_i, i <= r
    // d(qt) boundary part: dO_I S_I^T
    f32x4 acc[NTk];
#pragma unroll
    for (int n = 0; n < NTk; ++n) acc[n] = zero4();
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
      stage_state(S, p);
      __syncthreads();
      dv_contract(acc, r0, nullptr, true, p);
      __syncthreads();
    }
#pragma unroll
    for (int n = 0; n < NTk; ++n) {
      const int j = wave * CWk + 16 * n + c16;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 4 * g + ii;
        const float Lr = sL[r][j];
        float val = acc[n][ii] * __expf(Lr - sB[I][j]);
        for (int i2 = 0; i2 <= r; ++i2) val += sLf[0][r][i2] * __expf(Lr - sL[i2][j]) * sK[i2][j];
        const size_t gi = gidx(r0 + r, j);
        dq[gi] = Elem<Tin>::load(gamma, gi) * val;
        dgamma[gi] = Elem<Tin>::load(q, gi) * val;
        dlog_a[gi] = sQT[r][j] * val;
      }
    }
    // S_{I+1} = diag(g_I) S_I + Ke_I^T Delta_I
#pragma unroll
    for (int s = 0; s < RT; ++s) {
      const frag ka = M::load(&sColOp[16 * s + c16][4 * g]);
      f32x4 gs;
#pragma unroll
      for (int i = 0; i < 4; ++i) gs[i] = sG[16 * s + 4 * g + i];
#pragma unroll
      for (int n = 0; n < NTv; ++n) S[s][n] = M::mma(ka, M::from_f32(Dl[n]), S[s][n] * gs);
    }
    __syncthreads();
  }

  // ================= R: reverse sweep ==================
  f32x4 D[RT][NTv];
#pragma unroll
  for (int s = 0; s < RT; ++s)
#pragma unroll
    for (int n = 0; n < NTv; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        D[s][n][i] = dSC[static_cast<size_t>(16 * s + 4 * g + i) * DV + wave * CWv + 16 * n + c16];

#pragma unroll 1
  for (int J = NB - 1; J >= 0; --J) {
    const int r0 = 16 * J;
    stage(J, 1);
    leaf();
    frag Ptf, Ttf;
    {
      f32x4 pv, tv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = M::to_f32(sP[4 * g + i][c16]);
        tv[i] = M::to_f32(sT[4 * g + i][c16]);
      }
      Ptf = M::from_f32(pv);
      Ttf = M::from_f32(tv);
    }
    frag dOf[NTv];
    f32x4 dRn[NTv];
#pragma unroll
    for (int n = 0; n < NTv; ++n) {
      const int colv = wave * CWv + 16 * n + c16;
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < RT; ++s) acc = M::mma(M::load(&sRowOp[c16][16 * s + 4 * g]), M::from_f32(D[s][n]), acc);
      f32x4 dov;
#pragma unroll
      for (int i = 0; i < 4; ++i) dov[i] = Elem<Tin>::load(dO, gidx(r0 + 4 * g + i, colv));
      dOf[n] = M::from_f32(dov);
      acc = M::mma(Ptf, dOf[n], acc);
      dRn[n] = M::mma(Ttf, M::from_f32(acc), zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t gi = gidx(r0 + 4 * g + i, colv);
        gdR[static_cast<size_t>(r0 + 4 * g + i) * DV + colv] = dRn[n][i];
        dwrite[gi] = Elem<Tin>::load(v, gi) * dRn[n][i];
        dv[gi] = Elem<Tin>::load(write, gi) * dRn[n][i];
      }
    }
    __syncthreads();
    if (wave == 0) leaf_dot(r0, nullptr, true, gDel, false, sLf[0]);  // dO_r . Delta_i, r >= i
    if (wave == 1) leaf_dot(r0, gdR, false, gDel, true, sLf[1]);      // dR_r . Delta_i, r > i
    // d(k) boundary part: Delta_J D^T
    f32x4 acc[NTk];
#pragma unroll
    for (int n = 0; n < NTk; ++n) acc[n] = zero4();
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
      stage_state(D, p);
      __syncthreads();
      dv_contract(acc, r0, gDel, false, p);
      __syncthreads();
    }
#pragma unroll
    for (int n = 0; n < NTk; ++n) {
      const int j = wave * CWk + 16 * n + c16;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 4 * g + ii;
        const float Li = sL[i][j];
        float val = acc[n][ii] * __expf(sB[J + 1][j] - Li);
        for (int r = i; r < 16; ++r)
          val += __expf(sL[r][j] - Li) * (sLf[0][r][i] * sQT[r][j] - sLf[1][r][i] * sEK[r][j]);
        const size_t gi = gidx(r0 + i, j);
        dk[gi] = val;
        dlog_a[gi] -= sK[i][j] * val;
      }
    }
    // D <- diag(g_J) D + Y_J^T dO_J - X_J^T dR_J
#pragma unroll
    for (int s = 0; s < RT; ++s) {
      const frag ya = M::load(&sYt[16 * s + c16][4 * g]);
      const frag xa = M::load(&sColOp[16 * s + c16][4 * g]);
      f32x4 gs;
#pragma unroll
      for (int i = 0; i < 4; ++i) gs[i] = sG[16 * s + 4 * g + i];
#pragma unroll
      for (int n = 0; n < NTv; ++n) {
        f32x4 t = M::mma(ya, dOf[n], D[s][n] * gs);
        D[s][n] = M::mma(xa, M::from_f32(-dRn[n]), t);
      }
    }
    __syncthreads();
  }

  // ================= F2: forward sweep ==================
#pragma unroll
  for (int s = 0; s < RT; ++s)
#pragma unroll
    for (int n = 0; n < NTv; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[s][n][i] = S0c[static_cast<size_t>(16 * s + 4 * g + i) * DV + wave * CWv + 16 * n + c16];
  float prefix[NTk];  // running sum of dLam over the finished blocks (per owned channel)
#pragma unroll
  for (int n = 0; n < NTk; ++n) prefix[n] = 0.f;

#pragma unroll 1
  for (int I = 0; I < NB; ++I) {
    const int r0 = 16 * I;
    stage(I, 2);
    if (wave == 0) leaf_dot(r0, gdR, false, gDel, true, sLf[1]);  // dR_r . Delta_i, i < r
    f32x4 acc[NTk];
#pragma unroll
    for (int n = 0; n < NTk; ++n) acc[n] = zero4();
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
      stage_state(S, p);
      __syncthreads();
      dv_contract(acc, r0, gdR, false, p);
      __syncthreads();
    }
#pragma unroll
    for (int n = 0; n < NTk; ++n) {
      const int j = wave * CWk + 16 * n + c16;
      float dl[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 4 * g + ii;
        const float Lr = sL[r][j];
        float val = acc[n][ii] * __expf(Lr - sB[I][j]);
        for (int i2 = 0; i2 < r; ++i2) val += sLf[1][r][i2] * __expf(Lr - sL[i2][j]) * sK[i2][j];
        const float dek = -val;
        const size_t gi = gidx(r0 + r, j);
        const float bj = Elem<Tin>::load(erase, gi);
        const float kj = sK[r][j];
        derase[gi] = kj * dek;
        dk[gi] = dk[gi] + bj * dek;
        dl[ii] = dlog_a[gi] + sEK[r][j] * dek;
      }
      // exclusive prefix of dLam over the chunk, in token order
      const float tsum = dl[0] + dl[1] + dl[2] + dl[3];
      const float t0 = __shfl(tsum, c16, 64);
      const float t1 = __shfl(tsum, c16 + 16, 64);
      const float t2 = __shfl(tsum, c16 + 32, 64);
      const float t3 = __shfl(tsum, c16 + 48, 64);
      float run = prefix[n] + (g > 0 ? t0 : 0.f) + (g > 1 ? t1 : 0.f) + (g > 2 ? t2 : 0.f);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        dlog_a[gidx(r0 + 4 * g + ii, j)] = run;
        run += dl[ii];
      }
      prefix[n] += t0 + t1 + t2 + t3;
    }
    // S_{I+1} = diag(g_I) S_I + Ke_I^T Delta_I
#pragma unroll
    for (int s = 0; s < RT; ++s) {
      const frag ka = M::load(&sColOp[16 * s + c16][4 * g]);
      f32x4 gs;
#pragma unroll
      for (int i = 0; i < 4; ++i) gs[i] = sG[16 * s + 4 * g + i];
#pragma unroll
      for (int n = 0; n < NTv; ++n) {
        const int colv = wave * CWv + 16 * n + c16;
        f32x4 dlt;
#pragma unroll
        for (int i = 0; i < 4; ++i) dlt[i] = gDel[static_cast<size_t>(r0 + 4 * g + i) * DV + colv];
        S[s][n] = M::mma(ka, M::from_f32(dlt), S[s][n] * gs);
      }
    }
    __syncthreads();
  }

  // ---- chunk-end term rowsum(S_C * dS_C), then dlog_a_i = total - exclusive prefix ----
  {
    float rs[RT][4];
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = 0.f;
#pragma unroll
        for (int n = 0; n < NTv; ++n)
          a += S[s][n][i] * dSC[static_cast<size_t>(16 * s + 4 * g + i) * DV + wave * CWv + 16 * n + c16];
        a += __shfl_xor(a, 1, 64);
        a += __shfl_xor(a, 2, 64);
        a += __shfl_xor(a, 4, 64);
        a += __shfl_xor(a, 8, 64);
        rs[s][i] = a;
      }
    if (c16 == 0) {
#pragma unroll
      for (int s = 0; s < RT; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) sRow[wave][16 * s + 4 * g + i] = rs[s][i];
    }
  }
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int n = 0; n < NTk; ++n) {
      const int j = wave * CWk + 16 * n + c16;
      float tot = prefix[n];
#pragma unroll
      for (int w = 0; w < 4; ++w) tot += sRow[w][j];
      sTot[j] = tot;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < C * DK; idx += BCH_THREADS) {
    const int r = idx / DK;
    const int j = idx - r * DK;
    const size_t gi = gidx(r, j);
    dlog_a[gi] = sTot[j] - dlog_a[gi];
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

hipError_t launch_bwd_chunk(const ChunkShape& s, const void* q, const void* k, const void* v,
                            const void* log_a, const void* erase, const void* write,
                            const void* gamma, const float* S_chunks, const float* dS_chunks,
                            const void* dO, float* dq, float* dk, float* dv, float* dlog_a,
                            float* derase, float* dwrite, float* dgamma, float* scratch,
                            hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(s.nchunks());
  if (grid == 0) return hipSuccess;
#define MUIR_BCH(TT, DD)                                                                          \
  hipLaunchKernelGGL((bwd_chunk_kernel<TT, DD>), dim3(grid), dim3(BCH_THREADS), 0, stream, s.T,    \
                     s.H, s.C, (const TT*)q, (const TT*)k, (const TT*)v, (const TT*)log_a,          \
                     (const TT*)erase, (const TT*)write, (const TT*)gamma, S_chunks, dS_chunks,     \
                     (const TT*)dO, dq, dk, dv, dlog_a, derase, dwrite, dgamma, scratch)
  if (s.bf16) {
    if (s.DK == 128) MUIR_BCH(uint16_t, 128);
    else MUIR_BCH(uint16_t, 64);
  } else {
    if (s.DK == 128) MUIR_BCH(float, 128);
    else MUIR_BCH(float, 64);
  }
#undef MUIR_BCH
  return hipGetLastError();
}

}  // namespace muir
