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

// Scratch of one chunk (fp32 unless noted): deltas [C][DV], their gradients
// [C][DV], then per 16-token block the leaf inverse T_II and readout leaf
// P_II as [16][16] in the compute type.
template <typename TC>
__host__ __device__ constexpr size_t bwd_scratch_elems_f32(int C, int DV) {
  return static_cast<size_t>(2) * C * DV + (static_cast<size_t>(C / 16) * 2 * 256 * sizeof(TC) + 3) / 4;
}

template <typename Tin, int DK, int C>
__global__ __launch_bounds__((2 * DK / 32) * 64) void bwd_chunk_kernel(
    int T, int H, const Tin* __restrict__ q, const Tin* __restrict__ k,
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
  constexpr int NW = 2 * DK / 32;      // waves: wave w owns state column / gradient channel 16w + lane%16
  constexpr int NTH = 64 * NW;
  constexpr int RT = DK / 16;
  constexpr int TPC = NTH / DK;        // elementwise: threads per key channel (4 tokens each)
  constexpr int NB = C / 16;
  constexpr int SPLIT = (sizeof(TC) == 4 && DK == 128) ? 2 : 1;  // staged state in column passes
  constexpr int SW = DV / SPLIT;
  constexpr int PT = DK + 4;
  constexpr int PS = SW + 4;
  static_assert(NW * 16 == DV && TPC == 4, "wave / thread layout");

  const int NC = T / C;
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
  const int colv = 16 * wave + c16;   // state column (dv) and gradient channel (dk) of this lane
  const int ej = tid % DK;
  const int part = tid / DK;

  const size_t rowbase = (static_cast<size_t>(b) * T + static_cast<size_t>(c) * C) * H + h;
  auto gidx = [&](int t, int j) -> size_t { return (rowbase + static_cast<size_t>(t) * H) * DK + j; };
  float* gDel = scratch + static_cast<size_t>(chunk) * bwd_scratch_elems_f32<TC>(C, DV);
  float* gdR = gDel + static_cast<size_t>(C) * DV;
  TC* gTP = reinterpret_cast<TC*>(gdR + static_cast<size_t>(C) * DV);  // [NB][2][16][16]
  const float* S0c = S_chunks + static_cast<size_t>(chunk) * DK * DV;
  const float* dSC = dS_chunks + static_cast<size_t>(chunk) * DK * DV;

  __shared__ float sB[NB + 1][DK];
  __shared__ float sBsum[NB][DK];
  __shared__ float sBsuf[NB][DK];
  __shared__ float sTmp[TPC][DK];
  __shared__ float sLam[16][DK + 1];                         // log_a of the block
  __shared__ float sF[16][DK + 1];                           // per-element factor of the sweep
  __shared__ __attribute__((aligned(16))) TC sRowA[16][PT];  // F1: X rows   R: Ke rows
  __shared__ __attribute__((aligned(16))) TC sUn1[16 * PT > DK * 20 ? 16 * PT : DK * 20];  // F1: Y rows  R: Y^T
  __shared__ __attribute__((aligned(16))) TC sUn2[16 * PT > DK * 20 ? 16 * PT : DK * 20];  // F1: Z rows  R: Yhat^T
  __shared__ __attribute__((aligned(16))) TC sTA[DK][20];    // F1, F2: Ke^T   R: X^T
  __shared__ __attribute__((aligned(16))) TC sTZ[DK][20];    // F1, F2: Z^T    R: Xhat^T
  __shared__ __attribute__((aligned(16))) TC sU[DV][20];     // F1: (write*v)^T
  __shared__ float sAw[16][17];
  __shared__ float sPw[16][17];
  __shared__ float sTw[16][17];
  __shared__ float sPf[16][17];
  __shared__ __attribute__((aligned(16))) TC sSD[DK][PS];    // staged S or D columns, [dk][dv]
  __shared__ float sLf[2][16][17];
  __shared__ float sG[DK];
  __shared__ float sRow[NW][DK];
  __shared__ float sTot[DK];
  TC (*sRowB)[PT] = reinterpret_cast<TC (*)[PT]>(sUn1);
  TC (*sRowZ)[PT] = reinterpret_cast<TC (*)[PT]>(sUn2);
  TC (*sTB)[20] = reinterpret_cast<TC (*)[20]>(sUn1);
  TC (*sTY)[20] = reinterpret_cast<TC (*)[20]>(sUn2);

  // ---- block sums of the log-decay, prefix and suffix over blocks ----
#pragma unroll
  for (int I = part; I < NB; I += TPC) {
    float sacc = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sacc += Elem<Tin>::load(log_a, gidx(16 * I + rr, ej));
    sBsum[I][ej] = sacc;
  }
  __syncthreads();
  if (tid < DK) {
    float acc = 0.f;
    sB[0][tid] = 0.f;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      acc += sBsum[I][tid];
      sB[I + 1][tid] = acc;
    }
    float suf = 0.f;
#pragma unroll
    for (int I = NB - 1; I >= 0; --I) {
      suf += sBsum[I][tid];
      sBsuf[I][tid] = suf;
    }
  }
  __syncthreads();

  // Per-block tiles (elementwise; thread = channel ej, tokens 4*part..+3).
  // mode 0 (F1): sF = exp(Lam - B_I); X, Y, Z rows; Ke^T, Z^T, U^T
  // mode 1 (R):  sF = exp(B_{I+1} - Lam); Ke rows; X^T, Y^T, Xhat^T, Yhat^T
  // mode 2 (F2): sF = exp(Lam - B_I); Ke^T, Z^T
  // with X = ek exp(Lam - B_I), Y = qt exp(Lam - B_I), Ke = k exp(B_{I+1} - Lam),
  // Z = k exp(B_I - Lam), Xhat = ek exp(Lam - B_{I+1}), Yhat = qt exp(Lam - B_{I+1});
  // Z, Xhat, Yhat (>= 1) only for leaves whose decay stays within LEAF_SAFE_RANGE.
  auto stage = [&](int I, int mode) -> int {
    const int r0 = 16 * I;
    float kv[4], ev[4], qv[4], gv[4], lv[4], uv[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const size_t gi = gidx(r0 + 4 * part + rr, ej);
      kv[rr] = Elem<Tin>::load(k, gi);
      ev[rr] = Elem<Tin>::load(erase, gi);
      qv[rr] = Elem<Tin>::load(q, gi);
      gv[rr] = Elem<Tin>::load(gamma, gi);
      lv[rr] = Elem<Tin>::load(log_a, gi);
      uv[rr] = mode == 0 ? Elem<Tin>::load(write, gi) * Elem<Tin>::load(v, gi) : 0.f;
    }
    float cs[4], sf[4];
    {
      float run = 0.f;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        run += lv[rr];
        cs[rr] = run;
      }
      sTmp[part][ej] = run;
      sf[3] = 0.f;
      sf[2] = lv[3];
      sf[1] = lv[3] + lv[2];
      sf[0] = lv[3] + lv[2] + lv[1];
    }
    const float bsum = sBsum[I][ej];
    const int safe = __syncthreads_and(-bsum <= LEAF_SAFE_RANGE);
    float excl = 0.f, exsuf = 0.f;
    for (int p = 0; p < TPC; ++p) {
      if (p < part) excl += sTmp[p][ej];
      if (p > part) exsuf += sTmp[p][ej];
    }
    if (part == 0) sG[ej] = __expf(bsum);
    f32x4 tA, tZ, tB, tY;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * part + rr;
      const float loc = excl + cs[rr];   // Lam_r - B_I
      const float suf = sf[rr] + exsuf;  // B_{I+1} - Lam_r
      const float fs = __expf(loc);
      const float fe = __expf(suf);
      const float ek = ev[rr] * kv[rr];
      const float qt = gv[rr] * qv[rr];
      sLam[r][ej] = lv[rr];
      if (mode == 0) {
        const float z = safe ? kv[rr] * __expf(-loc) : 0.f;
        sF[r][ej] = fs;
        sRowA[r][ej] = M::cvt(ek * fs);
        sRowB[r][ej] = M::cvt(qt * fs);
        sRowZ[r][ej] = M::cvt(z);
        tA[rr] = kv[rr] * fe;
        tZ[rr] = z;
        tB[rr] = uv[rr];
      } else if (mode == 1) {
        const float ie = safe ? __expf(-suf) : 0.f;
        sF[r][ej] = fe;
        sRowA[r][ej] = M::cvt(kv[rr] * fe);
        tA[rr] = ek * fs;
        tB[rr] = qt * fs;
        tZ[rr] = ek * ie;
        tY[rr] = qt * ie;
      } else {
        sF[r][ej] = fs;
        tA[rr] = kv[rr] * fe;
        tZ[rr] = safe ? kv[rr] * __expf(-loc) : 0.f;
      }
    }
    store4(&sTA[ej][4 * part], tA);
    store4(&sTZ[ej][4 * part], tZ);
    if (mode == 0) store4(&sU[ej][4 * part], tB);
    if (mode == 1) {
      store4(&sTB[ej][4 * part], tB);
      store4(&sTY[ej][4 * part], tY);
    }
    __syncthreads();
    return safe;
  };

  // exp(sum of log_a over tokens (i, r] of the staged block, channel j), r >= i
  auto pair_factor = [&](int r, int i, int j) -> float {
    float ls = 0.f;
    for (int x = i + 1; x <= r; ++x) ls += sLam[x][j];
    return __expf(ls);
  };

  // out[r][i] = sum over dv of Arow[token r0+r] . Brow[token r0+i], masked to
  // i <= r (or i < r when strict); rows come from [C][DV] fp32 scratch or dO.
  auto leaf_dot = [&](int r0, const float* Arow, bool a_is_dO, const float* Brow, bool strict,
                      float (*dst)[17]) {
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < DV / 16; ++kk) {
      const f32x4 av = a_is_dO ? load4(dO + gidx(r0 + c16, 16 * kk + 4 * g))
                               : load4(Arow + static_cast<size_t>(r0 + c16) * DV + 16 * kk + 4 * g);
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

  // stage columns [p*SW, (p+1)*SW) of a state (rows 16s+4g+i, column colv) into sSD
  auto stage_state = [&](const f32x4* st, int p) {
    const int col = colv - p * SW;
    if (col >= 0 && col < SW) {
#pragma unroll
      for (int s = 0; s < RT; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) sSD[16 * s + 4 * g + i][col] = M::cvt(st[s][i]);
    }
  };

  // acc += Arow[token r0+c16][staged columns] . sSD[channel colv][staged columns]
  auto dv_contract = [&](f32x4 acc, int r0, const float* Arow, bool a_is_dO, int p) -> f32x4 {
#pragma unroll
    for (int kk = 0; kk < SW / 16; ++kk) {
      const int col = p * SW + 16 * kk + 4 * g;
      const f32x4 av = a_is_dO ? load4(dO + gidx(r0 + c16, col))
                               : load4(Arow + static_cast<size_t>(r0 + c16) * DV + col);
      acc = M::mma(M::from_f32(av), M::load(&sSD[colv][16 * kk + 4 * g]), acc);
    }
    return acc;
  };

  auto load_state = [&](f32x4* st, const float* src) {
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[s][i] = src[static_cast<size_t>(16 * s + 4 * g + i) * DV + colv];
  };

  // ================= F1: forward sweep: deltas, d(qt) ==================
  f32x4 S[RT];
  load_state(S, S0c);
#pragma unroll 1
  for (int I = 0; I < NB; ++I) {
    const int r0 = 16 * I;
    const int safe = stage(I, 0);
    // leaf A_II, P_II and T_II; kept in the chunk scratch for the reverse sweep
    if (safe) {
      if (wave == 0) {
        f32x4 a = zero4(), pp = zero4();
#pragma unroll
        for (int s = 0; s < RT; ++s) {
          const frag zb = M::load(&sRowZ[c16][16 * s + 4 * g]);
          a = M::mma(M::load(&sRowA[c16][16 * s + 4 * g]), zb, a);
          pp = M::mma(M::load(&sRowB[c16][16 * s + 4 * g]), zb, pp);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          sAw[r][c16] = c16 < r ? a[i] : 0.f;
          sPf[r][c16] = c16 <= r ? pp[i] : 0.f;
        }
      }
    } else {
      for (int pr = tid; pr < 256; pr += NTH) {
        const int r = pr >> 4;
        const int i = pr & 15;
        float a = 0.f, pp = 0.f;
        if (i <= r) {
          for (int j = 0; j < DK; ++j) {
            const size_t gr = gidx(r0 + r, j);
            const float kk = Elem<Tin>::load(k, gidx(r0 + i, j)) * pair_factor(r, i, j);
            a += Elem<Tin>::load(erase, gr) * Elem<Tin>::load(k, gr) * kk;
            pp += Elem<Tin>::load(gamma, gr) * Elem<Tin>::load(q, gr) * kk;
          }
        }
        sAw[r][i] = i < r ? a : 0.f;
        sPf[r][i] = pp;
      }
      __syncthreads();
    }
    if (wave == 0) {
      const f32x4 t = neumann16(sAw, sPw, sTw);
      TC* tp = gTP + static_cast<size_t>(I) * 512;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tp[(4 * g + i) * 16 + c16] = M::cvt(t[i]);
        tp[256 + (4 * g + i) * 16 + c16] = M::cvt(sPf[4 * g + i][c16]);
      }
    }
    __syncthreads();
    // Delta_I = T_II (U_I - X_I S_I)
    f32x4 Dl;
    {
      f32x4 xs = zero4();
#pragma unroll
      for (int s = 0; s < RT; ++s) xs = M::mma(M::load(&sRowA[c16][16 * s + 4 * g]), M::from_f32(S[s]), xs);
      const TC* tp = gTP + static_cast<size_t>(I) * 512;
      const frag ta = M::load(tp + c16 * 16 + 4 * g);
      const f32x4 rhs = load4(&sU[colv][4 * g]) - xs;
      Dl = M::mma(ta, M::from_f32(rhs), zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) gDel[static_cast<size_t>(r0 + 4 * g + i) * DV + colv] = Dl[i];
    }
    __syncthreads();
    if (wave == 0) leaf_dot(r0, nullptr, true, gDel, false, sLf[0]);  // dO_r . Delta_i, i <= r
    // d(qt)_r = exp(Lam_r - B_I) [ S_I dO_r + sum_{i<=r} (dO_r . Delta_i) Z_i ]
    f32x4 acc = zero4();
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
      stage_state(S, p);
      __syncthreads();
      acc = dv_contract(acc, r0, nullptr, true, p);
      if (p + 1 < SPLIT) __syncthreads();
    }
    if (safe) {
      f32x4 lf;
#pragma unroll
      for (int i = 0; i < 4; ++i) lf[i] = sLf[0][c16][4 * g + i];
      acc = M::mma(M::from_f32(lf), M::load(&sTZ[colv][4 * g]), acc);
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int r = 4 * g + ii;
      const int j = colv;
      float val = sF[r][j] * acc[ii];
      if (!safe)
        for (int i2 = 0; i2 <= r; ++i2)
          val += sLf[0][r][i2] * pair_factor(r, i2, j) * Elem<Tin>::load(k, gidx(r0 + i2, j));
      const size_t gi = gidx(r0 + r, j);
      const float qq = Elem<Tin>::load(q, gi);
      const float gg = Elem<Tin>::load(gamma, gi);
      dq[gi] = gg * val;
      dgamma[gi] = qq * val;
      dlog_a[gi] = gg * qq * val;
    }
    // S_{I+1} = diag(exp(B_{I+1} - B_I)) S_I + Ke_I^T Delta_I
    {
      const frag df = M::from_f32(Dl);
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        f32x4 gs;
#pragma unroll
        for (int i = 0; i < 4; ++i) gs[i] = sG[16 * s + 4 * g + i];
        S[s] = M::mma(M::load(&sTA[16 * s + c16][4 * g]), df, S[s] * gs);
      }
    }
    __syncthreads();
  }

  // ================= R: reverse sweep: dR, d(k) ==================
  f32x4 D[RT];
  load_state(D, dSC);
#pragma unroll 1
  for (int J = NB - 1; J >= 0; --J) {
    const int r0 = 16 * J;
    const int safe = stage(J, 1);
    const TC* tp = gTP + static_cast<size_t>(J) * 512;
    frag ptf, ttf;
    {
      f32x4 pv, tv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tv[i] = M::to_f32(tp[(4 * g + i) * 16 + c16]);
        pv[i] = M::to_f32(tp[256 + (4 * g + i) * 16 + c16]);
      }
      ptf = M::from_f32(pv);
      ttf = M::from_f32(tv);
    }
    // dR_J = T_JJ^T (Ke_J D + P_JJ^T dO_J)
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < RT; ++s) acc = M::mma(M::load(&sRowA[c16][16 * s + 4 * g]), M::from_f32(D[s]), acc);
    f32x4 dov;
#pragma unroll
    for (int i = 0; i < 4; ++i) dov[i] = Elem<Tin>::load(dO, gidx(r0 + 4 * g + i, colv));
    const frag dOf = M::from_f32(dov);
    acc = M::mma(ptf, dOf, acc);
    const f32x4 dRn = M::mma(ttf, M::from_f32(acc), zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t gi = gidx(r0 + 4 * g + i, colv);
      gdR[static_cast<size_t>(r0 + 4 * g + i) * DV + colv] = dRn[i];
      dwrite[gi] = Elem<Tin>::load(v, gi) * dRn[i];
      dv[gi] = Elem<Tin>::load(write, gi) * dRn[i];
    }
    __syncthreads();
    if (wave == 0) leaf_dot(r0, nullptr, true, gDel, false, sLf[0]);  // dO_r . Delta_i, r >= i
    if (wave == 1 % NW) leaf_dot(r0, gdR, false, gDel, true, sLf[1]); // dR_r . Delta_i, r > i
    // d(k)_i = exp(B_{J+1} - Lam_i) [ D Delta_i + sum_{r>=i} (dO_r.Delta_i) Yhat_r - sum_{r>i} (dR_r.Delta_i) Xhat_r ]
    f32x4 acc2 = zero4();
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
      stage_state(D, p);
      __syncthreads();
      acc2 = dv_contract(acc2, r0, gDel, false, p);
      if (p + 1 < SPLIT) __syncthreads();
    }
    if (safe) {
      f32x4 l1, l2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l1[i] = sLf[0][4 * g + i][c16];
        l2[i] = -sLf[1][4 * g + i][c16];
      }
      acc2 = M::mma(M::from_f32(l1), M::load(&sTY[colv][4 * g]), acc2);
      acc2 = M::mma(M::from_f32(l2), M::load(&sTZ[colv][4 * g]), acc2);
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 4 * g + ii;
      const int j = colv;
      float val = sF[i][j] * acc2[ii];
      if (!safe)
        for (int r = i; r < 16; ++r) {
          const size_t gr = gidx(r0 + r, j);
          const float f = pair_factor(r, i, j);
          val += f * (sLf[0][r][i] * Elem<Tin>::load(gamma, gr) * Elem<Tin>::load(q, gr) -
                      sLf[1][r][i] * Elem<Tin>::load(erase, gr) * Elem<Tin>::load(k, gr));
        }
      const size_t gi = gidx(r0 + i, j);
      dk[gi] = val;
      dlog_a[gi] -= Elem<Tin>::load(k, gi) * val;
    }
    // D <- diag(exp(B_{J+1} - B_J)) D + Y_J^T dO_J - X_J^T dR_J
    {
      const frag dRf = M::from_f32(-dRn);
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        f32x4 gs;
#pragma unroll
        for (int i = 0; i < 4; ++i) gs[i] = sG[16 * s + 4 * g + i];
        const f32x4 t = M::mma(M::load(&sTB[16 * s + c16][4 * g]), dOf, D[s] * gs);
        D[s] = M::mma(M::load(&sTA[16 * s + c16][4 * g]), dRf, t);
      }
    }
    __syncthreads();
  }

  // ================= F2: forward sweep: d(ek), totals ==================
  load_state(S, S0c);
  float prefix = 0.f;  // sum of dLam over the finished blocks, channel colv
#pragma unroll 1
  for (int I = 0; I < NB; ++I) {
    const int r0 = 16 * I;
    const int safe = stage(I, 2);
    if (wave == 0) leaf_dot(r0, gdR, false, gDel, true, sLf[1]);  // dR_r . Delta_i, i < r
    f32x4 acc = zero4();
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
      stage_state(S, p);
      __syncthreads();
      acc = dv_contract(acc, r0, gdR, false, p);
      if (p + 1 < SPLIT) __syncthreads();
    }
    if (safe) {
      f32x4 lf;
#pragma unroll
      for (int i = 0; i < 4; ++i) lf[i] = sLf[1][c16][4 * g + i];
      acc = M::mma(M::from_f32(lf), M::load(&sTZ[colv][4 * g]), acc);
    }
    float dl[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int r = 4 * g + ii;
      const int j = colv;
      float val = sF[r][j] * acc[ii];
      if (!safe)
        for (int i2 = 0; i2 < r; ++i2)
          val += sLf[1][r][i2] * pair_factor(r, i2, j) * Elem<Tin>::load(k, gidx(r0 + i2, j));
      const float dek = -val;  // d(ek)_r = -S'_r dR_r
      const size_t gi = gidx(r0 + r, j);
      const float bj = Elem<Tin>::load(erase, gi);
      const float kj = Elem<Tin>::load(k, gi);
      derase[gi] = kj * dek;
      dk[gi] = dk[gi] + bj * dek;
      dl[ii] = dlog_a[gi] + bj * kj * dek;
    }
    // exclusive prefix of dLam over the chunk, in token order
    {
      const float tsum = dl[0] + dl[1] + dl[2] + dl[3];
      const float t0 = __shfl(tsum, c16, 64);
      const float t1 = __shfl(tsum, c16 + 16, 64);
      const float t2 = __shfl(tsum, c16 + 32, 64);
      const float t3 = __shfl(tsum, c16 + 48, 64);
      float run = prefix + (g > 0 ? t0 : 0.f) + (g > 1 ? t1 : 0.f) + (g > 2 ? t2 : 0.f);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        dlog_a[gidx(r0 + 4 * g + ii, colv)] = run;
        run += dl[ii];
      }
      prefix += t0 + t1 + t2 + t3;
    }
    // S_{I+1} = diag(g_I) S_I + Ke_I^T Delta_I
    {
      f32x4 dlt;
#pragma unroll
      for (int i = 0; i < 4; ++i) dlt[i] = gDel[static_cast<size_t>(r0 + 4 * g + i) * DV + colv];
      const frag df = M::from_f32(dlt);
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        f32x4 gs;
#pragma unroll
        for (int i = 0; i < 4; ++i) gs[i] = sG[16 * s + 4 * g + i];
        S[s] = M::mma(M::load(&sTA[16 * s + c16][4 * g]), df, S[s] * gs);
      }
    }
    __syncthreads();
  }

  // ---- chunk-end term rowsum(S_C * dS_C); dlog_a_i = total - exclusive prefix ----
#pragma unroll
  for (int s = 0; s < RT; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = S[s][i] * dSC[static_cast<size_t>(16 * s + 4 * g + i) * DV + colv];
      a += __shfl_xor(a, 1, 64);
      a += __shfl_xor(a, 2, 64);
      a += __shfl_xor(a, 4, 64);
      a += __shfl_xor(a, 8, 64);
      if (c16 == 0) sRow[wave][16 * s + 4 * g + i] = a;
    }
  __syncthreads();
  if (g == 0) {
    float tot = prefix;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += sRow[w][colv];
    sTot[colv] = tot;
  }
  __syncthreads();
  for (int idx = tid; idx < C * DK; idx += NTH) {
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
#define MUIR_BCH1(TT, DD, CC)                                                                      \
  hipLaunchKernelGGL((bwd_chunk_kernel<TT, DD, CC>), dim3(grid), dim3((2 * DD / 32) * 64), 0,      \
                     stream, s.T, s.H, (const TT*)q, (const TT*)k, (const TT*)v, (const TT*)log_a, \
                     (const TT*)erase, (const TT*)write, (const TT*)gamma, S_chunks, dS_chunks,    \
                     (const TT*)dO, dq, dk, dv, dlog_a, derase, dwrite, dgamma, scratch)
#define MUIR_BCH(TT, DD)                         \
  do {                                           \
    if (s.C == 64) MUIR_BCH1(TT, DD, 64);        \
    else if (s.C == 128) MUIR_BCH1(TT, DD, 128); \
    else MUIR_BCH1(TT, DD, 256);                 \
  } while (0)
  if (s.bf16) {
    if (s.DK == 128) MUIR_BCH(uint16_t, 128);
    else MUIR_BCH(uint16_t, 64);
  } else {
    if (s.DK == 128) MUIR_BCH(float, 128);
    else MUIR_BCH(float, 64);
  }
#undef MUIR_BCH
#undef MUIR_BCH1
  return hipGetLastError();
}

size_t bwd_chunk_scratch_bytes(const ChunkShape& s) {
  return 4 * (s.bf16 ? bwd_scratch_elems_f32<uint16_t>(s.C, s.DV) : bwd_scratch_elems_f32<float>(s.C, s.DV));
}

}  // namespace muir
