// Per-chunk gradients of the Muir gated delta rule (gfx950).
//
// One workgroup per chunk gets the chunk's initial state S0 and the gradient
// dS_C of its end state (from the reverse scan in bwd.hip) and forms every
// input gradient with three sweeps over the chunk's 16-token blocks, with the
// block-boundary pivots of the forward (fwd.hip):
//   F1 (forward): Delta_I = T_II (U_I - X_I S_I), S_{I+1} = g_I S_I + Ke_I^T Delta_I,
//                 d(qt)_r = S_r dO_r                     (S_r: state after token r)
//   R  (reverse): D, the state gradient at the block's end, from dS_C;
//                 dR_J = T_JJ^T (Ke_J D + P_JJ^T dO_J)   (gradient of write*v),
//                 d(k)_i = E_i Delta_i                    (E_i: state gradient at i),
//                 D <- g_J D + Y_J^T dO_J - X_J^T dR_J
//   F2 (forward): d(ek)_r = -S'_r dR_r                   (S'_r: decayed state before r)
// with ek = erase*k, qt = gamma*q, then
//   dLam_r = ek_r d(ek)_r + qt_r d(qt)_r - k_r d(k)_r (+ rowsum(S_C * dS_C) at the last token),
//   dlog_a_i = sum_{r >= i in the chunk} dLam_r,
//   derase = k d(ek), dk = d(k) + erase d(ek), dq = gamma d(qt), dgamma = q d(qt),
//   dv = write dR, dwrite = v dR.
// (arXiv 2611.08376 states only that a custom backward pass is used, in its
// Methodology section and the fig:kernel caption; this is the adjoint of the
// chunkwise forward.)
//
// Each per-token product splits into a boundary part, a tile product with S_I,
// D or the deltas scaled by exp(.) <= 1, and a 16 x 16 leaf part.  On leaves
// whose decay stays within LEAF_SAFE_RANGE the leaf part is one more 16-wide
// MFMA product folded into the same accumulator; steeper leaves use per-pair
// factors in (0, 1].
//
// Latency: every global read a step needs (the block's inputs, dO rows,
// deltas, their gradients, the leaf inverse, the gradient partials) is issued
// one step ahead into registers and committed to LDS when the step starts, so
// a step's compute phase touches only LDS and registers.
#include "chunk_common.h"
#include "kernels.h"
#include "mma.h"

namespace muir {

namespace {

// Per-chunk scratch: deltas [C][DV] and their gradients [C][DV], then T_II and
// P_II of every 16-token block as [16][16], all in the compute type.
template <typename TC>
__host__ __device__ constexpr size_t bwd_scratch_bytes_tc(int C, int DV) {
  return (static_cast<size_t>(2) * C * DV + static_cast<size_t>(C / 16) * 512) * sizeof(TC);
}

template <typename Tin, int DK, int C>
__global__ __launch_bounds__((2 * DK / 32) * 64) void bwd_chunk_kernel(
    int T, int H, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ log_a, const Tin* __restrict__ erase,
    const Tin* __restrict__ write, const Tin* __restrict__ gamma,
    const float* __restrict__ S_chunks, const float* __restrict__ dS_chunks,
    const Tin* __restrict__ dO, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dlog_a, float* __restrict__ derase,
    float* __restrict__ dwrite, float* __restrict__ dgamma, char* __restrict__ scratch) {
  typedef Tin TC;
  typedef MM<TC> M;
  typedef typename M::frag frag;
  constexpr int DV = DK;
  constexpr int NW = 2 * DK / 32;    // wave w owns state column / gradient channel 16w + lane%16
  constexpr int NTH = 64 * NW;
  constexpr int RT = DK / 16;
  constexpr int TPC = NTH / DK;      // elementwise: 4 threads per key channel, 4 tokens each
  constexpr int NB = C / 16;
  constexpr int NSTEP = 3 * NB;
  constexpr bool LEAN = sizeof(TC) == 4 && DK == 128;  // q, gamma re-read from global (LDS budget)
  constexpr int SPLIT = LEAN ? 4 : 2;                  // staged state in column passes
  constexpr int SW = DV / SPLIT;
  constexpr int PT = DK + 4;
  constexpr int PV = DV + 4;
  constexpr int PS = SW + 4;
  constexpr int RC = DV / 4;         // threads per row of a [16][DV] tile
  static_assert(NW * 16 == DV && TPC == 4 && NTH == 16 * RC, "thread layout");

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
  const int colv = 16 * wave + c16;  // MFMA-output mapping: state column / gradient channel
  const int ej = tid % DK;           // elementwise mapping: channel, tokens 4*part..+3
  const int part = tid / DK;
  const int prow = tid / RC;         // row-tile mapping: row, columns 4*pc..+3
  const int pc4 = (tid % RC) * 4;

  const size_t rowbase = (static_cast<size_t>(b) * T + static_cast<size_t>(c) * C) * H + h;
  auto gidx = [&](int t, int j) -> size_t { return (rowbase + static_cast<size_t>(t) * H) * DK + j; };
  TC* gDel = reinterpret_cast<TC*>(scratch + static_cast<size_t>(chunk) * bwd_scratch_bytes_tc<TC>(C, DV));
  TC* gdR = gDel + static_cast<size_t>(C) * DV;
  TC* gTP = gdR + static_cast<size_t>(C) * DV;  // [NB][2][16][16]
  const float* S0c = S_chunks + static_cast<size_t>(chunk) * DK * DV;
  const float* dSC = dS_chunks + static_cast<size_t>(chunk) * DK * DV;

  constexpr int UNI = 16 * PT > DK * 20 ? 16 * PT : DK * 20;
  constexpr int UNU = DV * 20 > 16 * PV ? DV * 20 : 16 * PV;
  __shared__ float sBsum[NB][DK];                            // sum of log_a over block I
  __shared__ float sTmp[TPC][DK];
  __shared__ float sF[16][DK + 1];                           // per-element factor of the sweep
  __shared__ float sLam[16][DK + 1];                         // log_a of the block (per-pair leaves)
  __shared__ __attribute__((aligned(16))) TC sK[16][PT];     // raw k of the block
  __shared__ __attribute__((aligned(16))) TC sE[16][PT];     // raw erase
  __shared__ __attribute__((aligned(16))) TC sQ[LEAN ? 1 : 16][PT];   // raw q
  __shared__ __attribute__((aligned(16))) TC sGm[LEAN ? 1 : 16][PT];  // raw gamma
  __shared__ __attribute__((aligned(16))) TC sRowA[16][PT];  // F1: X rows   R: Ke rows
  __shared__ __attribute__((aligned(16))) TC sUn1[UNI];      // F1: Y rows   R: Y^T
  __shared__ __attribute__((aligned(16))) TC sUn2[UNI];      // F1: Z rows   R: Yhat^T
  __shared__ __attribute__((aligned(16))) TC sTA[DK][20];    // F1, F2: Ke^T   R: X^T
  __shared__ __attribute__((aligned(16))) TC sTZ[DK][20];    // F1, F2: Z^T    R: Xhat^T
  __shared__ __attribute__((aligned(16))) TC sUnU[UNU];      // F1: (write*v)^T   R, F2: dR rows
  __shared__ __attribute__((aligned(16))) TC sDO[16][PV];    // dO rows of the block
  __shared__ __attribute__((aligned(16))) TC sDL[16][PV];    // delta rows of the block
  __shared__ float sAw[16][17];
  __shared__ float sPw[16][17];
  __shared__ float sTw[16][17];
  __shared__ float sPf[16][17];
  __shared__ __attribute__((aligned(16))) TC sT[16][20];     // T_II of the block
  __shared__ __attribute__((aligned(16))) TC sP[16][20];     // P_II of the block
  __shared__ __attribute__((aligned(16))) TC sSD[DK][PS];    // staged S or D columns, [dk][dv]
  __shared__ float sLf[2][16][17];                           // leaf gradient matrices
  __shared__ float sG[DK];
  __shared__ float sRow[NW][DK];
  __shared__ float sTot[DK];
  TC (*sRowB)[PT] = reinterpret_cast<TC (*)[PT]>(sUn1);
  TC (*sRowZ)[PT] = reinterpret_cast<TC (*)[PT]>(sUn2);
  TC (*sTB)[20] = reinterpret_cast<TC (*)[20]>(sUn1);
  TC (*sTY)[20] = reinterpret_cast<TC (*)[20]>(sUn2);
  TC (*sU)[20] = reinterpret_cast<TC (*)[20]>(sUnU);
  TC (*sDR)[PV] = reinterpret_cast<TC (*)[PV]>(sUnU);

  // ---- block sums of the log-decay ----
#pragma unroll
  for (int I = part; I < NB; I += TPC) {
    float sacc = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sacc += Elem<Tin>::load(log_a, gidx(16 * I + rr, ej));
    sBsum[I][ej] = sacc;
  }

  auto step_sweep = [](int s) { return s / NB; };
  auto step_block = [](int s) { return (s / NB) == 1 ? NB - 1 - (s - NB) : s % NB; };

  // ---- prefetch registers ----
  float pk[4], pe[4], pq[4], pg[4], pl[4], pu[4];  // inputs of channel ej, tokens 4*part..+3
  f32x4 pdo, pdl, pdr;                             // row tiles: row prow, columns pc4..+3
  float ptp[512 / NTH];                            // T_II, P_II elements
  float pvv[4], pww[4];                            // R: v, write at (token 4g+i, column colv)
  float pdk[4], pdla[4];                           // F2: partial d(k), partial dLam at the same
  float pq2[4], pg2[4];                            // LEAN F1: q, gamma at the same

  auto prefetch = [&](int s) {
    if (s >= NSTEP) return;
    const int sw = step_sweep(s);
    const int I = step_block(s);
    const int r0 = 16 * I;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const size_t gi = gidx(r0 + 4 * part + rr, ej);
      pk[rr] = Elem<Tin>::load(k, gi);
      pe[rr] = Elem<Tin>::load(erase, gi);
      pq[rr] = Elem<Tin>::load(q, gi);
      pg[rr] = Elem<Tin>::load(gamma, gi);
      pl[rr] = Elem<Tin>::load(log_a, gi);
      pu[rr] = sw == 0 ? Elem<Tin>::load(write, gi) * Elem<Tin>::load(v, gi) : 0.f;
    }
    if (sw != 2) pdo = load4(dO + gidx(r0 + prow, pc4));
    // deltas: not for F1; for R's first block and F2's first block they are
    // still in LDS from the step before (which computed or loaded them)
    if ((sw == 1 && I != NB - 1) || (sw == 2 && I != 0))
      pdl = load4(gDel + static_cast<size_t>(r0 + prow) * DV + pc4);
    if (sw == 2 && I != 0) pdr = load4(gdR + static_cast<size_t>(r0 + prow) * DV + pc4);
    if (sw == 1 && I != NB - 1) {
#pragma unroll
      for (int e = 0; e < 512 / NTH; ++e) ptp[e] = M::to_f32(gTP[static_cast<size_t>(I) * 512 + tid + e * NTH]);
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const size_t go = gidx(r0 + 4 * g + ii, colv);
      if (sw == 1) {
        pvv[ii] = Elem<Tin>::load(v, go);
        pww[ii] = Elem<Tin>::load(write, go);
      }
      if (sw == 2) {
        pdla[ii] = dlog_a[go];
        if (I != 0) pdk[ii] = dk[go];  // F2's block 0: kept from R's last step
      }
      if (LEAN && sw == 0) {
        pq2[ii] = Elem<Tin>::load(q, go);
        pg2[ii] = Elem<Tin>::load(gamma, go);
      }
    }
  };

  // Commit the prefetched step into LDS and form the block's factor tiles.
  // F1: sF = exp(Lam - B_I); X, Y, Z rows; Ke^T, Z^T, U^T
  // R:  sF = exp(B_{I+1} - Lam); Ke rows; X^T, Y^T, Xhat^T, Yhat^T
  // F2: sF = exp(Lam - B_I); Ke^T, Z^T
  // X = ek exp(Lam - B_I), Y = qt exp(Lam - B_I), Ke = k exp(B_{I+1} - Lam),
  // Z = k exp(B_I - Lam), Xhat = ek exp(Lam - B_{I+1}), Yhat = qt exp(Lam - B_{I+1});
  // Z, Xhat, Yhat (>= 1) only on leaves within LEAF_SAFE_RANGE.  Returns that flag.
  auto commit = [&](int s) -> int {
    const int sw = step_sweep(s);
    const int I = step_block(s);
    float cs[4], sf[4];
    {
      float run = 0.f;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        run += pl[rr];
        cs[rr] = run;
      }
      sTmp[part][ej] = run;
      sf[3] = 0.f;
      sf[2] = pl[3];
      sf[1] = pl[3] + pl[2];
      sf[0] = pl[3] + pl[2] + pl[1];
    }
    const float bsum = sBsum[I][ej];
    const int safe = __syncthreads_and(-bsum <= LEAF_SAFE_RANGE);
    float excl = 0.f, exsuf = 0.f;
#pragma unroll
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
      const float ek = pe[rr] * pk[rr];
      const float qt = pg[rr] * pq[rr];
      sLam[r][ej] = pl[rr];
      sK[r][ej] = M::cvt(pk[rr]);
      sE[r][ej] = M::cvt(pe[rr]);
      if (!LEAN) {
        sQ[r][ej] = M::cvt(pq[rr]);
        sGm[r][ej] = M::cvt(pg[rr]);
      }
      if (sw == 0) {
        const float z = safe ? pk[rr] * __expf(-loc) : 0.f;
        sF[r][ej] = fs;
        sRowA[r][ej] = M::cvt(ek * fs);
        sRowB[r][ej] = M::cvt(qt * fs);
        sRowZ[r][ej] = M::cvt(z);
        tA[rr] = pk[rr] * fe;
        tZ[rr] = z;
        tB[rr] = pu[rr];
      } else if (sw == 1) {
        const float ie = safe ? __expf(-suf) : 0.f;
        sF[r][ej] = fe;
        sRowA[r][ej] = M::cvt(pk[rr] * fe);
        tA[rr] = ek * fs;
        tB[rr] = qt * fs;
        tZ[rr] = ek * ie;
        tY[rr] = qt * ie;
      } else {
        sF[r][ej] = fs;
        tA[rr] = pk[rr] * fe;
        tZ[rr] = safe ? pk[rr] * __expf(-loc) : 0.f;
      }
    }
    store4(&sTA[ej][4 * part], tA);
    store4(&sTZ[ej][4 * part], tZ);
    if (sw == 0) store4(&sU[ej][4 * part], tB);
    if (sw == 1) {
      store4(&sTB[ej][4 * part], tB);
      store4(&sTY[ej][4 * part], tY);
    }
    if (sw != 2) store4(&sDO[prow][pc4], pdo);
    if ((sw == 1 && I != NB - 1) || (sw == 2 && I != 0)) store4(&sDL[prow][pc4], pdl);
    if (sw == 2 && I != 0) store4(&sDR[prow][pc4], pdr);
    if (sw == 1 && I != NB - 1) {
#pragma unroll
      for (int e = 0; e < 512 / NTH; ++e) {
        const int idx = tid + e * NTH;
        if (idx < 256)
          sT[idx >> 4][idx & 15] = M::cvt(ptp[e]);
        else
          sP[(idx - 256) >> 4][idx & 15] = M::cvt(ptp[e]);
      }
    }
    __syncthreads();
    return safe;
  };

  // exp(sum of log_a over tokens (i, r] of the block, channel j), r >= i
  auto pair_factor = [&](int r, int i, int j) -> float {
    float ls = 0.f;
    for (int x = i + 1; x <= r; ++x) ls += sLam[x][j];
    return __expf(ls);
  };
  auto in_q = [&](int r0, int r, int j) -> float {
    if constexpr (LEAN) return Elem<Tin>::load(q, gidx(r0 + r, j));
    else return M::to_f32(sQ[LEAN ? 0 : r][j]);
  };
  auto in_g = [&](int r0, int r, int j) -> float {
    if constexpr (LEAN) return Elem<Tin>::load(gamma, gidx(r0 + r, j));
    else return M::to_f32(sGm[LEAN ? 0 : r][j]);
  };

  // out[r][i] = A_r . B_i over the DV columns of two row tiles, masked to
  // i <= r (or i < r when strict)
  auto leaf_dot = [&](const TC (*A)[PV], const TC (*Bm)[PV], bool strict, float (*dst)[17]) {
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < DV / 16; ++kk)
      acc = M::mma(M::load(&A[c16][16 * kk + 4 * g]), M::load(&Bm[c16][16 * kk + 4 * g]), acc);
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

  // acc += A[token c16][staged columns] . sSD[channel colv][staged columns]
  auto dv_contract = [&](f32x4 acc, const TC (*A)[PV], int p) -> f32x4 {
#pragma unroll
    for (int kk = 0; kk < SW / 16; ++kk)
      acc = M::mma(M::load(&A[c16][p * SW + 16 * kk + 4 * g]), M::load(&sSD[colv][16 * kk + 4 * g]), acc);
    return acc;
  };

  // contraction of a state with rows of a [16][DV] tile over dv, all column passes
  auto state_rows = [&](const f32x4* st, const TC (*A)[PV]) -> f32x4 {
    f32x4 acc = zero4();
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
      stage_state(st, p);
      __syncthreads();
      acc = dv_contract(acc, A, p);
      __syncthreads();
    }
    return acc;
  };

  auto load_state = [&](f32x4* st, const float* src) {
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[s][i] = src[static_cast<size_t>(16 * s + 4 * g + i) * DV + colv];
  };

  auto decay_update = [&](f32x4* st, int s, const frag& a, const frag& bfr) {
    f32x4 gs;
#pragma unroll
    for (int i = 0; i < 4; ++i) gs[i] = sG[16 * s + 4 * g + i];
    st[s] = M::mma(a, bfr, st[s] * gs);
  };

  f32x4 S[RT];
  load_state(S, S0c);
  prefetch(0);
  __syncthreads();  // sBsum

  // ================= F1: forward sweep: deltas, d(qt) ==================
#pragma unroll 1
  for (int I = 0; I < NB; ++I) {
    const int r0 = 16 * I;
    const int safe = commit(I);
    float qcur[4], gcur[4];  // LEAN: this step's q, gamma (prefetch registers are reused next)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      qcur[ii] = pq2[ii];
      gcur[ii] = pg2[ii];
    }
    prefetch(I + 1);
    // leaf A_II, P_II, T_II (also kept in the scratch for the reverse sweep)
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
            const float kk = M::to_f32(sK[i][j]) * pair_factor(r, i, j);
            a += M::to_f32(sE[r][j]) * M::to_f32(sK[r][j]) * kk;
            pp += in_g(r0, r, j) * in_q(r0, r, j) * kk;
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
        const int r = 4 * g + i;
        const TC tv = M::cvt(t[i]);
        const TC pv = M::cvt(sPf[r][c16]);
        sT[r][c16] = tv;
        sP[r][c16] = pv;
        tp[r * 16 + c16] = tv;
        tp[256 + r * 16 + c16] = pv;
      }
    }
    __syncthreads();
    // Delta_I = T_II (U_I - X_I S_I)
    f32x4 Dl;
    {
      f32x4 xs = zero4();
#pragma unroll
      for (int s = 0; s < RT; ++s) xs = M::mma(M::load(&sRowA[c16][16 * s + 4 * g]), M::from_f32(S[s]), xs);
      f32x4 rhs = load4(&sU[colv][4 * g]);
      rhs -= xs;
      Dl = M::mma(M::load(&sT[c16][4 * g]), M::from_f32(rhs), zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const TC dt = M::cvt(Dl[i]);
        sDL[4 * g + i][colv] = dt;
        gDel[static_cast<size_t>(r0 + 4 * g + i) * DV + colv] = dt;
      }
    }
    __syncthreads();
    if (wave == 0) leaf_dot(sDO, sDL, false, sLf[0]);  // dO_r . Delta_i, i <= r
    // d(qt)_r = exp(Lam_r - B_I) [ S_I dO_r + sum_{i<=r} (dO_r . Delta_i) Z_i ]
    f32x4 acc = state_rows(S, sDO);
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
        for (int i2 = 0; i2 <= r; ++i2) val += sLf[0][r][i2] * pair_factor(r, i2, j) * M::to_f32(sK[i2][j]);
      const float qq = LEAN ? qcur[ii] : in_q(r0, r, j);
      const float gg = LEAN ? gcur[ii] : in_g(r0, r, j);
      const size_t gi = gidx(r0 + r, j);
      dq[gi] = gg * val;
      dgamma[gi] = qq * val;
      dlog_a[gi] = gg * qq * val;
    }
    // S_{I+1} = diag(exp(B_{I+1} - B_I)) S_I + Ke_I^T Delta_I
    {
      const frag df = M::from_f32(Dl);
#pragma unroll
      for (int s = 0; s < RT; ++s) decay_update(S, s, M::load(&sTA[16 * s + c16][4 * g]), df);
    }
    __syncthreads();
  }

  // ================= R: reverse sweep: dR, d(k) ==================
  f32x4 D[RT];
  load_state(D, dSC);
#pragma unroll 1
  for (int J = NB - 1; J >= 0; --J) {
    const int r0 = 16 * J;
    const int st = NB + (NB - 1 - J);
    const int safe = commit(st);
    float vcur[4], wcur[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      vcur[ii] = pvv[ii];
      wcur[ii] = pww[ii];
    }
    prefetch(st + 1);
    frag ptf, ttf;
    {
      f32x4 pv, tv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tv[i] = M::to_f32(sT[4 * g + i][c16]);
        pv[i] = M::to_f32(sP[4 * g + i][c16]);
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
    for (int i = 0; i < 4; ++i) dov[i] = M::to_f32(sDO[4 * g + i][colv]);
    const frag dOf = M::from_f32(dov);
    acc = M::mma(ptf, dOf, acc);
    const f32x4 dRn = M::mma(ttf, M::from_f32(acc), zero4());
    // dR rows replace the delta gradient tile; deltas of this block stay in sDL
    __syncthreads();  // all waves are done reading sU-overlapping data of the step before
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      const TC dt = M::cvt(dRn[i]);
      sDR[r][colv] = dt;
      gdR[static_cast<size_t>(r0 + r) * DV + colv] = dt;
      const size_t gi = gidx(r0 + r, colv);
      dwrite[gi] = vcur[i] * dRn[i];
      dv[gi] = wcur[i] * dRn[i];
    }
    __syncthreads();
    if (wave == 0) leaf_dot(sDO, sDL, false, sLf[0]);      // dO_r . Delta_i, r >= i
    if (wave == 1 % NW) leaf_dot(sDR, sDL, true, sLf[1]);  // dR_r . Delta_i, r > i
    // d(k)_i = exp(B_{J+1} - Lam_i) [ D Delta_i + sum_{r>=i} (dO_r.Delta_i) Yhat_r - sum_{r>i} (dR_r.Delta_i) Xhat_r ]
    f32x4 acc2 = state_rows(D, sDL);
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
          const float f = pair_factor(r, i, j);
          const float qt = in_g(r0, r, j) * in_q(r0, r, j);
          const float ek = M::to_f32(sE[r][j]) * M::to_f32(sK[r][j]);
          val += f * (sLf[0][r][i] * qt - sLf[1][r][i] * ek);
        }
      dk[gidx(r0 + i, j)] = val;
      if (J == 0) pdk[ii] = val;  // the next step (F2, block 0) reads it from here
    }
    // D <- diag(exp(B_{J+1} - B_J)) D + Y_J^T dO_J - X_J^T dR_J
    {
      const frag dRf = M::from_f32(-dRn);
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        decay_update(D, s, M::load(&sTB[16 * s + c16][4 * g]), dOf);
        D[s] = M::mma(M::load(&sTA[16 * s + c16][4 * g]), dRf, D[s]);
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
    const int st = 2 * NB + I;
    const int safe = commit(st);
    float dkcur[4], dlcur[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      dkcur[ii] = pdk[ii];
      dlcur[ii] = pdla[ii];
    }
    prefetch(st + 1);
    if (wave == 0) leaf_dot(sDR, sDL, true, sLf[1]);  // dR_r . Delta_i, i < r
    f32x4 acc = state_rows(S, sDR);
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
        for (int i2 = 0; i2 < r; ++i2) val += sLf[1][r][i2] * pair_factor(r, i2, j) * M::to_f32(sK[i2][j]);
      const float dek = -val;  // d(ek)_r = -S'_r dR_r
      const float kj = M::to_f32(sK[r][j]);
      const float bj = M::to_f32(sE[r][j]);
      const size_t gi = gidx(r0 + r, j);
      derase[gi] = kj * dek;
      dk[gi] = dkcur[ii] + bj * dek;
      dl[ii] = dlcur[ii] - kj * dkcur[ii] + bj * kj * dek;
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
      for (int i = 0; i < 4; ++i) dlt[i] = M::to_f32(sDL[4 * g + i][colv]);
      const frag df = M::from_f32(dlt);
#pragma unroll
      for (int s = 0; s < RT; ++s) decay_update(S, s, M::load(&sTA[16 * s + c16][4 * g]), df);
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

size_t bwd_chunk_scratch_bytes(const ChunkShape& s) {
  return s.bf16 ? bwd_scratch_bytes_tc<uint16_t>(s.C, s.DV) : bwd_scratch_bytes_tc<float>(s.C, s.DV);
}

hipError_t launch_bwd_chunk(const ChunkShape& s, const void* q, const void* k, const void* v,
                            const void* log_a, const void* erase, const void* write,
                            const void* gamma, const float* S_chunks, const float* dS_chunks,
                            const void* dO, float* dq, float* dk, float* dv, float* dlog_a,
                            float* derase, float* dwrite, float* dgamma, void* scratch,
                            hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(s.nchunks());
  if (grid == 0) return hipSuccess;
#define MUIR_BCH1(TT, DD, CC)                                                                      \
  hipLaunchKernelGGL((bwd_chunk_kernel<TT, DD, CC>), dim3(grid), dim3((2 * DD / 32) * 64), 0,      \
                     stream, s.T, s.H, (const TT*)q, (const TT*)k, (const TT*)v, (const TT*)log_a, \
                     (const TT*)erase, (const TT*)write, (const TT*)gamma, S_chunks, dS_chunks,    \
                     (const TT*)dO, dq, dk, dv, dlog_a, derase, dwrite, dgamma, (char*)scratch)
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

}  // namespace muir
