// Chunkwise forward of the Muir gated delta rule (gfx950).
//
// arXiv 2611.08376, Methodology and the fig:kernel caption: each chunk is a
// triangular system; cumulative log-decay is split at interval boundaries so
// every exponential factor lies in (0, 1]; the per-chunk systems are inverted
// without division (block-Neumann products at the leaves).
//
// Notation for one chunk of C tokens (b, h fixed), Lam_r = sum_{s<=r} log_a_s
// (chunk-local), u_r = write_r*v_r, ek_r = erase_r*k_r, qt_r = gamma_r*q_r:
//   A_ri = sum_j ek_rj k_ij exp(Lam_rj - Lam_ij)   (i < r)      erase system
//   P_ri = sum_j qt_rj k_ij exp(Lam_rj - Lam_ij)   (i <= r)     readout kernel
//   [U~ | W] = (I + A)^-1 [U | exp(Lam) * ek]
//   Q' = exp(Lam) * qt - P W ,  O~ = P U~ ,  Kbar_i = exp(Lam_C - Lam_i) * k_i
// so that with S the state at the chunk start
//   o = O~ + Q' S ,  Delta = U~ - W S ,  S_next = diag(exp(Lam_C)) S + Kbar^T Delta.
//
// Kernel 1 (fwd_prep, one workgroup per chunk) computes the chunk summary
// (W, Q', Kbar, U~, O~, exp(Lam_C)).  It never forms the C x C matrices:
// the chunk is walked in 16-token blocks with an inner state
//   H_I = sum_{i < 16 I} (k_i exp(B_I - Lam_i)) (x) [U~_i | W_i]     (dk x (dv+dk))
// pivoted at the block boundary B_I = Lam_{16 I - 1}, so that for block I
//   [U~|W]_I = T_II ([U|K~]_I - X_I H_I),   X_r = ek_r exp(Lam_r - B_I)
//   [O~|P W]_I = Y_I H_I + P_II [U~|W]_I,   Y_r = qt_r exp(Lam_r - B_I)
//   H_{I+1} = diag(exp(B_{I+1} - B_I)) H_I + Ke_I^T [U~|W]_I,  Ke_i = k_i exp(B_{I+1} - Lam_i)
// All factors are exponentials of non-positive numbers.  The 16 x 16 leaf
// blocks A_II, P_II are formed directly from per-pair factors
// exp(Lam_r - Lam_i), r >= i, and T_II = (I + A_II)^-1 is the exact Neumann
// product (I - A)(I + A^2)(I + A^4)(I + A^8) (A_II^16 = 0).
//
// The sequential scan over chunks (o and the chunk states from the summary)
// is in scan.hip.
#include "chunk_common.h"
#include "kernels.h"
#include "mma.h"

namespace muir {

namespace {

template <typename TC>
struct SummaryView {
  TC* W;     // [C][DK]
  TC* Qp;    // [C][DK]
  TC* KbT;   // [DK][C]
  TC* UtT;   // [DV][C]
  TC* OtT;   // [DV][C]
  float* gC; // [DK]
  TC* TP;    // [C/16][2][16][16]: T_II, P_II of each 16-token block
  __device__ SummaryView(char* base, int C, int DK, int DV) {
    TC* b = reinterpret_cast<TC*>(base);
    W = b + summary_part(SP_W, C, DK, DV);
    Qp = b + summary_part(SP_QP, C, DK, DV);
    KbT = b + summary_part(SP_KBT, C, DK, DV);
    UtT = b + summary_part(SP_UTT, C, DK, DV);
    OtT = b + summary_part(SP_OTT, C, DK, DV);
    gC = reinterpret_cast<float*>(b + summary_part(SP_END, C, DK, DV));
    TP = reinterpret_cast<TC*>(gC + DK);
  }
};

// Work split: NW = (DK + DV) / 32 waves; wave w owns columns [32w, 32w + 32)
// of the inner state [U~ | W].  For the elementwise work each thread owns one
// key channel and 4 consecutive tokens of the current block.
template <typename Tin, int DK, int C>
__global__ __launch_bounds__((2 * DK / 32) * 64) void fwd_prep_kernel(
    int T, int H, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ log_a, const Tin* __restrict__ erase,
    const Tin* __restrict__ write, const Tin* __restrict__ gamma, char* __restrict__ summ,
    size_t summ_bytes, int gmode, const int32_t* __restrict__ ncu) {
  typedef Tin TC;
  typedef MM<TC> M;
  typedef typename M::frag frag;
  constexpr int DV = DK;
  constexpr int NH = DV + DK;    // columns of the inner state: [U~ | W]
  constexpr int NW = NH / 32;    // waves
  constexpr int NTH = 64 * NW;
  constexpr int NT = 2;          // column tiles per wave
  constexpr int RT = DK / 16;    // row tiles of the inner state
  constexpr int TPC = NTH / DK;  // threads per key channel in the elementwise phase
  constexpr int NB = C / 16;     // 16-token blocks per chunk
  constexpr int PT = DK + 4;     // row stride of [16][DK] operand tiles
  static_assert(TPC == 4, "each thread owns 4 tokens of a block");

  const int NC = T / C;
  const int chunk = blockIdx.x;
  const int bh = chunk / NC;
  const int c = chunk - bh * NC;
  if (ncu && c >= *ncu) return;  // packed documents: a chunk past those in use
  const int b = bh / H;
  const int h = bh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int ej = tid % DK;       // elementwise: key channel
  const int part = tid / DK;     // elementwise: tokens 4*part .. 4*part+3 of the block

  SummaryView<TC> out(summ + static_cast<size_t>(chunk) * summ_bytes, C, DK, DV);
  // workgroup-uniform bases of the chunk; element (t, j) is at t * HD + j
  const size_t ebase = ((static_cast<size_t>(b) * T + static_cast<size_t>(c) * C) * H + h) * DK;
  const uint32_t HD = static_cast<uint32_t>(H) * DK;
  const Tin* qb = q + ebase;
  const Tin* kb = k + ebase;
  const Tin* vb = v + ebase;
  const Tin* lb = log_a + ebase;
  const Tin* eb = erase + ebase;
  const Tin* wb = write + ebase;
  // readout gate: element (t, j) at gsel + t * gts + j, with gsel and gts
  // uniform -- per token (the gate's chunk base, stride H*dk), static (the
  // head's row, stride 0), or none (q's chunk base; the value is not used)
  const Tin* gsel = gmode == GAMMA_TOKEN ? gamma + ebase
                    : gmode == GAMMA_STATIC ? gamma + static_cast<size_t>(h) * DK : q + ebase;
  const uint32_t gts = gmode == GAMMA_STATIC ? 0u : HD;
  auto gi = [&](int t, int j) -> uint32_t { return static_cast<uint32_t>(t) * HD + static_cast<uint32_t>(j); };

  // per block I and channel: B_I = Lam at the end of block I-1 (B_0 = 0)
  __shared__ float sPart[NB][TPC][DK]; // sum of log_a over each part's 4 tokens of block I
  __shared__ float sEB[NB][DK];        // exp(B_I)
  __shared__ float sEBS[NB][DK];       // exp(Lam_C - B_{I+1})
  __shared__ float sGB[NB][DK];        // exp(B_{I+1} - B_I)
  __shared__ int sUnsafe;              // bit I: block I beyond LEAF_SAFE_RANGE
  // per-block operand tiles; in bf16 double-buffered (block I in buffer I & 1)
  // so that the elementwise work of block I+1 runs beside block I's products
  // (fp32 tiles take one buffer within the LDS and the two phases alternate)
  constexpr bool PIPE = sizeof(TC) == 2;
  constexpr int NBUF = PIPE ? 2 : 1;
  __shared__ float sL[NBUF][16][DK + 1];     // log_a of the block's tokens (per-pair fallback)
  __shared__ __attribute__((aligned(16))) TC sX[NBUF][16][PT];   // ek * exp(Lam - B_I)
  __shared__ __attribute__((aligned(16))) TC sY[NBUF][16][PT];   // qt * exp(Lam - B_I)
  __shared__ __attribute__((aligned(16))) TC sZ[NBUF][16][PT];   // k * exp(B_I - Lam)   (leaf only)
  __shared__ __attribute__((aligned(16))) TC sKe[NBUF][DK][20];  // (k * exp(B_{I+1} - Lam))^T
  __shared__ __attribute__((aligned(16))) TC sR[NBUF][NH][20];   // [U | K~]^T
  __shared__ __attribute__((aligned(16))) TC sQh[NBUF][DK][20];  // (qt * exp(Lam))^T
  __shared__ float sAw[16][17];  // A_II and P_II of a leaf beyond the safe range
  __shared__ float sPf[16][17];
  // T_II, P_II of the block (bf16: in buffer I & 1, since block I+1's are
  // formed while block I's are read)
  __shared__ __attribute__((aligned(16))) TC sT[NBUF][16][20];
  __shared__ __attribute__((aligned(16))) TC sP[NBUF][16][20];
  // W and Q' rows of a block on their way to the summary; in bf16 one buffer
  // per block parity, so a block's copy-out needs no closing barrier (the
  // buffer is written again two blocks later, after two barriers)
  __shared__ __attribute__((aligned(16))) TC sStage[NBUF][16][2 * DK + 8];

  // ---- the next block's inputs are loaded one block ahead (4 tokens of
  // channel ej), kept raw until used (a conversion at the load would wait
  // for it); no load is under a branch, so they stay in flight.  The first
  // block's are issued before the prologue's own loads, so that both wait
  // on one round trip ----
  Tin pk[4], pe[4], pq[4], pg[4], pv[4], pw[4], pl[4];
  // 64-token chunks (bf16): the block sums' log_a words are kept and used by
  // the blocks' elementwise work instead of a second read
  constexpr bool KEEPL = PIPE && NB == 4;
  i16x4 lk0, lk1, lk2, lk3;  // (named, not an array: a private array would be placed in LDS)
  auto prefetch = [&](int I) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const uint32_t o = gi(16 * I + 4 * part + rr, ej);
      pk[rr] = *at(kb, o);
      pe[rr] = *at(eb, o);
      pq[rr] = *at(qb, o);
      pg[rr] = *at(gsel, static_cast<uint32_t>(16 * I + 4 * part + rr) * gts + static_cast<uint32_t>(ej));
      pv[rr] = *at(vb, o);
      pw[rr] = *at(wb, o);
      if constexpr (!KEEPL) pl[rr] = *at(lb, o);
    }
  };

  prefetch(0);

  // ---- sums of the log-decay over each part of each block, the block
  // boundaries' factors, and the blocks beyond LEAF_SAFE_RANGE ----
  if (tid == 0) sUnsafe = 0;
#pragma unroll
  for (int I = 0; I < NB; ++I) {
    float sacc = 0.f;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const Tin raw = *at(lb, gi(16 * I + 4 * part + rr, ej));
      if constexpr (KEEPL) {
        const short w = static_cast<short>(raw);
        if (I == 0) lk0[rr] = w;
        else if (I == 1) lk1[rr] = w;
        else if (I == 2) lk2[rr] = w;
        else lk3[rr] = w;
      }
      sacc += M::to_f32(raw);
    }
    sPart[I][part][ej] = sacc;
  }
  __syncthreads();
  if (tid < DK) {
    float bsum[NB];
    unsigned mask = 0;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      float bs = 0.f;
#pragma unroll
      for (int p = 0; p < TPC; ++p) bs += sPart[I][p][tid];
      bsum[I] = bs;
      sGB[I][tid] = __expf(bs);
      if (!(-bs <= LEAF_SAFE_RANGE)) mask |= 1u << I;
    }
    float acc = 0.f;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      sEB[I][tid] = __expf(acc);
      acc += bsum[I];
    }
    out.gC[tid] = __expf(acc);
    float suf = 0.f;
#pragma unroll
    for (int I = NB - 1; I >= 0; --I) {
      sEBS[I][tid] = __expf(suf);
      suf += bsum[I];
    }
    if (mask) atomicOr(&sUnsafe, static_cast<int>(mask));
  }
  __syncthreads();

  f32x4 Hs[RT][NT];
#pragma unroll
  for (int s = 0; s < RT; ++s)
#pragma unroll
    for (int n = 0; n < NT; ++n) Hs[s][n] = zero4();

  // ---- elementwise work of block I (4 tokens of channel ej) into its
  // buffer: the scaled operand rows and transposed tiles, Kbar of the summary;
  // consumes the prefetched inputs and issues the next block's loads ----
  auto elementwise = [&](int I) {
    const int bb = PIPE ? I & 1 : 0;
    const int r0 = 16 * I;
    float kv[4], ev[4], qv[4], gv[4], vv[4], wv[4], lv[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      kv[rr] = M::to_f32(pk[rr]);
      ev[rr] = M::to_f32(pe[rr]);
      qv[rr] = M::to_f32(pq[rr]);
      gv[rr] = gmode == GAMMA_NONE ? 1.f : M::to_f32(pg[rr]);
      vv[rr] = M::to_f32(pv[rr]);
      wv[rr] = M::to_f32(pw[rr]);
      if constexpr (KEEPL) {
        // block I's words by selects (no run-time index into the register array)
        const short x = I == 0 ? lk0[rr] : I == 1 ? lk1[rr] : I == 2 ? lk2[rr] : lk3[rr];
        lv[rr] = M::to_f32(static_cast<Tin>(x));
      } else {
        lv[rr] = M::to_f32(pl[rr]);
      }
    }
    prefetch(I + 1 < NB ? I + 1 : I);
    // direct partial sums (never differences of cumulative sums): prefix of
    // the block up to and including each token, and suffix after it
    float cs[4], sf[4];
    {
      float run = 0.f;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        run += lv[rr];
        cs[rr] = run;
      }
      sf[3] = 0.f;
      sf[2] = lv[3];
      sf[1] = lv[3] + lv[2];
      sf[0] = lv[3] + lv[2] + lv[1];
    }
    const int safe = !((sUnsafe >> I) & 1);
    float excl = 0.f, exsuf = 0.f;  // (selects, not branches: see sL below)
#pragma unroll
    for (int p = 0; p < TPC; ++p) {
      const float ps = sPart[I][p][ej];
      excl += p < part ? ps : 0.f;
      exsuf += p > part ? ps : 0.f;
    }
    const float eBI = sEB[I][ej];    // exp(B_I)
    const float eBS = sEBS[I][ej];   // exp(Lam_C - B_{I+1})
    f32x4 keT, uT, ktT, qhT, kbT;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * part + rr;
      const float loc = excl + cs[rr];         // Lam_r - B_I        (<= 0)
      const float suf = sf[rr] + exsuf;        // B_{I+1} - Lam_r    (<= 0)
      const float fs = __expf(loc);            // exp(Lam_r - B_I)
      const float GL = eBI * fs;               // exp(Lam_r)
      const float fe = __expf(suf);            // exp(B_{I+1} - Lam_r)
      const float kbf = fe * eBS;              // exp(Lam_C - Lam_r)
      const float ek = ev[rr] * kv[rr];
      const float qt = gv[rr] * qv[rr];
      sL[bb][r][ej] = lv[rr];  // (unconditional: a branch here would make the
                               // compiler drain every load and store in flight)
      sX[bb][r][ej] = M::cvt(ek * fs);
      sY[bb][r][ej] = M::cvt(qt * fs);
      sZ[bb][r][ej] = M::cvt(safe ? kv[rr] * __expf(-loc) : 0.f);
      keT[rr] = kv[rr] * fe;
      uT[rr] = wv[rr] * vv[rr];
      ktT[rr] = ek * GL;
      qhT[rr] = qt * GL;
      kbT[rr] = kv[rr] * kbf;
    }
    store4(&sKe[bb][ej][4 * part], keT);
    store4(&sR[bb][ej][4 * part], uT);
    store4(&sR[bb][DV + ej][4 * part], ktT);
    store4(&sQh[bb][ej][4 * part], qhT);
    store4(out.KbT + tpart_index(ej, r0 + 4 * part, DK), kbT);
  };

  // T_II = (I + A_II)^-1 from A_II (both lane layouts, see neumann16), with
  // P_II (accumulator layout), into sT, sP and the summary, by wave 0
  auto leaf_inverse = [&](int I, f32x4 a_acc, f32x4 a_tr, f32x4 p_acc) {
    const f32x4 t = neumann16(a_acc, a_tr);
    const int tb = PIPE ? I & 1 : 0;
    TC* tp = out.TP + static_cast<size_t>(I) * 512;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      const TC tv = M::cvt(t[i]);
      const TC pv = M::cvt(p_acc[i]);
      sT[tb][r][c16] = tv;
      sP[tb][r][c16] = pv;
      tp[r * 16 + c16] = tv;  // kept for the backward
      tp[256 + r * 16 + c16] = pv;
    }
  };
  // the leaf of block I within LEAF_SAFE_RANGE from its operand tiles: A = X Z^T
  // and P = Y Z^T in the accumulator layout, and A^T = Z X^T (A in the other
  // layout, from the same operands swapped); by wave 0
  auto leaf_safe = [&](int I) {
    const int lb2 = PIPE ? I & 1 : 0;
    f32x4 a = zero4(), at = zero4(), p = zero4();
#pragma unroll
    for (int s = 0; s < RT; s += 2) {
      const frag zb = M::load(&sZ[lb2][c16][16 * s + 4 * g]);
      const frag xa = M::load(&sX[lb2][c16][16 * s + 4 * g]);
      const frag ya = M::load(&sY[lb2][c16][16 * s + 4 * g]);
      const frag zb1 = M::load(&sZ[lb2][c16][16 * s + 16 + 4 * g]);
      const frag xa1 = M::load(&sX[lb2][c16][16 * s + 16 + 4 * g]);
      const frag ya1 = M::load(&sY[lb2][c16][16 * s + 16 + 4 * g]);
      a = M::mma2(xa, zb, xa1, zb1, a);
      at = M::mma2(zb, xa, zb1, xa1, at);
      p = M::mma2(ya, zb, ya1, zb1, p);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      a[i] = c16 < r ? a[i] : 0.f;    // A[r][c16], strictly lower
      at[i] = r < c16 ? at[i] : 0.f;  // A[c16][r]
      p[i] = c16 <= r ? p[i] : 0.f;
    }
    leaf_inverse(I, a, at, p);
  };

  if (PIPE) {
    elementwise(0);
    __syncthreads();
    // block 0's leaf (each later block's is formed during the block before it)
    if (!(sUnsafe & 1) && wave == 0) leaf_safe(0);
  }

#pragma unroll 1
  for (int I = 0; I < NB; ++I) {
    const int r0 = 16 * I;
    const int bb = PIPE ? I & 1 : 0;
    const int safe = !((sUnsafe >> I) & 1);
    if (!PIPE) {
      elementwise(I);
      __syncthreads();
    }

    // ---- X H and Y H for this wave's columns ----
    f32x4 XH[NT], YH[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      XH[n] = zero4();
      YH[n] = zero4();
    }
    if (I > 0) {
#pragma unroll
      for (int s = 0; s < RT; s += 2) {
        const frag xa = M::load(&sX[bb][c16][16 * s + 4 * g]);
        const frag ya = M::load(&sY[bb][c16][16 * s + 4 * g]);
        const frag xa1 = M::load(&sX[bb][c16][16 * s + 16 + 4 * g]);
        const frag ya1 = M::load(&sY[bb][c16][16 * s + 16 + 4 * g]);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const frag hb = M::from_f32(Hs[s][n]);
          const frag hb1 = M::from_f32(Hs[s + 1][n]);
          XH[n] = M::mma2(xa, hb, xa1, hb1, XH[n]);
          YH[n] = M::mma2(ya, hb, ya1, hb1, YH[n]);
        }
      }
    }
    // ---- leaf: A_II, P_II, T_II (wave 0, when the leaf is within range;
    // in bf16 it was formed during the previous block) ----
    if (!PIPE && safe && wave == 0) leaf_safe(I);
    // ---- the next block's elementwise work, beside this block's products ----
    if (PIPE && I + 1 < NB) elementwise(I + 1);
    if (!safe) {
      // per-pair factors exp(Lam_r - Lam_i) = exp(sum of log_a over (i, r]) in (0, 1]
      for (int pr = tid; pr < 256; pr += NTH) {
        const int r = pr >> 4;
        const int i = pr & 15;
        float a = 0.f, p = 0.f;
        if (i <= r) {
          for (int j = 0; j < DK; ++j) {
            const uint32_t gr = gi(r0 + r, j), gq = gi(r0 + i, j);
            float ls = 0.f;
            for (int x = i + 1; x <= r; ++x) ls += sL[bb][x][j];
            const float kk = ldv(kb, gq) * __expf(ls);
            a += ldv(eb, gr) * ldv(kb, gr) * kk;
            const float gr_ = gmode == GAMMA_NONE ? 1.f : ldv(gsel, static_cast<uint32_t>(r0 + r) * gts + j);
            p += gr_ * ldv(qb, gr) * kk;
          }
        }
        sAw[r][i] = i < r ? a : 0.f;
        sPf[r][i] = p;
      }
      __syncthreads();
      if (wave == 0) {
        f32x4 a, at, p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = sAw[4 * g + i][c16];
          at[i] = sAw[c16][4 * g + i];
          p[i] = sPf[4 * g + i][c16];
        }
        leaf_inverse(I, a, at, p);
      }
    }
    __syncthreads();

    // ---- the next block's leaf (bf16), beside this block's products ----
    if (PIPE && I + 1 < NB && !((sUnsafe >> (I + 1)) & 1) && wave == 0) leaf_safe(I + 1);
    // ---- [U~|W]_I = T_II (R_I - X_I H_I);  [O~|PW]_I = Y_I H_I + P_II [U~|W]_I ----
    const int tb = PIPE ? I & 1 : 0;
    const frag ta = M::load(&sT[tb][c16][4 * g]);
    const frag pa = M::load(&sP[tb][c16][4 * g]);
    f32x4 UW[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int colg = wave * 32 + 16 * n + c16;
      const f32x4 rhs = load4(&sR[bb][colg][4 * g]) - XH[n];
      const f32x4 uw = M::mma(ta, M::from_f32(rhs), zero4());
      const f32x4 op = M::mma(pa, M::from_f32(uw), YH[n]);
      UW[n] = uw;
      if (colg < DV) {
        store4(out.UtT + tpart_index(colg, r0 + 4 * g, DV), uw);
        store4(out.OtT + tpart_index(colg, r0 + 4 * g, DV), op);
      } else {
        const int j = colg - DV;
        const f32x4 qv = load4(&sQh[bb][j][4 * g]) - op;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sStage[tb][4 * g + i][j] = M::cvt(uw[i]);
          sStage[tb][4 * g + i][DK + j] = M::cvt(qv[i]);
        }
      }
    }
    // ---- advance the inner state to the next block boundary ----
    if (I + 1 < NB) {
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        const frag ka = M::load(&sKe[bb][16 * s + c16][4 * g]);
        f32x4 gs;
#pragma unroll
        for (int i = 0; i < 4; ++i) gs[i] = sGB[I][16 * s + 4 * g + i];
#pragma unroll
        for (int n = 0; n < NT; ++n) Hs[s][n] = M::mma(ka, M::from_f32(UW[n]), Hs[s][n] * gs);
      }
    }
    __syncthreads();
    {
      // W and Q' rows of the block, 4 elements per store
      for (int idx = tid; idx < 16 * DK / 4; idx += NTH) {
        const int r = idx / (DK / 4);
        const int j4 = (idx - r * (DK / 4)) * 4;
        typedef typename Raw4<TC>::type R4;
        *reinterpret_cast<R4*>(out.W + static_cast<size_t>(r0 + r) * DK + j4) =
            *reinterpret_cast<const R4*>(&sStage[tb][r][j4]);
        *reinterpret_cast<R4*>(out.Qp + static_cast<size_t>(r0 + r) * DK + j4) =
            *reinterpret_cast<const R4*>(&sStage[tb][r][DK + j4]);
      }
      if (!PIPE) __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_fwd_prep(const ChunkShape& s, const void* q, const void* k, const void* v,
                           const void* log_a, const void* erase, const void* write,
                           const void* gamma, void* summ, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(s.nchunks());
  if (grid == 0) return hipSuccess;
#define MUIR_PREP1(TT, DD, CC)                                                                     \
  hipLaunchKernelGGL((fwd_prep_kernel<TT, DD, CC>), dim3(grid), dim3((2 * DD / 32) * 64), 0,         \
                     stream, s.T, s.H, (const TT*)q, (const TT*)k, (const TT*)v, (const TT*)log_a, \
                     (const TT*)erase, (const TT*)write, (const TT*)gamma, (char*)summ,            \
                     s.summary_bytes(), s.gmode, s.ncu)
#define MUIR_PREP(TT, DD)                         \
  do {                                            \
    if (s.C == 64) MUIR_PREP1(TT, DD, 64);        \
    else if (s.C == 128) MUIR_PREP1(TT, DD, 128); \
    else MUIR_PREP1(TT, DD, 256);                 \
  } while (0)
  if (s.bf16) {
    if (s.DK == 128) MUIR_PREP(uint16_t, 128);
    else MUIR_PREP(uint16_t, 64);
  } else {
    if (s.DK == 128) MUIR_PREP(float, 128);
    else MUIR_PREP(float, 64);
  }
#undef MUIR_PREP
#undef MUIR_PREP1
  return hipGetLastError();
}

}  // namespace muir
