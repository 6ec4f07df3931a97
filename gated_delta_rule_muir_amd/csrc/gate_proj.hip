// Gate prologue of the Muir operator: the fused low-rank gate projection and
// the SiLU + L2 normalisation of the query / key pathways, forward and
// backward (arXiv 2611.08376; wolonglab summary page, §Methodology: one
// down-projection shared by the five gates, five up-projections at ranks
// (64, 64, 128, 128, 128) with channel biases; fig:arch (b), (c)).
//
// The gates' up-projections run in gate_up_kernel (the rank-64/128
// contraction with the activation, or its gradient and the bias sums, fused
// into the epilogue).  Every other product runs through one grouped GEMM
// kernel: up to five independent problems per launch, 128 x BN tiles on four
// waves, bf16 (v_mfma_f32_16x16x32_bf16) or fp32 (v_mfma_f32_16x16x4_f32)
// with fp32 accumulation, and an epilogue chosen at compile time:
//   EPI_STORE     C = acc, in the compute type
//   EPI_PARTIAL   fp32 partial of one split of the contraction
// Operands are read either along their contiguous axis (k contiguous: rows of
// A, columns of B^T) or across it (k strided), the latter transposed on the
// way into LDS, so every product here -- x W_down^T, dpre U, dz W_down,
// dz^T x, dpre^T z -- runs without an explicit transpose.
#include <algorithm>
#include <type_traits>

#include "kernels.h"
#include "mma.h"

namespace muir {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int GEMM_THREADS = 256;
constexpr int UP_THREADS = 256;
constexpr int UP_BN = 64;  // columns per tile of the up-projection kernel
constexpr int UP_CT = 8;   // consecutive column tiles per workgroup of the up-projection kernel

enum Epi {
  EPI_STORE = 0,     // general GEMM: C = acc in the compute type
  EPI_GATE = 1,      // up-projection: gate = act(acc + bias)
  EPI_GATE_BWD = 2,  // up-projection: dpre = dG * act'(acc + bias), with per-tile column sums
  EPI_PARTIAL = 3    // general GEMM: fp32 partial of one split of the contraction
};

// Per-compute-type GEMM fragment: bf16 contracts 32 per MFMA (8 values per
// lane at k = 8*(lane/16) + i), fp32 contracts 16 per group of four MFMAs
// (4 values per lane at k = 4*(lane/16) + i, the MM<float> placement).
template <typename TC> struct GF;
template <> struct GF<uint16_t> {
  static constexpr int KF = 32;
  static constexpr int PAD = 8;
  typedef bf16x8 frag;
  static __device__ __forceinline__ frag load(const uint16_t* p) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(p));
  }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct GF<float> {
  static constexpr int KF = 16;
  static constexpr int PAD = 4;
  typedef f32x4 frag;
  static __device__ __forceinline__ frag load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) { return MM<float>::mma(a, b, c); }
};

// Hardware exp2 / log2 / reciprocal (v_exp_f32, v_log_f32, v_rcp_f32, about
// 1 ulp; denormal results flush to zero), far inside the tolerance of the
// compute types.
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-LOG2E * x));
}

// Gate activations (readings of the pages: log-decay = log sigmoid; erase,
// write and the output gate sigmoid; the readout gain 2 sigmoid).
// log sigmoid(x) = min(x, 0) - log(1 + e^-|x|); the logarithm of 1 + e with
// e <= 1 loses at most e ~ 6e-8 (absolute) when e is below fp32 resolution.
__device__ __forceinline__ float act_fwd(int act, float x) {
  switch (act) {
    case GATE_ACT_LOGSIG:
      return fminf(x, 0.f) - LN2 * __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-LOG2E * fabsf(x)));
    case GATE_ACT_SIG: return sigmoidf_(x);
    case GATE_ACT_SIG2: return 2.f * sigmoidf_(x);
    default: return x;
  }
}
__device__ __forceinline__ float act_grad(int act, float x) {
  switch (act) {
    case GATE_ACT_LOGSIG: return sigmoidf_(-x);
    case GATE_ACT_SIG: {
      const float s = sigmoidf_(x);
      return s - s * s;
    }
    case GATE_ACT_SIG2: {
      const float s = sigmoidf_(x);
      return 2.f * (s - s * s);
    }
    default: return 1.f;
  }
}

// Arguments of the gates' up-projection kernel (all five gates in one launch).
template <typename TC> struct GateUpArgs {
  const TC* z;     // [M, 512]
  const TC* U;     // packed up matrices
  const TC* bias;  // packed biases
  TC* out[5];      // gates (forward) or their pre-activation gradients (backward), [M, W_i]
  const TC* dG[5];  // backward: the gates' gradients, [M, W_i]
  float* colsum;   // backward: per-tile column sums [m tiles][colsum_ld]
  int colsum_ld;
  int M;
  int r[5], W[5], zoff[5], act[5], csoff[5];
  size_t woff[5], boff[5];
};

template <typename TC> struct GemmStep;
template <> struct GemmStep<uint16_t> { static constexpr int BK = 64; };
template <> struct GemmStep<float> { static constexpr int BK = 32; };

// Transposes a block of 16-byte words: in[r] holds KR consecutive-k rows of E
// columns; out[c] receives column c's KR values (k ascending).  bf16: 8 x 8
// (byte permutes pair up the 16-bit halves), fp32: 4 x 4 (register moves).
__device__ __forceinline__ void transpose_block(const uint4 (&in)[8], uint4 (&out)[8]) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(in);  // w[4*r + c/2]
  uint32_t* o = reinterpret_cast<uint32_t*>(out);             // o[4*c + p]
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = w[4 * (2 * p) + c / 2], hi = w[4 * (2 * p + 1) + c / 2];
      o[4 * c + p] = __builtin_amdgcn_perm(hi, lo, (c & 1) ? 0x07060302u : 0x05040100u);
    }
}
__device__ __forceinline__ void transpose_block(const uint4 (&in)[4], uint4 (&out)[4]) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(in);  // w[4*r + c]
  uint32_t* o = reinterpret_cast<uint32_t*>(out);             // o[4*c + r]
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[4 * c + r] = w[4 * r + c];
}

// Grouped GEMM, C_g = A_g B_g for the problems of `batch` (blockIdx.y picks
// problem and contraction split).  128 x BN tile on four waves (2 x 2), each
// wave 64 x BN/2 as 16 x 16 MFMA tiles.  The MFMA is issued with the B tile
// as its row operand, so each lane ends with four consecutive output columns
// of one row (lane (g, c16): row c16, columns 4g .. 4g+3 of each 16 x 16
// tile) and the epilogue stores straight from registers.
template <typename TC, int BM, int BN, bool A_KC, bool B_KC, int EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(GemmBatch batch) {
  typedef GF<TC> F;
  constexpr int BK = GemmStep<TC>::BK;
  constexpr int E = 16 / sizeof(TC);  // elements per 16-byte word
  constexpr int LDK = BK + F::PAD;    // LDS row pitch of an operand tile (elements)
  constexpr int TM = BM / 32, TN = BN / 32;  // 16 x 16 tiles per wave
  __shared__ __align__(16) TC sA[BM * LDK];
  __shared__ __align__(16) TC sB[BN * LDK];

  const int grp = blockIdx.y / batch.ksplit;
  const int split = blockIdx.y - grp * batch.ksplit;
  const GemmProblem& P = batch.p[grp];
  // XCD-aware tile order: consecutive workgroup ids go to different XCDs, so
  // each XCD is given a contiguous run of tiles, n fastest: the A rows of a
  // tile row are then reused from that XCD's L2.
  // (The grid's x extent is a multiple of 8, so blockIdx.x % 8 is the XCD.)
  const int mt = (P.M + BM - 1) / BM, nt = (P.N + BN - 1) / BN;
  const int ntile = mt * nt;
  const int per_xcd = (ntile + 7) / 8;
  const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (static_cast<int>(blockIdx.x / 8) >= per_xcd || t >= ntile) return;
  const int m0 = (t / nt) * BM;
  const int n0 = (t % nt) * BN;
  const int kbeg = split * batch.kchunk;
  const int kend = min(P.K, kbeg + batch.kchunk);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = (wave >> 1) * (BM / 2);
  const int wn = (wave & 1) * (BN / 2);
  const TC* __restrict__ gA = static_cast<const TC*>(P.A);
  const TC* __restrict__ gB = static_cast<const TC*>(P.B);

  // ---- global -> register staging --------------------------------------------
  // k-contiguous operand: R rows of BK values as 16-byte words, 8 per row
  // (row r, word w at tile index r * 8 + w).
  constexpr int KCW_A = BM * BK / E / GEMM_THREADS, KCW_B = BN * BK / E / GEMM_THREADS;
  // k-strided operand: blocks of KR k rows x E columns, staged by up to 128
  // threads each (A: threads 0.., B: 128.. when A is k-strided too, else 0..).
  constexpr int KR = 16 / sizeof(TC);
  constexpr int KSB_A = (BK / KR) * (BM / E), KSB_B = (BK / KR) * (BN / E);
  constexpr int KST_A = KSB_A < 128 ? KSB_A : 128, KST_B = KSB_B < 128 ? KSB_B : 128;
  static_assert(A_KC || KSB_A % KST_A == 0, "k-strided A tile must split over its threads");
  static_assert(B_KC || KSB_B % KST_B == 0, "k-strided B tile must split over its threads");
  constexpr int KS_PER_A = A_KC ? 0 : KSB_A / KST_A;
  constexpr int KS_PER_B = B_KC ? 0 : KSB_B / KST_B;
  constexpr int NRA = A_KC ? KCW_A : KS_PER_A * KR;
  constexpr int NRB = B_KC ? KCW_B : KS_PER_B * KR;
  static_assert(NRA >= 1 && NRB >= 1, "tile too small for the thread count");
  uint4 ra[NRA], rb[NRB];
  constexpr int B_BASE = A_KC ? 0 : 128;
  const bool a_ks_thread = !A_KC && tid < KST_A;
  const bool b_ks_thread = !B_KC && tid >= B_BASE && tid < B_BASE + KST_B;

  auto load_kc = [&](const TC* g, int ld, int rows_valid, int r0, int k0, uint4* r, int nw) {
    constexpr int WPR = BK / E;
    for (int w = 0; w < nw; ++w) {
      const int idx = tid + w * GEMM_THREADS;
      const int row = idx / WPR;
      const int gk = k0 + (idx % WPR) * E;
      uint4 v = {0u, 0u, 0u, 0u};
      if (r0 + row < rows_valid && gk < kend)
        v = *reinterpret_cast<const uint4*>(g + static_cast<size_t>(r0 + row) * ld + gk);
      r[w] = v;
    }
  };
  auto store_kc = [&](TC* s, const uint4* r, int nw) {
    constexpr int WPR = BK / E;
    for (int w = 0; w < nw; ++w) {
      const int idx = tid + w * GEMM_THREADS;
      *reinterpret_cast<uint4*>(s + (idx / WPR) * LDK + (idx % WPR) * E) = r[w];
    }
  };
  // block b: k block kb = b % (BK / KR) (so the 8 lanes of a store phase write
  // different k blocks of one column group: no LDS bank conflicts), column
  // block cb = b / (BK / KR).
  auto load_ks = [&](const TC* g, int ld, int cols_valid, int c0, int k0, uint4* r, int nb, int ks_tid, int nthr) {
    for (int i = 0; i < nb; ++i) {
      const int b = ks_tid + i * nthr;
      const int kb = b % (BK / KR), cb = b / (BK / KR);
      const int gc = c0 + cb * E;
#pragma unroll
      for (int rr = 0; rr < KR; ++rr) {
        const int gk = k0 + kb * KR + rr;
        uint4 v = {0u, 0u, 0u, 0u};
        if (gc < cols_valid && gk < kend) v = *reinterpret_cast<const uint4*>(g + static_cast<size_t>(gk) * ld + gc);
        r[i * KR + rr] = v;
      }
    }
  };
  auto store_ks = [&](TC* s, const uint4* r, int nb, int ks_tid, int nthr) {
    for (int i = 0; i < nb; ++i) {
      const int b = ks_tid + i * nthr;
      const int kb = b % (BK / KR), cb = b / (BK / KR);
      uint4 in[KR], out[KR];
#pragma unroll
      for (int rr = 0; rr < KR; ++rr) in[rr] = r[i * KR + rr];
      transpose_block(in, out);
#pragma unroll
      for (int c = 0; c < E; ++c) *reinterpret_cast<uint4*>(s + (cb * E + c) * LDK + kb * KR) = out[c];
    }
  };
  auto load_tiles = [&](int k0) {
    if constexpr (A_KC) load_kc(gA, P.lda, P.M, m0, k0, ra, NRA);
    else if (a_ks_thread) load_ks(gA, P.lda, P.M, m0, k0, ra, KS_PER_A, tid, KST_A);
    if constexpr (B_KC) load_kc(gB, P.ldb, P.N, n0, k0, rb, NRB);
    else if (b_ks_thread) load_ks(gB, P.ldb, P.N, n0, k0, rb, KS_PER_B, tid - B_BASE, KST_B);
  };
  auto store_tiles = [&]() {
    if constexpr (A_KC) store_kc(sA, ra, NRA);
    else if (a_ks_thread) store_ks(sA, ra, KS_PER_A, tid, KST_A);
    if constexpr (B_KC) store_kc(sB, rb, NRB);
    else if (b_ks_thread) store_ks(sB, rb, KS_PER_B, tid - B_BASE, KST_B);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero4();

  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const int fr = lane & 15;
  const int fk = (F::KF / 4) * (lane >> 4);
  if (nk > 0) load_tiles(kbeg);
  for (int kt = 0; kt < nk; ++kt) {
    store_tiles();
    __syncthreads();
    if (kt + 1 < nk) load_tiles(kbeg + (kt + 1) * BK);  // lands while this step computes
#pragma unroll
    for (int ks = 0; ks < BK; ks += F::KF) {
      typename F::frag fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = F::load(sA + (wm + 16 * i + fr) * LDK + ks + fk);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = F::load(sB + (wn + 16 * j + fr) * LDK + ks + fk);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = F::mma(fb[j], fa[i], acc[i][j]);
    }
    __syncthreads();
  }

  // ---- epilogue, from registers ------------------------------------------------
  // acc[i][j][r] = C[m0 + wm + 16i + fr][n0 + wn + 16j + 4g + r], g = lane / 16
  const int g4 = 4 * (lane >> 4);
  if constexpr (EPI == EPI_PARTIAL) {
    float* out = static_cast<float*>(P.C) + static_cast<size_t>(split) * batch.split_stride;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int gm = m0 + wm + 16 * i + fr;
      if (gm >= P.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int gn = n0 + wn + 16 * j + g4;
        if (gn < P.N) *reinterpret_cast<f32x4*>(out + static_cast<size_t>(gm) * P.ldc + gn) = acc[i][j];
      }
    }
  } else {
    TC* out = static_cast<TC*>(P.C);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int gm = m0 + wm + 16 * i + fr;
      if (gm >= P.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int gn = n0 + wn + 16 * j + g4;
        if (gn < P.N) store4(out + static_cast<size_t>(gm) * P.ldc + gn, acc[i][j]);
      }
    }
  }
}

// Activation as a template argument (one instance per gate form).
template <int ACT> __device__ __forceinline__ float act_fwd_t(float x) { return act_fwd(ACT, x); }
template <int ACT> __device__ __forceinline__ float act_grad_t(float x) { return act_grad(ACT, x); }

// One column tile's operands of the up-projection kernel, to registers: the
// U block (BN rows of the gate's rank, as 16-byte words; words past the
// block repeat its last) and, for the backward (DG), this thread's staged
// words of the upstream gradient (rows dgrow0 + s * RSTEP, clamped to the
// last row; rows past it are not used).
template <typename TC, bool DG, int MAXW, int SW, int RSTEP>
__device__ __forceinline__ void up_load_tile(u32x4 (&rb)[MAXW], u32x4 (&dgw)[SW], const TC* __restrict__ U,
                                             const TC* __restrict__ dG, int n0, int r, int W, int nwords, int tid,
                                             int dgrow0, int M, int scol) {
  constexpr int E = 16 / sizeof(TC);
  const int wpr = r / E;
#pragma unroll
  for (int w = 0; w < MAXW; ++w) {
    const int idx = min(tid + w * UP_THREADS, nwords - 1);
    rb[w] = *reinterpret_cast<const u32x4*>(U + static_cast<size_t>(n0 + idx / wpr) * r + (idx % wpr) * E);
  }
  if constexpr (DG) {
#pragma unroll
    for (int sw = 0; sw < SW; ++sw) {
      const int gm = min(dgrow0 + sw * RSTEP, M - 1);
      dgw[sw] = *reinterpret_cast<const u32x4*>(dG + static_cast<size_t>(gm) * W + n0 + scol);
    }
  }
}

// The gates' up-projections (contraction over one gate's rank, 64 or 128):
// C = z_i U_i^T + c_i with an activation epilogue (EPI_GATE) or its gradient
// (EPI_GATE_BWD).  A workgroup of 4 waves owns a 128-row block of one gate
// and UP_CT consecutive 64-column tiles; wave w owns rows 32 w .. +31.  The
// wave's rows of z are loaded once, straight into MFMA fragments, and stay in
// registers across the tiles (one tile per workgroup read each row block of z
// once per tile).  Each tile's U_i block (64 rows of [width, rank], rank
// contiguous) and, in the backward, its upstream gradients are loaded during
// the previous tile's products and written to LDS at the tile's start.  The
// next tile's loads are issued before this tile's stores and without a branch
// (addresses clamped), so no wait on them sits behind this workgroup's own
// stores (loads and stores share one counter).  The gradient tile is read,
// and the output tile written, through an LDS staging tile in whole 128-byte
// rows (8 lanes per row), not in the MFMA layout's 32-byte pieces.
// blockIdx.x: the row block (fastest), then the group of column tiles;
// blockIdx.y: the gate.
template <typename TC, int EPI>
__global__ __launch_bounds__(UP_THREADS) void gate_up_kernel(GateUpArgs<TC> a) {
  typedef GF<TC> F;
  constexpr int E = 16 / sizeof(TC);
  constexpr int RMAX = 128;
  constexpr int LDK = RMAX + F::PAD;
  constexpr int BM = 128, BN = UP_BN, TM = 2, TN = BN / 16;
  constexpr int KSTEPS = RMAX / F::KF;
  constexpr int MAXW = BN * (RMAX / E) / UP_THREADS;  // 16-byte words of the U tile per thread
  constexpr int LDS_ = BN + E;                         // staging pitch (elements): one 16-byte pad per row
  constexpr int WPR = BN / E;                          // 16-byte words per staged row
  constexpr int SW = BM * WPR / UP_THREADS;            // staged words per thread
  __shared__ __align__(16) TC sB[2][BN * LDK];  // U blocks of the current and the next tile
  __shared__ __align__(16) TC sS[BM * LDS_];
  __shared__ float red[2][4 * BN];

  const int gi = blockIdx.y;
  const int r = a.r[gi];
  const int W = a.W[gi];
  const int mt = (a.M + BM - 1) / BM;
  const int ntiles = W / BN;
  const int ngrp = (ntiles + UP_CT - 1) / UP_CT;
  if (static_cast<int>(blockIdx.x) >= mt * ngrp) return;
  const int mtile = blockIdx.x % mt;
  const int t0 = (blockIdx.x / mt) * UP_CT;
  const int t1 = min(ntiles, t0 + UP_CT);
  const int m0 = mtile * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = 32 * wave;
  const int fr = lane & 15, fk = (F::KF / 4) * (lane >> 4), g4 = 4 * (lane >> 4);
  const TC* __restrict__ z = a.z + a.zoff[gi];
  const TC* __restrict__ U = a.U + a.woff[gi];
  const TC* __restrict__ bias = a.bias + a.boff[gi];
  TC* __restrict__ out = a.out[gi];
  const int ksteps = r / F::KF;
  // staged words of this wave's 32 rows: word s of the thread is row
  // wm + s * (64 / WPR) + lane / WPR, columns (lane % WPR) * E ..
  auto srow = [&](int sw) { return wm + sw * (64 / WPR) + lane / WPR; };
  const int scol = (lane % WPR) * E;
  const int wpr = r / E;
  const int nwords = BN * wpr;

  // the wave's rows of z, once
  typename F::frag fa[TM][KSTEPS];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int gm = m0 + wm + 16 * i + fr;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint4 v = {0u, 0u, 0u, 0u};
      if (gm < a.M && ks < ksteps)
        v = *reinterpret_cast<const uint4*>(z + static_cast<size_t>(gm) * GATE_RTOT + ks * F::KF + fk);
      fa[i][ks] = __builtin_bit_cast(typename F::frag, v);
    }
  }
  // a tile's U block and upstream gradients, to registers
  u32x4 rb[MAXW];
  u32x4 dgw[SW];
  const int dgrow0 = m0 + wm + lane / WPR;
  constexpr bool BWD = EPI == EPI_GATE_BWD;
  auto put_tile = [&](TC* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < MAXW; ++w) {
      const int idx = min(tid + w * UP_THREADS, nwords - 1);
      *reinterpret_cast<u32x4*>(&dst[(idx / wpr) * LDK + (idx % wpr) * E]) = rb[w];
    }
    if constexpr (BWD) {
#pragma unroll
      for (int sw = 0; sw < SW; ++sw) *reinterpret_cast<u32x4*>(&sS[srow(sw) * LDS_ + scol]) = dgw[sw];
    }
  };
  // the four waves' column sums of a tile's dpre, from its partial-sum buffer
  auto put_colsum = [&](int t, const float* rd) __attribute__((always_inline)) {
    if (tid < BN)
      a.colsum[static_cast<size_t>(mtile) * a.colsum_ld + a.csoff[gi] + t * BN + tid] =
          rd[tid] + rd[BN + tid] + rd[2 * BN + tid] + rd[3 * BN + tid];
  };
  up_load_tile<TC, BWD, MAXW, SW, 64 / WPR>(rb, dgw, U, a.dG[gi], t0 * BN, r, W, nwords, tid, dgrow0, a.M, scol);
  put_tile(sB[0]);

#pragma unroll 1
  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    const int n0 = t * BN;
    // tile t's U block is in sB[buf] (and its dG words in sS); every wave is
    // done with tile t - 1, so sB[buf ^ 1] and red[buf ^ 1] are free once read
    __syncthreads();
    if constexpr (BWD) {
      if (t > t0) put_colsum(t - 1, red[buf ^ 1]);
    }
    // the next tile's operands, in flight during this one
    up_load_tile<TC, BWD, MAXW, SW, 64 / WPR>(rb, dgw, U, a.dG[gi], (t + 1 < t1 ? t + 1 : t) * BN, r, W, nwords,
                                              tid, dgrow0, a.M, scol);

    // accumulators start from the bias (lane: columns 16j + 4g .. + 3)
    f32x4 acc[TM][TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const f32x4 bv = load4(bias + n0 + 16 * j + g4);
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i][j] = bv;
    }
    const TC* sb = sB[buf];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (ks < ksteps) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const typename F::frag fb = F::load(&sb[(16 * j + fr) * LDK + ks * F::KF + fk]);
#pragma unroll
          for (int i = 0; i < TM; ++i) acc[i][j] = F::mma(fb, fa[i][ks], acc[i][j]);
        }
      }
    }

    // epilogue in the MFMA layout (lane: row wm + 16i + fr, columns 16j + 4g ..
    // + 3 of the tile), through this wave's rows of the staging tile
    float* rd = red[buf];
    auto epilogue = [&](auto act_tag) {
      constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int c = 16 * j + g4;
        float cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = wm + 16 * i + fr;
          f32x4 v = acc[i][j];
          if constexpr (!BWD) {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = act_fwd_t<ACT>(v[q]);
          } else {
            const f32x4 gv = load4(&sS[row * LDS_ + c]);
            const bool row_ok = m0 + row < a.M;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              v[q] = gv[q] * act_grad_t<ACT>(v[q]);
              cs[q] += row_ok ? v[q] : 0.f;
            }
          }
          store4(&sS[row * LDS_ + c], v);
        }
        if constexpr (BWD) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float sm = sum16(cs[q]);
            if (fr == 0) rd[wave * BN + c + q] = sm;
          }
        }
      }
    };
    switch (a.act[gi]) {
      case GATE_ACT_LOGSIG: epilogue(std::integral_constant<int, GATE_ACT_LOGSIG>{}); break;
      case GATE_ACT_SIG: epilogue(std::integral_constant<int, GATE_ACT_SIG>{}); break;
      case GATE_ACT_SIG2: epilogue(std::integral_constant<int, GATE_ACT_SIG2>{}); break;
      default: epilogue(std::integral_constant<int, GATE_ACT_NONE>{}); break;
    }
    // this wave's rows back out in whole rows (the wave wrote them itself: LDS
    // operations of one wave complete in order)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    TC* o = out + n0 + scol;
#pragma unroll
    for (int sw = 0; sw < SW; ++sw) {
      const int row = srow(sw);
      if (m0 + row < a.M)
        *reinterpret_cast<uint4*>(o + static_cast<size_t>(m0 + row) * W) =
            *reinterpret_cast<const uint4*>(&sS[row * LDS_ + scol]);
    }
    // the next tile's operands to LDS: sB[buf ^ 1] was last read in tile t - 1,
    // which every wave finished before this tile's barrier; the dG words go to
    // this wave's own staging rows after its reads of them above
    if (t + 1 < t1) put_tile(sB[buf ^ 1]);
  }
  if constexpr (BWD) {
    __syncthreads();
    put_colsum(t1 - 1, red[(t1 - 1 - t0) & 1]);
  }
}

// Column sums of a [rows][ncols] fp32 array (the bias gradient from the
// per-row-tile partial sums): 32 columns per block, the rows split over 8
// thread groups, then combined in LDS in a fixed order.
__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ part, int rows, int ncols,
                                                     float* __restrict__ out) {
  __shared__ float red[8][32];
  const int c = blockIdx.x * 32 + (threadIdx.x & 31);
  const int g = threadIdx.x >> 5;
  float s = 0.f;
  if (c < ncols)
    for (int r = g; r < rows; r += 8) s += part[static_cast<size_t>(r) * ncols + c];
  red[g][threadIdx.x & 31] = s;
  __syncthreads();
  if (threadIdx.x < 32 && c < ncols) {
    float t = 0.f;
    for (int k = 0; k < 8; ++k) t += red[k][threadIdx.x];
    out[c] = t;
  }
}

// Sum of `nsplit` fp32 partials of n values each (stride `stride`) into out.
__global__ void split_sum_kernel(const float* __restrict__ part, int nsplit, size_t stride, size_t n,
                                 float* __restrict__ out) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    float s = 0.f;
    for (int k = 0; k < nsplit; ++k) s += part[k * stride + i];
    out[i] = s;
  }
}

// One 16-byte word of a row as fp32 values, and back (bf16: the hardware
// round-to-nearest-even conversion, as every other bf16 store here).
template <typename TC> struct QkWord;
template <> struct QkWord<uint16_t> {
  static constexpr int V = 8;
  static __device__ __forceinline__ void unpack(u32x4 w, float (&x)[V]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float (&x)[V]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    return w;
  }
};
template <> struct QkWord<float> {
  static constexpr int V = 4;
  // (whole-vector casts: a bit cast of one subscripted vector element was
  // compiled as a cast of element 0)
  static __device__ __forceinline__ void unpack(u32x4 w, float (&x)[V]) {
    const f32x4 f = __builtin_bit_cast(f32x4, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = f[i];
  }
  static __device__ __forceinline__ u32x4 pack(const float (&x)[V]) {
    const f32x4 f = {x[0], x[1], x[2], x[3]};
    return __builtin_bit_cast(u32x4, f);
  }
};

constexpr int QK_THREADS = 256;
constexpr int QK_RPT = 4;  // rows per thread group, all loaded before the first use
template <typename TC, int D> struct QkShape {
  static constexpr int V = QkWord<TC>::V;     // values per lane (one 16-byte word)
  static constexpr int G = D / V;             // lanes per row
  static constexpr int RB = QK_THREADS / G;   // rows per pass of the workgroup
  static constexpr int ROWS = RB * QK_RPT;    // rows per workgroup
};

// SiLU then L2 normalisation over each row of D values (one head of q or k):
// y = s / sqrt(sum s^2 + eps), s = u sigmoid(u).  A row is G lanes of one
// 16-byte word each; the row sums are taken with lane shuffles inside the
// group.  Each lane group handles QK_RPT rows, RB apart, and issues all their
// loads first, so that several words per lane are in flight.
template <typename TC, int D>
__global__ __launch_bounds__(QK_THREADS) void qk_norm_fwd_kernel(const TC* __restrict__ u, TC* __restrict__ y,
                                                                 long long rows) {
  typedef QkShape<TC, D> S;
  typedef QkWord<TC> W;
  const int l = threadIdx.x % S::G;
  const long long r0 = static_cast<long long>(blockIdx.x) * S::ROWS + threadIdx.x / S::G;
  // rows past the end read the last row (rows >= 1) and are not stored
  u32x4 w[QK_RPT];
#pragma unroll
  for (int k = 0; k < QK_RPT; ++k)
    w[k] = *reinterpret_cast<const u32x4*>(u + min(r0 + k * S::RB, rows - 1) * D + S::V * l);
#pragma unroll
  for (int k = 0; k < QK_RPT; ++k) {
    const long long row = r0 + k * S::RB;
    float x[S::V];
    W::unpack(w[k], x);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < S::V; ++i) {
      x[i] = x[i] * sigmoidf_(x[i]);
      ss += x[i] * x[i];
    }
#pragma unroll
    for (int off = S::G / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = rsqrtf(ss + QK_L2_EPS);
#pragma unroll
    for (int i = 0; i < S::V; ++i) x[i] *= inv;
    if (row < rows) *reinterpret_cast<u32x4*>(y + row * D + S::V * l) = W::pack(x);
  }
}

// Reverse mode: du = (dy - y (y . dy)) / n * silu'(u), rows as in the forward.
template <typename TC, int D>
__global__ __launch_bounds__(QK_THREADS) void qk_norm_bwd_kernel(const TC* __restrict__ u, const TC* __restrict__ dy,
                                                                 TC* __restrict__ du, long long rows) {
  typedef QkShape<TC, D> S;
  typedef QkWord<TC> W;
  const int l = threadIdx.x % S::G;
  const long long r0 = static_cast<long long>(blockIdx.x) * S::ROWS + threadIdx.x / S::G;
  // rows past the end read the last row (rows >= 1) and are not stored
  u32x4 wu[QK_RPT], wg[QK_RPT];
#pragma unroll
  for (int k = 0; k < QK_RPT; ++k) {
    const long long off = min(r0 + k * S::RB, rows - 1) * D + S::V * l;
    wu[k] = *reinterpret_cast<const u32x4*>(u + off);
    wg[k] = *reinterpret_cast<const u32x4*>(dy + off);
  }
#pragma unroll
  for (int k = 0; k < QK_RPT; ++k) {
    const long long row = r0 + k * S::RB;
    float x[S::V], g[S::V], s[S::V], sg[S::V];
    W::unpack(wu[k], x);
    W::unpack(wg[k], g);
    float ss = 0.f, sd = 0.f;
#pragma unroll
    for (int i = 0; i < S::V; ++i) {
      sg[i] = sigmoidf_(x[i]);
      s[i] = x[i] * sg[i];
      ss += s[i] * s[i];
      sd += s[i] * g[i];
    }
#pragma unroll
    for (int off = S::G / 2; off >= 1; off >>= 1) {
      ss += __shfl_xor(ss, off, 64);
      sd += __shfl_xor(sd, off, 64);
    }
    const float inv = rsqrtf(ss + QK_L2_EPS);
    const float ydy = sd * inv;  // y . dy
    float r[S::V];
#pragma unroll
    for (int i = 0; i < S::V; ++i) {
      const float ds = (g[i] - s[i] * inv * ydy) * inv;
      r[i] = ds * (sg[i] * (1.f + x[i] * (1.f - sg[i])));
    }
    if (row < rows) *reinterpret_cast<u32x4*>(du + row * D + S::V * l) = W::pack(r);
  }
}

template <typename TC, int BM, int BN, bool A_KC, bool B_KC, int EPI>
hipError_t run_gemm(const GemmBatch& b, hipStream_t stream) {
  int tiles = 0;
  for (int i = 0; i < b.n; ++i) tiles = std::max(tiles, ((b.p[i].M + BM - 1) / BM) * ((b.p[i].N + BN - 1) / BN));
  if (tiles == 0) return hipSuccess;
  const int grid = (tiles + 7) / 8 * 8;  // whole rounds of the 8 XCDs
  hipLaunchKernelGGL((gemm_kernel<TC, BM, BN, A_KC, B_KC, EPI>), dim3(grid, b.n * b.ksplit), dim3(GEMM_THREADS), 0,
                     stream, b);
  return hipGetLastError();
}

}  // namespace

// ---- gate projection: launch sequences --------------------------------------------

namespace {

struct GateLayout {
  int M, d, W[5], r[5], zoff[5];
  size_t woff[5], boff[5];
};

GateLayout gate_layout(const GateShape& s) {
  GateLayout L;
  const int ranks[5] = {64, 64, 128, 128, 128};
  const int wk = s.H * s.dk, wv = s.H * s.dv;
  const int widths[5] = {wk, wk, wv, wv, wk};
  L.M = s.M;
  L.d = s.d;
  int z = 0;
  size_t w = 0, bo = 0;
  for (int i = 0; i < 5; ++i) {
    L.r[i] = ranks[i];
    L.W[i] = widths[i];
    L.zoff[i] = z;
    L.woff[i] = w;
    L.boff[i] = bo;
    z += ranks[i];
    w += static_cast<size_t>(ranks[i]) * widths[i];
    bo += widths[i];
  }
  return L;
}

const int kActs[5] = {GATE_ACT_LOGSIG, GATE_ACT_SIG, GATE_ACT_SIG, GATE_ACT_SIG, GATE_ACT_SIG2};

template <typename TC>
GateUpArgs<TC> gate_up_args(const GateLayout& L, const TC* z, const TC* U, const TC* bias) {
  GateUpArgs<TC> u = {};
  u.z = z;
  u.U = U;
  u.bias = bias;
  u.M = L.M;
  for (int i = 0; i < 5; ++i) {
    u.r[i] = L.r[i];
    u.W[i] = L.W[i];
    u.zoff[i] = L.zoff[i];
    u.woff[i] = L.woff[i];
    u.boff[i] = L.boff[i];
    u.act[i] = kActs[i];
  }
  return u;
}

template <typename TC, int EPI>
hipError_t run_gate_up(const GateUpArgs<TC>& u, hipStream_t stream) {
  int gx = 0;
  for (int i = 0; i < 5; ++i) gx = std::max(gx, ((u.M + 127) / 128) * ((u.W[i] / UP_BN + UP_CT - 1) / UP_CT));
  if (gx == 0) return hipSuccess;
  hipLaunchKernelGGL((gate_up_kernel<TC, EPI>), dim3(gx, 5), dim3(UP_THREADS), 0, stream, u);
  return hipGetLastError();
}

template <typename TC>
hipError_t gate_fwd_typed(const GateShape& s, const void* x, const void* W_down, const void* W_up, const void* bias,
                          void* z, void* const gates[5], hipStream_t stream) {
  const GateLayout L = gate_layout(s);
  const TC* Wu = static_cast<const TC*>(W_up);
  const TC* bs = static_cast<const TC*>(bias);
  GemmBatch b = {};
  b.n = 1;
  b.ksplit = 1;
  b.kchunk = s.d;
  b.p[0] = GemmProblem{x, W_down, z, s.M, GATE_RTOT, s.d, s.d, s.d, GATE_RTOT};  // z = x W_down^T
  hipError_t e = run_gemm<TC, 128, 128, true, true, EPI_STORE>(b, stream);
  if (e != hipSuccess) return e;
  GateUpArgs<TC> u = gate_up_args<TC>(L, static_cast<const TC*>(z), Wu, bs);
  for (int i = 0; i < 5; ++i) u.out[i] = static_cast<TC*>(gates[i]);
  return run_gate_up<TC, EPI_GATE>(u, stream);
}

template <typename TC>
hipError_t gate_bwd_typed(const GateShape& s, const void* x, const void* W_down, const void* W_up, const void* bias,
                          const void* z_in, const void* const dgates[5], void* dx, float* dW_down, float* dW_up,
                          float* dbias, char* ws, hipStream_t stream) {
  const GateLayout L = gate_layout(s);
  const GateWorkspace W = gate_workspace(s);
  const TC* Wu = static_cast<const TC*>(W_up);
  const TC* bs = static_cast<const TC*>(bias);
  TC* z = reinterpret_cast<TC*>(ws + W.z_off);
  TC* dpre = reinterpret_cast<TC*>(ws + W.dpre_off);
  TC* dz = reinterpret_cast<TC*>(ws + W.dz_off);
  float* part = reinterpret_cast<float*>(ws + W.part_off);
  float* csum = reinterpret_cast<float*>(ws + W.colsum_off);
  hipError_t e;
  const TC* zr = static_cast<const TC*>(z_in);
  if (!zr) {
    // the forward's z is not given: recompute it
    GemmBatch b = {};
    b.n = 1;
    b.ksplit = 1;
    b.kchunk = s.d;
    b.p[0] = GemmProblem{x, W_down, z, s.M, GATE_RTOT, s.d, s.d, s.d, GATE_RTOT};
    if ((e = run_gemm<TC, 128, 128, true, true, EPI_STORE>(b, stream)) != hipSuccess) return e;
    zr = z;
  }
  size_t dpo[5];
  size_t acc = 0;
  for (int i = 0; i < 5; ++i) {
    dpo[i] = acc;
    acc += static_cast<size_t>(s.M) * L.W[i];
  }
  // 1. dpre_i = dG_i * act'(z_i U_i + c_i), with per-tile column sums
  {
  GateUpArgs<TC> u = gate_up_args<TC>(L, zr, Wu, bs);
    u.colsum = csum;
    u.colsum_ld = W.colsum_ld;
    int coff = 0;
    for (int i = 0; i < 5; ++i) {
      u.out[i] = dpre + dpo[i];
      u.dG[i] = static_cast<const TC*>(dgates[i]);
      u.csoff[i] = coff;
      coff += L.W[i];
    }
    if ((e = run_gate_up<TC, EPI_GATE_BWD>(u, stream)) != hipSuccess) return e;
  }
  // 2. dz[:, slice_i] = dpre_i U_i
  {
    GemmBatch u = {};
    u.n = 5;
    u.ksplit = 1;
    u.kchunk = std::max(L.W[0], L.W[2]);
    for (int i = 0; i < 5; ++i)
      u.p[i] = GemmProblem{dpre + dpo[i], Wu + L.woff[i], dz + L.zoff[i], s.M, L.r[i], L.W[i], L.W[i], L.r[i],
                           GATE_RTOT};
    if ((e = run_gemm<TC, 128, 128, true, false, EPI_STORE>(u, stream)) != hipSuccess) return e;
  }
  // 3. dx = dz W_down
  {
    GemmBatch b = {};
    b.n = 1;
    b.ksplit = 1;
    b.kchunk = GATE_RTOT;
    b.p[0] = GemmProblem{dz, W_down, dx, s.M, s.d, GATE_RTOT, GATE_RTOT, s.d, s.d};
    if ((e = run_gemm<TC, 128, 128, true, false, EPI_STORE>(b, stream)) != hipSuccess) return e;
  }
  // 4. dW_down = dz^T x (split over tokens), 5. dW_up_i = dpre_i^T z_i (split over tokens)
  {
    GemmBatch b = {};
    b.n = 1;
    b.ksplit = W.ksplit;
    b.kchunk = W.kchunk;
    b.split_stride = W.part_stride;
    b.p[0] = GemmProblem{dz, x, part, GATE_RTOT, s.d, s.M, GATE_RTOT, s.d, s.d};
    if ((e = run_gemm<TC, 128, 128, false, false, EPI_PARTIAL>(b, stream)) != hipSuccess) return e;
    const size_t n = static_cast<size_t>(s.d) * GATE_RTOT;
    hipLaunchKernelGGL(split_sum_kernel, dim3(static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 4096))), dim3(256),
                       0, stream, part, W.ksplit, W.part_stride, n, dW_down);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    GemmBatch u = {};
    u.n = 5;
    u.ksplit = W.ksplit;
    u.kchunk = W.kchunk;
    u.split_stride = W.part_stride;
    for (int i = 0; i < 5; ++i)
      u.p[i] = GemmProblem{dpre + dpo[i], zr + L.zoff[i], part + L.woff[i], L.W[i], L.r[i], s.M, L.W[i], GATE_RTOT,
                           L.r[i]};
    if ((e = run_gemm<TC, 128, 128, false, false, EPI_PARTIAL>(u, stream)) != hipSuccess) return e;
    const size_t n = L.woff[4] + static_cast<size_t>(L.r[4]) * L.W[4];
    hipLaunchKernelGGL(split_sum_kernel, dim3(static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 4096))), dim3(256),
                       0, stream, part, W.ksplit, W.part_stride, n, dW_up);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 6. dbias = column sums over the token tiles
  {
    hipLaunchKernelGGL(colsum_kernel, dim3(static_cast<unsigned>((W.colsum_ld + 31) / 32)), dim3(256), 0, stream,
                       csum, W.mtiles, W.colsum_ld, dbias);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t gate_up_numel(const GateShape& s) {
  const GateLayout L = gate_layout(s);
  return L.woff[4] + static_cast<size_t>(L.r[4]) * L.W[4];
}

GateWorkspace gate_workspace(const GateShape& s) {
  GateWorkspace w = {};
  const GateLayout L = gate_layout(s);
  const size_t tc = s.bf16 ? 2 : 4;
  auto r256 = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  size_t off = 0;
  w.z_off = off;
  off += r256(static_cast<size_t>(s.M) * GATE_RTOT * tc);
  w.dpre_off = off;
  size_t dp = 0;
  for (int i = 0; i < 5; ++i) dp += static_cast<size_t>(s.M) * L.W[i];
  off += r256(dp * tc);
  w.dz_off = off;
  off += r256(static_cast<size_t>(s.M) * GATE_RTOT * tc);
  // the token contraction of the weight gradients is split so that the
  // launches fill the chip: about 4096 tokens per split, at most 16 splits
  w.ksplit = std::max(1, std::min(16, (s.M + 4095) / 4096));
  w.kchunk = ((s.M + w.ksplit - 1) / w.ksplit + 63) / 64 * 64;  // whole main-loop steps
  const size_t up = L.woff[4] + static_cast<size_t>(L.r[4]) * L.W[4];
  w.part_stride = r256(std::max(static_cast<size_t>(s.d) * GATE_RTOT, up) * 4) / 4;
  w.part_off = off;
  off += static_cast<size_t>(w.ksplit) * w.part_stride * 4;
  w.mtiles = (s.M + 127) / 128;
  w.colsum_ld = 0;
  for (int i = 0; i < 5; ++i) w.colsum_ld += L.W[i];
  w.colsum_off = off;
  off += r256(static_cast<size_t>(w.mtiles) * w.colsum_ld * 4);
  w.bytes = off;
  return w;
}

hipError_t launch_gate_fwd(const GateShape& s, const void* x, const void* W_down, const void* W_up, const void* bias,
                           void* z, void* const gates[5], hipStream_t stream) {
  return s.bf16 ? gate_fwd_typed<uint16_t>(s, x, W_down, W_up, bias, z, gates, stream)
                : gate_fwd_typed<float>(s, x, W_down, W_up, bias, z, gates, stream);
}

hipError_t launch_gate_bwd(const GateShape& s, const void* x, const void* W_down, const void* W_up, const void* bias,
                           const void* z, const void* const dgates[5], void* dx, float* dW_down, float* dW_up,
                           float* dbias, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  return s.bf16 ? gate_bwd_typed<uint16_t>(s, x, W_down, W_up, bias, z, dgates, dx, dW_down, dW_up, dbias, ws, stream)
                : gate_bwd_typed<float>(s, x, W_down, W_up, bias, z, dgates, dx, dW_down, dW_up, dbias, ws, stream);
}

hipError_t launch_qk_norm(long long rows, int D, bool bf16, const void* u, const void* dy, void* out,
                          hipStream_t stream) {
  if (rows == 0) return hipSuccess;
#define MUIR_QKN(TC, DD)                                                                                        \
  {                                                                                                              \
    const unsigned blocks = static_cast<unsigned>((rows + QkShape<TC, DD>::ROWS - 1) / QkShape<TC, DD>::ROWS);   \
    if (dy)                                                                                                      \
      hipLaunchKernelGGL((qk_norm_bwd_kernel<TC, DD>), dim3(blocks), dim3(QK_THREADS), 0, stream,                \
                         static_cast<const TC*>(u), static_cast<const TC*>(dy), static_cast<TC*>(out), rows);    \
    else                                                                                                         \
      hipLaunchKernelGGL((qk_norm_fwd_kernel<TC, DD>), dim3(blocks), dim3(QK_THREADS), 0, stream,                \
                         static_cast<const TC*>(u), static_cast<TC*>(out), rows);                                \
  }
  if (bf16) {
    if (D == 64) { MUIR_QKN(uint16_t, 64) } else { MUIR_QKN(uint16_t, 128) }
  } else {
    if (D == 64) { MUIR_QKN(float, 64) } else { MUIR_QKN(float, 128) }
  }
#undef MUIR_QKN
  return hipGetLastError();
}

}  // namespace muir
