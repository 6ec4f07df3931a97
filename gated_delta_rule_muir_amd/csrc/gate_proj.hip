// Gate prologue of the Muir operator: the fused low-rank gate projection and
// the SiLU + L2 normalisation of the query / key pathways, forward and
// backward (arXiv 2611.08376; wolonglab summary page, §Methodology: one
// down-projection shared by the five gates, five up-projections at ranks
// (64, 64, 128, 128, 128) with channel biases; fig:arch (b), (c)).
//
// The gates' up-projections run in gate_up_kernel (the rank-64/128
// contraction with the activation, or its gradient and the bias sums, fused
// into the epilogue).  The bf16 backward runs two bodies in one launch
// (gate_bwd_up_kernel): dpre with dz = dpre U, and dU = dpre^T z with the
// bias sums, each recomputing dpre from z, so dpre is never stored.  Every
// other product runs through a grouped GEMM:
// up to five independent problems per launch, 128 x 128 tiles on four waves,
// bf16 (v_mfma_f32_16x16x32_bf16) or fp32 (v_mfma_f32_16x16x4_f32) with fp32
// accumulation, and an epilogue chosen at compile time:
//   EPI_STORE     C = acc, in the compute type
//   EPI_PARTIAL   fp32 partial of one split of the contraction
// (The two plain bf16 products without a split, x W_down^T and dz W_down, go
// to hipBLASLt instead: see lt_gemm.)  Operands are read either along their
// contiguous axis (k contiguous: rows of A, columns of B^T) or across it (k
// strided), so every product here -- x W_down^T, dz W_down, dz^T x, and in
// fp32 dpre U and dpre^T z -- runs without an explicit transpose: bf16 tiles go straight from global memory
// into LDS (gemm_lds_kernel) and k-strided ones are read with transposing LDS
// reads; the register-staged gemm_kernel (fp32, and bf16 shapes that are not
// whole 64-deep steps) transposes them on the way into LDS.
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
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
  EPI_PARTIAL = 3,   // general GEMM: fp32 partial of one split of the contraction
  EPI_GATE_DZ = 4    // up-projection: dpre as EPI_GATE_BWD (no column sums), and dz = dpre U over the whole width
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
  TC* out[5];      // gates (forward) or their pre-activation gradients (EPI_GATE_BWD), [M, W_i]
  TC* dz;          // EPI_GATE_DZ: [M, 512], gate i's slice at its z offset
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

// GEMM epilogue, from registers: acc[i][j][r] = C[mw + 16i + fr][nw + 16j + 4g
// + r] (g = lane / 16, fr = lane % 16), stored in the compute type or as
// split s's fp32 partial.
template <typename TC, int TM, int TN, int EPI>
__device__ __forceinline__ void gemm_store(const f32x4 (&acc)[TM][TN], const GemmProblem& P, const GemmBatch& batch,
                                           int split, int mw, int nw, int lane) {
  const int fr = lane & 15, g4 = 4 * (lane >> 4);
  if constexpr (EPI == EPI_PARTIAL) {
    float* out = static_cast<float*>(P.C) + static_cast<size_t>(split) * batch.split_stride;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int gm = mw + 16 * i + fr;
      if (gm >= P.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int gn = nw + 16 * j + g4;
        if (gn < P.N) *reinterpret_cast<f32x4*>(out + static_cast<size_t>(gm) * P.ldc + gn) = acc[i][j];
      }
    }
  } else {
    TC* out = static_cast<TC*>(P.C);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int gm = mw + 16 * i + fr;
      if (gm >= P.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int gn = nw + 16 * j + g4;
        if (gn < P.N) store4(out + static_cast<size_t>(gm) * P.ldc + gn, acc[i][j]);
      }
    }
  }
}

// Grouped GEMM, C_g = A_g B_g for the problems of `batch` (blockIdx.y picks
// problem and contraction split).  128 x BN tile on four waves (2 x 2), each
// wave 64 x BN/2 as 16 x 16 MFMA tiles.  The MFMA is issued with the B tile
// as its row operand, so each lane ends with four consecutive output columns
// of one row (lane (g, c16): row c16, columns 4g .. 4g+3 of each 16 x 16
// tile) and the epilogue stores straight from registers.
template <typename TC, int BM, int BN, bool A_KC, bool B_KC, int EPI, int BK>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(GemmBatch batch) {
  typedef GF<TC> F;
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

  gemm_store<TC, TM, TN, EPI>(acc, P, batch, split, m0 + wm, n0 + wn, lane);
}

// The bf16 grouped GEMM with its operand tiles moved straight from global
// memory into LDS (global_load_lds_dwordx4): no register staging and no
// transposes.  Tile, waves and epilogue as gemm_kernel (128 x 128 on four
// waves, 64-deep steps).  Two LDS stages, each its own __shared__ array: the
// compiler then sees that one step's loads into one stage do not write what
// the step reads from the other (it would otherwise wait for those loads
// before every LDS read), and the loop is unrolled by two so that each
// step names its stages statically.  A step waits for its own stage's loads
// (vmcnt 0) and meets the other waves at a barrier, issues the next step's
// loads into the other stage (which every wave finished reading in the
// previous step), then forms its products.
// Stage layouts, with each row's 16-byte words permuted so that both the
// direct writes (1 KB contiguous per wave instruction) and the fragment
// reads are free of bank conflicts:
//   k-contiguous operand: [128 rows][64 k], 128-byte rows; word w of row r
//     at position w ^ ((r >> 1) & 7); fragments by ds_read_b128;
//   k-strided operand: [64 k][128 columns], 256-byte rows; word w of row r
//     at position w ^ 2 ((r & 3) + 4 ((r >> 3) & 1)); fragments by two
//     transposing reads (ds_read_b64_tr_b16) of four k rows each.
// Every split's contraction range is whole 64-deep steps (the launcher
// checks; other shapes take gemm_kernel).  Rows and columns past M and N
// read the last valid ones and are not stored.
template <bool A_KC, bool B_KC, int EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_lds_kernel(GemmBatch batch) {
  typedef uint16_t TC;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int BM = 128, BN = 128, BK = 64, TM = BM / 32, TN = BN / 32;
  constexpr int TILE = 128 * BK;
  __shared__ __align__(16) TC sA0[TILE];
  __shared__ __align__(16) TC sA1[TILE];
  __shared__ __align__(16) TC sB0[TILE];
  __shared__ __align__(16) TC sB1[TILE];

  const int grp = blockIdx.y / batch.ksplit;
  const int split = blockIdx.y - grp * batch.ksplit;
  const GemmProblem& P = batch.p[grp];
  const int mt = (P.M + BM - 1) / BM, nt = (P.N + BN - 1) / BN;
  const int ntile = mt * nt;
  const int per_xcd = (ntile + 7) / 8;
  const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (static_cast<int>(blockIdx.x / 8) >= per_xcd || t >= ntile) return;
  const int m0 = (t / nt) * BM;
  const int n0 = (t % nt) * BN;
  const int kbeg = split * batch.kchunk;
  const int kend = min(P.K, kbeg + batch.kchunk);
  const int nk = kend > kbeg ? (kend - kbeg) / BK : 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = (wave >> 1) * (BM / 2);
  const int wn = (wave & 1) * (BN / 2);
  const TC* __restrict__ gA = static_cast<const TC*>(P.A);
  const TC* __restrict__ gB = static_cast<const TC*>(P.B);

  // one operand tile into a stage: k-contiguous rows r0.. (k along the row)
  auto load_kc = [&](TC* dst, const TC* g, int ld, int rows_valid, int r0, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 32 * wave + 8 * j + (lane >> 3);
      const int w = (lane & 7) ^ ((row >> 1) & 7);
      const TC* src = g + static_cast<size_t>(min(r0 + row, rows_valid - 1)) * ld + k0 + 8 * w;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + (32 * wave + 8 * j) * BK), 16, 0, 0);
    }
  };
  // ... or k-strided: k rows k0 .., columns c0 .. c0 + 127
  auto load_ks = [&](TC* dst, const TC* g, int ld, int cols_valid, int c0, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * wave + 4 * j + (lane >> 4);
      const int w = (lane & 15) ^ (2 * ((row & 3) + 4 * ((row >> 3) & 1)));
      const TC* src = g + static_cast<size_t>(k0 + row) * ld + min(c0 + 8 * w, cols_valid - 8);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + (16 * wave + 4 * j) * 128), 16, 0, 0);
    }
  };
  auto load_step = [&](TC* a, TC* b, int k0) __attribute__((always_inline)) {
    if constexpr (A_KC) load_kc(a, gA, P.lda, P.M, m0, k0);
    else load_ks(a, gA, P.lda, P.M, m0, k0);
    if constexpr (B_KC) load_kc(b, gB, P.ldb, P.N, n0, k0);
    else load_ks(b, gB, P.ldb, P.N, n0, k0);
  };
  // fragment of row / column `rc` of a stage, k = 32 ks + 8 (lane / 16) .. + 7
  auto frag = [&](const TC* st, int rc, int ks, auto kc_tag) __attribute__((always_inline)) -> bf16x8 {
    constexpr bool KC = decltype(kc_tag)::value;
    const int g = lane >> 4;
    if constexpr (KC) {
      const int r = rc + (lane & 15);
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(st + r * BK + 8 * ((4 * ks + g) ^ ((r >> 1) & 7))));
    } else {
      const int l = lane & 15;
      const int w = (rc >> 3) + ((l & 3) >> 1);
      i16x4 h[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int rr = 32 * ks + 8 * g + 4 * hh + (l >> 2);
        h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(st + rr * 128 + 8 * (w ^ (2 * ((rr & 3) + 4 * ((rr >> 3) & 1)))) + 4 * (l & 1)));
      }
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero4();

  auto step = [&](const TC* a, const TC* b, TC* an, TC* bn, int kt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of this stage are in LDS
    __syncthreads();                      // and every wave's
    if (kt + 1 < nk) load_step(an, bn, kbeg + (kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = frag(a, wm + 16 * i, ks, std::integral_constant<bool, A_KC>{});
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = frag(b, wn + 16 * j, ks, std::integral_constant<bool, B_KC>{});
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
  };
  if (nk > 0) load_step(sA0, sB0, kbeg);
#pragma unroll 1
  for (int kt = 0; kt < nk; kt += 2) {
    step(sA0, sB0, sA1, sB1, kt);
    if (kt + 1 < nk) step(sA1, sB1, sA0, sB0, kt + 1);
  }
  gemm_store<TC, TM, TN, EPI>(acc, P, batch, split, m0 + wm, n0 + wn, lane);
}

// Activation as a template argument (one instance per gate form).
template <int ACT> __device__ __forceinline__ float act_fwd_t(float x) { return act_fwd(ACT, x); }
template <int ACT> __device__ __forceinline__ float act_grad_t(float x) { return act_grad(ACT, x); }

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
// blockIdx.y: the gate.  The gate's rank and activation are template
// arguments of the body (one instance per form), so its loops carry no
// run-time bounds.
//
// EPI_GATE_DZ (bf16) also forms the gate's slice of dz = dpre U: a workgroup
// then takes every column tile of its row block, and each tile's dpre, still
// in registers, is the right operand of a product with U's block read
// transposed from LDS (ds_read_b64_tr_b16): the lane's four consecutive
// columns of the tile are four consecutive contraction indices, so two
// tiles' values make one 32-deep product.  dz stays in registers until the
// row block is done, and dpre need not be re-read for it.
template <typename TC, int EPI> struct UpShape {
  static constexpr int RMAX = 128;
  // U block rows: 272 bytes, or 288 for the transposing reads of EPI_GATE_DZ
  // (an odd number of 32-byte units: the four rows of each lane group's read
  // fall on distinct banks)
  static constexpr int LDK = RMAX + (EPI == EPI_GATE_DZ ? 16 : GF<TC>::PAD);
  static constexpr int BM = 128;
  static constexpr int LDS_ = UP_BN + 16 / static_cast<int>(sizeof(TC));  // staging pitch: one 16-byte pad per row
};

template <typename TC, int EPI, int R, int ACT>
__device__ __forceinline__ void gate_up_body(const GateUpArgs<TC>& a, int gi, TC* __restrict__ sBm, TC* __restrict__ sS,
                                             float* __restrict__ redm) {
  typedef GF<TC> F;
  typedef UpShape<TC, EPI> S;
  constexpr bool DZ = EPI == EPI_GATE_DZ;
  constexpr bool BWD = EPI == EPI_GATE_BWD || DZ;
  // per-tile column sums of dpre (the bias gradient); with EPI_GATE_DZ the
  // weight-gradient kernel forms them instead
  constexpr bool CS = BWD && !DZ;
  static_assert(!DZ || sizeof(TC) == 2, "the fused dz product is bf16");
  constexpr int E = 16 / sizeof(TC);
  constexpr int LDK = S::LDK, LDS_ = S::LDS_;
  constexpr int BM = S::BM, BN = UP_BN, TM = 2, TN = BN / 16;
  constexpr int KSTEPS = R / F::KF;
  constexpr int WPU = R / E;                   // 16-byte words per U row
  constexpr int MAXW = BN * WPU / UP_THREADS;  // 16-byte words of the U block per thread
  constexpr int WPR = BN / E;                  // 16-byte words per staged row
  constexpr int SW = BM * WPR / UP_THREADS;    // staged words per thread
  static_assert(MAXW * UP_THREADS == BN * WPU && SW * UP_THREADS == BM * WPR && R <= S::RMAX, "tile layout");

  const int W = a.W[gi];
  const int mt = (a.M + BM - 1) / BM;
  const int ntiles = W / BN;
  const int ct = DZ ? ntiles : UP_CT;  // column tiles per workgroup
  const int ngrp = (ntiles + ct - 1) / ct;
  if (static_cast<int>(blockIdx.x) >= mt * ngrp) return;
  const int mtile = blockIdx.x % mt;
  const int t0 = (blockIdx.x / mt) * ct;
  const int t1 = min(ntiles, t0 + ct);
  const int m0 = mtile * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = 32 * wave;
  const int fr = lane & 15, fk = (F::KF / 4) * (lane >> 4), g4 = 4 * (lane >> 4);
  const TC* __restrict__ z = a.z + a.zoff[gi];
  const TC* __restrict__ U = a.U + a.woff[gi];
  const TC* __restrict__ bias = a.bias + a.boff[gi];
  const TC* __restrict__ dG = a.dG[gi];
  TC* __restrict__ out = a.out[gi];
  // staged words of this wave's 32 rows: word s of the thread is row
  // wm + s * (64 / WPR) + lane / WPR, columns (lane % WPR) * E ..
  auto srow = [&](int sw) { return wm + sw * (64 / WPR) + lane / WPR; };
  const int scol = (lane % WPR) * E;

  // the wave's rows of z, once
  typename F::frag fa[TM][KSTEPS];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int gm = m0 + wm + 16 * i + fr;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint4 v = {0u, 0u, 0u, 0u};
      if (gm < a.M) v = *reinterpret_cast<const uint4*>(z + static_cast<size_t>(gm) * GATE_RTOT + ks * F::KF + fk);
      fa[i][ks] = __builtin_bit_cast(typename F::frag, v);
    }
  }
  // a tile's U block and, for the backward, this thread's staged words of the
  // upstream gradient (rows clamped to the last; rows past it are not used)
  u32x4 rb[MAXW];
  u32x4 dgw[BWD ? SW : 1];
  const int dgrow0 = m0 + wm + lane / WPR;
  auto load_tile = [&](int n0) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < MAXW; ++w) {
      const int idx = tid + w * UP_THREADS;
      rb[w] = *reinterpret_cast<const u32x4*>(U + static_cast<size_t>(n0 + idx / WPU) * R + (idx % WPU) * E);
    }
    if constexpr (BWD) {
#pragma unroll
      for (int sw = 0; sw < SW; ++sw) {
        const int gm = min(dgrow0 + sw * (64 / WPR), a.M - 1);
        dgw[sw] = *reinterpret_cast<const u32x4*>(dG + static_cast<size_t>(gm) * W + n0 + scol);
      }
    }
  };
  auto put_tile = [&](TC* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < MAXW; ++w) {
      const int idx = tid + w * UP_THREADS;
      *reinterpret_cast<u32x4*>(&dst[(idx / WPU) * LDK + (idx % WPU) * E]) = rb[w];
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
  // EPI_GATE_DZ: dz^T of the wave's rows, [rank tile s][row tile i] in the MFMA
  // layout (lane: rank 16s + 4g .. + 3, row wm + 16i + fr), and the tile's
  // dpre as bf16 operands (lane: columns 16j + 4g .. + 3, row wm + 16i + fr)
  constexpr int RTZ = DZ ? R / 16 : 1;
  f32x4 dzacc[RTZ][TM];
  typename MM<TC>::frag dp[DZ ? TM : 1][DZ ? TN : 1];
  if constexpr (DZ) {
#pragma unroll
    for (int s2 = 0; s2 < RTZ; ++s2)
#pragma unroll
      for (int i = 0; i < TM; ++i) dzacc[s2][i] = zero4();
  }

  load_tile(t0 * BN);
  put_tile(sBm);

#pragma unroll 1
  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    const int n0 = t * BN;
    const TC* sb = sBm + buf * BN * LDK;
    float* rd = redm + buf * 4 * BN;
    // tile t's U block is in buffer buf (and its dG words in sS); every wave is
    // done with tile t - 1, so the other buffers are free once read
    __syncthreads();
    if constexpr (CS) {
      if (t > t0) put_colsum(t - 1, redm + (buf ^ 1) * 4 * BN);
    }
    // the next tile's operands, in flight during this one
    load_tile((t + 1 < t1 ? t + 1 : t) * BN);

    // accumulators start from the bias (lane: columns 16j + 4g .. + 3)
    f32x4 acc[TM][TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const f32x4 bv = load4(bias + n0 + 16 * j + g4);
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i][j] = bv;
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const typename F::frag fb = F::load(&sb[(16 * j + fr) * LDK + ks * F::KF + fk]);
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][j] = F::mma(fb, fa[i][ks], acc[i][j]);
      }
    }

    // epilogue in the MFMA layout (lane: row wm + 16i + fr, columns 16j + 4g ..
    // + 3 of the tile), through this wave's rows of the staging tile
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
            if constexpr (CS) cs[q] += row_ok ? v[q] : 0.f;
          }
          if constexpr (DZ) dp[i][j] = MM<TC>::from_f32(v);
        }
        if constexpr (!DZ) store4(&sS[row * LDS_ + c], v);
      }
      if constexpr (CS) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sm = sum16(cs[q]);
          if (fr == 0) rd[wave * BN + c + q] = sm;
        }
      }
    }
    // this wave's rows back out in whole rows (the wave wrote them itself: LDS
    // operations of one wave complete in order); EPI_GATE_DZ keeps no dpre
    if constexpr (!DZ) {
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      TC* o = out + n0 + scol;
#pragma unroll
      for (int sw = 0; sw < SW; ++sw) {
        const int row = srow(sw);
        if (m0 + row < a.M)
          *reinterpret_cast<uint4*>(o + static_cast<size_t>(m0 + row) * W) =
              *reinterpret_cast<const uint4*>(&sS[row * LDS_ + scol]);
      }
    }
    if constexpr (DZ) {
      // dz^T[16s.., rows] += U_block^T dpre^T: the U block's rows 16jj + 4g ..
      // + 3 (and the next tile's) of rank column 16s + fr, read transposed
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      const TC* ub = sb + (4 * (lane >> 4) + ((lane & 15) >> 2)) * LDK + 4 * (lane & 3);
#pragma unroll
      for (int s2 = 0; s2 < RTZ; ++s2) {
#pragma unroll
        for (int jj = 0; jj < TN; jj += 2) {
          const i16x4 u0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ub + 16 * jj * LDK + 16 * s2));
          const i16x4 u1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ub + (16 * jj + 16) * LDK + 16 * s2));
#pragma unroll
          for (int i = 0; i < TM; ++i) dzacc[s2][i] = MM<TC>::mma2(u0, dp[i][jj], u1, dp[i][jj + 1], dzacc[s2][i]);
        }
      }
    }
    // the next tile's operands to LDS: the other U buffer was last read in
    // tile t - 1, which every wave finished before this tile's barrier; the dG
    // words go to this wave's own staging rows after its reads of them above
    if (t + 1 < t1) put_tile(sBm + (buf ^ 1) * BN * LDK);
  }
  if constexpr (CS) {
    __syncthreads();
    put_colsum(t1 - 1, redm + ((t1 - 1 - t0) & 1) * 4 * BN);
  }
  if constexpr (DZ) {
    // lane: dz[row wm + 16i + fr][z offset + 16s + 4g .. + 3]
    TC* dzo = a.dz + a.zoff[gi] + g4;
#pragma unroll
    for (int s2 = 0; s2 < RTZ; ++s2) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int gm = m0 + wm + 16 * i + fr;
        if (gm < a.M) store4(dzo + static_cast<size_t>(gm) * GATE_RTOT + 16 * s2, dzacc[s2][i]);
      }
    }
  }
}

// One body instance per (rank, activation); the gates' ranks are 64 or 128.
#define MUIR_GATE_FORMS(BODY)                                       \
  switch (a.act[gi]) {                                              \
    case GATE_ACT_LOGSIG:                                           \
      if (r == 64) BODY(64, GATE_ACT_LOGSIG); else BODY(128, GATE_ACT_LOGSIG); \
      break;                                                        \
    case GATE_ACT_SIG:                                              \
      if (r == 64) BODY(64, GATE_ACT_SIG); else BODY(128, GATE_ACT_SIG); \
      break;                                                        \
    case GATE_ACT_SIG2:                                             \
      if (r == 64) BODY(64, GATE_ACT_SIG2); else BODY(128, GATE_ACT_SIG2); \
      break;                                                        \
    default:                                                        \
      if (r == 64) BODY(64, GATE_ACT_NONE); else BODY(128, GATE_ACT_NONE); \
      break;                                                        \
  }

template <typename TC, int EPI>
__global__ __launch_bounds__(UP_THREADS) __attribute__((amdgpu_waves_per_eu(EPI == EPI_GATE_DZ ? 2 : 1))) void
gate_up_kernel(GateUpArgs<TC> a) {
  typedef UpShape<TC, EPI> S;
  __shared__ __align__(16) TC sB[2 * UP_BN * S::LDK];  // U blocks of the current and the next tile
  __shared__ __align__(16) TC sS[S::BM * S::LDS_];
  __shared__ float red[2 * 4 * UP_BN];
  const int gi = blockIdx.y;
  const int r = a.r[gi];
#define MUIR_UP_BODY(RR, AA) gate_up_body<TC, EPI, RR, AA>(a, gi, sB, sS, red)
  MUIR_GATE_FORMS(MUIR_UP_BODY)
#undef MUIR_UP_BODY
}

// Arguments of the up-projections' weight-gradient kernel (bf16).
struct GateDwArgs {
  const uint16_t* z;      // [M, 512]
  const uint16_t* U;      // packed up matrices ([W_i, r_i] each, rank contiguous)
  const uint16_t* bias;   // packed biases
  const uint16_t* dG[5];  // the gates' gradients, [M, W_i]
  float* part;            // fp32 partials, split s at part + s * split_stride, gate i at woff[i]
  size_t split_stride;
  float* colsum;          // the bias gradient's partials: split s, gate i at colsum + s * colsum_ld + csoff[i]
  int colsum_ld;
  int csoff[5];
  int M, ksplit, kchunk;
  int r[5], W[5], zoff[5], act[5];
  size_t woff[5], boff[5];
};

// dU_i = dpre_i^T z_i, summed over one split of the tokens, with
// dpre_i = dG_i * act'(z_i U_i^T + c_i) recomputed from z instead of read
// back (bf16).  A workgroup owns 128 columns of one gate's width (32 per
// wave, two 16-column tiles that share every z operand read) and runs
// through its split in blocks of 64 tokens.  Per block:
//   pre[t][w] (MFMA layout: lane holds tokens 4g .. + 3 of one column w),
//     z rows from LDS times the lane's column of U, held in registers;
//   dpre = dG * act'(pre), with dG read transposed from LDS into the same
//     layout, so the values are already the right operand of
//   dU^T[r][w] += z^T dpre, z read transposed from LDS (ds_read_b64_tr_b16):
//     four consecutive tokens per lane, two token tiles per 32-deep product.
// The next block's z and dG rows are loaded while this block computes and
// stored into the other LDS buffer after it: one barrier per block.  Tokens
// past M are zero (dG = 0 gives dpre = 0).  The lane's four dpre values of
// each token tile are also summed in place, for the bias gradient's partial
// sum over the split (in-lane adds; the four token groups meet at the end).
// Workgroups of one split sit on
// one XCD, so its z rows are fetched into that XCD's L2 once.  The rank and
// activation are template arguments of the body.
constexpr int DW_WPW = 2;               // 16-column tiles per wave
constexpr int DW_WB = 64 * DW_WPW, DW_TB = 64;
constexpr int DW_PZ = 128 + 16;         // z rows: 288 bytes (an odd number of 32-byte units)
constexpr int DW_PG = DW_WB + 16;       // dG rows: 288 bytes
constexpr int DW_SPLIT_TOKENS = 2048;   // tokens per split of the weight-gradient kernel

template <int R, int ACT>
__device__ __forceinline__ void gate_dw_body(const GateDwArgs& a, int gi, uint16_t* __restrict__ sZm,
                                             uint16_t* __restrict__ sGm) {
  typedef uint16_t TC;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  constexpr int WB = DW_WB, TB = DW_TB, PZ = DW_PZ, PG = DW_PG, WPW = DW_WPW;
  constexpr int RW = R / 8;                 // 16-byte words per z row of the gate
  constexpr int GWR = WB / 8;               // 16-byte words per dG row
  constexpr int ZW = TB * RW / 256;         // 16-byte z words per thread and block
  constexpr int GW = TB * GWR / 256;        // 16-byte dG words per thread and block
  constexpr int KS = R / 32, RT = R / 16;
  static_assert(ZW * 256 == TB * RW && GW * 256 == TB * GWR, "block layout");

  const int W = a.W[gi];
  const int nwt = (W + WB - 1) / WB;  // (W is a multiple of 64: the last group may be half)
  const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
  const int wt = j % nwt;
  const int split = (j / nwt) * 8 + xcd;
  if (split >= a.ksplit) return;
  const int w0 = wt * WB;
  const int kbeg = split * a.kchunk;
  const int kend = min(a.M, kbeg + a.kchunk);
  const int nblk = kend > kbeg ? (kend - kbeg + TB - 1) / TB : 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int wl = 16 * WPW * wave;  // the wave's first column within the workgroup's
  const TC* __restrict__ z = a.z + a.zoff[gi];
  const TC* __restrict__ U = a.U + a.woff[gi];
  const TC* __restrict__ dG = a.dG[gi];

  // the lane's columns of U as right operands of the pre product (k = r)
  bf16x8 ub[WPW][KS];
  float cb[WPW];
#pragma unroll
  for (int u = 0; u < WPW; ++u) {
    const int wcol = min(w0 + wl + 16 * u + c16, W - 1);  // columns past W: zero dG, not stored
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ub[u][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(U + static_cast<size_t>(wcol) * R + 32 * ks + 8 * g));
    cb[u] = bf16_to_f32(a.bias[a.boff[gi] + wcol]);
  }

  // Rows past the split's end are read at its last row (no branch around the
  // loads); their dG words are then zeroed, which makes their dpre zero.
  u32x4 zr[ZW], gr[GW];
  auto load_block = [&](int b) __attribute__((always_inline)) {
    const int t0 = kbeg + b * TB;
#pragma unroll
    for (int u = 0; u < ZW; ++u) {
      const int idx = tid + 256 * u;
      const int row = min(t0 + idx / RW, kend - 1), c = idx % RW;
      zr[u] = *reinterpret_cast<const u32x4*>(z + static_cast<size_t>(row) * GATE_RTOT + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < GW; ++u) {
      const int idx = tid + 256 * u;
      const int row = t0 + idx / GWR, col = w0 + 8 * (idx % GWR);
      const u32x4 v = *reinterpret_cast<const u32x4*>(dG + static_cast<size_t>(min(row, kend - 1)) * W + (col < W ? col : w0));
      const u32x4 zero = {0u, 0u, 0u, 0u};
      gr[u] = row < kend && col < W ? v : zero;
    }
  };
  auto store_block = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < ZW; ++u) {
      const int idx = tid + 256 * u;
      *reinterpret_cast<u32x4*>(&sZm[buf * TB * PZ + (idx / RW) * PZ + 8 * (idx % RW)]) = zr[u];
    }
#pragma unroll
    for (int u = 0; u < GW; ++u) {
      const int idx = tid + 256 * u;
      *reinterpret_cast<u32x4*>(&sGm[buf * TB * PG + (idx / GWR) * PG + 8 * (idx % GWR)]) = gr[u];
    }
  };

  f32x4 du[RT][WPW];
#pragma unroll
  for (int s2 = 0; s2 < RT; ++s2)
#pragma unroll
    for (int u = 0; u < WPW; ++u) du[s2][u] = zero4();
  float csum[WPW];  // sum of dpre over the lane's tokens, the lane's column
#pragma unroll
  for (int u = 0; u < WPW; ++u) csum[u] = 0.f;

  if (nblk > 0) {
    load_block(0);
    store_block(0);
  }
  __syncthreads();
#pragma unroll 1
  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    if (b + 1 < nblk) load_block(b + 1);
    const TC* zb = sZm + buf * TB * PZ;
    const TC* gb = sGm + buf * TB * PG;
    i16x4 dpf[TB / 16][WPW];
#pragma unroll
    for (int tt = 0; tt < TB / 16; ++tt) {
      bf16x8 za[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        za[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&zb[(16 * tt + c16) * PZ + 32 * ks + 8 * g]));
#pragma unroll
      for (int u = 0; u < WPW; ++u) {
        f32x4 acc = {cb[u], cb[u], cb[u], cb[u]};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za[ks], ub[u][ks], acc, 0, 0, 0);
        // dG at (tokens 16tt + 4g .. + 3, the lane's column)
        const i16x4 gq = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(gb + (16 * tt + 4 * g + (c16 >> 2)) * PG + wl + 16 * u + 4 * (c16 & 3)));
        f32x4 dv;
#pragma unroll
        for (int q = 0; q < 4; ++q) dv[q] = bf16_to_f32(static_cast<uint16_t>(gq[q])) * act_grad_t<ACT>(acc[q]);
        dpf[tt][u] = pack4(dv);
        csum[u] += (dv[0] + dv[1]) + (dv[2] + dv[3]);
      }
    }
    // dU^T[16s + 4g .., columns] += z^T dpre over the block's tokens
    const TC* zt = zb + (4 * g + (c16 >> 2)) * PZ + 4 * (c16 & 3);
#pragma unroll
    for (int s2 = 0; s2 < RT; ++s2) {
#pragma unroll
      for (int tt = 0; tt < TB / 16; tt += 2) {
        const i16x4 z0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(zt + 16 * tt * PZ + 16 * s2));
        const i16x4 z1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(zt + (16 * tt + 16) * PZ + 16 * s2));
#pragma unroll
        for (int u = 0; u < WPW; ++u) du[s2][u] = mma32_bf16(z0, dpf[tt][u], z1, dpf[tt + 1][u], du[s2][u]);
      }
    }
    // the next block into the other buffer: every wave finished reading it
    // before this block's barrier
    if (b + 1 < nblk) store_block(buf ^ 1);
    __syncthreads();
  }
  // lane: dU[column][16s + 4g .. + 3]; the bias partial from the lanes of
  // the column's four token groups (c16 + 16g)
#pragma unroll
  for (int u = 0; u < WPW; ++u) {
    const int wcol = w0 + wl + 16 * u + c16;
    float cg = csum[u] + __shfl_xor(csum[u], 16, 64);
    cg += __shfl_xor(cg, 32, 64);
    if (w0 + wl + 16 * u >= W) continue;
    if (g == 0) a.colsum[static_cast<size_t>(split) * a.colsum_ld + a.csoff[gi] + wcol] = cg;
    float* out = a.part + static_cast<size_t>(split) * a.split_stride + a.woff[gi] + static_cast<size_t>(wcol) * R + 4 * g;
#pragma unroll
    for (int s2 = 0; s2 < RT; ++s2) *reinterpret_cast<f32x4*>(out + 16 * s2) = du[s2][u];
  }
}

// The bf16 backward of the up-projections in one launch: blockIdx.y = 2 i
// runs the fused dpre / dz body (EPI_GATE_DZ) of gate i, blockIdx.y = 2 i + 1
// the weight-gradient body of gate i.  The two parts are independent (both
// recompute dpre from z; one writes dz, the other the split partials of dU
// and of the bias gradient).  Either alone ends in a partly filled round of
// the CUs' workgroup slots (1,280 workgroups each at the 4K layer, two per
// CU); in one launch the second part's workgroups fill the slots the first
// part's last round leaves free.  Workgroups are dispatched in blockIdx.y
// order, so both parts of one gate run one after the other: the second
// part's reads of the gate's gradient (134 MB at the 4K layer) then find it
// in the 256 MB Infinity Cache instead of HBM, which the order gate by gate
// and part by part did not allow (the four other gates' gradients passed
// between the two reads).  The LDS is one buffer, laid out per part.
constexpr int BWDUP_LDS_UP =
    (2 * UP_BN * UpShape<uint16_t, EPI_GATE_DZ>::LDK + UpShape<uint16_t, EPI_GATE_DZ>::BM * UpShape<uint16_t, EPI_GATE_DZ>::LDS_) * 2 +
    2 * 4 * UP_BN * 4;
constexpr int BWDUP_LDS_DW = 2 * DW_TB * (DW_PZ + DW_PG) * 2;
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gate_bwd_up_kernel(GateUpArgs<uint16_t> ua,
                                                                                               GateDwArgs da) {
  typedef UpShape<uint16_t, EPI_GATE_DZ> S;
  static_assert(UP_THREADS == 256, "one block size for both parts");
  __shared__ __align__(16) char smem[BWDUP_LDS_UP > BWDUP_LDS_DW ? BWDUP_LDS_UP : BWDUP_LDS_DW];
  if ((blockIdx.y & 1) == 0) {
    const GateUpArgs<uint16_t>& a = ua;
    const int gi = blockIdx.y >> 1;
    const int r = a.r[gi];
    uint16_t* sB = reinterpret_cast<uint16_t*>(smem);
    uint16_t* sS = sB + 2 * UP_BN * S::LDK;
    float* red = reinterpret_cast<float*>(sS + S::BM * S::LDS_);
#define MUIR_UP_BODY(RR, AA) gate_up_body<uint16_t, EPI_GATE_DZ, RR, AA>(a, gi, sB, sS, red)
    MUIR_GATE_FORMS(MUIR_UP_BODY)
#undef MUIR_UP_BODY
  } else {
    const GateDwArgs& a = da;
    const int gi = blockIdx.y >> 1;
    const int r = a.r[gi];
    uint16_t* sZ = reinterpret_cast<uint16_t*>(smem);
    uint16_t* sG = sZ + 2 * DW_TB * DW_PZ;
#define MUIR_DW_BODY(RR, AA) gate_dw_body<RR, AA>(a, gi, sZ, sG)
    MUIR_GATE_FORMS(MUIR_DW_BODY)
#undef MUIR_DW_BODY
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

template <typename TC, int BM, int BN, bool A_KC, bool B_KC, int EPI, int BK = GemmStep<TC>::BK>
hipError_t run_gemm(const GemmBatch& b, hipStream_t stream) {
  int tiles = 0;
  for (int i = 0; i < b.n; ++i) tiles = std::max(tiles, ((b.p[i].M + BM - 1) / BM) * ((b.p[i].N + BN - 1) / BN));
  if (tiles == 0) return hipSuccess;
  const int grid = (tiles + 7) / 8 * 8;  // whole rounds of the 8 XCDs
  if constexpr (sizeof(TC) == 2 && BM == 128 && BN == 128 && BK == 64) {
    // whole 64-deep steps in every split, 16-byte rows: the LDS-direct kernel
    bool whole = b.kchunk % BK == 0;
    for (int i = 0; i < b.n; ++i)
      whole = whole && b.p[i].K % BK == 0 && b.p[i].lda % 8 == 0 && b.p[i].ldb % 8 == 0 && b.p[i].M >= 8 &&
              b.p[i].N >= 8;
    if (whole) {
      hipLaunchKernelGGL((gemm_lds_kernel<A_KC, B_KC, EPI>), dim3(grid, b.n * b.ksplit), dim3(GEMM_THREADS), 0, stream,
                         b);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<TC, BM, BN, A_KC, B_KC, EPI, BK>), dim3(grid, b.n * b.ksplit), dim3(GEMM_THREADS), 0,
                     stream, b);
  return hipGetLastError();
}

// ---- plain bf16 products through hipBLASLt ----------------------------------------
//
// z = x W_down^T and dx = dz W_down are plain GEMMs (no epilogue, no split of
// the contraction).  For bf16 they go to hipBLASLt, whose kernels measured
// faster on these shapes at the 4K layer (z: about 70 against 95 us; dx:
// about 100 against 120 us).  The token contraction dW_down = dz^T x keeps the split
// kernel above (105 us against 208 us for the library's single product).
// The problems are row-major; hipBLASLt is column-major, so C^T = B^T A^T is
// issued: the library's first operand is B, its second A.  One handle per
// device and one algorithm per shape (the heuristic's first), made on first
// use and kept for the process; no workspace is given, so the chosen
// algorithm needs none and the call allocates nothing.
struct LtPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
  bool ok = false;
};
constexpr int kLtMaxDevices = 64;
std::mutex g_lt_mu;
hipblasLtHandle_t g_lt_handle[kLtMaxDevices] = {};
std::map<std::tuple<int, int, int, int, int, int, int, bool, bool>, LtPlan> g_lt_plans;

// The plan of C[M][N] = A[M][K] B[K][N] (bf16, fp32 accumulation; A_KC: A's
// rows are k-contiguous, else A is stored k-major; B_KC: B is stored as B^T's
// rows, k-contiguous, else as B's rows).  nullptr when the library has no
// algorithm for it.
const LtPlan* lt_plan(int dev, const GemmProblem& p, bool a_kc, bool b_kc) {
  std::lock_guard<std::mutex> lock(g_lt_mu);
  if (!g_lt_handle[dev] && hipblasLtCreate(&g_lt_handle[dev]) != HIPBLAS_STATUS_SUCCESS) {
    g_lt_handle[dev] = nullptr;
    return nullptr;
  }
  const auto key = std::make_tuple(dev, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, a_kc, b_kc);
  auto it = g_lt_plans.find(key);
  if (it != g_lt_plans.end()) return it->second.ok ? &it->second : nullptr;
  LtPlan& pl = g_lt_plans[key];
  // column-major: C^T [N x M] = op(B-buffer) [N x K] . op(A-buffer) [K x M]
  const hipblasOperation_t opa = b_kc ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  const hipblasOperation_t opb = a_kc ? HIPBLAS_OP_N : HIPBLAS_OP_T;
  bool ok = hipblasLtMatmulDescCreate(&pl.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(pl.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(pl.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&pl.la, HIP_R_16BF, b_kc ? p.K : p.N, b_kc ? p.N : p.K, p.ldb) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&pl.lb, HIP_R_16BF, a_kc ? p.K : p.M, a_kc ? p.M : p.K, p.lda) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&pl.lc, HIP_R_16BF, p.N, p.M, p.ldc) == HIPBLAS_STATUS_SUCCESS;
  if (ok) {
    hipblasLtMatmulPreference_t pref = nullptr;
    uint64_t wsmax = 0;
    ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsmax,
                                               sizeof(wsmax)) == HIPBLAS_STATUS_SUCCESS;
    hipblasLtMatmulHeuristicResult_t res[1];
    int nres = 0;
    ok = ok && hipblasLtMatmulAlgoGetHeuristic(g_lt_handle[dev], pl.desc, pl.la, pl.lb, pl.lc, pl.lc, pref, 1, res,
                                               &nres) == HIPBLAS_STATUS_SUCCESS &&
         nres > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize == 0;
    if (ok) pl.algo = res[0].algo;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  }
  pl.ok = ok;
  return ok ? &pl : nullptr;
}

// C = A B through hipBLASLt (bf16); hipErrorNotSupported when the library
// has no algorithm for the shape (the caller then runs its own kernel).
hipError_t lt_gemm(const GemmProblem& p, bool a_kc, bool b_kc, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kLtMaxDevices) return hipErrorNotSupported;
  const LtPlan* pl = lt_plan(dev, p, a_kc, b_kc);
  if (!pl) return hipErrorNotSupported;
  const float alpha = 1.f, beta = 0.f;
  const hipblasStatus_t st = hipblasLtMatmul(g_lt_handle[dev], pl->desc, &alpha, p.B, pl->la, p.A, pl->lb, &beta, p.C,
                                             pl->lc, p.C, pl->lc, &pl->algo, nullptr, 0, stream);
  return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

// One plain product in the compute type: hipBLASLt for bf16 when it has an
// algorithm for the shape, else the kernels above.
template <typename TC, bool A_KC, bool B_KC>
hipError_t plain_gemm(const GemmProblem& p, hipStream_t stream) {
  if constexpr (sizeof(TC) == 2) {
    const hipError_t e = lt_gemm(p, A_KC, B_KC, stream);
    if (e != hipErrorNotSupported) return e;
  }
  GemmBatch b = {};
  b.n = 1;
  b.ksplit = 1;
  b.kchunk = p.K;
  b.p[0] = p;
  return run_gemm<TC, 128, 128, A_KC, B_KC, EPI_STORE>(b, stream);
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
  constexpr int ct = EPI == EPI_GATE_DZ ? 1 << 30 : UP_CT;  // EPI_GATE_DZ: every column tile in one workgroup
  int gx = 0;
  for (int i = 0; i < 5; ++i) gx = std::max(gx, ((u.M + 127) / 128) * ((u.W[i] / UP_BN + ct - 1) / ct));
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
  hipError_t e =
      plain_gemm<TC, true, true>(GemmProblem{x, W_down, z, s.M, GATE_RTOT, s.d, s.d, s.d, GATE_RTOT}, stream);  // z = x W_down^T
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
    e = plain_gemm<TC, true, true>(GemmProblem{x, W_down, z, s.M, GATE_RTOT, s.d, s.d, s.d, GATE_RTOT}, stream);
    if (e != hipSuccess) return e;
    zr = z;
  }
  size_t dpo[5];
  size_t acc = 0;
  for (int i = 0; i < 5; ++i) {
    dpo[i] = acc;
    acc += static_cast<size_t>(s.M) * L.W[i];
  }
  // 1. dpre_i = dG_i * act'(z_i U_i + c_i), and its column sums (the bias
  // gradient) per token tile (fp32) or per split (bf16)
  GateUpArgs<TC> u = gate_up_args<TC>(L, zr, Wu, bs);
  u.colsum = csum;
  u.colsum_ld = W.colsum_ld;
  {
    int coff = 0;
    for (int i = 0; i < 5; ++i) {
      u.out[i] = dpre + dpo[i];
      u.dG[i] = static_cast<const TC*>(dgates[i]);
      u.csoff[i] = coff;
      coff += L.W[i];
    }
  }
  if constexpr (sizeof(TC) == 2) {
    // bf16, one launch: dz[:, slice_i] = dpre_i U_i (2.) with dpre kept in
    // registers, and dU_i = dpre_i^T z_i (5.) with dpre recomputed from z;
    // dpre itself is never stored
    u.dz = dz;
    GateDwArgs d = {};
    d.z = zr;
    d.U = Wu;
    d.bias = bs;
    d.part = part + static_cast<size_t>(W.ksplit) * W.part_stride;  // after dW_down's partials
    d.split_stride = W.part_stride;
    d.colsum = csum;
    d.colsum_ld = W.colsum_ld;
    d.M = s.M;
    d.ksplit = W.dw_ksplit;
    d.kchunk = W.dw_kchunk;
    int nwt = 0;
    for (int i = 0; i < 5; ++i) {
      d.dG[i] = static_cast<const TC*>(dgates[i]);
      d.r[i] = L.r[i];
      d.W[i] = L.W[i];
      d.zoff[i] = L.zoff[i];
      d.act[i] = kActs[i];
      d.woff[i] = L.woff[i];
      d.boff[i] = L.boff[i];
      d.csoff[i] = u.csoff[i];
      nwt = std::max(nwt, (L.W[i] + DW_WB - 1) / DW_WB);
    }
    // x: the row blocks of the dz part (one workgroup takes all of a gate's
    // column tiles), or the weight-gradient part's column groups x splits
    const int gx = std::max((s.M + 127) / 128, 8 * nwt * ((W.dw_ksplit + 7) / 8));
    hipLaunchKernelGGL(gate_bwd_up_kernel, dim3(gx, 10), dim3(256), 0, stream, u, d);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    if ((e = run_gate_up<TC, EPI_GATE_BWD>(u, stream)) != hipSuccess) return e;
    // 2. dz[:, slice_i] = dpre_i U_i
    GemmBatch g = {};
    g.n = 5;
    g.ksplit = 1;
    g.kchunk = std::max(L.W[0], L.W[2]);
    for (int i = 0; i < 5; ++i)
      g.p[i] = GemmProblem{dpre + dpo[i], Wu + L.woff[i], dz + L.zoff[i], s.M, L.r[i], L.W[i], L.W[i], L.r[i],
                           GATE_RTOT};
    if ((e = run_gemm<TC, 128, 128, true, false, EPI_STORE>(g, stream)) != hipSuccess) return e;
  }
  // 3. dx = dz W_down
  e = plain_gemm<TC, true, false>(GemmProblem{dz, W_down, dx, s.M, s.d, GATE_RTOT, GATE_RTOT, s.d, s.d}, stream);
  if (e != hipSuccess) return e;
  // 4. dW_down = dz^T x (split over tokens)
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
  // 5. dW_up_i = dpre_i^T z_i (split over tokens; bf16: formed in 1.)
  {
    const float* upart = part;
    int upk = W.ksplit;
    if constexpr (sizeof(TC) == 2) {
      upart = part + static_cast<size_t>(W.ksplit) * W.part_stride;
      upk = W.dw_ksplit;
    } else {
      GemmBatch g = {};
      g.n = 5;
      g.ksplit = W.ksplit;
      g.kchunk = W.kchunk;
      g.split_stride = W.part_stride;
      for (int i = 0; i < 5; ++i)
        g.p[i] = GemmProblem{dpre + dpo[i], zr + L.zoff[i], part + L.woff[i], L.W[i], L.r[i], s.M, L.W[i], GATE_RTOT,
                             L.r[i]};
      if ((e = run_gemm<TC, 128, 128, false, false, EPI_PARTIAL>(g, stream)) != hipSuccess) return e;
    }
    const size_t n = L.woff[4] + static_cast<size_t>(L.r[4]) * L.W[4];
    hipLaunchKernelGGL(split_sum_kernel, dim3(static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 4096))), dim3(256),
                       0, stream, upart, upk, W.part_stride, n, dW_up);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 6. dbias = column sums over the token tiles (fp32) or the splits (bf16)
  {
    hipLaunchKernelGGL(colsum_kernel, dim3(static_cast<unsigned>((W.colsum_ld + 31) / 32)), dim3(256), 0, stream,
                       csum, sizeof(TC) == 2 ? W.dw_ksplit : W.mtiles, W.colsum_ld, dbias);
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
  // dpre is kept only by the fp32 path (bf16 recomputes it where it is used)
  w.dpre_off = off;
  size_t dp = 0;
  for (int i = 0; i < 5; ++i) dp += static_cast<size_t>(s.M) * L.W[i];
  if (!s.bf16) off += r256(dp * tc);
  w.dz_off = off;
  off += r256(static_cast<size_t>(s.M) * GATE_RTOT * tc);
  // the token contraction of the weight gradients is split so that the
  // launches fill the chip: about 4096 tokens per split, at most 16 splits
  w.ksplit = std::max(1, std::min(16, (s.M + 4095) / 4096));
  w.kchunk = ((s.M + w.ksplit - 1) / w.ksplit + 63) / 64 * 64;  // whole main-loop steps
  // the up-projections' weight-gradient kernel (bf16) has a split of its own
  w.dw_ksplit = s.bf16 ? std::max(1, std::min(64, (s.M + DW_SPLIT_TOKENS - 1) / DW_SPLIT_TOKENS)) : w.ksplit;
  w.dw_kchunk = ((s.M + w.dw_ksplit - 1) / w.dw_ksplit + 63) / 64 * 64;
  const size_t up = L.woff[4] + static_cast<size_t>(L.r[4]) * L.W[4];
  w.part_stride = r256(std::max(static_cast<size_t>(s.d) * GATE_RTOT, up) * 4) / 4;
  w.part_off = off;
  // dW_down's split partials, then (bf16) the up-projections' own, which the
  // combined kernel writes before dW_down's are formed
  off += static_cast<size_t>(w.ksplit + (s.bf16 ? w.dw_ksplit : 0)) * w.part_stride * 4;
  w.mtiles = (s.M + 127) / 128;
  w.colsum_ld = 0;
  for (int i = 0; i < 5; ++i) w.colsum_ld += L.W[i];
  w.colsum_off = off;
  off += r256(static_cast<size_t>(std::max(w.mtiles, w.dw_ksplit)) * w.colsum_ld * 4);
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
