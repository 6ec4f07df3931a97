// Gate prologue of the Muir operator: the fused low-rank gate projection and
// the SiLU + L2 normalisation of the query / key pathways, forward and
// backward (arXiv 2611.08376; wolonglab summary page, §Methodology: one
// down-projection shared by the five gates, five up-projections at ranks
// (64, 64, 128, 128, 128) with channel biases; fig:arch (b), (c)).
//
// All projections run through one grouped GEMM kernel: up to five
// independent problems per launch (one per gate), 128 x BN tiles on four
// waves, bf16 (v_mfma_f32_16x16x32_bf16) or fp32 (v_mfma_f32_16x16x4_f32)
// with fp32 accumulation, LDS double buffering, and an epilogue chosen at
// compile time:
//   EPI_STORE     C = acc, in the compute type
//   EPI_GATE      C = act(acc + bias), in the compute type
//   EPI_GATE_BWD  dpre = dG * act'(acc + bias) stored in the compute type,
//                 with per-tile column sums of dpre (the bias gradient)
//   EPI_PARTIAL   fp32 partial of one split of the contraction
// Operands are read either along their contiguous axis (k contiguous: rows of
// A, columns of B^T) or across it (k strided), the latter transposed on the
// way into LDS, so every product here -- x W, z U, dpre U^T, dz W^T, x^T dz,
// z^T dpre -- runs without an explicit transpose.
#include <algorithm>

#include "kernels.h"
#include "mma.h"

namespace muir {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int GEMM_THREADS = 256;
constexpr int BK = 32;

enum Epi { EPI_STORE = 0, EPI_GATE = 1, EPI_GATE_BWD = 2, EPI_PARTIAL = 3 };

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

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

// Gate activations (readings of the pages: log-decay = log sigmoid; erase,
// write and the output gate sigmoid; the readout gain 2 sigmoid).
__device__ __forceinline__ float act_fwd(int act, float x) {
  switch (act) {
    case GATE_ACT_LOGSIG: return fminf(x, 0.f) - log1pf(__expf(-fabsf(x)));
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
      return s * (1.f - s);
    }
    case GATE_ACT_SIG2: {
      const float s = sigmoidf_(x);
      return 2.f * s * (1.f - s);
    }
    default: return 1.f;
  }
}

template <typename TC, int BM, int BN, bool A_KC, bool B_KC, int EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(GemmBatch batch) {
  typedef GF<TC> F;
  constexpr int E = 16 / sizeof(TC);  // elements per 16-byte word
  constexpr int LDK = BK + F::PAD;    // LDS row pitch of an operand tile (elements)
  constexpr int TM = BM / 32, TN = BN / 32;  // 16 x 16 tiles per wave (2 x 2 waves)
  constexpr size_t OPS_BYTES = 2 * static_cast<size_t>(BM + BN) * LDK * sizeof(TC);
  constexpr int LDC = BN + 4;  // fp32 pitch of the staged output tile
  constexpr size_t EPI_BYTES = static_cast<size_t>(BM) * LDC * 4;
  constexpr size_t SMEM = OPS_BYTES > EPI_BYTES ? OPS_BYTES : EPI_BYTES;
  __shared__ __align__(16) char smem[SMEM];
  TC* sA = reinterpret_cast<TC*>(smem);                          // [2][BM][LDK]
  TC* sB = reinterpret_cast<TC*>(smem) + 2 * BM * LDK;           // [2][BN][LDK]
  float* sC = reinterpret_cast<float*>(smem);                    // [BM][LDC] after the main loop

  const int grp = blockIdx.z / batch.ksplit;
  const int split = blockIdx.z - grp * batch.ksplit;
  const GemmProblem& P = batch.p[grp];
  const int m0 = blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  if (m0 >= P.M || n0 >= P.N) return;
  const int kchunk = batch.kchunk;
  const int kbeg = split * kchunk;
  const int kend = min(P.K, kbeg + kchunk);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = (wave >> 1) * (BM / 2);
  const int wn = (wave & 1) * (BN / 2);
  const TC* __restrict__ gA = static_cast<const TC*>(P.A);
  const TC* __restrict__ gB = static_cast<const TC*>(P.B);

  // ---- global -> register staging --------------------------------------------
  // k-contiguous operand: R rows of BK values, 16-byte words.
  constexpr int KC_WORDS_A = BM * BK / E / GEMM_THREADS;
  constexpr int KC_WORDS_B = BN * BK / E / GEMM_THREADS;
  // k-strided operand: pairs of k rows x E columns.
  constexpr int KS_ITEMS_A = (BK / 2) * (BM / E) / GEMM_THREADS;
  constexpr int KS_ITEMS_B = (BK / 2) * (BN / E) / GEMM_THREADS;
  constexpr int NA = A_KC ? KC_WORDS_A : 2 * KS_ITEMS_A;
  constexpr int NB = B_KC ? KC_WORDS_B : 2 * KS_ITEMS_B;
  static_assert(NA >= 1 && NB >= 1, "tile too small for the thread count");
  uint4 ra[NA], rb[NB];

  auto load_kc = [&](const TC* g, int ld, int rows_valid, int r0, int k0, uint4* r, int nwords) {
    constexpr int WPR = BK / E;  // words per row
    for (int w = 0; w < nwords; ++w) {
      const int idx = tid + w * GEMM_THREADS;
      const int row = idx / WPR;
      const int kk = (idx - row * WPR) * E;
      const int gr = r0 + row;
      const int gk = k0 + kk;
      uint4 v = {0u, 0u, 0u, 0u};
      if (gr < rows_valid && gk < kend) v = *reinterpret_cast<const uint4*>(g + static_cast<size_t>(gr) * ld + gk);
      r[w] = v;
    }
  };
  auto load_ks = [&](const TC* g, int ld, int cols_valid, int c0, int k0, uint4* r, int nitems, int R) {
    const int CPR = R / E;  // column words per k row
    for (int it = 0; it < nitems; ++it) {
      const int idx = tid + it * GEMM_THREADS;
      const int kp = idx / CPR;
      const int cw = idx - kp * CPR;
      const int gk = k0 + 2 * kp;
      const int gc = c0 + cw * E;
      uint4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
      if (gc < cols_valid) {
        if (gk < kend) v0 = *reinterpret_cast<const uint4*>(g + static_cast<size_t>(gk) * ld + gc);
        if (gk + 1 < kend) v1 = *reinterpret_cast<const uint4*>(g + static_cast<size_t>(gk + 1) * ld + gc);
      }
      r[2 * it] = v0;
      r[2 * it + 1] = v1;
    }
  };
  auto store_kc = [&](TC* s, const uint4* r, int nwords) {
    constexpr int WPR = BK / E;
    for (int w = 0; w < nwords; ++w) {
      const int idx = tid + w * GEMM_THREADS;
      const int row = idx / WPR;
      const int kk = (idx - row * WPR) * E;
      *reinterpret_cast<uint4*>(s + row * LDK + kk) = r[w];
    }
  };
  // k-strided words land transposed: column c's values for k and k+1 side by side.
  auto store_ks = [&](TC* s, const uint4* r, int nitems, int R) {
    const int CPR = R / E;
    for (int it = 0; it < nitems; ++it) {
      const int idx = tid + it * GEMM_THREADS;
      const int kp = idx / CPR;
      const int cw = idx - kp * CPR;
      const TC* v0 = reinterpret_cast<const TC*>(&r[2 * it]);
      const TC* v1 = reinterpret_cast<const TC*>(&r[2 * it + 1]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        TC* dst = s + (cw * E + e) * LDK + 2 * kp;
        if constexpr (sizeof(TC) == 2) {
          const uint32_t pr = static_cast<uint32_t>(v0[e]) | (static_cast<uint32_t>(v1[e]) << 16);
          *reinterpret_cast<uint32_t*>(dst) = pr;
        } else {
          f32x2 pr = {v0[e], v1[e]};
          *reinterpret_cast<f32x2*>(dst) = pr;
        }
      }
    }
  };
  auto load_tiles = [&](int k0) {
    if constexpr (A_KC) load_kc(gA, P.lda, P.M, m0, k0, ra, NA);
    else load_ks(gA, P.lda, P.M, m0, k0, ra, KS_ITEMS_A, BM);
    if constexpr (B_KC) load_kc(gB, P.ldb, P.N, n0, k0, rb, NB);
    else load_ks(gB, P.ldb, P.N, n0, k0, rb, KS_ITEMS_B, BN);
  };
  auto store_tiles = [&](int buf) {
    TC* a = sA + buf * BM * LDK;
    TC* b = sB + buf * BN * LDK;
    if constexpr (A_KC) store_kc(a, ra, NA);
    else store_ks(a, ra, KS_ITEMS_A, BM);
    if constexpr (B_KC) store_kc(b, rb, NB);
    else store_ks(b, rb, KS_ITEMS_B, BN);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero4();

  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  if (nk > 0) {
    load_tiles(kbeg);
    store_tiles(0);
  }
  __syncthreads();
  const int fr = lane & 15;
  const int fk = (F::KF / 4) * (lane >> 4);
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) load_tiles(kbeg + (kt + 1) * BK);
    const TC* a = sA + (kt & 1) * BM * LDK;
    const TC* b = sB + (kt & 1) * BN * LDK;
#pragma unroll
    for (int ks = 0; ks < BK; ks += F::KF) {
      typename F::frag fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = F::load(a + (wm + 16 * i + fr) * LDK + ks + fk);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = F::load(b + (wn + 16 * j + fr) * LDK + ks + fk);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = F::mma(fa[i], fb[j], acc[i][j]);
    }
    if (more) store_tiles((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: stage the fp32 tile in LDS, then write coalesced -------------
  // accumulator (i, j) of the wave: rows wm+16i + 4*(lane/16) + r, column wn+16j + lane%16
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) sC[(wm + 16 * i + 4 * (lane >> 4) + r) * LDC + wn + 16 * j + fr] = acc[i][j][r];
  __syncthreads();

  if constexpr (EPI == EPI_PARTIAL) {
    float* out = static_cast<float*>(P.C) + static_cast<size_t>(split) * batch.split_stride;
    constexpr int WPR = BN / 4;
    for (int idx = tid; idx < BM * WPR; idx += GEMM_THREADS) {
      const int row = idx / WPR;
      const int c = (idx - row * WPR) * 4;
      if (m0 + row < P.M && n0 + c < P.N) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(sC + row * LDC + c);
        *reinterpret_cast<f32x4*>(out + static_cast<size_t>(m0 + row) * P.ldc + n0 + c) = v;
      }
    }
  } else {
    // 8 (bf16) or 4 (fp32) consecutive columns per thread and row
    constexpr int WPR = BN / E;
    constexpr int ROWS_PER_PASS = GEMM_THREADS / WPR;
    const int cw = tid % WPR;
    const int rr = tid / WPR;
    const int c = cw * E;
    const bool col_ok = n0 + c < P.N;
    float bias[E];
    int act = P.act;
    if constexpr (EPI == EPI_GATE || EPI == EPI_GATE_BWD) {
      const TC* bp = static_cast<const TC*>(P.bias);
#pragma unroll
      for (int e = 0; e < E; ++e) bias[e] = col_ok ? Elem<TC>::load(bp, n0 + c + e) : 0.f;
    }
    float csum[E];
#pragma unroll
    for (int e = 0; e < E; ++e) csum[e] = 0.f;
    TC* out = static_cast<TC*>(P.C);
    for (int row = rr; row < BM; row += ROWS_PER_PASS) {
      const int gm = m0 + row;
      if (gm >= P.M || !col_ok) continue;
      float v[E];
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = sC[row * LDC + c + e];
      const size_t o = static_cast<size_t>(gm) * P.ldc + n0 + c;
      if constexpr (EPI == EPI_GATE) {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = act_fwd(act, v[e] + bias[e]);
      } else if constexpr (EPI == EPI_GATE_BWD) {
        uint4 graw = *reinterpret_cast<const uint4*>(static_cast<const TC*>(P.dG) + o);
        const TC* gv = reinterpret_cast<const TC*>(&graw);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          v[e] = Elem<TC>::load(gv, e) * act_grad(act, v[e] + bias[e]);
          csum[e] += v[e];
        }
      }
      uint4 w;
      TC* wv = reinterpret_cast<TC*>(&w);
#pragma unroll
      for (int e = 0; e < E; ++e) Elem<TC>::store(wv, e, v[e]);
      *reinterpret_cast<uint4*>(out + o) = w;
    }
    if constexpr (EPI == EPI_GATE_BWD) {
      // column sums of this tile's dpre: reduce the ROWS_PER_PASS row groups in LDS
      __syncthreads();
      float* red = sC;  // [ROWS_PER_PASS][BN]
#pragma unroll
      for (int e = 0; e < E; ++e) red[rr * BN + c + e] = csum[e];
      __syncthreads();
      if (tid < BN && n0 + tid < P.N) {
        float s = 0.f;
        for (int g = 0; g < ROWS_PER_PASS; ++g) s += red[g * BN + tid];
        batch.colsum[static_cast<size_t>(blockIdx.x) * batch.colsum_ld + P.colsum_off + n0 + tid] = s;
      }
    }
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

// SiLU then L2 normalisation over each row of D values (one head of q or k):
// y = s / sqrt(sum s^2 + eps), s = u sigmoid(u).  D / 4 lanes per row, four
// values per lane; the row sums are taken with lane shuffles inside the group.
template <typename TC, int D>
__global__ __launch_bounds__(256) void qk_norm_fwd_kernel(const TC* __restrict__ u, TC* __restrict__ y,
                                                          long long rows) {
  constexpr int G = D / 4;  // lanes per row
  const long long row = (static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x) / G;
  const int l = threadIdx.x % G;
  const bool ok = row < rows;
  f32x4 s = zero4();
  if (ok) {
    const f32x4 x = load4(u + row * D + 4 * l);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = x[i] * sigmoidf_(x[i]);
  }
  float ss = s[0] * s[0] + s[1] * s[1] + s[2] * s[2] + s[3] * s[3];
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float inv = rsqrtf(ss + QK_L2_EPS);
  if (ok) store4(y + row * D + 4 * l, s * inv);
}

// Reverse mode: du = (dy - y (y . dy)) / n * silu'(u).
template <typename TC, int D>
__global__ __launch_bounds__(256) void qk_norm_bwd_kernel(const TC* __restrict__ u, const TC* __restrict__ dy,
                                                          TC* __restrict__ du, long long rows) {
  constexpr int G = D / 4;
  const long long row = (static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x) / G;
  const int l = threadIdx.x % G;
  const bool ok = row < rows;
  f32x4 x = zero4(), g = zero4(), s, sg;
  if (ok) {
    x = load4(u + row * D + 4 * l);
    g = load4(dy + row * D + 4 * l);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sg[i] = sigmoidf_(x[i]);
    s[i] = x[i] * sg[i];
  }
  float ss = s[0] * s[0] + s[1] * s[1] + s[2] * s[2] + s[3] * s[3];
  float sd = s[0] * g[0] + s[1] * g[1] + s[2] * g[2] + s[3] * g[3];
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) {
    ss += __shfl_xor(ss, off, 64);
    sd += __shfl_xor(sd, off, 64);
  }
  const float n2 = ss + QK_L2_EPS;
  const float inv = rsqrtf(n2);
  const float ydy = sd * inv;  // y . dy
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float ds = (g[i] - s[i] * inv * ydy) * inv;
    r[i] = ds * (sg[i] * (1.f + x[i] * (1.f - sg[i])));
  }
  if (ok) store4(du + row * D + 4 * l, r);
}

template <typename TC, int BM, int BN, bool A_KC, bool B_KC, int EPI>
hipError_t run_gemm(const GemmBatch& b, hipStream_t stream) {
  int mt = 0, nt = 0;
  for (int i = 0; i < b.n; ++i) {
    mt = std::max(mt, (b.p[i].M + BM - 1) / BM);
    nt = std::max(nt, (b.p[i].N + BN - 1) / BN);
  }
  if (mt == 0 || nt == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<TC, BM, BN, A_KC, B_KC, EPI>), dim3(mt, nt, b.n * b.ksplit), dim3(GEMM_THREADS),
                     0, stream, b);
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
hipError_t gate_fwd_typed(const GateShape& s, const void* x, const void* W_down, const void* W_up, const void* bias,
                          void* z, void* const gates[5], hipStream_t stream) {
  const GateLayout L = gate_layout(s);
  const TC* Wu = static_cast<const TC*>(W_up);
  const TC* bs = static_cast<const TC*>(bias);
  GemmBatch b = {};
  b.n = 1;
  b.ksplit = 1;
  b.kchunk = s.d;
  b.p[0] = GemmProblem{x, W_down, z, s.M, GATE_RTOT, s.d, s.d, GATE_RTOT, GATE_RTOT};
  hipError_t e = run_gemm<TC, 128, 128, true, false, EPI_STORE>(b, stream);
  if (e != hipSuccess) return e;
  GemmBatch u = {};
  u.n = 5;
  u.ksplit = 1;
  u.kchunk = 128;
  for (int i = 0; i < 5; ++i) {
    GemmProblem& p = u.p[i];
    p = GemmProblem{static_cast<const TC*>(z) + L.zoff[i], Wu + L.woff[i], gates[i], s.M, L.W[i], L.r[i],
                    GATE_RTOT, L.W[i], L.W[i]};
    p.bias = bs + L.boff[i];
    p.act = kActs[i];
  }
  return run_gemm<TC, 128, 128, true, false, EPI_GATE>(u, stream);
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
    b.p[0] = GemmProblem{x, W_down, z, s.M, GATE_RTOT, s.d, s.d, GATE_RTOT, GATE_RTOT};
    if ((e = run_gemm<TC, 128, 128, true, false, EPI_STORE>(b, stream)) != hipSuccess) return e;
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
    GemmBatch u = {};
    u.n = 5;
    u.ksplit = 1;
    u.kchunk = 128;
    u.colsum = csum;
    u.colsum_ld = W.colsum_ld;
    int coff = 0;
    for (int i = 0; i < 5; ++i) {
      GemmProblem& p = u.p[i];
      p = GemmProblem{zr + L.zoff[i], Wu + L.woff[i], dpre + dpo[i], s.M, L.W[i], L.r[i], GATE_RTOT, L.W[i],
                      L.W[i]};
      p.bias = bs + L.boff[i];
      p.act = kActs[i];
      p.dG = dgates[i];
      p.colsum_off = coff;
      coff += L.W[i];
    }
    if ((e = run_gemm<TC, 128, 128, true, false, EPI_GATE_BWD>(u, stream)) != hipSuccess) return e;
  }
  // 2. dz[:, slice_i] = dpre_i U_i^T
  {
    GemmBatch u = {};
    u.n = 5;
    u.ksplit = 1;
    u.kchunk = std::max(L.W[0], L.W[2]);
    for (int i = 0; i < 5; ++i)
      u.p[i] = GemmProblem{dpre + dpo[i], Wu + L.woff[i], dz + L.zoff[i], s.M, L.r[i], L.W[i], L.W[i], L.W[i],
                           GATE_RTOT};
    if ((e = run_gemm<TC, 128, 64, true, true, EPI_STORE>(u, stream)) != hipSuccess) return e;
  }
  // 3. dx = dz W_down^T
  {
    GemmBatch b = {};
    b.n = 1;
    b.ksplit = 1;
    b.kchunk = GATE_RTOT;
    b.p[0] = GemmProblem{dz, W_down, dx, s.M, s.d, GATE_RTOT, GATE_RTOT, GATE_RTOT, s.d};
    if ((e = run_gemm<TC, 128, 128, true, true, EPI_STORE>(b, stream)) != hipSuccess) return e;
  }
  // 4. dW_down = x^T dz (split over tokens), 5. dW_up_i = z_i^T dpre_i (split over tokens)
  {
    GemmBatch b = {};
    b.n = 1;
    b.ksplit = W.ksplit;
    b.kchunk = W.kchunk;
    b.split_stride = W.part_stride;
    b.p[0] = GemmProblem{x, dz, part, s.d, GATE_RTOT, s.M, s.d, GATE_RTOT, GATE_RTOT};
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
      u.p[i] = GemmProblem{zr + L.zoff[i], dpre + dpo[i], part + L.woff[i], L.r[i], L.W[i], s.M, GATE_RTOT, L.W[i],
                           L.W[i]};
    if ((e = run_gemm<TC, 128, 128, false, false, EPI_PARTIAL>(u, stream)) != hipSuccess) return e;
    const size_t n = L.woff[4] + static_cast<size_t>(L.r[4]) * L.W[4];
    hipLaunchKernelGGL(split_sum_kernel, dim3(static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 4096))), dim3(256),
                       0, stream, part, W.ksplit, W.part_stride, n, dW_up);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 6. dbias = column sums over the token tiles
  {
    const size_t n = W.colsum_ld;
    hipLaunchKernelGGL(split_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, csum,
                       W.mtiles, static_cast<size_t>(W.colsum_ld), n, dbias);
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
  w.kchunk = ((s.M + w.ksplit - 1) / w.ksplit + BK - 1) / BK * BK;
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
  const long long threads = rows * (D / 4);
  const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
#define MUIR_QKN(TC, DD)                                                                                        \
  if (dy)                                                                                                        \
    hipLaunchKernelGGL((qk_norm_bwd_kernel<TC, DD>), dim3(blocks), dim3(256), 0, stream,                         \
                       static_cast<const TC*>(u), static_cast<const TC*>(dy), static_cast<TC*>(out), rows);      \
  else                                                                                                           \
    hipLaunchKernelGGL((qk_norm_fwd_kernel<TC, DD>), dim3(blocks), dim3(256), 0, stream,                         \
                       static_cast<const TC*>(u), static_cast<TC*>(out), rows);
  if (bf16) {
    if (D == 64) { MUIR_QKN(uint16_t, 64) } else { MUIR_QKN(uint16_t, 128) }
  } else {
    if (D == 64) { MUIR_QKN(float, 64) } else { MUIR_QKN(float, 128) }
  }
#undef MUIR_QKN
  return hipGetLastError();
}

}  // namespace muir
