// Sequential chunk scans of the Muir gated delta rule (gfx950): the forward
// state scan with the chunk output, and the reverse scan of the state
// gradient.
//
// arXiv 2611.08376, Methodology: chunks are processed in order and the state
// carries the recurrence across chunk boundaries.  With the chunk summary
// (W, Q', Kbar, U~, O~, Gamma_C) of the chunkwise forward (fwd.hip), which
// both scans read:
//   forward:  o = O~ + Q' S,  S_next = diag(Gamma_C) S + Kbar^T (U~ - W S)
//   backward: dS = diag(Gamma_C) dS_next + Q'^T dO - W^T (Kbar dS_next)
// (the backward is the adjoint of the forward update; the pages state only
// that a custom backward pass is used).
//
// Work split: one workgroup per (b, h, NV = 16 NW state columns), one wave
// per 16 columns; the state stays in MFMA accumulators (fp32) for the whole
// sequence.  Chunks are walked in units of SB tokens.  A unit's summary tiles
// are loaded one unit ahead into registers as 16-byte words (no load is under
// a branch, so they stay in flight across the current unit's products) and
// written to LDS tiles whose 16-byte chunks are XOR-permuted per row, so that
// the fragment reads of 16 lanes on 16 rows fall on distinct banks.
#include "kernels.h"
#include "mma.h"

namespace muir {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Byte offset of (row, byte) in an LDS tile with rows of L bytes (a power of
// two >= 32), 16-byte chunks permuted per row.
template <int L> __device__ __forceinline__ int swz(int row, int byte) {
  constexpr int CPR = L / 16;
  const int key = CPR >= 16 ? (row & 15) : ((row / (16 / CPR)) & (CPR - 1));
  return row * L + (((byte >> 4) ^ key) << 4) + (byte & 15);
}

template <int WORDS, int NTH> constexpr int words_per_thread() { return (WORDS + NTH - 1) / NTH; }

// Tokens per unit: 16 NW (bf16) or 8 NW (fp32), at least 16; a unit's tiles
// then take 16 words of 16 bytes per thread at d = 128.
template <typename TC, int NW> constexpr int scan_unit() {
  return (sizeof(TC) == 2 ? 16 : 8) * NW < 16 ? 16 : (sizeof(TC) == 2 ? 16 : 8) * NW;
}

template <typename TC> __device__ __forceinline__ typename MM<TC>::frag identity_frag(int g, int c16) {
  f32x4 idv;
#pragma unroll
  for (int i = 0; i < 4; ++i) idv[i] = (4 * g + i == c16) ? 1.f : 0.f;
  return MM<TC>::from_f32(idv);
}

// ---------------------------------------------------------------------------
// Forward.  Reads W [C][DK], Q' [C][DK], Kbar^T [DK][C], U~^T [DV][C],
// O~^T [DV][C] and Gamma_C of each chunk summary (SummaryPart).
template <typename Tin, int DK, int NW>
__global__ __launch_bounds__(64 * NW) void fwd_scan_kernel(
    int T, int H, int C, const char* __restrict__ summ, size_t summ_bytes,
    const float* __restrict__ S0, Tin* __restrict__ o, float* __restrict__ S_chunks,
    float* __restrict__ S_T, char* __restrict__ dsumm, size_t dl_offset) {
  typedef Tin TC;
  typedef MM<TC> M;
  typedef typename M::frag frag;
  constexpr int DV = DK;
  constexpr int RT = DK / 16;
  constexpr int NV = 16 * NW;
  constexpr int NTH = 64 * NW;
  constexpr int SZ = sizeof(TC);
  constexpr int SB = scan_unit<TC, NW>();
  constexpr int LW = DK * SZ;       // bytes per W / Q' row
  constexpr int LK = SB * SZ;       // bytes per unit segment of a Kbar^T / U~^T / O~^T row
  constexpr int CW = LW / 16;
  constexpr int CK = LK / 16;
  constexpr int W_WORDS = SB * CW;  // also Q'
  constexpr int K_WORDS = DK * CK;
  constexpr int U_WORDS = NV * CK;  // also O~
  constexpr int G_WORDS = DK / 4;
  constexpr int PW = words_per_thread<W_WORDS, NTH>();
  constexpr int PK = words_per_thread<K_WORDS, NTH>();
  constexpr int PU = words_per_thread<U_WORDS, NTH>();
  constexpr int PG = words_per_thread<G_WORDS, NTH>();

  const int NC = T / C;
  const int NSB = C / SB;
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
  const int col0 = vb * NV + 16 * wave;  // this wave's first state column
  const int colg = col0 + c16;

  __shared__ __attribute__((aligned(16))) char sW[SB * LW];
  __shared__ __attribute__((aligned(16))) char sQ[SB * LW];
  __shared__ __attribute__((aligned(16))) char sK[DK * LK];
  __shared__ __attribute__((aligned(16))) char sU[NV * LK];
  __shared__ __attribute__((aligned(16))) char sO[NV * LK];
  __shared__ __attribute__((aligned(16))) float sgC[DK];

  const char* hsum = summ + static_cast<size_t>(bh) * NC * summ_bytes;  // this head's summaries
  u32x4 rw[PW], rq[PW], rk[PK], ru[PU], ro[PU], rg[PG];

  auto prefetch = [&](int u) {
    const int c = u / NSB;
    const int sb = u - c * NSB;
    const char* base = hsum + static_cast<size_t>(c) * summ_bytes;
    auto part = [&](int p) { return static_cast<uint32_t>(summary_part(p, C, DK, DV) * SZ); };
    const uint32_t wofs = part(SP_W) + static_cast<uint32_t>(sb * SB * LW);
    const uint32_t qofs = part(SP_QP) + static_cast<uint32_t>(sb * SB * LW);
    const uint32_t kofs = part(SP_KBT) + static_cast<uint32_t>(sb * LK);
    const uint32_t uofs = part(SP_UTT) + static_cast<uint32_t>(vb * NV * C * SZ + sb * LK);
    const uint32_t oofs = part(SP_OTT) + static_cast<uint32_t>(vb * NV * C * SZ + sb * LK);
    const uint32_t gofs = part(SP_END);
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int w = min(tid + k * NTH, W_WORDS - 1);
      rw[k] = *reinterpret_cast<const u32x4*>(at(base, wofs + 16 * w));
      rq[k] = *reinterpret_cast<const u32x4*>(at(base, qofs + 16 * w));
    }
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      const int w = min(tid + k * NTH, K_WORDS - 1);
      rk[k] = *reinterpret_cast<const u32x4*>(at(base, kofs + (w / CK) * C * SZ + 16 * (w % CK)));
    }
#pragma unroll
    for (int k = 0; k < PU; ++k) {
      const int w = min(tid + k * NTH, U_WORDS - 1);
      const uint32_t ro_ = (w / CK) * C * SZ + 16 * (w % CK);
      ru[k] = *reinterpret_cast<const u32x4*>(at(base, uofs + ro_));
      ro[k] = *reinterpret_cast<const u32x4*>(at(base, oofs + ro_));
    }
#pragma unroll
    for (int k = 0; k < PG; ++k) {
      const int w = min(tid + k * NTH, G_WORDS - 1);
      rg[k] = *reinterpret_cast<const u32x4*>(at(base, gofs + 16 * w));
    }
  };

  auto commit = [&]() {
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int w = min(tid + k * NTH, W_WORDS - 1);
      const int a = swz<LW>(w / CW, 16 * (w % CW));
      *reinterpret_cast<u32x4*>(sW + a) = rw[k];
      *reinterpret_cast<u32x4*>(sQ + a) = rq[k];
    }
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      const int w = min(tid + k * NTH, K_WORDS - 1);
      *reinterpret_cast<u32x4*>(sK + swz<LK>(w / CK, 16 * (w % CK))) = rk[k];
    }
#pragma unroll
    for (int k = 0; k < PU; ++k) {
      const int w = min(tid + k * NTH, U_WORDS - 1);
      const int a = swz<LK>(w / CK, 16 * (w % CK));
      *reinterpret_cast<u32x4*>(sU + a) = ru[k];
      *reinterpret_cast<u32x4*>(sO + a) = ro[k];
    }
#pragma unroll
    for (int k = 0; k < PG; ++k) {
      const int w = min(tid + k * NTH, G_WORDS - 1);
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(sgC) + 16 * w) = rg[k];
    }
  };

  const frag ident = identity_frag<TC>(g, c16);
  const size_t sbase = static_cast<size_t>(bh) * DK * DV;
  f32x4 S[RT];
#pragma unroll
  for (int s = 0; s < RT; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[s][i] = S0 ? S0[sbase + static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] : 0.f;
  frag Sf[RT];
  f32x4 dS[RT];

  const int U = NC * NSB;
  if (U > 0) prefetch(0);
#pragma unroll 1
  for (int u = 0; u < U; ++u) {
    const int c = u / NSB;
    const int sb = u - c * NSB;
    __syncthreads();  // the previous unit's LDS reads are done
    commit();
    prefetch(u + 1 < U ? u + 1 : u);
    __syncthreads();
    if (sb == 0) {
      if (S_chunks) {
        float* dst = S_chunks + (static_cast<size_t>(bh) * NC + c) * DK * DV;
#pragma unroll
        for (int s = 0; s < RT; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] = S[s][i];
      }
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        Sf[s] = M::from_f32(S[s]);
        dS[s] = zero4();
      }
    }
    // token t of the unit is sequence position c*C + sb*SB + t
    const size_t obase = ((static_cast<size_t>(b) * T + static_cast<size_t>(c) * C + sb * SB) * H + h) * DV;
    // this chunk's deltas [C][DV] in its summary (when they are kept)
    TC* dlc = dsumm ? reinterpret_cast<TC*>(dsumm + (static_cast<size_t>(bh) * NC + c) * summ_bytes + dl_offset)
                    : nullptr;
#pragma unroll 2
    for (int m = 0; m < SB / 16; ++m) {
      f32x4 Oa = zero4(), Da = zero4();
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        const int a = swz<LW>(16 * m + c16, (16 * s + 4 * g) * SZ);
        if (o) Oa = M::mma(M::load(reinterpret_cast<const TC*>(sQ + a)), Sf[s], Oa);
        Da = M::mma(M::load(reinterpret_cast<const TC*>(sW + a)), Sf[s], Da);
      }
      const int au = swz<LK>(16 * wave + c16, (16 * m + 4 * g) * SZ);
      if (o) {
        const f32x4 ot = load4(reinterpret_cast<const TC*>(sO + au));
        // tokens 4g+i, column c16 -> token c16, columns 4g..4g+3
        const f32x4 tt = M::mma(M::from_f32(Oa + ot), ident, zero4());
        store4(at(o + obase, static_cast<uint32_t>((16 * m + c16) * H * DV + col0 + 4 * g)), tt);
      }
      const f32x4 ut = load4(reinterpret_cast<const TC*>(sU + au));
      const frag df = M::from_f32(ut - Da);
      if (dlc) {
        // the deltas in the compute type, as token rows (exact: a product with the identity)
        const f32x4 tt = M::mma(df, ident, zero4());
        store4(at(dlc, static_cast<uint32_t>((sb * SB + 16 * m + c16) * DV + col0 + 4 * g)), tt);
      }
#pragma unroll
      for (int s = 0; s < RT; ++s)
        dS[s] = M::mma(M::load(reinterpret_cast<const TC*>(sK + swz<LK>(16 * s + c16, (16 * m + 4 * g) * SZ))),
                       df, dS[s]);
    }
    if (sb == NSB - 1) {
#pragma unroll
      for (int s = 0; s < RT; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[s][i] = sgC[16 * s + 4 * g + i] * S[s][i] + dS[s][i];
    }
  }
  if (S_T) {
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) S_T[sbase + static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] = S[s][i];
  }
}

// ---------------------------------------------------------------------------
// Backward, on the same summaries: reads W^T [DK][C], Q'^T [DK][C] and
// Kbar [C][DK] (the orientations whose contraction index is contiguous for
// these products) and Gamma_C.
template <typename Tin, int DK, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_scan_kernel(
    int T, int H, int C, const char* __restrict__ summ, size_t summ_bytes,
    const Tin* __restrict__ dO, const float* __restrict__ dS_T, Tin* __restrict__ dS_chunks,
    float* __restrict__ dS0) {
  typedef Tin TC;
  typedef MM<TC> M;
  typedef typename M::frag frag;
  constexpr int DV = DK;
  constexpr int RT = DK / 16;
  constexpr int NV = 16 * NW;
  constexpr int NTH = 64 * NW;
  constexpr int SZ = sizeof(TC);
  constexpr int SB = scan_unit<TC, NW>();
  constexpr int LW = DK * SZ;       // bytes per Kbar row
  constexpr int LK = SB * SZ;       // bytes per unit segment of a W^T / Q'^T row
  constexpr int LO = NV * SZ;       // bytes per dO row segment of this workgroup
  constexpr int CW = LW / 16;
  constexpr int CK = LK / 16;
  constexpr int CO = LO / 16;
  constexpr int K_WORDS = SB * CW;  // Kbar
  constexpr int T_WORDS = DK * CK;  // W^T, also Q'^T
  constexpr int O_WORDS = SB * CO;
  constexpr int G_WORDS = DK / 4;
  constexpr int PK = words_per_thread<K_WORDS, NTH>();
  constexpr int PT = words_per_thread<T_WORDS, NTH>();
  constexpr int PO = words_per_thread<O_WORDS, NTH>();
  constexpr int PG = words_per_thread<G_WORDS, NTH>();
  static_assert(LO >= 32, "dO row segment");

  const int NC = T / C;
  const int NSB = C / SB;
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

  __shared__ __attribute__((aligned(16))) char sWt[DK * LK];
  __shared__ __attribute__((aligned(16))) char sQt[DK * LK];
  __shared__ __attribute__((aligned(16))) char sKb[SB * LW];
  __shared__ __attribute__((aligned(16))) char sDO[SB * LO];
  __shared__ __attribute__((aligned(16))) float sgC[DK];

  const char* hsum = summ + static_cast<size_t>(bh) * NC * summ_bytes;
  u32x4 rt[PT], rq[PT], rk[PK], rd[PO], rg[PG];

  // unit u walks the chunks in reverse, and each chunk's units in reverse
  auto unit_c = [&](int u) { return NC - 1 - u / NSB; };
  auto unit_sb = [&](int u) { return NSB - 1 - (u - (u / NSB) * NSB); };

  auto prefetch = [&](int u) {
    const int c = unit_c(u);
    const int sb = unit_sb(u);
    const char* base = hsum + static_cast<size_t>(c) * summ_bytes;
    auto part = [&](int p) { return static_cast<uint32_t>(summary_part(p, C, DK, DV) * SZ); };
    const uint32_t tofs = part(SP_WT) + static_cast<uint32_t>(sb * LK);
    const uint32_t qofs = part(SP_QT) + static_cast<uint32_t>(sb * LK);
    const uint32_t kofs = part(SP_KB) + static_cast<uint32_t>(sb * SB * LW);
    const uint32_t gofs = part(SP_END);
    const char* dob = reinterpret_cast<const char*>(
        dO + ((static_cast<size_t>(b) * T + static_cast<size_t>(c) * C + sb * SB) * H + h) * DV + vb * NV);
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      const int w = min(tid + k * NTH, T_WORDS - 1);
      const uint32_t r = (w / CK) * C * SZ + 16 * (w % CK);
      rt[k] = *reinterpret_cast<const u32x4*>(at(base, tofs + r));
      rq[k] = *reinterpret_cast<const u32x4*>(at(base, qofs + r));
    }
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      const int w = min(tid + k * NTH, K_WORDS - 1);
      rk[k] = *reinterpret_cast<const u32x4*>(at(base, kofs + 16 * w));
    }
#pragma unroll
    for (int k = 0; k < PO; ++k) {
      const int w = min(tid + k * NTH, O_WORDS - 1);
      rd[k] = *reinterpret_cast<const u32x4*>(at(dob, static_cast<uint32_t>((w / CO) * H * DV * SZ + 16 * (w % CO))));
    }
#pragma unroll
    for (int k = 0; k < PG; ++k) {
      const int w = min(tid + k * NTH, G_WORDS - 1);
      rg[k] = *reinterpret_cast<const u32x4*>(at(base, gofs + 16 * w));
    }
  };

  auto commit = [&]() {
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      const int w = min(tid + k * NTH, T_WORDS - 1);
      const int a = swz<LK>(w / CK, 16 * (w % CK));
      *reinterpret_cast<u32x4*>(sWt + a) = rt[k];
      *reinterpret_cast<u32x4*>(sQt + a) = rq[k];
    }
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      const int w = min(tid + k * NTH, K_WORDS - 1);
      *reinterpret_cast<u32x4*>(sKb + swz<LW>(w / CW, 16 * (w % CW))) = rk[k];
    }
#pragma unroll
    for (int k = 0; k < PO; ++k) {
      const int w = min(tid + k * NTH, O_WORDS - 1);
      *reinterpret_cast<u32x4*>(sDO + swz<LO>(w / CO, 16 * (w % CO))) = rd[k];
    }
#pragma unroll
    for (int k = 0; k < PG; ++k) {
      const int w = min(tid + k * NTH, G_WORDS - 1);
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(sgC) + 16 * w) = rg[k];
    }
  };

  const frag ident = identity_frag<TC>(g, c16);
  const size_t sbase = static_cast<size_t>(bh) * DK * DV;
  f32x4 dS[RT];
#pragma unroll
  for (int s = 0; s < RT; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dS[s][i] = dS_T ? dS_T[sbase + static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] : 0.f;
  frag dSf[RT];
  f32x4 Z[RT];

  const int U = NC * NSB;
  if (U > 0) prefetch(0);
#pragma unroll 1
  for (int u = 0; u < U; ++u) {
    const int c = unit_c(u);
    const int sb = unit_sb(u);
    __syncthreads();
    commit();
    prefetch(u + 1 < U ? u + 1 : u);
    __syncthreads();
    if (sb == NSB - 1) {
      // gradient at the end of chunk c, in the compute type, as transposed
      // 16-row tiles (the lane's four rows of column colg are contiguous)
      TC* dst = dS_chunks + (static_cast<size_t>(bh) * NC + c) * DK * DV;
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        store4(at(dst, static_cast<uint32_t>((s * DV + colg) * 16 + 4 * g)), dS[s]);
        dSf[s] = M::from_f32(dS[s]);
        Z[s] = zero4();
      }
    }
#pragma unroll 2
    for (int m = 0; m < SB / 16; ++m) {
      // X = Kbar_m dS_next (16 tokens x this wave's 16 columns)
      f32x4 X = zero4();
#pragma unroll
      for (int s = 0; s < RT; ++s)
        X = M::mma(M::load(reinterpret_cast<const TC*>(sKb + swz<LW>(16 * m + c16, (16 * s + 4 * g) * SZ))), dSf[s], X);
      // dO rows as the right operand (tokens along the contraction): one
      // identity product turns the row fragment around
      const f32x4 dot = M::mma(
          M::load(reinterpret_cast<const TC*>(sDO + swz<LO>(16 * m + c16, (16 * wave + 4 * g) * SZ))), ident,
          zero4());
      const frag dof = M::from_f32(dot);
      const frag xf = M::from_f32(-X);
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        const int a = swz<LK>(16 * s + c16, (16 * m + 4 * g) * SZ);
        Z[s] = M::mma(M::load(reinterpret_cast<const TC*>(sQt + a)), dof, Z[s]);
        Z[s] = M::mma(M::load(reinterpret_cast<const TC*>(sWt + a)), xf, Z[s]);
      }
    }
    if (sb == 0) {
#pragma unroll
      for (int s = 0; s < RT; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) dS[s][i] = sgC[16 * s + 4 * g + i] * dS[s][i] + Z[s][i];
    }
  }
  if (dS0) {
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) dS0[sbase + static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] = dS[s][i];
  }
}

}  // namespace

// Four waves (64 columns) per workgroup when that still fills the chip, else
// one wave (16 columns) per workgroup for more independent chains.
hipError_t launch_fwd_scan(const ChunkShape& s, const void* summ, const float* S0, void* o,
                           float* S_chunks, float* S_T, void* deltas, hipStream_t stream) {
  const int heads = s.B * s.H;
  if (heads == 0) return hipSuccess;
  const bool wide = static_cast<long long>(heads) * (s.DV / 64) >= 256;
#define MUIR_SCAN(TT, DD, NW)                                                                      \
  hipLaunchKernelGGL((fwd_scan_kernel<TT, DD, NW>), dim3(heads * (s.DV / (16 * NW))),              \
                     dim3(64 * NW), 0, stream, s.T, s.H, s.C, (const char*)summ, s.summary_bytes(), \
                     S0, (TT*)o, S_chunks, S_T, (char*)deltas, s.dl_offset())
  if (s.bf16) {
    if (s.DK == 128) {
      if (wide) MUIR_SCAN(uint16_t, 128, 4); else MUIR_SCAN(uint16_t, 128, 1);
    } else {
      if (wide) MUIR_SCAN(uint16_t, 64, 4); else MUIR_SCAN(uint16_t, 64, 1);
    }
  } else {
    if (s.DK == 128) {
      if (wide) MUIR_SCAN(float, 128, 4); else MUIR_SCAN(float, 128, 1);
    } else {
      if (wide) MUIR_SCAN(float, 64, 4); else MUIR_SCAN(float, 64, 1);
    }
  }
#undef MUIR_SCAN
  return hipGetLastError();
}

hipError_t launch_bwd_scan(const ChunkShape& s, const void* summ, const void* dO, const float* dS_T,
                           void* dS_chunks, float* dS0, hipStream_t stream) {
  const int heads = s.B * s.H;
  if (heads == 0) return hipSuccess;
  const bool wide = static_cast<long long>(heads) * (s.DV / 64) >= 256;
#define MUIR_BSCAN(TT, DD, NW)                                                                     \
  hipLaunchKernelGGL((bwd_scan_kernel<TT, DD, NW>), dim3(heads * (s.DV / (16 * NW))),              \
                     dim3(64 * NW), 0, stream, s.T, s.H, s.C, (const char*)summ, s.summary_bytes(), \
                     (const TT*)dO, dS_T, (TT*)dS_chunks, dS0)
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
