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

// LDS tile addressing.  A tile has rows of L bytes; its G-byte granules (G =
// 8 for bf16 fragments, read 8 bytes per lane, or 16 for fp32 ones) are
// XOR-permuted per row.  LDS serves a fragment read 128 bytes at a time (32
// banks of 4 bytes): 16 lanes of an 8-byte read, 8 of a 16-byte one, each lane
// on its own row at the same column.  The key spreads those rows over distinct
// granules of the 128-byte bank window (rows shorter than the window share
// it, and the key then runs over the rows of one window).  XOR on 16-byte
// chunks would leave 8-byte reads two-way conflicted.
template <int L, int G> __device__ __forceinline__ int swz_key(int row) {
  constexpr int S = L / G;                       // granules per row
  constexpr int WIN = 128 / G;                   // granules per bank window
  constexpr int RPW = S >= WIN ? 1 : WIN / S;    // rows per bank window
  constexpr int KS = S >= WIN ? WIN : S;
  return (row / RPW) & (KS - 1);
}
template <int L, int G> __device__ __forceinline__ int swz(int row, int byte) {
  return row * L + (((byte / G) ^ swz_key<L, G>(row)) * G) + (byte % G);
}
// Writes the 16-byte word holding bytes [16 c, 16 c + 16) of a row.  With
// 8-byte granules its halves land in one aligned 16-byte chunk, swapped when
// the key is odd.
template <int L, int G> __device__ __forceinline__ void put16(char* tile, int row, int c, u32x4 w) {
  if constexpr (G == 16) {
    *reinterpret_cast<u32x4*>(tile + swz<L, 16>(row, 16 * c)) = w;
  } else {
    const int key = swz_key<L, 8>(row);
    const u32x4 sw = {w[2], w[3], w[0], w[1]};
    *reinterpret_cast<u32x4*>(tile + row * L + ((c ^ (key >> 1)) << 4)) = (key & 1) ? sw : w;
  }
}

// Workgroup id -> (group, member): the nvb workgroups of one (head, segment)
// read the same chunk summaries, so they are placed on one XCD (consecutive
// workgroup ids go round-robin over the 8 XCDs, each with its own L2) and
// dispatched together: member k of group P is workgroup
// ((P / 8) * m + k) * 8 + P % 8.  A grid that is not a whole number of
// 8-group rounds keeps the plain order.
__device__ __forceinline__ int2 xcd_group(int id, int m, int ngroups) {
  if (ngroups % 8 != 0) return make_int2(id / m, id % m);
  const int xcd = id % 8, slot = id / 8;
  return make_int2((slot / m) * 8 + xcd, slot % m);
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
//
// Segments: the chunks of a sequence are split into nseg consecutive
// segments, one workgroup row each.  With TRANS the kernel runs the
// recurrence S <- (diag(Gamma_C) - Kbar^T W) S + Kbar^T U~ over its segment
// from [S | P] = [0 | I] (dk more state columns, whose U~ is zero) and writes
// the segment's offset E and transition P into trans[head][seg] ([dk][DV + DK]
// fp32); without it, segment seg > 0 starts from S_seg[head][seg] ([dk][dv]
// fp32, formed from those by seg_combine_kernel) and segment 0 from S0.
template <typename Tin, int DK, int NW, bool TRANS>
__global__ __launch_bounds__(64 * NW) void fwd_scan_kernel(
    int T, int H, int C, const char* __restrict__ summ, size_t summ_bytes,
    const float* __restrict__ S0, Tin* __restrict__ o, Tin* __restrict__ S_chunks,
    float* __restrict__ S_T, char* __restrict__ dsumm, size_t dl_offset, int nseg,
    const float* __restrict__ S_seg, float* __restrict__ trans) {
  typedef Tin TC;
  typedef MM<TC> M;
  typedef typename M::frag frag;
  constexpr int DV = DK;
  constexpr int RT = DK / 16;
  constexpr int NV = 16 * NW;
  constexpr int NTH = 64 * NW;
  constexpr int SZ = sizeof(TC);
  constexpr int GR = SZ == 2 ? 8 : 16;  // LDS swizzle granule: the fragment read size
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
  constexpr int NCOL = TRANS ? DV + DK : DV;  // state columns ([S | P] with TRANS)

  const int NC = T / C;
  const int NSB = C / SB;
  const int nvb = NCOL / NV;
  const int2 gm = xcd_group(blockIdx.x, nvb, static_cast<int>(gridDim.x) / nvb);
  const int bh = gm.x / nseg;
  const int seg = gm.x - bh * nseg;
  const int vb = gm.y;
  const int L = (NC + nseg - 1) / nseg;  // chunks per segment
  const int cbeg = min(NC, seg * L);
  const int cend = min(NC, cbeg + L);
  const bool pcols = TRANS && vb * NV >= DV;  // transition columns: no U~ (their loads read tile 0)
  const int vbu = pcols ? 0 : vb;
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
    // (the transposed parts in 16-token tiles: row r, word ww of the unit
    // is token sb * SB + ww * (16 / SZ))
    const uint32_t kofs = part(SP_KBT);
    const uint32_t uofs = part(SP_UTT);
    const uint32_t oofs = part(SP_OTT);
    auto tofs = [&](int r, int ww, int D) {
      return static_cast<uint32_t>(tpart_index(r, sb * SB + ww * (16 / SZ), D) * SZ);
    };
    const uint32_t gofs = part(SP_END);
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int w = min(tid + k * NTH, W_WORDS - 1);
      rw[k] = *reinterpret_cast<const u32x4*>(at(base, wofs + 16 * w));
      if constexpr (!TRANS) rq[k] = *reinterpret_cast<const u32x4*>(at(base, qofs + 16 * w));
    }
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      const int w = min(tid + k * NTH, K_WORDS - 1);
      rk[k] = *reinterpret_cast<const u32x4*>(at(base, kofs + tofs(w / CK, w % CK, DK)));
    }
#pragma unroll
    for (int k = 0; k < PU; ++k) {
      const int w = min(tid + k * NTH, U_WORDS - 1);
      const uint32_t ro_ = tofs(vbu * NV + w / CK, w % CK, DV);
      ru[k] = *reinterpret_cast<const u32x4*>(at(base, uofs + ro_));
      if constexpr (!TRANS) ro[k] = *reinterpret_cast<const u32x4*>(at(base, oofs + ro_));
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
      put16<LW, GR>(sW, w / CW, w % CW, rw[k]);
      if constexpr (!TRANS) put16<LW, GR>(sQ, w / CW, w % CW, rq[k]);
    }
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      const int w = min(tid + k * NTH, K_WORDS - 1);
      put16<LK, GR>(sK, w / CK, w % CK, rk[k]);
    }
#pragma unroll
    for (int k = 0; k < PU; ++k) {
      const int w = min(tid + k * NTH, U_WORDS - 1);
      const u32x4 zw = {0u, 0u, 0u, 0u};
      put16<LK, GR>(sU, w / CK, w % CK, pcols ? zw : ru[k]);
      if constexpr (!TRANS) put16<LK, GR>(sO, w / CK, w % CK, ro[k]);
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
  {
    // the segment's start: [0 | I] with TRANS, else S0 or the segment state
    const float* src = seg == 0 ? (S0 ? S0 + sbase : nullptr)
                                : S_seg + (static_cast<size_t>(bh) * nseg + seg) * DK * DV;
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * s + 4 * g + i;
        if constexpr (TRANS) S[s][i] = (pcols && row == colg - DV) ? 1.f : 0.f;
        else S[s][i] = src ? src[static_cast<size_t>(row) * DV + colg] : 0.f;
      }
  }
  frag Sf[RT];
  f32x4 dS[RT];

  const int U0 = cbeg * NSB, U1 = cend * NSB;
  if (U0 < U1) prefetch(U0);
#pragma unroll 1
  for (int u = U0; u < U1; ++u) {
    const int c = u / NSB;
    const int sb = u - c * NSB;
    // The chunk-start state is stored first, ahead of this unit's commit and
    // the next unit's loads: vector memory instructions issue in order, so
    // stores queued behind a unit of loads wait for them.  (Measured at B = 8,
    // T = 4096, H = 16, d = 128, bf16: 304 us here, 321 us between the commit
    // and the prefetch, 328 us after the prefetch.)
    if (sb == 0) {
      if (!TRANS && S_chunks) {
        // the chunk-start state, kept for the backward in the compute type
        Tin* dst = S_chunks + (static_cast<size_t>(bh) * NC + c) * DK * DV;
        if constexpr (sizeof(Tin) == 4) {
#pragma unroll
          for (int s = 0; s < RT; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] = S[s][i];
        } else {
          // rounded once, then turned onto rows by an identity product (exact):
          // row 16s + c16, four columns per lane
#pragma unroll
          for (int s = 0; s < RT; ++s)
            store4(at(dst, static_cast<uint32_t>((16 * s + c16) * DV + col0 + 4 * g)),
                   M::mma(M::from_f32(S[s]), ident, zero4()));
        }
      }
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        Sf[s] = M::from_f32(S[s]);
        dS[s] = zero4();
      }
    }
    __syncthreads();  // the previous unit's LDS reads are done
    commit();
    prefetch(u + 1 < U1 ? u + 1 : u);
    __syncthreads();
    // token t of the unit is sequence position c*C + sb*SB + t
    const size_t obase = ((static_cast<size_t>(b) * T + static_cast<size_t>(c) * C + sb * SB) * H + h) * DV;
    // this chunk's deltas [C][DV] in its summary (when they are kept)
    TC* dlc = (!TRANS && dsumm)
                  ? reinterpret_cast<TC*>(dsumm + (static_cast<size_t>(bh) * NC + c) * summ_bytes + dl_offset)
                  : nullptr;
#pragma unroll 2
    for (int m = 0; m < SB / 16; ++m) {
      // two accumulators per product (even and odd key tiles): independent
      // MFMA chains of half the length
      f32x4 Oa0 = zero4(), Oa1 = zero4(), Da0 = zero4(), Da1 = zero4();
#pragma unroll
      for (int s = 0; s < RT; s += 2) {
        const int a0 = swz<LW, GR>(16 * m + c16, (16 * s + 4 * g) * SZ);
        const int a1 = swz<LW, GR>(16 * m + c16, (16 * (s + 1) + 4 * g) * SZ);
        if constexpr (!TRANS) {
          Oa0 = M::mma(M::load(reinterpret_cast<const TC*>(sQ + a0)), Sf[s], Oa0);
          Oa1 = M::mma(M::load(reinterpret_cast<const TC*>(sQ + a1)), Sf[s + 1], Oa1);
        }
        Da0 = M::mma(M::load(reinterpret_cast<const TC*>(sW + a0)), Sf[s], Da0);
        Da1 = M::mma(M::load(reinterpret_cast<const TC*>(sW + a1)), Sf[s + 1], Da1);
      }
      const f32x4 Oa = Oa0 + Oa1, Da = Da0 + Da1;
      const int au = swz<LK, GR>(16 * wave + c16, (16 * m + 4 * g) * SZ);
      if (!TRANS && o) {
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
        dS[s] = M::mma(M::load(reinterpret_cast<const TC*>(sK + swz<LK, GR>(16 * s + c16, (16 * m + 4 * g) * SZ))),
                       df, dS[s]);
    }
    if (sb == NSB - 1) {
#pragma unroll
      for (int s = 0; s < RT; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[s][i] = sgC[16 * s + 4 * g + i] * S[s][i] + dS[s][i];
    }
  }
  if constexpr (TRANS) {
    float* dst = trans + (static_cast<size_t>(bh) * nseg + seg) * DK * NCOL;
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[static_cast<size_t>(16 * s + 4 * g + i) * NCOL + colg] = S[s][i];
  } else if (S_T && seg == nseg - 1) {
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
//
// Segments as in the forward, walked in reverse: with TRANS the kernel runs
// dS <- (diag(Gamma_C) - W^T Kbar) dS + Q'^T dO over its segment from
// [0 | I] (dk more columns, whose dO is zero) into trans[head][seg]; without
// it, the last segment starts from dS_T and segment seg from dS_seg[head][seg]
// (the gradient at the segment's end), and segment 0 writes dS0.
template <typename Tin, int DK, int NW, bool TRANS>
__global__ __launch_bounds__(64 * NW) void bwd_scan_kernel(
    int T, int H, int C, const char* __restrict__ summ, size_t summ_bytes,
    const Tin* __restrict__ dO, const float* __restrict__ dS_T, Tin* __restrict__ dS_chunks,
    float* __restrict__ dS0, int nseg, const float* __restrict__ dS_seg, float* __restrict__ trans) {
  typedef Tin TC;
  typedef MM<TC> M;
  typedef typename M::frag frag;
  constexpr int DV = DK;
  constexpr int RT = DK / 16;
  constexpr int NV = 16 * NW;
  constexpr int NTH = 64 * NW;
  constexpr int SZ = sizeof(TC);
  constexpr int GR = SZ == 2 ? 8 : 16;  // LDS swizzle granule: the fragment read size
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
  constexpr int NCOL = TRANS ? DV + DK : DV;  // state-gradient columns ([dS | P] with TRANS)

  const int NC = T / C;
  const int NSB = C / SB;
  const int nvb = NCOL / NV;
  const int2 gm = xcd_group(blockIdx.x, nvb, static_cast<int>(gridDim.x) / nvb);
  const int bh = gm.x / nseg;
  const int seg = gm.x - bh * nseg;
  const int vb = gm.y;
  const int L = (NC + nseg - 1) / nseg;  // chunks per segment
  const int cbeg = min(NC, seg * L);
  const int cend = min(NC, cbeg + L);
  const bool pcols = TRANS && vb * NV >= DV;  // transition columns: no dO (their loads read tile 0)
  const int vbu = pcols ? 0 : vb;
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

  // unit u walks the segment's chunks in reverse, and each chunk's units in reverse
  auto unit_c = [&](int u) { return cend - 1 - u / NSB; };
  auto unit_sb = [&](int u) { return NSB - 1 - (u - (u / NSB) * NSB); };

  auto prefetch = [&](int u) {
    const int c = unit_c(u);
    const int sb = unit_sb(u);
    const char* base = hsum + static_cast<size_t>(c) * summ_bytes;
    auto part = [&](int p) { return static_cast<uint32_t>(summary_part(p, C, DK, DV) * SZ); };
    const uint32_t tofs = part(SP_WT);  // (16-token tiles, as in the forward scan)
    const uint32_t qofs = part(SP_QT);
    const uint32_t kofs = part(SP_KB) + static_cast<uint32_t>(sb * SB * LW);
    const uint32_t gofs = part(SP_END);
    const char* dob = reinterpret_cast<const char*>(
        dO + ((static_cast<size_t>(b) * T + static_cast<size_t>(c) * C + sb * SB) * H + h) * DV + vbu * NV);
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      const int w = min(tid + k * NTH, T_WORDS - 1);
      const uint32_t r = static_cast<uint32_t>(tpart_index(w / CK, sb * SB + (w % CK) * (16 / SZ), DK) * SZ);
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
      put16<LK, GR>(sWt, w / CK, w % CK, rt[k]);
      put16<LK, GR>(sQt, w / CK, w % CK, rq[k]);
    }
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      const int w = min(tid + k * NTH, K_WORDS - 1);
      put16<LW, GR>(sKb, w / CW, w % CW, rk[k]);
    }
#pragma unroll
    for (int k = 0; k < PO; ++k) {
      const int w = min(tid + k * NTH, O_WORDS - 1);
      const u32x4 zw = {0u, 0u, 0u, 0u};
      put16<LO, GR>(sDO, w / CO, w % CO, pcols ? zw : rd[k]);
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
  {
    // the segment's end: [0 | I] with TRANS, else dS_T or the segment state
    const float* src = seg == nseg - 1 ? (dS_T ? dS_T + sbase : nullptr)
                                       : dS_seg + (static_cast<size_t>(bh) * nseg + seg) * DK * DV;
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * s + 4 * g + i;
        if constexpr (TRANS) dS[s][i] = (pcols && row == colg - DV) ? 1.f : 0.f;
        else dS[s][i] = src ? src[static_cast<size_t>(row) * DV + colg] : 0.f;
      }
  }
  frag dSf[RT];
  f32x4 Z[RT];

  const int U = (cend - cbeg) * NSB;
  if (U > 0) prefetch(0);
#pragma unroll 1
  for (int u = 0; u < U; ++u) {
    const int c = unit_c(u);
    const int sb = unit_sb(u);
    __syncthreads();
    commit();
    // The chunk-end gradient is stored after the commit, before the next
    // unit's loads are issued.  (Measured at B = 8, T = 4096, H = 16, d = 128,
    // bf16: 206 us here, 238 us ahead of the commit, where the commit's waits
    // then also wait for these stores, 210 us after the prefetch.)
    if (sb == NSB - 1) {
      // gradient at the end of chunk c, in the compute type, as transposed
      // 16-row tiles (the lane's four rows of column colg are contiguous)
      TC* dst = dS_chunks + (static_cast<size_t>(bh) * NC + c) * DK * DV;
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        if constexpr (!TRANS) store4(at(dst, static_cast<uint32_t>((s * DV + colg) * 16 + 4 * g)), dS[s]);
        dSf[s] = M::from_f32(dS[s]);
        Z[s] = zero4();
      }
    }
    prefetch(u + 1 < U ? u + 1 : u);
    __syncthreads();
    // (the unit's token tiles fully unrolled: their X products are independent,
    // so their MFMA chains interleave)
#pragma unroll
    for (int m = 0; m < SB / 16; ++m) {
      // X = Kbar_m dS_next (16 tokens x this wave's 16 columns)
      f32x4 X0 = zero4(), X1 = zero4();  // even and odd key tiles: two independent chains
#pragma unroll
      for (int s = 0; s < RT; s += 2) {
        X0 = M::mma(M::load(reinterpret_cast<const TC*>(sKb + swz<LW, GR>(16 * m + c16, (16 * s + 4 * g) * SZ))), dSf[s],
                    X0);
        X1 = M::mma(M::load(reinterpret_cast<const TC*>(sKb + swz<LW, GR>(16 * m + c16, (16 * (s + 1) + 4 * g) * SZ))),
                    dSf[s + 1], X1);
      }
      const f32x4 X = X0 + X1;
      // dO rows as the right operand (tokens along the contraction): one
      // identity product turns the row fragment around
      const f32x4 dot = M::mma(
          M::load(reinterpret_cast<const TC*>(sDO + swz<LO, GR>(16 * m + c16, (16 * wave + 4 * g) * SZ))), ident,
          zero4());
      const frag dof = M::from_f32(dot);
      const frag xf = M::from_f32(-X);
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        const int a = swz<LK, GR>(16 * s + c16, (16 * m + 4 * g) * SZ);
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
  if constexpr (TRANS) {
    float* dst = trans + (static_cast<size_t>(bh) * nseg + seg) * DK * NCOL;
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[static_cast<size_t>(16 * s + 4 * g + i) * NCOL + colg] = dS[s][i];
  } else if (dS0 && seg == 0) {
#pragma unroll
    for (int s = 0; s < RT; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) dS0[sbase + static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] = dS[s][i];
  }
}

// ---------------------------------------------------------------------------
// The segment recurrence of a split scan: x_next = P_g x + E_g with
// [E_g | P_g] = trans[head][g] ([dk][DV + DK] fp32, from a TRANS scan),
// applied from x0 (NULL: zero) over the segments in order (reverse: from the
// last segment down); the value that starts each later segment (reverse: each
// earlier one) goes to xseg[head][segment] ([dk][dv] fp32).  fp32 MFMA; four
// waves of 16 columns per workgroup.
template <int DK>
__global__ __launch_bounds__(256) void seg_combine_kernel(int nseg, int reverse, const float* __restrict__ x0,
                                                          const float* __restrict__ trans,
                                                          float* __restrict__ xseg) {
  typedef MM<float> MF;
  constexpr int DV = DK;
  constexpr int RT = DK / 16;
  constexpr int NCOL = DV + DK;
  const int nvb = DV / 64;
  const int bh = blockIdx.x / nvb;
  const int vb = blockIdx.x - bh * nvb;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int colg = vb * 64 + 16 * wave + c16;
  f32x4 X[RT];
#pragma unroll
  for (int s = 0; s < RT; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      X[s][i] = x0 ? x0[static_cast<size_t>(bh) * DK * DV + static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] : 0.f;
#pragma unroll 1
  for (int st = 0; st + 1 < nseg; ++st) {
    const int gs = reverse ? nseg - 1 - st : st;  // the segment whose map applies
    const int gd = reverse ? gs - 1 : gs + 1;     // the segment its result starts
    const float* tr = trans + (static_cast<size_t>(bh) * nseg + gs) * DK * NCOL;
    f32x4 Y[RT];
#pragma unroll
    for (int s = 0; s < RT; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Y[s][i] = tr[static_cast<size_t>(16 * s + 4 * g + i) * NCOL + colg];
#pragma unroll
      for (int kk = 0; kk < RT; ++kk) {
        // P rows 16s + c16, columns 16kk + 4g..4g+3 as the left operand
        const f32x4 a = *reinterpret_cast<const f32x4*>(tr + static_cast<size_t>(16 * s + c16) * NCOL + DV + 16 * kk + 4 * g);
        Y[s] = MF::mma(a, X[kk], Y[s]);
      }
    }
    float* dst = xseg + (static_cast<size_t>(bh) * nseg + gd) * DK * DV;
#pragma unroll
    for (int s = 0; s < RT; ++s) {
      X[s] = Y[s];
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] = X[s][i];
    }
  }
}

}  // namespace

// One scan over every head: four waves (64 columns) per workgroup when that
// fills the chip; with fewer heads the sequence is split into segments
// (ChunkShape::scan_segments): each segment's transition, the segment
// recurrence, then every segment's scan from its start -- else one wave (16
// columns) per workgroup.
template <typename TT, int DD>
hipError_t fwd_scan_typed(const ChunkShape& s, const void* summ, const float* S0, void* o,
                          void* S_chunks_v, float* S_T, void* deltas, float* split, hipStream_t stream) {
  TT* S_chunks = static_cast<TT*>(S_chunks_v);
  const int heads = s.B * s.H;
  const int nseg = s.scan_segments();
  const size_t sb = s.summary_bytes();
  if (nseg > 1) {
    float* trans = split;
    float* sseg = split + static_cast<size_t>(heads) * nseg * DD * (2 * DD);
    hipLaunchKernelGGL((fwd_scan_kernel<TT, DD, 4, true>), dim3(heads * nseg * (2 * DD / 64)), dim3(256), 0,
                       stream, s.T, s.H, s.C, (const char*)summ, sb, S0, (TT*)nullptr, (TT*)nullptr,
                       (float*)nullptr, (char*)nullptr, size_t(0), nseg, (const float*)nullptr, trans);
    hipLaunchKernelGGL((seg_combine_kernel<DD>), dim3(heads * (DD / 64)), dim3(256), 0, stream, nseg, 0, S0,
                       (const float*)trans, sseg);
    hipLaunchKernelGGL((fwd_scan_kernel<TT, DD, 4, false>), dim3(heads * nseg * (DD / 64)), dim3(256), 0, stream,
                       s.T, s.H, s.C, (const char*)summ, sb, S0, (TT*)o, S_chunks, S_T, (char*)deltas,
                       s.dl_offset(), nseg, (const float*)sseg, (float*)nullptr);
  } else if (static_cast<long long>(heads) * (DD / 64) >= 256) {
    hipLaunchKernelGGL((fwd_scan_kernel<TT, DD, 4, false>), dim3(heads * (DD / 64)), dim3(256), 0, stream, s.T,
                       s.H, s.C, (const char*)summ, sb, S0, (TT*)o, S_chunks, S_T, (char*)deltas, s.dl_offset(), 1,
                       (const float*)nullptr, (float*)nullptr);
  } else {
    hipLaunchKernelGGL((fwd_scan_kernel<TT, DD, 1, false>), dim3(heads * (DD / 16)), dim3(64), 0, stream, s.T,
                       s.H, s.C, (const char*)summ, sb, S0, (TT*)o, S_chunks, S_T, (char*)deltas, s.dl_offset(), 1,
                       (const float*)nullptr, (float*)nullptr);
  }
  return hipGetLastError();
}

template <typename TT, int DD>
hipError_t bwd_scan_typed(const ChunkShape& s, const void* summ, const void* dO, const float* dS_T,
                          void* dS_chunks, float* dS0, float* split, hipStream_t stream) {
  const int heads = s.B * s.H;
  const int nseg = s.scan_segments();
  const size_t sb = s.summary_bytes();
  if (nseg > 1) {
    float* trans = split;
    float* sseg = split + static_cast<size_t>(heads) * nseg * DD * (2 * DD);
    hipLaunchKernelGGL((bwd_scan_kernel<TT, DD, 4, true>), dim3(heads * nseg * (2 * DD / 64)), dim3(256), 0,
                       stream, s.T, s.H, s.C, (const char*)summ, sb, (const TT*)dO, dS_T, (TT*)dS_chunks,
                       (float*)nullptr, nseg, (const float*)nullptr, trans);
    hipLaunchKernelGGL((seg_combine_kernel<DD>), dim3(heads * (DD / 64)), dim3(256), 0, stream, nseg, 1, dS_T,
                       (const float*)trans, sseg);
    hipLaunchKernelGGL((bwd_scan_kernel<TT, DD, 4, false>), dim3(heads * nseg * (DD / 64)), dim3(256), 0, stream,
                       s.T, s.H, s.C, (const char*)summ, sb, (const TT*)dO, dS_T, (TT*)dS_chunks, dS0, nseg,
                       (const float*)sseg, (float*)nullptr);
  } else if (static_cast<long long>(heads) * (DD / 64) >= 256) {
    hipLaunchKernelGGL((bwd_scan_kernel<TT, DD, 4, false>), dim3(heads * (DD / 64)), dim3(256), 0, stream, s.T,
                       s.H, s.C, (const char*)summ, sb, (const TT*)dO, dS_T, (TT*)dS_chunks, dS0, 1,
                       (const float*)nullptr, (float*)nullptr);
  } else {
    hipLaunchKernelGGL((bwd_scan_kernel<TT, DD, 1, false>), dim3(heads * (DD / 16)), dim3(64), 0, stream, s.T,
                       s.H, s.C, (const char*)summ, sb, (const TT*)dO, dS_T, (TT*)dS_chunks, dS0, 1,
                       (const float*)nullptr, (float*)nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_scan(const ChunkShape& s, const void* summ, const float* S0, void* o,
                           void* S_chunks, float* S_T, void* deltas, float* split, hipStream_t stream) {
  if (s.B * s.H == 0) return hipSuccess;
  if (s.bf16) {
    return s.DK == 128 ? fwd_scan_typed<uint16_t, 128>(s, summ, S0, o, S_chunks, S_T, deltas, split, stream)
                       : fwd_scan_typed<uint16_t, 64>(s, summ, S0, o, S_chunks, S_T, deltas, split, stream);
  }
  return s.DK == 128 ? fwd_scan_typed<float, 128>(s, summ, S0, o, S_chunks, S_T, deltas, split, stream)
                     : fwd_scan_typed<float, 64>(s, summ, S0, o, S_chunks, S_T, deltas, split, stream);
}

hipError_t launch_bwd_scan(const ChunkShape& s, const void* summ, const void* dO, const float* dS_T,
                           void* dS_chunks, float* dS0, float* split, hipStream_t stream) {
  if (s.B * s.H == 0) return hipSuccess;
  if (s.bf16) {
    return s.DK == 128 ? bwd_scan_typed<uint16_t, 128>(s, summ, dO, dS_T, dS_chunks, dS0, split, stream)
                       : bwd_scan_typed<uint16_t, 64>(s, summ, dO, dS_T, dS_chunks, dS0, split, stream);
  }
  return s.DK == 128 ? bwd_scan_typed<float, 128>(s, summ, dO, dS_T, dS_chunks, dS0, split, stream)
                     : bwd_scan_typed<float, 64>(s, summ, dO, dS_T, dS_chunks, dS0, split, stream);
}

}  // namespace muir
