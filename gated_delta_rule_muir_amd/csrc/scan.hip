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

// Tiles read transposed (the reverse scan): rows r hold the forward's
// orientation, and a fragment needs, in lane (c16, g), the four values at rows
// k0 + 4g .. k0 + 4g + 3 of column n0 + c16 -- the MFMA operand whose
// contraction runs along the rows.
//   bf16: one ds_read_b64_tr_b16.  Lane l of each 16-lane group reads the
//   8 bytes at row k0 + 4g + l/4, columns n0 + 4 (l%4) .. + 3; the
//   instruction hands lane c16 of the group the four values of column
//   n0 + c16, one from each of the four rows, in row order.  Two groups (32
//   lanes, eight rows x 32 bytes) are served together from 256 bytes of banks
//   (a timing loop at full LDS load: no slower than 64 lanes reading 512
//   contiguous bytes), so rows of 128 bytes or more are padded by 32 bytes:
//   a pitch of an odd number of 32-byte units puts eight consecutive rows'
//   pieces on distinct banks.  (Rows of 256 bytes XOR-permuted by 4 (row % 4)
//   granules measured 20% slower, rows padded by 16 bytes the same.)
//   fp32: four 4-byte reads, unpadded rows.
template <int SZ> constexpr int tpitch(int L) { return SZ == 2 && L >= 128 ? L + 32 : L; }
// Writes the 16-byte word c of row `row` of a transposed-read tile of pitch P.
template <int P> __device__ __forceinline__ void put_t(char* tile, int row, int c, u32x4 w) {
  *reinterpret_cast<u32x4*>(tile + row * P + 16 * c) = w;
}
template <typename TC, int P> __device__ __forceinline__ typename MM<TC>::frag frag_t(const char* tile, int k0, int n0,
                                                                                   int lane) {
  const int g = lane >> 4, l = lane & 15;
  if constexpr (sizeof(TC) == 2) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(tile + (k0 + 4 * g + (l >> 2)) * P + 2 * (n0 + 4 * (l & 3))));
  } else {
    f32x4 a;
#pragma unroll
    for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const float*>(tile + (k0 + 4 * g + t) * P + 4 * (n0 + l));
    return a;
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
// DOCS: packed documents (cinfo, ncu given; see ChunkShape).  A separate
// instance, so that the fixed-length scans carry none of its registers.
template <typename Tin, int DK, int NW, bool TRANS, int RS, bool DOCS>
__global__ __launch_bounds__(64 * NW * RS) __attribute__((amdgpu_waves_per_eu(TRANS ? 2 : 1))) void fwd_scan_kernel(
    int T, int H, int C, const char* __restrict__ summ, size_t summ_bytes,
    const float* __restrict__ S0, Tin* __restrict__ o, Tin* __restrict__ S_chunks,
    float* __restrict__ S_T, char* __restrict__ dsumm, size_t dl_offset, int nseg,
    const float* __restrict__ S_seg, float* __restrict__ trans, const int32_t* __restrict__ cinfo,
    const int32_t* __restrict__ ncu) {
  typedef Tin TC;
  typedef MM<TC> M;
  typedef typename M::frag frag;
  constexpr int DV = DK;
  constexpr int RT = DK / 16;
  constexpr int NV = 16 * NW;
  constexpr int NTH = 64 * NW * RS;
  constexpr int RTW = RT / RS;  // row tiles of the state per wave
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
  constexpr int NM = SB / 16;                 // 16-token tiles per unit
  static_assert(RTW % 2 == 0 && (RS == 1 || RS == 2), "row split");

  const int NC = T / C;
  const int NCU = DOCS ? min(*ncu, NC) : NC;  // chunks in use (packed documents: see ChunkShape)
  const int NSB = C / SB;
  const int nvb = NCOL / NV;
  const int2 gm = xcd_group(blockIdx.x, nvb, static_cast<int>(gridDim.x) / nvb);
  const int bh = gm.x / nseg;
  const int seg = gm.x - bh * nseg;
  const int vb = gm.y;
  const int L = (NCU + nseg - 1) / nseg;  // chunks per segment
  const int cbeg = min(NCU, seg * L);
  const int cend = min(NCU, cbeg + L);
  const bool pcols = TRANS && vb * NV >= DV;  // transition columns: no U~ (their loads read tile 0)
  const int vbu = pcols ? 0 : vb;
  const int b = bh / H;
  const int h = bh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wc = RS == 1 ? wave : wave % NW;  // this wave's 16 state columns within the workgroup's NV
  const int wr = RS == 1 ? 0 : wave / NW;     // and its share of the rows: tiles s0 .. s0 + RTW - 1
  const int s0 = wr * RTW;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int col0 = vb * NV + 16 * wc;  // this wave's first state column
  const int colg = col0 + c16;

  __shared__ __attribute__((aligned(16))) char sW[SB * LW];
  __shared__ __attribute__((aligned(16))) char sQ[SB * LW];
  __shared__ __attribute__((aligned(16))) char sK[DK * LK];
  __shared__ __attribute__((aligned(16))) char sU[NV * LK];
  __shared__ __attribute__((aligned(16))) char sO[NV * LK];
  __shared__ __attribute__((aligned(16))) float sgC[DK];
  // row split: each wave's partial Q'S and W S over its rows, for its partner
  __shared__ f32x4 sXo[RS > 1 ? NW * RS : 1][RS > 1 ? NM : 1][2][64];

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
  f32x4 S[RTW];  // rows 16 (s0 + sl) + 4g + i, column colg
  {
    // the segment's start: [0 | I] with TRANS, else S0 or the segment state
    const float* src = seg == 0 ? (S0 ? S0 + sbase : nullptr)
                                : S_seg + (static_cast<size_t>(bh) * nseg + seg) * DK * DV;
#pragma unroll
    for (int s = 0; s < RTW; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * (s0 + s) + 4 * g + i;
        if constexpr (TRANS) S[s][i] = (pcols && row == colg - DV) ? 1.f : 0.f;
        else S[s][i] = src ? src[static_cast<size_t>(row) * DV + colg] : 0.f;
      }
  }
  frag Sf[RTW];
  f32x4 dS[RTW];

  const int U0 = cbeg * NSB, U1 = cend * NSB;
  if (U0 < U1) prefetch(U0);
  // packed documents: this chunk's table entry, and the next chunk's, loaded
  // a chunk ahead
  int cinf = 0, cinf_next = 0;
  if constexpr (DOCS) cinf_next = cbeg < cend ? cinfo[cbeg] : 0;
#pragma unroll 1
  for (int u = U0; u < U1; ++u) {
    const int c = u / NSB;
    const int sb = u - c * NSB;
    if (DOCS && sb == 0) {
      cinf = cinf_next;
      cinf_next = c + 1 < cend ? cinfo[c + 1] : 0;
      if (cinf & CI_START) {
        // a document's first chunk: its S0 (zero without one); in the
        // transition pass [S | P] = [S0 | 0], since no earlier state reaches
        // past this chunk
        const float* src = S0 ? S0 + (static_cast<size_t>(cinf & CI_DOC) * H + h) * DK * DV : nullptr;
#pragma unroll
        for (int s = 0; s < RTW; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * (s0 + s) + 4 * g + i;
            S[s][i] = (src && !pcols) ? src[static_cast<size_t>(row) * DV + colg] : 0.f;
          }
      }
    }
    // The chunk-start state is stored first, ahead of this unit's commit and
    // the next unit's loads: vector memory instructions issue in order, so
    // stores queued behind a unit of loads wait for them.  (Measured at B = 8,
    // T = 4096, H = 16, d = 128, bf16: 304 us here, 321 us between the commit
    // and the prefetch, 328 us after the prefetch.)
    if (sb == 0) {
      if (!TRANS && S_chunks) {
        // the chunk-start state, kept for the backward in the compute type
        // (as 16 x 16 tiles, stile_index)
        Tin* dst = S_chunks + (static_cast<size_t>(bh) * NC + c) * DK * DV;
        if constexpr (sizeof(Tin) == 4) {
#pragma unroll
          for (int s = 0; s < RTW; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[stile_index(16 * (s0 + s) + 4 * g + i, colg, DV)] = S[s][i];
        } else {
          // rounded once, then turned onto rows by an identity product (exact):
          // row 16s + c16, four columns per lane -- one 512-byte tile per store
#pragma unroll
          for (int s = 0; s < RTW; ++s)
            store4(at(dst, stile_index(16 * (s0 + s) + c16, col0 + 4 * g, DV)),
                   M::mma(M::from_f32(S[s]), ident, zero4()));
        }
      }
#pragma unroll
      for (int s = 0; s < RTW; ++s) {
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
    // One 16-token tile of the unit from its full Q'S and W S: o (by the
    // first row half) and the deltas (by the last) stored; returns the deltas
    // as the operand of the state update.
    auto tile_out = [&](int m, const f32x4& Oa, const f32x4& Da) -> frag {
      const int au = swz<LK, GR>(16 * wc + c16, (16 * m + 4 * g) * SZ);
      if (!TRANS && o && wr == 0) {
        const f32x4 ot = load4(reinterpret_cast<const TC*>(sO + au));
        // tokens 4g+i, column c16 -> token c16, columns 4g..4g+3
        const f32x4 tt = M::mma(M::from_f32(Oa + ot), ident, zero4());
        store4(at(o + obase, static_cast<uint32_t>((16 * m + c16) * H * DV + col0 + 4 * g)), tt);
      }
      const f32x4 ut = load4(reinterpret_cast<const TC*>(sU + au));
      const frag df = M::from_f32(ut - Da);
      if (dlc && wr == RS - 1) {
        // the deltas in the compute type, as token rows (exact: a product with the identity)
        const f32x4 tt = M::mma(df, ident, zero4());
        store4(at(dlc, static_cast<uint32_t>((sb * SB + 16 * m + c16) * DV + col0 + 4 * g)), tt);
      }
      return df;
    };
    if constexpr (RS == 1) {
      // each 16-token tile of the unit in turn, its products used at once
#pragma unroll 2
      for (int m = 0; m < NM; ++m) {
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
        const frag df = tile_out(m, Oa0 + Oa1, Da0 + Da1);
#pragma unroll
        for (int s = 0; s < RT; ++s)
          dS[s] = M::mma(M::load(reinterpret_cast<const TC*>(sK + swz<LK, GR>(16 * s + c16, (16 * m + 4 * g) * SZ))),
                         df, dS[s]);
      }
    } else {
      // Q'S and W S of the unit's token tiles over this wave's rows (two
      // independent chains: even and odd key tiles)
      f32x4 Oa[NM], Da[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        f32x4 Oa0 = zero4(), Oa1 = zero4(), Da0 = zero4(), Da1 = zero4();
#pragma unroll
        for (int sl = 0; sl < RTW; sl += 2) {
          const int s = s0 + sl;
          const int a0 = swz<LW, GR>(16 * m + c16, (16 * s + 4 * g) * SZ);
          const int a1 = swz<LW, GR>(16 * m + c16, (16 * (s + 1) + 4 * g) * SZ);
          if constexpr (!TRANS) {
            Oa0 = M::mma(M::load(reinterpret_cast<const TC*>(sQ + a0)), Sf[sl], Oa0);
            Oa1 = M::mma(M::load(reinterpret_cast<const TC*>(sQ + a1)), Sf[sl + 1], Oa1);
          }
          Da0 = M::mma(M::load(reinterpret_cast<const TC*>(sW + a0)), Sf[sl], Da0);
          Da1 = M::mma(M::load(reinterpret_cast<const TC*>(sW + a1)), Sf[sl + 1], Da1);
        }
        Oa[m] = Oa0 + Oa1;
        Da[m] = Da0 + Da1;
      }
      if constexpr (RS == 2) {
        // the two row halves exchange their partial sums through LDS (the
        // same sum on both sides: addition commutes)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          if constexpr (!TRANS) sXo[wave][m][0][lane] = Oa[m];
          sXo[wave][m][1][lane] = Da[m];
        }
        __syncthreads();
        const int pw = wc + NW * (1 - wr);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          if constexpr (!TRANS) Oa[m] += sXo[pw][m][0][lane];
          Da[m] += sXo[pw][m][1][lane];
        }
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const frag df = tile_out(m, Oa[m], Da[m]);
#pragma unroll
        for (int sl = 0; sl < RTW; ++sl)
          dS[sl] = M::mma(
              M::load(reinterpret_cast<const TC*>(sK + swz<LK, GR>(16 * (s0 + sl) + c16, (16 * m + 4 * g) * SZ))), df,
              dS[sl]);
      }
    }
    if (sb == NSB - 1) {
#pragma unroll
      for (int s = 0; s < RTW; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[s][i] = sgC[16 * (s0 + s) + 4 * g + i] * S[s][i] + dS[s][i];
      if (DOCS && !TRANS && (cinf & CI_END) && S_T) {
        // a document's last chunk: its final state
        float* dst = S_T + (static_cast<size_t>(cinf & CI_DOC) * H + h) * DK * DV;
#pragma unroll
        for (int s = 0; s < RTW; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[static_cast<size_t>(16 * (s0 + s) + 4 * g + i) * DV + colg] = S[s][i];
      }
    }
  }
  if constexpr (TRANS) {
    float* dst = trans + (static_cast<size_t>(bh) * nseg + seg) * DK * NCOL;
#pragma unroll
    for (int s = 0; s < RTW; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[static_cast<size_t>(16 * (s0 + s) + 4 * g + i) * NCOL + colg] = S[s][i];
  } else if (S_T && seg == nseg - 1 && !DOCS) {
#pragma unroll
    for (int s = 0; s < RTW; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_T[sbase + static_cast<size_t>(16 * (s0 + s) + 4 * g + i) * DV + colg] = S[s][i];
  }
}

// ---------------------------------------------------------------------------
// Backward, on the same summaries: reads W [C][DK], Q' [C][DK], Kbar^T and
// Gamma_C, the forward scan's operands, and takes W^T, Q'^T and Kbar as
// transposed fragment reads of the staged tiles (frag_t).
//
// Segments as in the forward, walked in reverse: with TRANS the kernel runs
// dS <- (diag(Gamma_C) - W^T Kbar) dS + Q'^T dO over its segment from zero
// and writes the segment's offset E into columns 0 .. DV-1 of
// trans[head][seg] ([dk][DV + DK] fp32, the forward's layout).  The
// segment's transition is not formed here: it is the transpose of the
// forward's, Prod_c M_c^T = (Prod_c M_c)^T with M_c = diag(Gamma_C) - Kbar^T W
// taken in the opposite order, and seg_combine_kernel reads it from the
// forward's trans.  Without TRANS, the last segment starts from dS_T and
// segment seg from dS_seg[head][seg] (the gradient at the segment's end), and
// segment 0 writes dS0.
template <typename Tin, int DK, int NW, bool TRANS, int RS, bool DOCS>
__global__ __launch_bounds__(64 * NW * RS) void bwd_scan_kernel(
    int T, int H, int C, const char* __restrict__ summ, size_t summ_bytes,
    const Tin* __restrict__ dO, const float* __restrict__ dS_T, Tin* __restrict__ dS_chunks,
    float* __restrict__ dS0, int nseg, const float* __restrict__ dS_seg, float* __restrict__ trans,
    const int32_t* __restrict__ cinfo, const int32_t* __restrict__ ncu) {
  typedef Tin TC;
  typedef MM<TC> M;
  typedef typename M::frag frag;
  constexpr int DV = DK;
  constexpr int RT = DK / 16;
  constexpr int NV = 16 * NW;
  constexpr int NTH = 64 * NW * RS;
  constexpr int RTW = RT / RS;  // row tiles of the state gradient per wave
  constexpr int SZ = sizeof(TC);
  constexpr int GR = SZ == 2 ? 8 : 16;  // LDS swizzle granule: the fragment read size
  constexpr int SB = scan_unit<TC, NW>();
  constexpr int LW = DK * SZ;       // bytes per W / Q' row
  constexpr int LK = SB * SZ;       // bytes per unit segment of a Kbar^T row
  constexpr int PWT = tpitch<SZ>(LW), PKT = tpitch<SZ>(LK);  // their LDS pitches
  constexpr int LO = NV * SZ;       // bytes per dO row segment of this workgroup
  constexpr int CW = LW / 16;
  constexpr int CK = LK / 16;
  constexpr int CO = LO / 16;
  constexpr int W_WORDS = SB * CW;  // W, also Q'
  constexpr int K_WORDS = DK * CK;  // Kbar^T
  constexpr int O_WORDS = SB * CO;
  constexpr int G_WORDS = DK / 4;
  constexpr int PK = words_per_thread<K_WORDS, NTH>();
  constexpr int PW = words_per_thread<W_WORDS, NTH>();
  constexpr int PO = words_per_thread<O_WORDS, NTH>();
  constexpr int PG = words_per_thread<G_WORDS, NTH>();
  static_assert(LO >= 32, "dO row segment");
  constexpr int TS = DV + DK;  // row stride of trans
  constexpr int NM = SB / 16;  // 16-token tiles per unit
  static_assert(RTW % 2 == 0 && (RS == 1 || RS == 2), "row split");

  const int NC = T / C;
  const int NCU = DOCS ? min(*ncu, NC) : NC;  // chunks in use (packed documents: see ChunkShape)
  const int NSB = C / SB;
  const int nvb = DV / NV;
  const int2 gm = xcd_group(blockIdx.x, nvb, static_cast<int>(gridDim.x) / nvb);
  const int bh = gm.x / nseg;
  const int seg = gm.x - bh * nseg;
  const int vb = gm.y;
  const int L = (NCU + nseg - 1) / nseg;  // chunks per segment
  const int cbeg = min(NCU, seg * L);
  const int cend = min(NCU, cbeg + L);
  const int b = bh / H;
  const int h = bh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wc = RS == 1 ? wave : wave % NW;  // this wave's 16 columns within the workgroup's NV
  const int wr = RS == 1 ? 0 : wave / NW;     // and its share of the rows: tiles s0 .. s0 + RTW - 1
  const int s0 = wr * RTW;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int colg = vb * NV + 16 * wc + c16;

  __shared__ __attribute__((aligned(16))) char sW[SB * PWT];   // read transposed (frag_t)
  __shared__ __attribute__((aligned(16))) char sQ[SB * PWT];   // read transposed
  __shared__ __attribute__((aligned(16))) char sKt[DK * PKT];  // read transposed
  __shared__ __attribute__((aligned(16))) char sDO[SB * LO];
  __shared__ __attribute__((aligned(16))) float sgC[DK];
  // row split: each wave's partial Kbar dS over its rows, for its partner
  __shared__ f32x4 sXb[RS > 1 ? NW * RS : 1][RS > 1 ? NM : 1][64];

  const char* hsum = summ + static_cast<size_t>(bh) * NC * summ_bytes;
  u32x4 rw[PW], rq[PW], rk[PK], rd[PO], rg[PG];

  // unit u walks the segment's chunks in reverse, and each chunk's units in reverse
  auto unit_c = [&](int u) { return cend - 1 - u / NSB; };
  auto unit_sb = [&](int u) { return NSB - 1 - (u - (u / NSB) * NSB); };

  auto prefetch = [&](int u) {
    const int c = unit_c(u);
    const int sb = unit_sb(u);
    const char* base = hsum + static_cast<size_t>(c) * summ_bytes;
    auto part = [&](int p) { return static_cast<uint32_t>(summary_part(p, C, DK, DV) * SZ); };
    const uint32_t wofs = part(SP_W) + static_cast<uint32_t>(sb * SB * LW);
    const uint32_t qofs = part(SP_QP) + static_cast<uint32_t>(sb * SB * LW);
    const uint32_t kofs = part(SP_KBT);  // (16-token tiles, as in the forward scan)
    const uint32_t gofs = part(SP_END);
    const char* dob = reinterpret_cast<const char*>(
        dO + ((static_cast<size_t>(b) * T + static_cast<size_t>(c) * C + sb * SB) * H + h) * DV + vb * NV);
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int w = min(tid + k * NTH, W_WORDS - 1);
      rw[k] = *reinterpret_cast<const u32x4*>(at(base, wofs + 16 * w));
      rq[k] = *reinterpret_cast<const u32x4*>(at(base, qofs + 16 * w));
    }
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      const int w = min(tid + k * NTH, K_WORDS - 1);
      const uint32_t r = static_cast<uint32_t>(tpart_index(w / CK, sb * SB + (w % CK) * (16 / SZ), DK) * SZ);
      rk[k] = *reinterpret_cast<const u32x4*>(at(base, kofs + r));
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
    for (int k = 0; k < PW; ++k) {
      const int w = min(tid + k * NTH, W_WORDS - 1);
      put_t<PWT>(sW, w / CW, w % CW, rw[k]);
      put_t<PWT>(sQ, w / CW, w % CW, rq[k]);
    }
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      const int w = min(tid + k * NTH, K_WORDS - 1);
      put_t<PKT>(sKt, w / CK, w % CK, rk[k]);
    }
#pragma unroll
    for (int k = 0; k < PO; ++k) {
      const int w = min(tid + k * NTH, O_WORDS - 1);
      put16<LO, GR>(sDO, w / CO, w % CO, rd[k]);
    }
#pragma unroll
    for (int k = 0; k < PG; ++k) {
      const int w = min(tid + k * NTH, G_WORDS - 1);
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(sgC) + 16 * w) = rg[k];
    }
  };

  const frag ident = identity_frag<TC>(g, c16);
  const size_t sbase = static_cast<size_t>(bh) * DK * DV;
  f32x4 dS[RTW];  // rows 16 (s0 + sl) + 4g + i, column colg
  {
    // the segment's end: zero with TRANS, else dS_T or the segment state
    const float* src = TRANS ? nullptr
                       : seg == nseg - 1 ? ((dS_T && !DOCS) ? dS_T + sbase : nullptr)
                                         : dS_seg + (static_cast<size_t>(bh) * nseg + seg) * DK * DV;
#pragma unroll
    for (int s = 0; s < RTW; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dS[s][i] = src ? src[static_cast<size_t>(16 * (s0 + s) + 4 * g + i) * DV + colg] : 0.f;
  }
  frag dSf[RTW];
  f32x4 Z[RTW];

  const int U = (cend - cbeg) * NSB;
  if (U > 0) prefetch(0);
  // packed documents: this chunk's table entry, and the next one's (the chunk
  // before it), loaded a chunk ahead
  int cinf = 0, cinf_next = 0;
  if constexpr (DOCS) cinf_next = U > 0 ? cinfo[cend - 1] : 0;
#pragma unroll 1
  for (int u = 0; u < U; ++u) {
    const int c = unit_c(u);
    const int sb = unit_sb(u);
    if (DOCS && sb == NSB - 1) {
      cinf = cinf_next;
      cinf_next = c - 1 >= cbeg ? cinfo[c - 1] : 0;
      if (cinf & CI_END) {
        // a document's last chunk: the gradient at its end is the document's
        // dS_T (zero without one)
        const float* src = dS_T ? dS_T + (static_cast<size_t>(cinf & CI_DOC) * H + h) * DK * DV : nullptr;
#pragma unroll
        for (int s = 0; s < RTW; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dS[s][i] = src ? src[static_cast<size_t>(16 * (s0 + s) + 4 * g + i) * DV + colg] : 0.f;
      }
    }
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
      for (int s = 0; s < RTW; ++s) {
        if constexpr (!TRANS) store4(at(dst, static_cast<uint32_t>(((s0 + s) * DV + colg) * 16 + 4 * g)), dS[s]);
        dSf[s] = M::from_f32(dS[s]);
        Z[s] = zero4();
      }
    }
    prefetch(u + 1 < U ? u + 1 : u);
    __syncthreads();
    // X = Kbar_m dS_next over this wave's rows, for each token tile m of the
    // unit (independent products, so their MFMA chains interleave)
    f32x4 X[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if constexpr (SZ == 2) {
        // bf16: pairs of key tiles in one 32-deep product
        X[m] = zero4();
#pragma unroll
        for (int sl = 0; sl < RTW; sl += 2)
          X[m] = M::mma2(frag_t<TC, PKT>(sKt, 16 * (s0 + sl), 16 * m, lane), dSf[sl],
                         frag_t<TC, PKT>(sKt, 16 * (s0 + sl + 1), 16 * m, lane), dSf[sl + 1], X[m]);
      } else {
        f32x4 X0 = zero4(), X1 = zero4();  // even and odd key tiles: two independent chains
#pragma unroll
        for (int sl = 0; sl < RTW; sl += 2) {
          X0 = M::mma(frag_t<TC, PKT>(sKt, 16 * (s0 + sl), 16 * m, lane), dSf[sl], X0);
          X1 = M::mma(frag_t<TC, PKT>(sKt, 16 * (s0 + sl + 1), 16 * m, lane), dSf[sl + 1], X1);
        }
        X[m] = X0 + X1;
      }
    }
    if constexpr (RS == 2) {
      // the two row halves exchange their partial sums through LDS (the
      // same sum on both sides: addition commutes)
#pragma unroll
      for (int m = 0; m < NM; ++m) sXb[wave][m][lane] = X[m];
      __syncthreads();
      const int pw = wc + NW * (1 - wr);
#pragma unroll
      for (int m = 0; m < NM; ++m) X[m] += sXb[pw][m][lane];
    }
    // dO rows as the right operand (tokens along the contraction): one
    // identity product turns the row fragment around
    auto dO_frag = [&](int m) {
      return M::from_f32(M::mma(
          M::load(reinterpret_cast<const TC*>(sDO + swz<LO, GR>(16 * m + c16, (16 * wc + 4 * g) * SZ))), ident,
          zero4()));
    };
    if constexpr (SZ == 2 && NM % 2 == 0) {
      // bf16: token tiles in pairs, each pair of 16-deep products issued as
      // one 32-deep product
#pragma unroll
      for (int m = 0; m < NM; m += 2) {
        const frag dof0 = dO_frag(m), dof1 = dO_frag(m + 1);
        const frag xf0 = M::from_f32(-X[m]), xf1 = M::from_f32(-X[m + 1]);
#pragma unroll
        for (int sl = 0; sl < RTW; ++sl) {
          const int s = s0 + sl;
          Z[sl] = M::mma2(frag_t<TC, PWT>(sQ, 16 * m, 16 * s, lane), dof0,
                          frag_t<TC, PWT>(sQ, 16 * (m + 1), 16 * s, lane), dof1, Z[sl]);
          Z[sl] = M::mma2(frag_t<TC, PWT>(sW, 16 * m, 16 * s, lane), xf0,
                          frag_t<TC, PWT>(sW, 16 * (m + 1), 16 * s, lane), xf1, Z[sl]);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const frag dof = dO_frag(m);
        const frag xf = M::from_f32(-X[m]);
#pragma unroll
        for (int sl = 0; sl < RTW; ++sl) {
          Z[sl] = M::mma(frag_t<TC, PWT>(sQ, 16 * m, 16 * (s0 + sl), lane), dof, Z[sl]);
          Z[sl] = M::mma(frag_t<TC, PWT>(sW, 16 * m, 16 * (s0 + sl), lane), xf, Z[sl]);
        }
      }
    }
    if (sb == 0) {
#pragma unroll
      for (int s = 0; s < RTW; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) dS[s][i] = sgC[16 * (s0 + s) + 4 * g + i] * dS[s][i] + Z[s][i];
      if (DOCS && (cinf & CI_START)) {
        // a document's first chunk: the gradient at its start is the
        // document's dS0; none of it reaches the chunk before (another
        // document's), so the flow is cut there
        if (!TRANS && dS0) {
          float* dst = dS0 + (static_cast<size_t>(cinf & CI_DOC) * H + h) * DK * DV;
#pragma unroll
          for (int s = 0; s < RTW; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[static_cast<size_t>(16 * (s0 + s) + 4 * g + i) * DV + colg] = dS[s][i];
        }
#pragma unroll
        for (int s = 0; s < RTW; ++s) dS[s] = zero4();
      }
    }
  }
  if constexpr (TRANS) {
    float* dst = trans + (static_cast<size_t>(bh) * nseg + seg) * DK * TS;
#pragma unroll
    for (int s = 0; s < RTW; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[static_cast<size_t>(16 * (s0 + s) + 4 * g + i) * TS + colg] = dS[s][i];
  } else if (dS0 && seg == 0 && !DOCS) {
#pragma unroll
    for (int s = 0; s < RTW; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dS0[sbase + static_cast<size_t>(16 * (s0 + s) + 4 * g + i) * DV + colg] = dS[s][i];
  }
}

// ---------------------------------------------------------------------------
// The segment recurrence of a split scan, applied from x0 (NULL: zero) over
// the segments in order (reverse: from the last segment down); the value that
// starts each later segment (reverse: each earlier one) goes to
// xseg[head][segment] ([dk][dv] fp32).  E and P point to [head][g][dk][DV + DK]
// fp32 arrays (the TRANS scans' layout) holding the offset E_g in columns
// 0 .. DV-1 and, in P, the forward transition P_g in columns DV .. DV+DK-1:
// forward x_next = P_g x + E_g, reverse x_next = P_g^T x + E_g.  fp32 MFMA.
//
// The recurrence is a chain of nseg - 1 dependent products, so its length is
// what counts: one workgroup per (head, 16 columns) and one wave per 16 rows,
// each forming its 16 x 16 tile of the next value (16 fp32 MFMA products per
// 16-deep step of the contraction); the tiles meet in LDS, where every wave
// reads the whole column block as its right operand for the next segment.
// Each wave's P rows and E values of the next segment are loaded while the
// current one is formed.  The products are summed in the same order as by a
// single wave holding the whole column block.
template <int DK, bool REV>
__global__ __launch_bounds__(4 * DK) void seg_combine_kernel(int nseg, const float* __restrict__ x0,
                                                             const float* __restrict__ E,
                                                             const float* __restrict__ P,
                                                             float* __restrict__ xseg) {
  typedef MM<float> MF;
  constexpr int DV = DK;
  constexpr int RT = DK / 16;
  constexpr int NCOL = DV + DK;
  constexpr int NVB = DV / 16;
  const int bh = blockIdx.x / NVB;
  const int vb = blockIdx.x - bh * NVB;
  const int lane = threadIdx.x & 63;
  const int s = threadIdx.x >> 6;  // this wave's row tile
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int colg = vb * 16 + c16;
  // the current value, per row tile in the accumulator layout, double-buffered
  __shared__ f32x4 sX[2][RT][64];

  // the map applied at step st: rows 16s + c16, columns 16kk + 4g .. + 3 of
  // P_g (reverse: of P_g^T, four loads of 16 consecutive columns of P_g) as
  // the left operand, and E_g at rows 16s + 4g + i, column colg
  auto load_step = [&](int st, f32x4 (&a)[RT], f32x4& e) {
    const int gs = REV ? nseg - 1 - st : st;
    const size_t base = (static_cast<size_t>(bh) * nseg + gs) * DK * NCOL;
    const float* pg = P + base + DV;
    if constexpr (REV) {
#pragma unroll
      for (int kk = 0; kk < RT; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j) a[kk][j] = pg[static_cast<size_t>(16 * kk + 4 * g + j) * NCOL + 16 * s + c16];
    } else {
#pragma unroll
      for (int kk = 0; kk < RT; ++kk)
        a[kk] = *reinterpret_cast<const f32x4*>(pg + static_cast<size_t>(16 * s + c16) * NCOL + 16 * kk + 4 * g);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = E[base + static_cast<size_t>(16 * s + 4 * g + i) * NCOL + colg];
  };

  f32x4 a0[RT], e0;
  load_step(0, a0, e0);  // (nseg >= 2 whenever the kernel is launched)
  {
    f32x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = x0 ? x0[static_cast<size_t>(bh) * DK * DV + static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] : 0.f;
    sX[0][s][lane] = x;
  }
  __syncthreads();
  int cur = 0;
#pragma unroll 1
  for (int st = 0; st + 1 < nseg; ++st) {
    f32x4 a1[RT], e1;
    load_step(st + 2 < nseg ? st + 1 : st, a1, e1);  // the next step's map (clamped at the end)
    f32x4 y = e0;
#pragma unroll
    for (int kk = 0; kk < RT; ++kk) y = MF::mma(a0[kk], sX[cur][kk][lane], y);
    const int gd = REV ? nseg - 2 - st : st + 1;  // the segment this value starts
    float* dst = xseg + (static_cast<size_t>(bh) * nseg + gd) * DK * DV;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[static_cast<size_t>(16 * s + 4 * g + i) * DV + colg] = y[i];
    sX[cur ^ 1][s][lane] = y;
    __syncthreads();
    cur ^= 1;
#pragma unroll
    for (int kk = 0; kk < RT; ++kk) a0[kk] = a1[kk];
    e0 = e1;
  }
}

}  // namespace

// One scan over every head: four waves (64 columns) per workgroup when that
// fills the chip; with fewer heads the sequence is split into segments
// (ChunkShape::scan_segments): each segment's transition, the segment
// recurrence, then every segment's scan from its start -- else one wave (16
// columns) per workgroup.
// Each segment's offset and transition, [E_g | P_g], into trans.
// (S0 is read only at the first chunks of packed documents.)
template <typename TT, int DD, bool DOCS>
void fwd_trans_typed(const ChunkShape& s, const void* summ, const float* S0, float* trans, hipStream_t stream) {
  const int heads = s.B * s.H;
  const int nseg = s.scan_segments();
  hipLaunchKernelGGL((fwd_scan_kernel<TT, DD, 4, true, 1, DOCS>), dim3(heads * nseg * (2 * DD / 64)), dim3(256), 0, stream,
                     s.T, s.H, s.C, (const char*)summ, s.summary_bytes(), s.cinfo ? S0 : (const float*)nullptr,
                     (TT*)nullptr, (TT*)nullptr, (float*)nullptr, (char*)nullptr, size_t(0), nseg,
                     (const float*)nullptr, trans, s.cinfo, s.ncu);
}

template <typename TT, int DD, bool DOCS>
hipError_t fwd_scan_typed(const ChunkShape& s, const void* summ, const float* S0, void* o,
                          void* S_chunks_v, float* S_T, void* deltas, float* split, hipStream_t stream) {
  TT* S_chunks = static_cast<TT*>(S_chunks_v);
  const int heads = s.B * s.H;
  const int nseg = s.scan_segments();
  const size_t sb = s.summary_bytes();
  if (nseg > 1) {
    float* trans = split;
    float* sseg = split + static_cast<size_t>(heads) * nseg * DD * (2 * DD);
    fwd_trans_typed<TT, DD, DOCS>(s, summ, S0, trans, stream);
    // (packed documents: the first chunk starts a document, whose own S0 the
    // scan takes there)
    hipLaunchKernelGGL((seg_combine_kernel<DD, false>), dim3(heads * (DD / 16)), dim3(4 * DD), 0, stream, nseg,
                       s.cinfo ? (const float*)nullptr : S0, (const float*)trans, (const float*)trans, sseg);
    hipLaunchKernelGGL((fwd_scan_kernel<TT, DD, 4, false, 2, DOCS>), dim3(heads * nseg * (DD / 64)), dim3(512), 0, stream,
                       s.T, s.H, s.C, (const char*)summ, sb, S0, (TT*)o, S_chunks, S_T, (char*)deltas,
                       s.dl_offset(), nseg, (const float*)sseg, (float*)nullptr, s.cinfo, s.ncu);
  } else if (static_cast<long long>(heads) * (DD / 64) >= 256) {
    hipLaunchKernelGGL((fwd_scan_kernel<TT, DD, 4, false, 2, DOCS>), dim3(heads * (DD / 64)), dim3(512), 0, stream, s.T,
                       s.H, s.C, (const char*)summ, sb, S0, (TT*)o, S_chunks, S_T, (char*)deltas, s.dl_offset(), 1,
                       (const float*)nullptr, (float*)nullptr, s.cinfo, s.ncu);
  } else {
    hipLaunchKernelGGL((fwd_scan_kernel<TT, DD, 1, false, 1, DOCS>), dim3(heads * (DD / 16)), dim3(64), 0, stream, s.T,
                       s.H, s.C, (const char*)summ, sb, S0, (TT*)o, S_chunks, S_T, (char*)deltas, s.dl_offset(), 1,
                       (const float*)nullptr, (float*)nullptr, s.cinfo, s.ncu);
  }
  return hipGetLastError();
}

template <typename TT, int DD, bool DOCS>
hipError_t bwd_scan_typed(const ChunkShape& s, const void* summ, const void* dO, const float* dS_T,
                          void* dS_chunks, float* dS0, float* split, const float* ftrans, hipStream_t stream) {
  const int heads = s.B * s.H;
  const int nseg = s.scan_segments();
  const size_t sb = s.summary_bytes();
  if (nseg > 1) {
    // each segment's offset into the E columns of trans; the transitions are
    // the transposes of the forward's, read from ftrans
    float* trans = split;
    float* sseg = split + static_cast<size_t>(heads) * nseg * DD * (2 * DD);
    // (the transition pass takes each packed document's dS_T at its last chunk)
    hipLaunchKernelGGL((bwd_scan_kernel<TT, DD, 4, true, 2, DOCS>), dim3(heads * nseg * (DD / 64)), dim3(512), 0, stream,
                       s.T, s.H, s.C, (const char*)summ, sb, (const TT*)dO, dS_T, (TT*)dS_chunks, (float*)nullptr,
                       nseg, (const float*)nullptr, trans, s.cinfo, s.ncu);
    hipLaunchKernelGGL((seg_combine_kernel<DD, true>), dim3(heads * (DD / 16)), dim3(4 * DD), 0, stream, nseg,
                       s.cinfo ? (const float*)nullptr : dS_T, (const float*)trans, ftrans, sseg);
    hipLaunchKernelGGL((bwd_scan_kernel<TT, DD, 4, false, 2, DOCS>), dim3(heads * nseg * (DD / 64)), dim3(512), 0, stream,
                       s.T, s.H, s.C, (const char*)summ, sb, (const TT*)dO, dS_T, (TT*)dS_chunks, dS0, nseg,
                       (const float*)sseg, (float*)nullptr, s.cinfo, s.ncu);
  } else if (static_cast<long long>(heads) * (DD / 64) >= 256) {
    hipLaunchKernelGGL((bwd_scan_kernel<TT, DD, 4, false, 2, DOCS>), dim3(heads * (DD / 64)), dim3(512), 0, stream, s.T,
                       s.H, s.C, (const char*)summ, sb, (const TT*)dO, dS_T, (TT*)dS_chunks, dS0, 1,
                       (const float*)nullptr, (float*)nullptr, s.cinfo, s.ncu);
  } else {
    hipLaunchKernelGGL((bwd_scan_kernel<TT, DD, 1, false, 1, DOCS>), dim3(heads * (DD / 16)), dim3(64), 0, stream, s.T,
                       s.H, s.C, (const char*)summ, sb, (const TT*)dO, dS_T, (TT*)dS_chunks, dS0, 1,
                       (const float*)nullptr, (float*)nullptr, s.cinfo, s.ncu);
  }
  return hipGetLastError();
}

template <bool DOCS>
hipError_t fwd_scan_any(const ChunkShape& s, const void* summ, const float* S0, void* o, void* S_chunks,
                        float* S_T, void* deltas, float* split, hipStream_t stream) {
  if (s.bf16) {
    return s.DK == 128 ? fwd_scan_typed<uint16_t, 128, DOCS>(s, summ, S0, o, S_chunks, S_T, deltas, split, stream)
                       : fwd_scan_typed<uint16_t, 64, DOCS>(s, summ, S0, o, S_chunks, S_T, deltas, split, stream);
  }
  return s.DK == 128 ? fwd_scan_typed<float, 128, DOCS>(s, summ, S0, o, S_chunks, S_T, deltas, split, stream)
                     : fwd_scan_typed<float, 64, DOCS>(s, summ, S0, o, S_chunks, S_T, deltas, split, stream);
}

hipError_t launch_fwd_scan(const ChunkShape& s, const void* summ, const float* S0, void* o,
                           void* S_chunks, float* S_T, void* deltas, float* split, hipStream_t stream) {
  if (s.B * s.H == 0) return hipSuccess;
  return s.cinfo ? fwd_scan_any<true>(s, summ, S0, o, S_chunks, S_T, deltas, split, stream)
                 : fwd_scan_any<false>(s, summ, S0, o, S_chunks, S_T, deltas, split, stream);
}

hipError_t launch_fwd_trans(const ChunkShape& s, const void* summ, float* split, hipStream_t stream) {
  if (s.B * s.H == 0 || s.scan_segments() < 2) return hipSuccess;
  if (s.cinfo) return hipErrorInvalidValue;  // packed documents need their S0 here: launch_fwd_scan forms these
  if (s.bf16) {
    if (s.DK == 128) fwd_trans_typed<uint16_t, 128, false>(s, summ, nullptr, split, stream);
    else fwd_trans_typed<uint16_t, 64, false>(s, summ, nullptr, split, stream);
  } else {
    if (s.DK == 128) fwd_trans_typed<float, 128, false>(s, summ, nullptr, split, stream);
    else fwd_trans_typed<float, 64, false>(s, summ, nullptr, split, stream);
  }
  return hipGetLastError();
}

template <bool DOCS>
hipError_t bwd_scan_any(const ChunkShape& s, const void* summ, const void* dO, const float* dS_T, void* dS_chunks,
                        float* dS0, float* split, const float* ftrans, hipStream_t stream) {
  if (s.bf16) {
    return s.DK == 128 ? bwd_scan_typed<uint16_t, 128, DOCS>(s, summ, dO, dS_T, dS_chunks, dS0, split, ftrans, stream)
                       : bwd_scan_typed<uint16_t, 64, DOCS>(s, summ, dO, dS_T, dS_chunks, dS0, split, ftrans, stream);
  }
  return s.DK == 128 ? bwd_scan_typed<float, 128, DOCS>(s, summ, dO, dS_T, dS_chunks, dS0, split, ftrans, stream)
                     : bwd_scan_typed<float, 64, DOCS>(s, summ, dO, dS_T, dS_chunks, dS0, split, ftrans, stream);
}

hipError_t launch_bwd_scan(const ChunkShape& s, const void* summ, const void* dO, const float* dS_T,
                           void* dS_chunks, float* dS0, float* split, const float* ftrans, hipStream_t stream) {
  if (s.B * s.H == 0) return hipSuccess;
  return s.cinfo ? bwd_scan_any<true>(s, summ, dO, dS_T, dS_chunks, dS0, split, ftrans, stream)
                 : bwd_scan_any<false>(s, summ, dO, dS_T, dS_chunks, dS0, split, ftrans, stream);
}

}  // namespace muir
