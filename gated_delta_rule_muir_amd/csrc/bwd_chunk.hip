// Per-chunk gradients of the Muir gated delta rule (gfx950).
//
// One workgroup per chunk gets the chunk's initial state S0 and the gradient
// dS_C of its end state (from the reverse scan in scan.hip) and forms every
// input gradient with two sweeps over the chunk's 16-token blocks, with the
// block-boundary pivots of the forward (fwd.hip):
//   F (forward): Delta_I = T_II (U_I - X_I S_I),  S_{I+1} = g_I S_I + Ke_I^T Delta_I;
//                the deltas and the block-start states S_I go to the scratch
//   R (reverse): D, the state gradient at the block's end, starting from dS_C;
//                dR_J    = T_JJ^T (Ke_J D + P_JJ^T dO_J)   (gradient of write*v)
//                d(k)_i  = E_i Delta_i                     (E_i: state gradient at token i)
//                d(qt)_r = S_r dO_r                        (S_r: state after token r)
//                d(ek)_r = -S'_r dR_r                      (S'_r: decayed state before r's write)
//                D <- g_J D + Y_J^T dO_J - X_J^T dR_J
// with ek = erase*k, qt = gamma*q, and
//   dLam_r   = ek_r d(ek)_r + qt_r d(qt)_r - k_r d(k)_r,
//   dlog_a_i = sum_{r >= i in the chunk} dLam_r + rowsum(S_C * dS_C),
//   derase = k d(ek), dk = d(k) + erase d(ek), dq = gamma d(qt), dgamma = q d(qt),
//   dv = write dR, dwrite = v dR.
// Each gradient is written once: the reverse sweep carries the suffix sums of
// dLam from block to block.  (arXiv 2611.08376 states only that a custom
// backward pass is used, in its Methodology section and the fig:kernel
// caption; this is the adjoint of the chunkwise forward.)
//
// Each per-token product splits into a boundary part, a tile product with S_J,
// D or the deltas scaled by exp(.) <= 1, and a 16 x 16 leaf part.  On leaves
// whose decay stays within LEAF_SAFE_RANGE the leaf part is one more 16-wide
// MFMA product folded into the same accumulator; steeper leaves use per-pair
// factors in (0, 1].
//
// Latency: every global read a step needs (the block's inputs, dO rows,
// deltas, the leaf inverse, the block-start state) is issued one step ahead
// into registers (clamped at the ends of each sweep, so no load sits under a
// branch) and committed to LDS when the step starts.
#include "chunk_common.h"
#include "kernels.h"
#include "mma.h"

namespace muir {

namespace {

// Forms of the per-chunk backward:
//   0: two sweeps (fp32 inputs): a forward sweep over the 16-token blocks
//      solves for the deltas and keeps every block-start state, then the
//      reverse sweep;
//   1: direct (bf16, 64-token chunks): the chunk's deltas come from the
//      forward scan, and the reverse sweep forms every block-start state
//      from the chunk-start state and the deltas (Horner over the earlier
//      blocks);
//   2: direct over sub-chunks (bf16, 128- and 256-token chunks): a forward
//      pass over the chunk's 64-token sub-chunks carries the state with the
//      forward scan's deltas and keeps each later sub-chunk's start state;
//      the reverse sweep then runs form 1 within each sub-chunk.
enum BwdForm { BWD_TWO_SWEEP = 0, BWD_DIRECT = 1, BWD_SUB = 2 };

// Per-chunk scratch, in the compute type.  Form 0: deltas [C][DV], then the
// state at the start of every 16-token block [C/16][DK][DV] (row-major, as
// staged).  Form 2: the start state of sub-chunks 1 .. C/64 - 1, each
// [DK][DV] as 16 x 16 tiles like the saved chunk states (sub-chunk 0 starts
// from the chunk's own start state).  Form 1: none.
template <typename TC, int FORM>
__host__ __device__ constexpr size_t bwd_scratch_bytes_tc(int C, int DK, int DV) {
  return FORM == BWD_TWO_SWEEP ? (static_cast<size_t>(C) * DV + static_cast<size_t>(C / 16) * DK * DV) * sizeof(TC)
         : FORM == BWD_SUB     ? static_cast<size_t>(C / 64 - 1) * DK * DV * sizeof(TC)
                               : 0;
}

// LDS row padding (elements).  LDS serves a fragment read 128 bytes at a
// time (32 banks of 4 bytes): 16 lanes of an 8-byte bf16 read, 8 lanes of a
// 16-byte fp32 one, each on its own row at the same column.  Rows padded by 8
// bytes (bf16) or 16 bytes (fp32) put those rows on distinct banks; a 16-byte
// pad would leave the bf16 reads two-way conflicted.  bf16 rows are then only
// 8-byte aligned, so 16-byte words go into them as two 8-byte stores (put16).
template <typename TC> constexpr int row_pad() { return 4; }  // 8 bytes (bf16), 16 bytes (fp32)

// A 16-byte word into an LDS row that may be only 8-byte aligned.
__device__ __forceinline__ void put16(void* p, u32x4 w) {
  u32x2* q = reinterpret_cast<u32x2*>(p);
  const u32x2 lo = {w[0], w[1]}, hi = {w[2], w[3]};
  q[0] = lo;
  q[1] = hi;
}

// Column passes for the two staged states ([DK][DV / SPLIT] each), chosen so
// the kernel's LDS stays within 160 KB.
template <typename TC, int DK, int C> constexpr int stage_split() {
  return DK == 64 ? 1 : (sizeof(TC) == 2 ? (C == 64 ? 1 : 2) : (C == 64 ? 4 : 8));
}

// Tin: element type of the inputs, dO, the chunk states and the MFMA
// operands; Tg: element type of the per-token gradients (Tin, or fp32 for
// bf16 inputs); FORM: BwdForm.  PKO (packed documents, ChunkShape::docoff):
// the per-token gradients go straight to the caller's packed [T_total, H, D]
// tensors -- the chunk's rows from row cu[d] + (its first row - docoff[d]) of
// document d, the rows past the document's end not stored -- instead of to
// a chunk-aligned copy.
template <typename Tin, typename Tg, int DK, int C, int NW, int FORM, bool GTOK, bool PKO>
__global__ __launch_bounds__(64 * NW) void bwd_chunk_kernel(
    int T, int H, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ log_a, const Tin* __restrict__ erase,
    const Tin* __restrict__ write, const Tin* __restrict__ gamma, const char* __restrict__ summ,
    size_t summ_bytes, size_t tp_offset, size_t dl_offset, const Tin* __restrict__ S_chunks,
    const Tin* __restrict__ dS_chunks, const Tin* __restrict__ dO, Tg* __restrict__ dq,
    Tg* __restrict__ dk, Tg* __restrict__ dv, Tg* __restrict__ dlog_a,
    Tg* __restrict__ derase, Tg* __restrict__ dwrite, Tg* __restrict__ dgamma,
    char* __restrict__ scratch, int gmode, float* __restrict__ dgam_part, const int32_t* __restrict__ ncu,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ docoff, const int32_t* __restrict__ cinfo) {
  typedef Tin TC;
  typedef MM<TC> M;
  typedef typename M::frag frag;
  constexpr int DV = DK;
  constexpr int NTH = 64 * NW;
  constexpr int NT = DV / (16 * NW);  // 16-column tiles per wave (state columns, gradient channels)
  constexpr int RT = DK / 16;
  constexpr int TPC = NTH / DK;       // elementwise: threads per key channel
  constexpr int RPT = 16 / TPC;       // elementwise: consecutive tokens per thread
  constexpr int NB = C / 16;
  // the direct machinery (forms 1 and 2): the reverse sweep forms the state at
  // each block start within a span of NBS blocks (a 64-token chunk or
  // sub-chunk) from the span's start state
  constexpr bool DIRECT = FORM != BWD_TWO_SWEEP;
  constexpr bool SUB = FORM == BWD_SUB;
  constexpr int NBS = DIRECT ? 4 : NB;
  constexpr int NSUB = NB / NBS;
  static_assert(NB % NBS == 0 && (FORM != BWD_DIRECT || NB == 4) && (!SUB || NB > 4), "backward form");
  constexpr int SPLIT = DIRECT ? 1 : stage_split<TC, DK, C>();
  constexpr int SW = DV / SPLIT;
  constexpr int PT = DK + row_pad<TC>();
  constexpr int PV = DV + row_pad<TC>();
  constexpr int PS = SW + row_pad<TC>();
  constexpr int TP = 20;  // row length of the [.][16] transposed tiles (40 or 80 bytes: distinct banks over 16 or 8 rows)
  constexpr int EPT = 16 * DV / NTH;  // row-tile elements per thread
  constexpr int RC = DV / EPT;        // threads per row of a [16][DV] tile
  constexpr int EPW = 8 / static_cast<int>(sizeof(TC));  // elements per 8-byte word
  constexpr int RW = EPT / EPW;       // 8-byte words per thread of a row tile
  constexpr int TPW = 512 / EPW;      // threads that move a block's T_II, P_II words
  constexpr int SEW = 16 / static_cast<int>(sizeof(TC));  // elements per 16-byte word
  constexpr int SWR = DV / SEW;       // 16-byte words per state row
  constexpr int SPT = DK * SWR / NTH; // 16-byte words of a block-start state per thread
  static_assert(NT >= 1 && NW * NT * 16 == DV && TPC * RPT == 16 && RPT % 4 == 0 && RW >= 1 &&
                    EPT % EPW == 0 && TPW <= NTH && SPT * NTH == DK * SWR && SW % SEW == 0,
                "thread layout");
  static_assert(!DIRECT || SPLIT == 1, "the direct form stages S0 once, whole");

  const int NC = T / C;
  const int chunk = blockIdx.x;
  const int bh = chunk / NC;
  const int c = chunk - bh * NC;
  if (ncu && c >= *ncu) {
    // packed documents: a chunk past those in use adds nothing to a static
    // gate's gradient
    if (gmode == GAMMA_STATIC)
      for (int j = threadIdx.x; j < DK; j += NTH) dgam_part[static_cast<size_t>(chunk) * DK + j] = 0.f;
    return;
  }
  const int b = bh / H;
  const int h = bh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  // MFMA-output mapping: lane's state column / gradient channel of tile n
  auto colv = [&](int n) -> int { return 16 * (NT * wave + n) + c16; };
  auto col0 = [&](int n) -> int { return 16 * (NT * wave + n); };
  const int ej = tid % DK;            // elementwise mapping: channel, tokens RPT*part..+RPT-1
  const int part = tid / DK;
  const int prow = tid / RC;          // row-tile mapping: row, columns pc0..pc0+EPT-1
  const int pc0 = (tid % RC) * EPT;

  // Workgroup-uniform bases of the chunk; element (t, j) of a [B, T, H, D]
  // tensor is at index t * HD + j from them.
  const size_t ebase = ((static_cast<size_t>(b) * T + static_cast<size_t>(c) * C) * H + h) * DK;
  const uint32_t HD = static_cast<uint32_t>(H) * DK;
  const Tin* qb = q + ebase;
  const Tin* kb = k + ebase;
  const Tin* vb = v + ebase;
  const Tin* lb = log_a + ebase;
  const Tin* eb = erase + ebase;
  const Tin* wb = write + ebase;
  // readout gate: per token at gb (as the other inputs), static at the
  // head's row gst, or none (both then point into q; the value is not used)
  const Tin* gbase = gmode == GAMMA_NONE ? q : gamma;
  const Tin* gb = gbase + ebase;
  const Tin* gst = gbase + static_cast<size_t>(h) * DK;
  const Tin* dOb = dO + ebase;
  // the gradients' chunk base, and the chunk's rows that are stored
  size_t obase = ebase;
  int vrows = C;
  if constexpr (PKO) {
    const int d = cinfo[c] & CI_DOC;
    const int t0 = c * C - docoff[d];  // the chunk's first token within document d (B = 1)
    vrows = min(C, cu[d + 1] - cu[d] - t0);
    obase = ((static_cast<size_t>(cu[d]) + t0) * H + h) * DK;
  }
  Tg* dqb = dq + obase;
  Tg* dkb = dk + obase;
  Tg* dvb = dv + obase;
  Tg* dlb = dlog_a + obase;
  Tg* deb = derase + obase;
  Tg* dwb = dwrite + obase;
  Tg* dgb = dgamma + obase;
  auto gi = [&](int t, int j) -> uint32_t { return static_cast<uint32_t>(t) * HD + static_cast<uint32_t>(j); };
  // the readout gate of element (t, j) of the chunk (GTOK: per token, as the
  // other inputs; else static or none, chosen at run time)
  auto gam = [&](int t, int j) -> float {
    const uint32_t o = static_cast<uint32_t>(t) * HD + static_cast<uint32_t>(j);
    if constexpr (GTOK) return ldv(gb, o);
    const float x = ldv(gst, static_cast<uint32_t>(j));
    return gmode == GAMMA_NONE ? 1.f : x;
  };
  // the static gate's values this thread uses (channels colv(n) and ej; none:
  // 1), read once here, ahead of the prologue's own reads: a read per block
  // sat in the sweep's critical path (1,229 against 1,038 us per launch at
  // the 4K layer, static against per-token gate)
  float gsc[NT], gse = 1.f;
#pragma unroll
  for (int n = 0; n < NT; ++n) gsc[n] = 1.f;
  if constexpr (!GTOK) {
    if (gmode != GAMMA_NONE) {
#pragma unroll
      for (int n = 0; n < NT; ++n) gsc[n] = ldv(gst, static_cast<uint32_t>(colv(n)));
      gse = ldv(gst, static_cast<uint32_t>(ej));
    }
  }
  TC* gDel = reinterpret_cast<TC*>(scratch + static_cast<size_t>(chunk) * bwd_scratch_bytes_tc<TC, FORM>(C, DK, DV));
  TC* gS = gDel + static_cast<size_t>(C) * DV;  // form 0: [NB][DK][DV]
  TC* gSub = gDel;                              // form 2: [NSUB - 1] states as 16 x 16 tiles
  // T_II, P_II of the chunk's blocks, from the chunk summary, [NB][2][16][16]
  const TC* gTP = reinterpret_cast<const TC*>(summ + static_cast<size_t>(chunk) * summ_bytes + tp_offset);
  const Tin* S0c = S_chunks + static_cast<size_t>(chunk) * DK * DV;  // 16 x 16 tiles (stile_index), compute type
  const TC* dSC = dS_chunks + static_cast<size_t>(chunk) * DK * DV;  // transposed 16-row tiles

  __shared__ float sPart[NB][TPC][DK];                       // sum of log_a over each part's RPT tokens
  __shared__ int sUnsafe;                                    // bit I: block I beyond LEAF_SAFE_RANGE
  __shared__ __attribute__((aligned(16))) TC sRowA[16][PT];  // F: X rows   R: Ke rows
  __shared__ __attribute__((aligned(16))) TC sTA[DK][TP];    // F: Ke^T     R: X^T
  __shared__ __attribute__((aligned(16))) TC sTB[DK][TP];    // F: U^T      R: Y^T
  __shared__ __attribute__((aligned(16))) TC sDO[16][PV];    // dO rows of the block
  __shared__ __attribute__((aligned(16))) TC sDL[DIRECT ? 16 * NBS : 16][PV];  // delta rows (direct: of the span)
  __shared__ __attribute__((aligned(16))) TC sDR[16][PV];    // dR rows of the block
  __shared__ __attribute__((aligned(16))) TC sT[16][TP];     // T_II of the block
  __shared__ __attribute__((aligned(16))) TC sP[16][TP];     // P_II of the block
  __shared__ __attribute__((aligned(16))) TC sSD[DK][PS];    // staged D columns, [dk][dv]
  __shared__ __attribute__((aligned(16))) TC sSS[DIRECT ? 1 : DK][PS];  // staged S_J columns, [dk][dv] (two sweeps)
  // direct form: the block's inputs q, k, v, write, erase, log_a, gamma as
  // token rows, read by both the elementwise and the output mapping
  // (rows of 288 bytes for d = 128: read by transposing reads, tr_in, whose
  // eight rows of a 32-lane pass then fall on distinct banks)
  // Two buffers where they fit (64-token chunks): the next block's tiles are
  // then written before the closing barrier of the current one.
  constexpr int PVI = DIRECT ? DV + 16 : 1;
  constexpr int NIB = FORM == BWD_DIRECT ? 2 : 1;
  __shared__ __attribute__((aligned(16))) TC sIn[NIB][DIRECT ? 7 : 1][16][PVI];
  int ibuf = 0;  // the buffer of the block being processed
  __shared__ float sLf[2][16][17];                           // leaf matrices of steep blocks
  __shared__ float sG[DK];
  __shared__ float sGH[DIRECT ? NBS - 1 : 1][DK];             // direct: block decays exp(B_{I+1} - B_I)
  // The block's token-token products x_r . Delta_t over dv (x = dO, dR; r, t
  // tokens), each formed once by one wave and read by all: for the deltas of
  // the block itself masked to the leaf's triangle, in both orientations
  // (sGd: rows r, sGT: rows t, the dR part negated), and in the direct form
  // for each earlier block's deltas (sGh: rows r).
  constexpr int GP = 16 + row_pad<TC>();
  __shared__ __attribute__((aligned(16))) TC sGd[2][16][GP];
  __shared__ __attribute__((aligned(16))) TC sGT[2][16][GP];
  __shared__ __attribute__((aligned(16))) TC sGh[2][DIRECT ? NBS - 1 : 1][16][GP];
  // per-wave partial rowsums of S_C * dS_C, used once before the reverse
  // sweep (which then writes X^T over it)
  static_assert(NW * DK * sizeof(float) <= sizeof(TC) * DK * TP, "rowsum scratch");
  float (*sRow)[DK] = reinterpret_cast<float (*)[DK]>(&sTA[0][0]);

  // identity operand: a 16x16 product with it moves a tile's rows onto lanes
  frag ident;
  {
    f32x4 idv;
#pragma unroll
    for (int i = 0; i < 4; ++i) idv[i] = (4 * g + i == c16) ? 1.f : 0.f;
    ident = M::from_f32(idv);
  }

  // within-block prefix (through each token) and suffix (after it) of log_a,
  // channel ej, tokens RPT*part + rr: loc = Lam_r - B_I, suf = B_{I+1} - Lam_r
  auto block_sums = [&](int I, const float* xl, float* loc, float* suf) {
    float excl = 0.f, exsuf = 0.f, bs = 0.f;
#pragma unroll
    for (int p = 0; p < TPC; ++p) {
      const float ps = sPart[I][p][ej];
      if (p < part) excl += ps;
      if (p > part) exsuf += ps;
      bs += ps;
    }
    float run = 0.f;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      run += xl[rr];
      loc[rr] = excl + run;
    }
    float s2 = 0.f;
#pragma unroll
    for (int rr = RPT - 1; rr >= 0; --rr) {
      suf[rr] = s2 + exsuf;
      s2 += xl[rr];
    }
    if (part == 0) sG[ej] = __expf(bs);
  };

  // T_II, P_II words of block I into sT, sP
  auto tp_word = [&](int I) -> u32x2 {
    return *reinterpret_cast<const u32x2*>(
        at(gTP, static_cast<uint32_t>(I * 512 + (tid < TPW ? tid : TPW - 1) * EPW)));
  };
  auto tp_commit = [&](u32x2 w) {
    if (tid < TPW) {
      const int e0 = tid * EPW;
      TC* dst = e0 < 256 ? &sT[e0 >> 4][e0 & 15] : &sP[(e0 - 256) >> 4][e0 & 15];
      *reinterpret_cast<u32x2*>(dst) = w;
    }
  };

  // (A_m . B_n) over the DV columns of two [16][DV] row tiles, in the
  // MFMA-output layout: lane (g, c16) holds m = 4g+i, n = c16.  Read as the
  // left operand of a 16-wide product it is the matrix with n on the rows
  // and m along the contraction.
  auto leaf_pair = [&](const TC (*A)[PV], const TC (*Bm)[PV]) -> f32x4 {
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < DV / 16; kk += 2)
      acc = M::mma2(M::load(&A[c16][16 * kk + 4 * g]), M::load(&Bm[c16][16 * kk + 4 * g]),
                    M::load(&A[c16][16 * kk + 16 + 4 * g]), M::load(&Bm[c16][16 * kk + 16 + 4 * g]), acc);
    return acc;
  };
  // dst[r][i] = A_r . B_i, masked to i <= r (or i < r when strict): the leaf
  // matrices in LDS, for the per-pair sums of steep blocks
  auto leaf_dot = [&](const TC (*A)[PV], const TC (*Bm)[PV], bool strict, float (*dst)[17]) {
    const f32x4 acc = leaf_pair(A, Bm);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int r = 4 * g + ii;
      const bool keep = strict ? (c16 < r) : (c16 <= r);
      dst[r][c16] = keep ? acc[ii] : 0.f;
    }
  };
  // Steep leaves read the raw inputs from global memory (L2-resident: the
  // step's own loads brought them in).
  // exp(sum of log_a over tokens (i, r] of the block at r0, channel j), r >= i
  auto pair_factor = [&](int r0, int r, int i, int j) -> float {
    float ls = 0.f;
    for (int x = i + 1; x <= r; ++x) ls += ldv(lb, gi(r0 + x, j));
    return __expf(ls);
  };

  // a [16][16] tile held in MFMA-output layout (rows 4g+i, column c16), moved
  // by one identity product so that lane (g, c16) holds row c16, columns
  // 4g..4g+3
  auto turn = [&](f32x4 tile) -> f32x4 { return M::mma(M::from_f32(tile), ident, zero4()); };
  // a gradient tile in MFMA-output layout (tokens r0 + 4g+i, channel colv(n))
  // to its [B, T, H, D] tensor: bf16 gradients turned into token rows of four
  // channels by the bf16 identity product (which rounds to bf16 as the store
  // would; one 8-byte store per lane), fp32 gradients element by element (4
  // stores of 64-byte row pieces: measured 7% faster for the whole kernel than
  // turning the tile with an fp32 identity product for 16-byte stores)
  auto store_grad = [&](Tg* base, int r0, int n, f32x4 tile) {
    if constexpr (sizeof(Tg) == 2) {
      const f32x4 tt = turn(tile);
      if (!PKO || r0 + c16 < vrows) store4(at(base, gi(r0 + c16, col0(n) + 4 * g)), tt);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!PKO || r0 + 4 * g + i < vrows) *at(base, gi(r0 + 4 * g + i, colv(n))) = tile[i];
    }
  };

  // A saved state (16 x 16 tiles, stile_index) in the accumulator layout.
  // (the lane offset is made opaque per call so that the addresses are formed
  // where they are used instead of being kept live across the sweeps)
  auto load_state = [&](f32x4 (*st)[NT], const Tin* src) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if constexpr (sizeof(Tin) == 4) {
        uint32_t lo = stile_index(4 * g, colv(n), DV);
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int s = 0; s < RT; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[s][n][i] = *at(src, lo + static_cast<uint32_t>(s * (DV / 16) * 256 + 16 * i));
      } else {
        // row 16s + c16, columns col0(n) + 4g .. + 3 as one 8-byte word (the
        // wave reads one whole tile), turned onto the accumulator layout by an
        // identity product (exact)
        uint32_t lo = stile_index(c16, col0(n) + 4 * g, DV);
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int s = 0; s < RT; ++s) {
          const uint2 w = *reinterpret_cast<const uint2*>(at(src, lo + static_cast<uint32_t>(s * (DV / 16) * 256)));
          st[s][n] = M::mma(__builtin_bit_cast(frag, w), ident, zero4());
        }
      }
    }
  };
  // the chunk-end state gradient from its transposed 16-row tiles (the
  // lane's four rows of column colv(n) are one 8- or 16-byte word)
  auto load_dstate = [&](f32x4 (*st)[NT]) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      uint32_t lo = static_cast<uint32_t>(colv(n) * 16 + 4 * g);
      asm volatile("" : "+v"(lo));
#pragma unroll
      for (int s = 0; s < RT; ++s) st[s][n] = load4(at(dSC, lo + static_cast<uint32_t>(s * DV * 16)));
    }
  };

  auto decay_scale = [&](int s) -> f32x4 {
    f32x4 gs;
#pragma unroll
    for (int i = 0; i < 4; ++i) gs[i] = sG[16 * s + 4 * g + i];
    return gs;
  };

  // =========================== R: reverse sweep ===========================
  // slots: log_a, k, erase, q, gamma (channel ej, tokens RPT*part + rr);
  // dO and delta rows (raw words); T/P word; the block-start state (16-byte
  // words); q, gamma, v, write, k, erase, log_a at (token 4g+i, column colv(n))
  float xl[RPT], xk[RPT], xe[RPT], xq[RPT], xg[RPT];
  u32x2 rdo[RW], rdl[RW], rtp;
  u32x4 rss[SPT];
  float oq[NT][4], og[NT][4], ov[NT][4], ow[NT][4], ok[NT][4], oe[NT][4], ol[NT][4];
  auto prefetch_r = [&](int J) {
    const int r0 = 16 * J;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      if constexpr (!DIRECT) {
        const uint32_t o = gi(r0 + RPT * part + rr, ej);
        xl[rr] = ldv(lb, o);
        xk[rr] = ldv(kb, o);
        xe[rr] = ldv(eb, o);
        xq[rr] = ldv(qb, o);
        xg[rr] = GTOK ? gam(r0 + RPT * part + rr, ej) : gse;
      }
    }
#pragma unroll
    for (int e = 0; e < RW; ++e) {
      const int col = pc0 + e * EPW;
      rdo[e] = *reinterpret_cast<const u32x2*>(at(dOb, gi(r0 + prow, col)));
      if constexpr (!DIRECT)
        rdl[e] = *reinterpret_cast<const u32x2*>(at(gDel, static_cast<uint32_t>((r0 + prow) * DV + col)));
    }
    rtp = tp_word(J);
    if constexpr (!DIRECT) {
      const TC* sj = gS + static_cast<size_t>(J) * DK * DV;
#pragma unroll
      for (int k2 = 0; k2 < SPT; ++k2)
        rss[k2] = *reinterpret_cast<const u32x4*>(at(sj, static_cast<uint32_t>((tid + k2 * NTH) * SEW)));
    }
  };
  // the inputs at the output mapping: issued once the step's outputs are
  // written (their registers are then free)
  auto prefetch_r_out = [&](int J) {
    const int r0 = 16 * J;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const uint32_t o = gi(r0 + 4 * g + ii, colv(n));
        oq[n][ii] = ldv(qb, o);
        og[n][ii] = GTOK ? gam(r0 + 4 * g + ii, colv(n)) : gsc[n];
        ov[n][ii] = ldv(vb, o);
        ow[n][ii] = ldv(wb, o);
        ok[n][ii] = ldv(kb, o);
        oe[n][ii] = ldv(eb, o);
        ol[n][ii] = ldv(lb, o);
      }
  };
  // Direct form: the block's inputs into sIn.  Tensor t (q, k, v, write,
  // erase, log_a, gamma; gamma only when per token) is moved by wave t % NW,
  // 16 rows of DV values as 16-byte words, loaded a step ahead into registers.
  constexpr int NTEN = 7;
  constexpr int SPWV = (NTEN + NW - 1) / NW;  // tensors per wave
  constexpr int IWR = DV / SEW;               // 16-byte words per input row
  constexpr int IWT = 16 * IWR / 64;          // words per lane and tensor
  static_assert(!DIRECT || (16 * IWR) % 64 == 0, "input staging layout");
  u32x4 iw[DIRECT ? SPWV * IWT : 1];
  auto in_ptr = [&](int t) -> const Tin* {
    return t == 0 ? qb : t == 1 ? kb : t == 2 ? vb : t == 3 ? wb : t == 4 ? eb : t == 5 ? lb : gb;
  };
  auto load_in = [&](int J) {
    if constexpr (DIRECT) {
#pragma unroll
      for (int sl = 0; sl < SPWV; ++sl) {
        const int t = wave + sl * NW;  // wave-uniform
        if (t < (GTOK ? NTEN : NTEN - 1)) {
          const Tin* base = in_ptr(t);
#pragma unroll
          for (int k2 = 0; k2 < IWT; ++k2) {
            const int w = lane + 64 * k2;
            const int row = w / IWR;
            iw[sl * IWT + k2] = *reinterpret_cast<const u32x4*>(at(base, gi(16 * J + row, (w - row * IWR) * SEW)));
          }
        }
      }
    }
  };
  auto store_in = [&](int buf) {
    if constexpr (DIRECT) {
#pragma unroll
      for (int sl = 0; sl < SPWV; ++sl) {
        const int t = wave + sl * NW;
        if (t < (GTOK ? NTEN : NTEN - 1)) {
#pragma unroll
          for (int k2 = 0; k2 < IWT; ++k2) {
            const int w = lane + 64 * k2;
            const int row = w / IWR;
            put16(&sIn[buf][t][row][(w - row * IWR) * SEW], iw[sl * IWT + k2]);
          }
        }
      }
    }
  };
  // Direct form: four consecutive tokens of one channel of input tile x, by a
  // transposing read: lane l of each 16-lane group reads row row0 + l/4,
  // channels cb + 4 (l%4) .. + 3, and receives the four rows' values of
  // channel cb + l (cb: its group's first channel)
  auto tr_in = [&](int x, int row0, int cb) -> i16x4 {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int l = lane & 15;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(&sIn[ibuf][x][row0 + (l >> 2)][cb + 4 * (l & 3)]));
  };
  // bf16: rows 4g .. 4g+3 of column n0 + c16 of a [16][pitch] tile as a
  // fragment (the transposed read of a tile held as token rows)
  auto tr_tile = [&](const TC* tile, int pitch, int n0) -> i16x4 {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int l = lane & 15;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(tile + (4 * g + (l >> 2)) * pitch + n0 + 4 * (l & 3)));
  };
  // a static gate's value per channel (none: 1)
  auto gam_static = [&](int j) -> float { return gmode == GAMMA_NONE ? 1.f : ldv(gst, static_cast<uint32_t>(j)); };
  // Direct form: the block's inputs at the output mapping, from sIn
  auto in_out = [&]() {
    if constexpr (DIRECT) {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const float gs = GTOK ? 0.f : gsc[n];
        // tokens 4g .. 4g+3 of channel colv(n)
        const i16x4 fq = tr_in(0, 4 * g, col0(n)), fk = tr_in(1, 4 * g, col0(n)), fv = tr_in(2, 4 * g, col0(n)),
                    fw = tr_in(3, 4 * g, col0(n)), fe = tr_in(4, 4 * g, col0(n)), fl = tr_in(5, 4 * g, col0(n));
        i16x4 fg = fq;
        if constexpr (GTOK) fg = tr_in(6, 4 * g, col0(n));
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          oq[n][ii] = M::to_f32(static_cast<uint16_t>(fq[ii]));
          ok[n][ii] = M::to_f32(static_cast<uint16_t>(fk[ii]));
          ov[n][ii] = M::to_f32(static_cast<uint16_t>(fv[ii]));
          ow[n][ii] = M::to_f32(static_cast<uint16_t>(fw[ii]));
          oe[n][ii] = M::to_f32(static_cast<uint16_t>(fe[ii]));
          ol[n][ii] = M::to_f32(static_cast<uint16_t>(fl[ii]));
          og[n][ii] = GTOK ? M::to_f32(static_cast<uint16_t>(fg[ii])) : gs;
        }
      }
    }
  };
  // log-decay of channel colv(n) over the block at the output mapping (tokens
  // 4g+ii): loc = Lam - B_J (through the token), suf = B_{J+1} - Lam (after
  // it); the lane's four tokens, plus the token groups of lanes c16 + 16g'
  auto out_sums = [&](int n, float* loc, float* suf) {
    const float* l = ol[n];
    const float s4 = (l[0] + l[1]) + (l[2] + l[3]);
    const float t0 = __shfl(s4, c16, 64);
    const float t1 = __shfl(s4, c16 + 16, 64);
    const float t2 = __shfl(s4, c16 + 32, 64);
    const float t3 = __shfl(s4, c16 + 48, 64);
    float run = (g > 0 ? t0 : 0.f) + (g > 1 ? t1 : 0.f) + (g > 2 ? t2 : 0.f);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      run += l[ii];
      loc[ii] = run;
    }
    float after = (g < 3 ? t3 : 0.f) + (g < 2 ? t2 : 0.f) + (g < 1 ? t1 : 0.f);
#pragma unroll
    for (int ii = 3; ii >= 0; --ii) {
      suf[ii] = after;
      after += l[ii];
    }
  };
  // block-start state words of column pass p into sSS
  auto commit_state = [&](const u32x4* words, int p) {
#pragma unroll
    for (int k2 = 0; k2 < SPT; ++k2) {
      const int w = tid + k2 * NTH;
      const int row = w / SWR;
      const int colw = (w - row * SWR) * SEW;
      if (colw / SW == p) put16(&sSS[row][colw - p * SW], words[k2]);
    }
  };
  // Ke = k exp(B_{J+1} - Lam) rows; X = ek exp(Lam - B_J), Y = qt exp(Lam - B_J)
  // transposed.  Returns whether the block's leaf is within LEAF_SAFE_RANGE.
  auto commit_r = [&](int J) -> int {
    const int safe = !((sUnsafe >> J) & 1);
    if constexpr (DIRECT) {
      const float gs = GTOK ? 0.f : gse;
      // tokens RPT part .. + 3 of channel ej (the lane's channel within its
      // 16-lane group: ej % 16 == lane % 16)
      static_assert(RPT == 4 && DK % 64 == 0, "elementwise mapping of the transposing reads");
      const int cb = ej & ~15;
      const i16x4 fq = tr_in(0, RPT * part, cb), fk = tr_in(1, RPT * part, cb), fe = tr_in(4, RPT * part, cb),
                  fl = tr_in(5, RPT * part, cb);
      i16x4 fg = fq;
      if constexpr (GTOK) fg = tr_in(6, RPT * part, cb);
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) {
        xq[rr] = M::to_f32(static_cast<uint16_t>(fq[rr]));
        xk[rr] = M::to_f32(static_cast<uint16_t>(fk[rr]));
        xe[rr] = M::to_f32(static_cast<uint16_t>(fe[rr]));
        xl[rr] = M::to_f32(static_cast<uint16_t>(fl[rr]));
        xg[rr] = GTOK ? M::to_f32(static_cast<uint16_t>(fg[rr])) : gs;
      }
    }
    float loc[RPT], suf[RPT];
    block_sums(J, xl, loc, suf);
#pragma unroll
    for (int h4 = 0; h4 < RPT / 4; ++h4) {
      f32x4 tA, tB;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int rr = 4 * h4 + q4;
        const int r = RPT * part + rr;
        const float fs = __expf(loc[rr]);
        sRowA[r][ej] = M::cvt(xk[rr] * __expf(suf[rr]));
        tA[q4] = xe[rr] * xk[rr] * fs;
        tB[q4] = xg[rr] * xq[rr] * fs;
      }
      const int t0 = RPT * part + 4 * h4;
      store4(&sTA[ej][t0], tA);
      store4(&sTB[ej][t0], tB);
    }
#pragma unroll
    for (int e = 0; e < RW; ++e) {
      const int col = pc0 + e * EPW;
      *reinterpret_cast<u32x2*>(&sDO[prow][col]) = rdo[e];
      if constexpr (!DIRECT) *reinterpret_cast<u32x2*>(&sDL[prow][col]) = rdl[e];
    }
    tp_commit(rtp);
    if constexpr (!DIRECT) commit_state(rss, 0);
    __syncthreads();
    return safe;
  };

  // =========================== F: forward sweep ===========================
  // slots: log_a, k, erase, write, v (channel ej, tokens RPT*part + rr), T/P word
  float fl[RPT], fk[RPT], fe[RPT], fw[RPT], fv[RPT];
  u32x2 ftp;
  auto prefetch_f = [&](int I) {
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const uint32_t o = gi(16 * I + RPT * part + rr, ej);
      fl[rr] = ldv(lb, o);
      fk[rr] = ldv(kb, o);
      fe[rr] = ldv(eb, o);
      fw[rr] = ldv(wb, o);
      fv[rr] = ldv(vb, o);
    }
    ftp = tp_word(I);
  };
  // X = ek exp(Lam - B_I) rows, Ke = k exp(B_{I+1} - Lam) and U = write*v transposed
  auto commit_f = [&](int I) {
    float loc[RPT], suf[RPT];
    block_sums(I, fl, loc, suf);
#pragma unroll
    for (int h4 = 0; h4 < RPT / 4; ++h4) {
      f32x4 tA, tB;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int rr = 4 * h4 + q4;
        const int r = RPT * part + rr;
        sRowA[r][ej] = M::cvt(fe[rr] * fk[rr] * __expf(loc[rr]));
        tA[q4] = fk[rr] * __expf(suf[rr]);
        tB[q4] = fw[rr] * fv[rr];
      }
      const int t0 = RPT * part + 4 * h4;
      store4(&sTA[ej][t0], tA);
      store4(&sTB[ej][t0], tB);
    }
    tp_commit(ftp);
    __syncthreads();
  };

  f32x4 S[RT][NT];
  f32x4 D[RT][NT];
  // Direct form: the operands of the Horner steps in the reverse sweep,
  // Ke_I = k exp(B_{I+1} - Lam) at (token 4g+i of block I, channel colv(n)),
  // and the block decays exp(B_{I+1} - B_I) in sGH, for every block but the last.
  frag keH[DIRECT ? NBS - 1 : 1][NT];
  frag s0f[NT][DIRECT ? DV / 16 : 1];  // direct form: S0 rows of the wave's key channels
  // Direct form: every global read of the prologue is issued before the
  // first wait -- the chunk's deltas and Kbar^T (16-byte words), Gamma_C, the
  // Horner inputs, S0, dS_C and the first step's prefetch.
  constexpr int DWR = DV / SEW;        // 16-byte words per delta row
  constexpr int DWT = C * DWR / NTH;   // delta words per thread
  constexpr int KWR = C / SEW;         // 16-byte words per Kbar^T row
  constexpr int KWT = DK * KWR / NTH;  // Kbar^T words per thread
  u32x4 dw[DIRECT ? DWT : 1], kw[DIRECT ? KWT : 1], gcw;
  // direct form: log_a of every block and k of the earlier ones at (token
  // 4g+i of block I, channel colv(n)): the Horner inputs, and the per-part
  // decay sums (part p of the elementwise mapping is token group g = p here)
  float hl[DIRECT ? NBS : 1][NT][4], hk[DIRECT ? NBS - 1 : 1][NT][4];
  // The Horner operands of a span from hl, hk (keH, and the block decays in sGH).
  auto horner_setup = [&]() {
    if constexpr (DIRECT)
#pragma unroll
    for (int I = 0; I < NBS - 1; ++I)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const float* l = hl[I][n];
        // log-decay after each token to the block's end: within the lane's
        // four tokens, plus the token groups of the lanes c16 + 16g' (g' > g)
        const float s4 = (l[0] + l[1]) + (l[2] + l[3]);
        const float t1 = __shfl(s4, c16 + 16, 64);
        const float t2 = __shfl(s4, c16 + 32, 64);
        const float t3 = __shfl(s4, c16 + 48, 64);
        const float t0 = __shfl(s4, c16, 64);
        float later = (g < 3 ? t3 : 0.f) + (g < 2 ? t2 : 0.f) + (g < 1 ? t1 : 0.f);
        f32x4 kv;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          kv[i] = hk[I][n][i] * __expf(later);
          later += l[i];
        }
        keH[I][n] = M::from_f32(kv);
        if (g == 0) sGH[I][colv(n)] = __expf(((t0 + t1) + t2) + t3);
      }
  };
  // log_a of the span's blocks and k of all but its last, at (token 4g+i of
  // block I of the span starting at block I0, channel colv(n))
  auto horner_loads = [&](int I0) {
    if constexpr (DIRECT)
#pragma unroll
    for (int I = 0; I < NBS; ++I)
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t o = gi(16 * (I0 + I) + 4 * g + i, colv(n));
          hl[I][n][i] = ldv(lb, o);
          if (I < NBS - 1) hk[I < NBS - 1 ? I : 0][n][i] = ldv(kb, o);
        }
  };
  // the span's start state: its rows of this wave's key channels as the right
  // operands of the boundary products (rows colv(n), dv columns 16kk + 4g ..)
  auto load_s0f = [&](const Tin* src) {
    if constexpr (DIRECT)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int kk = 0; kk < DV / 16; ++kk)
        s0f[n][kk] = *reinterpret_cast<const frag*>(at(src, stile_index(col0(n) + c16, 16 * kk + 4 * g, DV)));
  };
  if constexpr (FORM == BWD_DIRECT) {
    static_assert(DWT * NTH == C * DWR && KWT * NTH == DK * KWR && DK / 4 <= NTH && NB == 4,
                  "direct-form prologue layout");
    static_assert(TPC == 4 && RPT == 4, "direct form: one elementwise part per token group of the output mapping");
    const char* cs = summ + static_cast<size_t>(chunk) * summ_bytes;
    const TC* gD = reinterpret_cast<const TC*>(cs + dl_offset);
    const TC* gKT = reinterpret_cast<const TC*>(cs) + summary_part(SP_KBT, C, DK, DV);
    const float* gGC = reinterpret_cast<const float*>(cs + summary_part(SP_END, C, DK, DV) * sizeof(TC));
#pragma unroll
    for (int k2 = 0; k2 < DWT; ++k2)
      dw[k2] = *reinterpret_cast<const u32x4*>(at(gD, static_cast<uint32_t>((tid + k2 * NTH) * SEW)));
#pragma unroll
    for (int k2 = 0; k2 < KWT; ++k2)
      kw[k2] = *reinterpret_cast<const u32x4*>(
          at(gKT, tpart_index((tid + k2 * NTH) / KWR, ((tid + k2 * NTH) % KWR) * SEW, DK)));  // 16-token tiles
    gcw = *reinterpret_cast<const u32x4*>(at(gGC, static_cast<uint32_t>(4 * min(tid, DK / 4 - 1))));
    horner_loads(0);
    load_state(S, S0c);
    load_s0f(S0c);
    load_dstate(D);
    prefetch_r(NB - 1);
    load_in(NB - 1);
  }

  // ---- sums of the log-decay over each block and each part of it, and the
  // blocks whose decay leaves LEAF_SAFE_RANGE (steep leaves) ----
  if (tid == 0) sUnsafe = 0;
  if constexpr (FORM == BWD_DIRECT) {
    // from the log-decay already in registers at the output mapping
#pragma unroll
    for (int I = 0; I < NB; ++I)
#pragma unroll
      for (int n = 0; n < NT; ++n) sPart[I][g][colv(n)] = (hl[I][n][0] + hl[I][n][1]) + (hl[I][n][2] + hl[I][n][3]);
  } else {
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      float sacc = 0.f;
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) sacc += ldv(lb, gi(16 * I + RPT * part + rr, ej));
      sPart[I][part][ej] = sacc;
    }
  }
  __syncthreads();
  if (part == 0) {
    unsigned mask = 0;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      float bs = 0.f;
#pragma unroll
      for (int p = 0; p < TPC; ++p) bs += sPart[I][p][ej];
      if (!(-bs <= LEAF_SAFE_RANGE)) mask |= 1u << I;
    }
    if (mask) atomicOr(&sUnsafe, static_cast<int>(mask));
  }

  if constexpr (FORM == BWD_DIRECT) {
    // deltas into sDL; Kbar^T into sSD (until the sweep stages D there);
    // Gamma_C into sG (until the sweep's block sums); the last block's inputs
    // into sIn
#pragma unroll
    for (int k2 = 0; k2 < DWT; ++k2) {
      const int w = tid + k2 * NTH;
      const int row = w / DWR;
      put16(&sDL[row][(w - row * DWR) * SEW], dw[k2]);
    }
#pragma unroll
    for (int k2 = 0; k2 < KWT; ++k2) {
      const int w = tid + k2 * NTH;
      const int row = w / KWR;
      put16(&sSD[row][(w - row * KWR) * SEW], kw[k2]);
    }
    if (tid < DK / 4) *reinterpret_cast<u32x4*>(&sG[4 * tid]) = gcw;
    store_in((NB - 1) % NIB);
    horner_setup();
    __syncthreads();  // sDL, sSD, sG, sIn, sGH
    // S becomes the chunk-end state S_C = diag(Gamma_C) S0 + Kbar^T Delta
    // (for the rowsum term below)
    {
      frag dcol[NB][NT];  // Delta at (token 4g+i of block m, column colv(n))
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          f32x4 t;
#pragma unroll
          for (int i = 0; i < 4; ++i) t[i] = M::to_f32(sDL[16 * m + 4 * g + i][colv(n)]);
          dcol[m][n] = M::from_f32(t);
        }
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        const f32x4 gc = decay_scale(s);
#pragma unroll
        for (int n = 0; n < NT; ++n) S[s][n] *= gc;
#pragma unroll
        for (int m = 0; m < NB; m += 2) {
          const frag ka = M::load(&sSD[16 * s + c16][16 * m + 4 * g]);
          const frag ka1 = M::load(&sSD[16 * s + c16][16 * m + 16 + 4 * g]);
#pragma unroll
          for (int n = 0; n < NT; ++n) S[s][n] = M::mma2(ka, dcol[m][n], ka1, dcol[m + 1][n], S[s][n]);
        }
      }
    }
  } else if constexpr (SUB) {
    // Forward pass over the 64-token sub-chunks:
    //   S_{g+1} = diag(Gamma_g) S_g + Kbar_g^T Delta_g,
    // with the deltas the forward scan kept in the chunk summary and
    // Kbar_g = k exp(Lam_end - Lam), the keys decayed to the sub-chunk's end
    // (every factor <= 1).  The start state of each later sub-chunk goes to the
    // scratch (compute type, [dk][dv] rows) for the reverse sweep; S ends as
    // the chunk-end state S_C.
    constexpr int SWT = 16 * NBS * DV / SEW / NTH;  // 16-byte delta words per thread and sub-chunk
    static_assert(SWT * NTH * SEW == 16 * NBS * DV && RPT == 4, "sub-chunk pass layout");
    const TC* gD = reinterpret_cast<const TC*>(summ + static_cast<size_t>(chunk) * summ_bytes + dl_offset);
    load_state(S, S0c);
    load_dstate(D);
    prefetch_r(NB - 1);
    load_in(NB - 1);
    __syncthreads();  // sPart
#pragma unroll 1
    for (int sg = 0; sg < NSUB; ++sg) {
      u32x4 dwl[SWT];
#pragma unroll
      for (int k2 = 0; k2 < SWT; ++k2)
        dwl[k2] = *reinterpret_cast<const u32x4*>(
            at(gD, static_cast<uint32_t>(16 * NBS * sg * DV + (tid + k2 * NTH) * SEW)));
      float fk[NBS][RPT], fl2[NBS][RPT];
#pragma unroll
      for (int bl = 0; bl < NBS; ++bl)
#pragma unroll
        for (int rr = 0; rr < RPT; ++rr) {
          const uint32_t o = gi(16 * (NBS * sg + bl) + RPT * part + rr, ej);
          fk[bl][rr] = ldv(kb, o);
          fl2[bl][rr] = ldv(lb, o);
        }
      // Kbar_g^T into sSD ([dk][tokens of the sub-chunk]), Gamma_g into sG
      float later = 0.f;  // log-decay of the sub-chunk's blocks after block bl (channel ej)
#pragma unroll
      for (int bl = NBS - 1; bl >= 0; --bl) {
        const int I = NBS * sg + bl;
        float exsuf = 0.f, bs = 0.f;
#pragma unroll
        for (int p = 0; p < TPC; ++p) {
          const float ps = sPart[I][p][ej];
          if (p > part) exsuf += ps;
          bs += ps;
        }
        float s2 = 0.f;
        f32x4 kv;
#pragma unroll
        for (int rr = RPT - 1; rr >= 0; --rr) {
          kv[rr] = fk[bl][rr] * __expf(s2 + exsuf + later);
          s2 += fl2[bl][rr];
        }
        store4(&sSD[ej][16 * bl + RPT * part], kv);
        later += bs;
      }
      if (part == 0) sG[ej] = __expf(later);
#pragma unroll
      for (int k2 = 0; k2 < SWT; ++k2) {
        const int w = tid + k2 * NTH;
        const int row = w / DWR;
        put16(&sDL[row][(w - row * DWR) * SEW], dwl[k2]);
      }
      __syncthreads();
      if (sg > 0) {
        // the sub-chunk's start state, rounded once, as 16 x 16 tiles
        TC* dst = gSub + static_cast<size_t>(sg - 1) * DK * DV;
#pragma unroll
        for (int s2 = 0; s2 < RT; ++s2)
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const f32x4 tt = M::mma(M::from_f32(S[s2][n]), ident, zero4());  // row 16s+c16, columns col0(n)+4g+i
            store4(at(dst, stile_index(16 * s2 + c16, col0(n) + 4 * g, DV)), tt);
          }
      }
      frag dcol[NBS][NT];  // Delta at (token 4g+i of block m, column colv(n))
#pragma unroll
      for (int m = 0; m < NBS; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          f32x4 t;
#pragma unroll
          for (int i = 0; i < 4; ++i) t[i] = M::to_f32(sDL[16 * m + 4 * g + i][colv(n)]);
          dcol[m][n] = M::from_f32(t);
        }
#pragma unroll
      for (int s2 = 0; s2 < RT; ++s2) {
        const f32x4 gc = decay_scale(s2);
#pragma unroll
        for (int n = 0; n < NT; ++n) S[s2][n] *= gc;
#pragma unroll
        for (int m = 0; m < NBS; m += 2) {
          const frag ka = M::load(&sSD[16 * s2 + c16][16 * m + 4 * g]);
          const frag ka1 = M::load(&sSD[16 * s2 + c16][16 * m + 16 + 4 * g]);
#pragma unroll
          for (int n = 0; n < NT; ++n) S[s2][n] = M::mma2(ka, dcol[m][n], ka1, dcol[m + 1][n], S[s2][n]);
        }
      }
      __syncthreads();  // sDL, sSD and sG are rewritten by the next sub-chunk
    }
    store_in((NB - 1) % NIB);  // the last block's inputs, for the reverse sweep
  } else {
    load_state(S, S0c);
    prefetch_f(0);
    __syncthreads();  // sPart, sUnsafe

#pragma unroll 1
    for (int I = 0; I < NB; ++I) {
      const int r0 = 16 * I;
      commit_f(I);
      prefetch_f(I + 1 < NB ? I + 1 : I);
      frag Sf[RT][NT];
#pragma unroll
      for (int s = 0; s < RT; ++s)
#pragma unroll
        for (int n = 0; n < NT; ++n) Sf[s][n] = M::from_f32(S[s][n]);
      // the block-start state, as [dk][dv] rows, for the reverse sweep
      {
        TC* dst = gS + static_cast<size_t>(I) * DK * DV;
#pragma unroll
        for (int s = 0; s < RT; ++s)
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const f32x4 tt = M::mma(Sf[s][n], ident, zero4());  // row 16s+c16, columns col0(n)+4g+i
            store4(at(dst, static_cast<uint32_t>((16 * s + c16) * DV + col0(n) + 4 * g)), tt);
          }
      }
      // Delta_I = T_II (U_I - X_I S_I)
      f32x4 Dl[NT];
      {
        f32x4 xs[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) xs[n] = zero4();
#pragma unroll
        for (int s = 0; s < RT; s += 2) {
          const frag xa = M::load(&sRowA[c16][16 * s + 4 * g]);
          const frag xa1 = M::load(&sRowA[c16][16 * s + 16 + 4 * g]);
#pragma unroll
          for (int n = 0; n < NT; ++n) xs[n] = M::mma2(xa, Sf[s][n], xa1, Sf[s + 1][n], xs[n]);
        }
        const frag ta = M::load(&sT[c16][4 * g]);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          f32x4 rhs = load4(&sTB[colv(n)][4 * g]);
          rhs -= xs[n];
          Dl[n] = M::mma(ta, M::from_f32(rhs), zero4());
          store4(at(gDel, static_cast<uint32_t>((r0 + c16) * DV + col0(n) + 4 * g)), turn(Dl[n]));
        }
      }
      // S_{I+1} = diag(exp(B_{I+1} - B_I)) S_I + Ke_I^T Delta_I
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        const frag ka = M::load(&sTA[16 * s + c16][4 * g]);
        const f32x4 gs = decay_scale(s);
#pragma unroll
        for (int n = 0; n < NT; ++n) S[s][n] = M::mma(ka, M::from_f32(Dl[n]), S[s][n] * gs);
      }
      __syncthreads();
    }
    prefetch_r(NB - 1);
    prefetch_r_out(NB - 1);
    load_dstate(D);
  }  // F sweep

  // chunk-end term rowsum(S_C * dS_C): S holds S_C here and D holds dS_C;
  // it enters dlog_a on every token of the chunk
#pragma unroll
  for (int s = 0; s < RT; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = 0.f;
#pragma unroll
      for (int n = 0; n < NT; ++n) a += S[s][n][i] * D[s][n][i];
      a = sum16(a);
      if (c16 == 0) sRow[wave][16 * s + 4 * g + i] = a;
    }
  __syncthreads();
  float carry[NT];  // sum of dLam over the finished (later) tokens, channel colv(n)
  float gsum[NT];   // static readout gate: this lane's share of the chunk's sum of dgamma
#pragma unroll
  for (int n = 0; n < NT; ++n) gsum[n] = 0.f;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += sRow[w][colv(n)];
    carry[n] = t;
  }
  __syncthreads();  // sRow is read before the first commit overwrites it

#pragma unroll 1
  for (int J = NB - 1; J >= 0; --J) {
    const int r0 = 16 * J;
    const int jl = J % NBS;  // the block within its span (direct forms)
    if constexpr (SUB) {
      if (jl == NBS - 1) {
        // a sub-chunk's last block: its start state (the chunk's, or from the
        // forward pass), its deltas and its Horner operands; the previous
        // step's closing barrier ended every read of the later sub-chunk's
        // and the commit below publishes these
        const int sg = J / NBS;
        constexpr int SWT = 16 * NBS * DV / SEW / NTH;
        const TC* gD = reinterpret_cast<const TC*>(summ + static_cast<size_t>(chunk) * summ_bytes + dl_offset);
        u32x4 dwl[SWT];
#pragma unroll
        for (int k2 = 0; k2 < SWT; ++k2)
          dwl[k2] = *reinterpret_cast<const u32x4*>(
              at(gD, static_cast<uint32_t>(16 * NBS * sg * DV + (tid + k2 * NTH) * SEW)));
        horner_loads(NBS * sg);
        load_s0f(sg == 0 ? S0c : gSub + static_cast<size_t>(sg - 1) * DK * DV);
#pragma unroll
        for (int k2 = 0; k2 < SWT; ++k2) {
          const int w = tid + k2 * NTH;
          const int row = w / DWR;
          put16(&sDL[row][(w - row * DWR) * SEW], dwl[k2]);
        }
        horner_setup();
      }
    }
    const TC (*dlJ)[PV] = DIRECT ? sDL + 16 * jl : sDL;  // the block's delta rows
    ibuf = J % NIB;
    const int safe = commit_r(J);
    u32x4 css[SPLIT > 1 ? SPT : 1];  // this block's state words for the later column passes
    if (SPLIT > 1) {
#pragma unroll
      for (int k2 = 0; k2 < SPT; ++k2) css[k2] = rss[k2];
    }
    prefetch_r(J > 0 ? J - 1 : 0);
    load_in(J > 0 ? J - 1 : 0);  // (direct form) the next block's inputs, written to sIn at the step's end
    in_out();                    // (direct form) this block's inputs at the output mapping
    // dR_J = T_JJ^T (Ke_J D + P_JJ^T dO_J)
    f32x4 dRn[NT];
    frag dOf[NT];
    {
      frag ptf, ttf;
      if constexpr (sizeof(TC) == 2) {
        ttf = __builtin_bit_cast(frag, tr_tile(&sT[0][0], TP, 0));
        ptf = __builtin_bit_cast(frag, tr_tile(&sP[0][0], TP, 0));
      } else {
        f32x4 pv, tv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          tv[i] = M::to_f32(sT[4 * g + i][c16]);
          pv[i] = M::to_f32(sP[4 * g + i][c16]);
        }
        ptf = M::from_f32(pv);
        ttf = M::from_f32(tv);
      }
      // key tiles in pairs, one 32-deep product each
      f32x4 acc[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = zero4();
#pragma unroll
      for (int s = 0; s < RT; s += 2) {
        const frag ka = M::load(&sRowA[c16][16 * s + 4 * g]);
        const frag kb2 = M::load(&sRowA[c16][16 * (s + 1) + 4 * g]);
#pragma unroll
        for (int n = 0; n < NT; ++n)
          acc[n] = M::mma2(ka, M::from_f32(D[s][n]), kb2, M::from_f32(D[s + 1][n]), acc[n]);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if constexpr (sizeof(TC) == 2) {
          dOf[n] = __builtin_bit_cast(frag, tr_tile(&sDO[0][0], PV, col0(n)));
        } else {
          f32x4 dov;
#pragma unroll
          for (int i = 0; i < 4; ++i) dov[i] = M::to_f32(sDO[4 * g + i][colv(n)]);
          dOf[n] = M::from_f32(dov);
        }
        acc[n] = M::mma(ptf, dOf[n], acc[n]);
        dRn[n] = M::mma(ttf, M::from_f32(acc[n]), zero4());
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      store4(&sDR[c16][col0(n) + 4 * g], turn(dRn[n]));
      f32x4 gw, gv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gw[i] = ov[n][i] * dRn[n][i];
        gv[i] = ow[n][i] * dRn[n][i];
      }
      store_grad(dwb, r0, n, gw);
      store_grad(dvb, r0, n, gv);
    }
    // Boundary parts, in column passes over dv:
    //   d(k)_i <- Delta_i . D rows,  d(qt)_r <- dO_r . S_J rows,  d(ek)_r <- dR_r . S_J rows
    f32x4 acck[NT], accq[NT], acce[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      acck[n] = zero4();
      accq[n] = zero4();
      acce[n] = zero4();
    }
    // The shared token-token products G = x . Delta_t (x = dO, dR rows of the
    // block), np of them, product pr by wave pr % NW: with the deltas of the
    // block itself (pr < 2), and in the direct forms of block pr/2 <= jl of
    // the span.  A wave whose pr >= np forms a product it does not store (no
    // branch in the contraction).
    constexpr int PPW = DIRECT ? (2 * NBS + NW - 1) / NW : (2 + NW - 1) / NW;
    const int np = DIRECT ? 2 * (jl + 1) : 2;
    f32x4 gacc[PPW];
#pragma unroll
    for (int q2 = 0; q2 < PPW; ++q2) gacc[q2] = zero4();
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) {
      if (p > 0) {
        __syncthreads();  // the previous pass's reads of the staging tiles are done
        commit_state(css, p);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int cb = col0(n) - p * SW;
        if (cb >= 0 && cb < SW) {
#pragma unroll
          for (int s = 0; s < RT; ++s) store4(&sSD[16 * s + c16][cb + 4 * g], turn(D[s][n]));
        }
      }
      __syncthreads();  // also publishes the dR rows
      // contraction tiles in pairs (one 32-deep product each) when the pass
      // holds an even number of them
      constexpr int KP = (SW / 16) % 2 == 0 ? 2 : 1;
      auto mmk = [&](const frag* a, const frag* b, f32x4 c) -> f32x4 {
        if constexpr (KP == 2) return M::mma2(a[0], b[0], a[1], b[1], c);
        else return M::mma(a[0], b[0], c);
      };
#pragma unroll
      for (int kk = 0; kk < SW / 16; kk += KP) {
        const int cc = p * SW + 16 * kk + 4 * g;
        frag al[KP], ao[KP], ar[KP];
#pragma unroll
        for (int u = 0; u < KP; ++u) {
          al[u] = M::load(&dlJ[c16][cc + 16 * u]);
          ao[u] = M::load(&sDO[c16][cc + 16 * u]);
          ar[u] = M::load(&sDR[c16][cc + 16 * u]);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          frag bd[KP], bs[KP];
#pragma unroll
          for (int u = 0; u < KP; ++u) {
            bd[u] = M::load(&sSD[colv(n)][16 * (kk + u) + 4 * g]);
            bs[u] = DIRECT ? s0f[n][kk + u] : M::load(&sSS[colv(n)][16 * (kk + u) + 4 * g]);
          }
          acck[n] = mmk(al, bd, acck[n]);
          accq[n] = mmk(ao, bs, accq[n]);
          acce[n] = mmk(ar, bs, acce[n]);
        }
        if constexpr (SPLIT == 1) {
          // this wave's shared products (dO or dR rows, the same operands)
#pragma unroll
          for (int q2 = 0; q2 < PPW; ++q2) {
            const int pr = wave + q2 * NW;
            frag bl[KP];
#pragma unroll
            for (int u = 0; u < KP; ++u) bl[u] = M::load(&sDL[(DIRECT ? 16 * (pr >> 1) : 0) + c16][cc + 16 * u]);
            gacc[q2] = mmk((pr & 1) ? ar : ao, bl, gacc[q2]);
          }
        }
      }
    }
    if constexpr (SPLIT > 1) {
      // (column passes: the products over the whole of dv, from the rows in LDS)
#pragma unroll
      for (int q2 = 0; q2 < PPW; ++q2) {
        const int pr = wave + q2 * NW;
        const TC (*xr)[PV] = (pr & 1) ? sDR : sDO;
#pragma unroll
        for (int kk = 0; kk < DV / 16; kk += 2) {
          const TC* dl = &sDL[(DIRECT ? 16 * (pr >> 1) : 0) + c16][16 * kk + 4 * g];
          gacc[q2] = M::mma2(M::load(&xr[c16][16 * kk + 4 * g]), M::load(dl), M::load(&xr[c16][16 * kk + 16 + 4 * g]),
                             M::load(dl + 16), gacc[q2]);
        }
      }
    }
#pragma unroll
    for (int q2 = 0; q2 < PPW; ++q2) {
      // lane (g, c16) of product pr: x_{4g+i} . Delta_{c16}, x = dO (pr even) or
      // dR rows, the deltas of block pr/2 of the span (direct forms) or of this block
      const int pr = wave + q2 * NW;
      const int x = pr & 1;
      const int I = DIRECT ? pr >> 1 : jl;
      if (pr < np) {
        if (I == jl) {
          // leaf triangle: t <= r for dO, t < r for dR (negated in the t-row copy)
          f32x4 gm, gt;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            const bool keep = x ? c16 < r : c16 <= r;
            gm[i] = keep ? gacc[q2][i] : 0.f;
            gt[i] = keep ? (x ? -gacc[q2][i] : gacc[q2][i]) : 0.f;
          }
          store4(&sGT[x][c16][4 * g], gt);
          store4(&sGd[x][c16][4 * g], turn(gm));
        } else {
          store4(&sGh[x][DIRECT ? I : 0][c16][4 * g], turn(gacc[q2]));
        }
      }
    }
    __syncthreads();  // the shared products
    if constexpr (DIRECT) {
      // d(qt), d(ek) boundary parts with S_J in place of S0:
      //   S_J = exp(B_J) S0 + sum_{I<J} diag(exp(B_J - B_{I+1})) Ke_I^T Delta_I,
      // so each row x of dO_J, dR_J takes, in Horner form over the earlier
      // blocks I, acc <- exp(B_{I+1} - B_I) acc + (x . Delta_t) Ke_I[t] (every factor <= 1)
#pragma unroll
      for (int I = 0; I < NBS - 1; ++I) {
        if (I < jl) {
          const frag mqf = M::load(&sGh[0][I][c16][4 * g]);  // rows r, contraction over block I's tokens
          const frag mef = M::load(&sGh[1][I][c16][4 * g]);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const float gb = sGH[I][colv(n)];
            accq[n] = M::mma(mqf, keH[I][n], accq[n] * gb);
            acce[n] = M::mma(mef, keH[I][n], acce[n] * gb);
          }
        }
      }
    }
    // log-decay sums at the output mapping (per-token factors and leaf operands)
    float oloc[NT][4], osuf[NT][4];
#pragma unroll
    for (int n = 0; n < NT; ++n) out_sums(n, oloc[n], osuf[n]);
    // Leaf parts
    if (safe) {
      // rows i on lanes, contraction over r:  (dO_r . Delta_i) Yhat_r, r >= i;  -(dR_r . Delta_i) Xhat_r, r > i
      // rows r on lanes, contraction over i:  (Delta_i . dO_r) Z_i, i <= r;  (Delta_i . dR_r) Z_i, i < r
      // with Yhat = qt exp(Lam - B_{J+1}), Xhat = ek exp(Lam - B_{J+1}), Z = k exp(B_J - Lam)
      // (>= 1, within LEAF_SAFE_RANGE) built at the lane's (tokens 4g+i, channel colv(n))
      const frag l0f = M::load(&sGT[0][c16][4 * g]), l1f = M::load(&sGT[1][c16][4 * g]);
      const frag m0f = M::load(&sGd[0][c16][4 * g]), m1f = M::load(&sGd[1][c16][4 * g]);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        f32x4 yh, xh, zz;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ie = __expf(-osuf[n][i]);
          yh[i] = og[n][i] * oq[n][i] * ie;
          xh[i] = oe[n][i] * ok[n][i] * ie;
          zz[i] = ok[n][i] * __expf(-oloc[n][i]);
        }
        const frag zb = M::from_f32(zz);
        acck[n] = M::mma2(l0f, M::from_f32(yh), l1f, M::from_f32(xh), acck[n]);
        accq[n] = M::mma(m0f, zb, accq[n]);
        acce[n] = M::mma(m1f, zb, acce[n]);
      }
    } else {
      if (wave == 0) leaf_dot(sDO, dlJ, false, sLf[0]);      // dO_r . Delta_i, i <= r
      if (wave == 1 % NW) leaf_dot(sDR, dlJ, true, sLf[1]);  // dR_r . Delta_i, i < r
      __syncthreads();
    }
    // per-token gradients; dlog_a as the suffix sum of dLam
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int j = colv(n);
      float dl[4];
      f32x4 gq, gg, ge, gk, gl;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int t = 4 * g + ii;  // token of the block
        const float fs = __expf(oloc[n][ii]);          // exp(Lam_t - B_J)
        float vk = __expf(osuf[n][ii]) * acck[n][ii];  // d(k)_t
        float vq = fs * accq[n][ii];                   // d(qt)_t
        float ve = fs * acce[n][ii];                   // -d(ek)_t
        if (!safe) {
          for (int r = t; r < 16; ++r) {
            const float f = pair_factor(r0, r, t, j);
            const uint32_t orj = gi(r0 + r, j);
            const float qt = gam(r0 + r, j) * ldv(qb, orj);
            const float ek = ldv(eb, orj) * ldv(kb, orj);
            vk += f * (sLf[0][r][t] * qt - sLf[1][r][t] * ek);
          }
          for (int i2 = 0; i2 <= t; ++i2) {
            const float f = pair_factor(r0, t, i2, j) * ldv(kb, gi(r0 + i2, j));
            vq += sLf[0][t][i2] * f;
            ve += sLf[1][t][i2] * f;
          }
        }
        const float dek = -ve;
        gq[ii] = og[n][ii] * vq;
        gg[ii] = oq[n][ii] * vq;
        ge[ii] = ok[n][ii] * dek;
        gk[ii] = vk + oe[n][ii] * dek;
        dl[ii] = oe[n][ii] * ok[n][ii] * dek + og[n][ii] * oq[n][ii] * vq - ok[n][ii] * vk;
      }
      // suffix sums over the block's tokens (4g..4g+3 in this lane, the other
      // token groups in lanes c16 + 16g')
      const float tsum = dl[0] + dl[1] + dl[2] + dl[3];
      const float t0 = __shfl(tsum, c16, 64);
      const float t1 = __shfl(tsum, c16 + 16, 64);
      const float t2 = __shfl(tsum, c16 + 32, 64);
      const float t3 = __shfl(tsum, c16 + 48, 64);
      float run = carry[n] + (g < 3 ? t3 : 0.f) + (g < 2 ? t2 : 0.f) + (g < 1 ? t1 : 0.f);
#pragma unroll
      for (int ii = 3; ii >= 0; --ii) {
        run += dl[ii];
        gl[ii] = run;
      }
      carry[n] += t0 + t1 + t2 + t3;
      store_grad(dqb, r0, n, gq);
      if constexpr (GTOK) store_grad(dgb, r0, n, gg);
      gsum[n] += (gg[0] + gg[1]) + (gg[2] + gg[3]);
      store_grad(deb, r0, n, ge);
      store_grad(dkb, r0, n, gk);
      store_grad(dlb, r0, n, gl);
    }
    if constexpr (!DIRECT) prefetch_r_out(J > 0 ? J - 1 : 0);
    // D <- diag(exp(B_{J+1} - B_J)) D + Y_J^T dO_J - X_J^T dR_J
    {
      frag dRf[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) dRf[n] = M::from_f32(-dRn[n]);
#pragma unroll
      for (int s = 0; s < RT; ++s) {
        const frag ya = M::load(&sTB[16 * s + c16][4 * g]);
        const frag xa = M::load(&sTA[16 * s + c16][4 * g]);
        const f32x4 gs = decay_scale(s);
#pragma unroll
        for (int n = 0; n < NT; ++n) D[s][n] = M::mma2(ya, dOf[n], xa, dRf[n], D[s][n] * gs);
      }
    }
    if (NIB == 2 && J > 0) store_in((J - 1) % NIB);  // the other buffer: its last reader was block J+1
    __syncthreads();
    if (NIB == 1 && DIRECT && J > 0) {
      store_in(0);  // the next block's inputs (every read of this block's is done)
      __syncthreads();
    }
  }
  if (gmode == GAMMA_STATIC) {
    // the chunk's sum of dgamma per key channel (lanes c16 + 16g' hold the token groups)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float t0 = __shfl(gsum[n], c16, 64), t1 = __shfl(gsum[n], c16 + 16, 64);
      const float t2 = __shfl(gsum[n], c16 + 32, 64), t3 = __shfl(gsum[n], c16 + 48, 64);
      if (g == 0) dgam_part[static_cast<size_t>(chunk) * DK + colv(n)] = ((t0 + t1) + t2) + t3;
    }
  }
}

}  // namespace

size_t bwd_chunk_scratch_bytes(const ChunkShape& s) {
  if (!s.bf16) return bwd_scratch_bytes_tc<float, BWD_TWO_SWEEP>(s.C, s.DK, s.DV);
  return s.C == 64 ? bwd_scratch_bytes_tc<uint16_t, BWD_DIRECT>(s.C, s.DK, s.DV)
                   : bwd_scratch_bytes_tc<uint16_t, BWD_SUB>(s.C, s.DK, s.DV);
}

hipError_t launch_bwd_chunk(const ChunkShape& s, const void* q, const void* k, const void* v,
                            const void* log_a, const void* erase, const void* write,
                            const void* gamma, const void* summ, const void* S_chunks,
                            const void* dS_chunks, const void* dO, void* dq, void* dk, void* dv,
                            void* dlog_a, void* derase, void* dwrite, void* dgamma, void* scratch,
                            float* dgam_part,
                            hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(s.nchunks());
  if (grid == 0) return hipSuccess;
#define MUIR_BCH2(TT, TG, DD, CC, NW, FORM, GT, PK)                                                          \
  hipLaunchKernelGGL((bwd_chunk_kernel<TT, TG, DD, CC, NW, FORM, GT, PK>), dim3(grid), dim3(64 * NW), 0, stream, s.T, \
                     s.H, (const TT*)q, (const TT*)k, (const TT*)v, (const TT*)log_a, (const TT*)erase,        \
                     (const TT*)write, (const TT*)gamma, (const char*)summ, s.summary_bytes(), s.tp_offset(),    \
                     s.dl_offset(), (const TT*)S_chunks, (const TT*)dS_chunks, (const TT*)dO, (TG*)dq, (TG*)dk,  \
                     (TG*)dv, (TG*)dlog_a, (TG*)derase, (TG*)dwrite, (TG*)dgamma, (char*)scratch, s.gmode,       \
                     dgam_part, s.ncu, s.cu, s.docoff, s.cinfo)
#define MUIR_BCH1(TT, TG, DD, CC, NW, FORM, PK)                              \
  do {                                                                       \
    if (s.gmode == GAMMA_TOKEN) MUIR_BCH2(TT, TG, DD, CC, NW, FORM, true, PK); \
    else MUIR_BCH2(TT, TG, DD, CC, NW, FORM, false, PK);                     \
  } while (0)
#define MUIR_BCH(TT, TG, DD, NW, F64, FL, PK)                    \
  do {                                                           \
    if (s.C == 64) MUIR_BCH1(TT, TG, DD, 64, NW, F64, PK);       \
    else if (s.C == 128) MUIR_BCH1(TT, TG, DD, 128, NW, FL, PK); \
    else MUIR_BCH1(TT, TG, DD, 256, NW, FL, PK);                 \
  } while (0)
  // one 16-column tile per wave: 8 waves at d = 128, 4 at d = 64; bf16 inputs
  // take the direct forms (their chunk deltas are kept by the forward scan,
  // ChunkShape::bwd_direct), fp32 inputs the two sweeps
  // (packed-document output straight to the caller's tensors: bf16 inputs
  // at d = 128 only; packed_output() tells the caller)
  const bool pko = s.docoff && s.bf16 && s.DK == 128;
  if (s.bf16 && s.gbf16) {
    if (s.DK == 128 && pko) MUIR_BCH(uint16_t, uint16_t, 128, 8, BWD_DIRECT, BWD_SUB, true);
    else if (s.DK == 128) MUIR_BCH(uint16_t, uint16_t, 128, 8, BWD_DIRECT, BWD_SUB, false);
    else MUIR_BCH(uint16_t, uint16_t, 64, 4, BWD_DIRECT, BWD_SUB, false);
  } else if (s.bf16) {
    if (s.DK == 128 && pko) MUIR_BCH(uint16_t, float, 128, 8, BWD_DIRECT, BWD_SUB, true);
    else if (s.DK == 128) MUIR_BCH(uint16_t, float, 128, 8, BWD_DIRECT, BWD_SUB, false);
    else MUIR_BCH(uint16_t, float, 64, 4, BWD_DIRECT, BWD_SUB, false);
  } else {
    if (s.DK == 128) MUIR_BCH(float, float, 128, 8, BWD_TWO_SWEEP, BWD_TWO_SWEEP, false);
    else MUIR_BCH(float, float, 64, 4, BWD_TWO_SWEEP, BWD_TWO_SWEEP, false);
  }
#undef MUIR_BCH
#undef MUIR_BCH1
#undef MUIR_BCH2
  return hipGetLastError();
}

namespace {
// dgamma of a static readout gate: per (head, key channel), the sum of the
// per-chunk partial sums over the batch and the chunks, in a fixed order.  A
// block takes 32 consecutive (head, channel) columns; the B*NC partials of
// each are split over 8 thread groups (rows r = grp, grp + 8, ...), each
// summing into four interleaved accumulators so that its loads stay in
// flight together, and the groups' sums are added in LDS in group order.
// (One thread per column summing its partials in sequence took about 150 us
// at the 4K layer: 512 dependent steps on 8 workgroups.)
__global__ __launch_bounds__(256) void gamma_sum_kernel(int B, int H, int NC, int DK,
                                                        const float* __restrict__ part,
                                                        float* __restrict__ dgamma) {
  __shared__ float red[8][32];
  const int jl = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int col = blockIdx.x * 32 + jl;
  const bool ok = col < H * DK;
  const int h = ok ? col / DK : 0;
  const int j = ok ? col - h * DK : 0;
  const int n = B * NC;  // partial row r = b NC + c at part[((b H + h) NC + c) DK + j]
  auto P = [&](int r) -> float {
    const int b = r / NC;
    const int c = r - b * NC;
    return part[((static_cast<size_t>(b) * H + h) * NC + c) * DK + j];
  };
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int r = grp;
  if (ok) {
    for (; r + 24 < n; r += 32) {
      a0 += P(r);
      a1 += P(r + 8);
      a2 += P(r + 16);
      a3 += P(r + 24);
    }
    for (; r < n; r += 8) a0 += P(r);
  }
  red[grp][jl] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (grp == 0 && ok) {
    float acc = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < 8; ++g2) acc += red[g2][jl];
    dgamma[col] = acc;
  }
}
}  // namespace

hipError_t launch_gamma_sum(const ChunkShape& s, const float* part, float* dgamma, hipStream_t stream) {
  const int n = s.H * s.DK;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gamma_sum_kernel, dim3((n + 31) / 32), dim3(256), 0, stream, s.B, s.H, s.NC(), s.DK, part,
                     dgamma);
  return hipGetLastError();
}

}  // namespace muir
