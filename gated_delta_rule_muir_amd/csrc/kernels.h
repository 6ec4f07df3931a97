// Host-side launchers of the Muir HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace muir {

// Parts of a chunk summary, in order; offsets in compute-type elements.
//   W [C][DK], Q' [C][DK], Kbar^T [DK][C], U~^T [DV][C], O~^T [DV][C]
// (the forward scan's orientations; the reverse scan contracts W, Q' and
// Kbar the other way and reads them transposed from LDS), then Gamma_C [DK] fp32, the
// leaf blocks T_II, P_II [C/16][2][16][16] (compute type) and the chunk's
// deltas U~ - W S [C][DV] (compute type; written by the forward scan when it
// saves the chunk states and the direct backward is used, see bwd_direct).
enum SummaryPart { SP_W, SP_QP, SP_KBT, SP_UTT, SP_OTT, SP_END };
__host__ __device__ constexpr size_t summary_part(int part, int C, int DK, int DV) {
  return part <= SP_UTT ? static_cast<size_t>(part) * C * DK
                        : static_cast<size_t>(3) * C * DK + static_cast<size_t>(part - SP_UTT) * C * DV;
}

// The transposed parts (Kbar^T, U~^T, O~^T: logically [D][C]) are
// stored as 16-token tiles [C/16][D][16], so that each 16-token block's tile
// is one contiguous run: element (row d, token t) is at this index.
__host__ __device__ constexpr uint32_t tpart_index(int d, int t, int D) {
  return (static_cast<uint32_t>(t >> 4) * static_cast<uint32_t>(D) + static_cast<uint32_t>(d)) * 16u +
         static_cast<uint32_t>(t & 15);
}

// A state kept for the backward (the chunk-start states S_chunks, and the
// backward's own sub-chunk start states) is stored as 16 x 16 tiles, row-major
// within a tile and tile-row-major over the state: element (r, j) of a
// [DK][DV] state is at this index.  Every access to these states (a lane's
// four consecutive columns of one row, for 16 rows and 16 columns at a time)
// then covers one contiguous 512-byte tile (bf16) instead of 32-byte pieces
// of 16 rows.
__host__ __device__ constexpr uint32_t stile_index(int r, int j, int DV) {
  return (static_cast<uint32_t>(r >> 4) * static_cast<uint32_t>(DV >> 4) + static_cast<uint32_t>(j >> 4)) * 256u +
         static_cast<uint32_t>(r & 15) * 16u + static_cast<uint32_t>(j & 15);
}

// Readout-gate forms: per token [B, T, H, dk]; static per (head, key channel)
// [H, dk]; none (gamma = 1, no pointer).
enum GammaMode { GAMMA_TOKEN = 0, GAMMA_STATIC = 1, GAMMA_NONE = 2 };

// Packed documents (variable-length calls) run as one sequence (B = 1) in
// which each document starts at a chunk boundary.  Per chunk of that
// sequence, cinfo holds the document's index (CI_DOC bits) and whether the
// chunk is the document's first (CI_START: the scans start the state from
// the document's S0, and the reverse scan cuts the gradient flowing into the
// chunk before it) or last (CI_END: the forward scan writes the document's
// S_T there, and the reverse scan starts the gradient from its dS_T).
constexpr int32_t CI_DOC = (1 << 29) - 1;
constexpr int32_t CI_START = 1 << 29;
constexpr int32_t CI_END = 1 << 30;

// Sizes and derived quantities of one chunkwise call, validated by the API.
struct ChunkShape {
  int B, T, H, DK, DV, C;
  bool bf16;
  bool gbf16;  // per-token gradients in bf16 (else fp32)
  int gmode;   // GammaMode
  // Packed documents only (else NULL): the per-chunk document table above,
  // and the number of chunks in use (device memory; the chunks past it, which
  // the launch sizes still count, are skipped by every kernel).  S0, S_T,
  // dS_T and dS0 are then per document, [N, H, dk, dv].
  const int32_t* cinfo = nullptr;
  const int32_t* ncu = nullptr;
  // Packed documents whose per-token gradients the chunk kernel writes
  // straight to the caller's packed tensors (packed_output()): the caller's
  // cu_seqlens and each document's first row in the packed sequence.
  const int32_t* cu = nullptr;
  const int32_t* docoff = nullptr;
  bool packed_output() const { return cinfo && bf16 && DK == 128; }
  // chunks per sequence, a partial last one included (the kernels only ever
  // run on shapes whose T is a multiple of C)
  int NC() const { return (T + C - 1) / C; }
  size_t nchunks() const { return static_cast<size_t>(B) * H * NC(); }
  size_t tc_bytes() const { return bf16 ? 2 : 4; }
  size_t tg_bytes() const { return gbf16 ? 2 : 4; }  // one per-token gradient element
  // Per-chunk block of the forward intermediates ("chunk summary"), see SummaryPart.
  size_t summary_elems() const { return summary_part(SP_END, C, DK, DV); }
  size_t gc_offset() const { return summary_elems() * tc_bytes(); }
  size_t tp_offset() const { return gc_offset() + static_cast<size_t>(DK) * 4; }
  size_t dl_offset() const { return tp_offset() + static_cast<size_t>(C / 16) * 512 * tc_bytes(); }
  size_t summary_bytes() const {
    size_t b = dl_offset() + static_cast<size_t>(C) * DV * tc_bytes();
    return (b + 255) & ~static_cast<size_t>(255);
  }
  size_t state_bytes() const { return static_cast<size_t>(DK) * DV * 4; }
  // The backward takes the chunk's deltas from the forward scan and forms the
  // states inside a chunk from S0 and those deltas (one reverse sweep over
  // its blocks; longer chunks first carry the state over their 64-token
  // sub-chunks), instead of a forward sweep that recomputes both: for bf16,
  // whose tiles then fit the LDS.
  bool bwd_direct() const { return bf16; }
  // Segments of the split scans: 1 when the heads' 64-column scans alone fill
  // the chip; else the sequence is cut into the fewest power-of-two segments
  // that do, with at least 4 chunks each.
  int scan_segments() const {
    const long long cols = static_cast<long long>(B) * H * (DV / 64);
    int n = 1;
    while (cols * n < 256 && NC() / (2 * n) >= 4) n *= 2;
    return n;
  }
  // Workspace of the split scans: per head and segment, the transition and
  // offset [dk][DV + DK] and the segment start [dk][dv], fp32.
  size_t scan_split_bytes() const {
    const int n = scan_segments();
    return n > 1 ? static_cast<size_t>(B) * H * n * DK * (2 * DV + DK) * 4 : 0;
  }
};

hipError_t launch_step(int N, int H, int dk, int dv, bool bf16, int gmode, const void* q,
                       const void* k, const void* v, const void* log_a, const void* erase,
                       const void* write, const void* gamma, float* S, void* o, hipStream_t stream);

// Chunk-parallel: per chunk summary (W, Q', Kbar, U~, O~, Gamma_C and the
// 16-token leaf blocks T_II, P_II) into `summ`.  `gamma` in the form s.gmode
// (unused, and may be NULL, for GAMMA_NONE).
hipError_t launch_fwd_prep(const ChunkShape& s, const void* q, const void* k, const void* v,
                           const void* log_a, const void* erase, const void* write,
                           const void* gamma, void* summ, hipStream_t stream);

// Sequential over chunks: o (may be NULL), S_chunks (may be NULL: the
// chunk-start states in the compute type, as 16 x 16 tiles, stile_index),
// S_T (may be NULL).  With `deltas` (the same summaries, writable) each
// chunk's deltas are written into its summary.  `split`: scan_split_bytes(s)
// of workspace; when the scan splits into segments it starts with each
// segment's offset and transition, [dk][dv + dk] fp32 per head and segment,
// which the reverse scan reads (ftrans).
hipError_t launch_fwd_scan(const ChunkShape& s, const void* summ, const float* S0, void* o,
                           void* S_chunks, float* S_T, void* deltas, float* split, hipStream_t stream);

// Only the segment transitions of launch_fwd_scan (into the start of
// `split`); nothing when the scan does not split.
hipError_t launch_fwd_trans(const ChunkShape& s, const void* summ, float* split, hipStream_t stream);

// Reverse sequential over chunks: dS_chunks[c] = gradient w.r.t. the state at the
// END of chunk c, in the compute type, as transposed 16-row tiles: element
// (r, j) at ((r / 16) * DV + j) * 16 + r % 16 of the chunk's DK * DV block;
// dS0 (fp32 [dk][dv], may be NULL).  When the scan splits into segments,
// `ftrans` holds the forward's segment transitions (the start of the split
// area of a launch_fwd_scan or launch_fwd_trans on the same summaries; it may
// be `split` itself, whose transition columns this call leaves unchanged).
hipError_t launch_bwd_scan(const ChunkShape& s, const void* summ, const void* dO,
                           const float* dS_T, void* dS_chunks, float* dS0, float* split,
                           const float* ftrans, hipStream_t stream);

// Chunk-parallel: all input gradients of every chunk (per-token ones in the
// element type s.gbf16 selects).  `summ` holds the
// chunk summaries (their leaf blocks are read; with bwd_direct also Kbar^T,
// Gamma_C and the deltas); `scratch` holds bwd_chunk_scratch_bytes(s) per
// chunk (the deltas and block-start states of the forward sweep; none with
// bwd_direct).
size_t bwd_chunk_scratch_bytes(const ChunkShape& s);
hipError_t launch_bwd_chunk(const ChunkShape& s, const void* q, const void* k, const void* v,
                            const void* log_a, const void* erase, const void* write,
                            const void* gamma, const void* summ, const void* S_chunks,
                            const void* dS_chunks,
                            const void* dO, void* dq, void* dk, void* dv, void* dlog_a,
                            void* derase, void* dwrite, void* dgamma, void* scratch,
                            float* dgam_part, hipStream_t stream);

// dgamma [H][dk] fp32 of a static readout gate from bwd_chunk's per-chunk
// partial sums ([nchunks][dk] fp32).
hipError_t launch_gamma_sum(const ChunkShape& s, const float* part, float* dgamma, hipStream_t stream);

// ---- gate prologue ---------------------------------------------------------------

// Channels of the shared down-projection (the five gate ranks 64 + 64 + 128 +
// 128 + 128) and the guard of the q / k L2 normalisation.
constexpr int GATE_RTOT = 512;
constexpr float QK_L2_EPS = 1e-6f;
enum GateAct { GATE_ACT_NONE = 0, GATE_ACT_LOGSIG = 1, GATE_ACT_SIG = 2, GATE_ACT_SIG2 = 3 };

// One product C = A B of a grouped GEMM launch (elements; A is M x K, B is
// K x N; the kernel instance fixes whether each operand is read along k or
// across it).
struct GemmProblem {
  const void* A;
  const void* B;
  void* C;
  int M, N, K;
  int lda, ldb, ldc;
};
struct GemmBatch {
  GemmProblem p[5];
  int n;                // problems in the launch
  int ksplit;           // splits of the contraction (fp32 partials)
  int kchunk;           // contraction length per split
  size_t split_stride;  // floats between the partials of consecutive splits
};

// Sizes of a gate-prologue call: M tokens of width d; H heads of dk key and
// dv value channels.
struct GateShape {
  int M, d, H, dk, dv;
  bool bf16;
};
// Backward workspace: recomputed z, dpre of the five gates (fp32 only), dz, split
// partials of the weight gradients and the bias gradient's partial column sums
// (per 128-token tile for fp32, per split for bf16).
struct GateWorkspace {
  size_t z_off, dpre_off, dz_off, part_off, colsum_off, bytes;
  size_t part_stride;
  int ksplit, kchunk, mtiles, colsum_ld;
  int dw_ksplit, dw_kchunk;  // the split of the bf16 weight-gradient kernel
};
GateWorkspace gate_workspace(const GateShape& s);
// Elements of the packed up-projection weights (sum of rank x width).
size_t gate_up_numel(const GateShape& s);
hipError_t launch_gate_fwd(const GateShape& s, const void* x, const void* W_down, const void* W_up,
                           const void* bias, void* z, void* const gates[5], hipStream_t stream);
hipError_t launch_gate_bwd(const GateShape& s, const void* x, const void* W_down, const void* W_up,
                           const void* bias, const void* z, const void* const dgates[5], void* dx,
                           float* dW_down, float* dW_up, float* dbias, void* workspace, hipStream_t stream);
// SiLU + L2 over rows of D in {64, 128} values: forward (dy == NULL, out = y)
// or reverse (out = du).
hipError_t launch_qk_norm(long long rows, int D, bool bf16, const void* u, const void* dy, void* out,
                          hipStream_t stream);

}  // namespace muir
