// Host-side launchers of the Muir HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace muir {

// Sizes and derived quantities of one chunkwise call, validated by the API.
struct ChunkShape {
  int B, T, H, DK, DV, C;
  bool bf16;
  int NC() const { return T / C; }
  size_t nchunks() const { return static_cast<size_t>(B) * H * NC(); }
  size_t tc_bytes() const { return bf16 ? 2 : 4; }
  // Per-chunk block of the forward intermediates ("chunk summary"):
  //   W  [C][DK], Qp [C][DK], Kb^T [DK][C], Ut^T [DV][C], Ot^T [DV][C] (compute type)
  //   gC [DK] fp32
  size_t summary_elems() const { return static_cast<size_t>(C) * (3 * DK + 2 * DV); }
  size_t summary_bytes() const {
    size_t b = summary_elems() * tc_bytes() + static_cast<size_t>(DK) * 4;
    return (b + 255) & ~static_cast<size_t>(255);
  }
  size_t state_bytes() const { return static_cast<size_t>(DK) * DV * 4; }
};

hipError_t launch_step(int N, int H, int dk, int dv, bool bf16, const void* q, const void* k,
                       const void* v, const void* log_a, const void* erase, const void* write,
                       const void* gamma, float* S, void* o, hipStream_t stream);

// Chunk-parallel: per chunk summary (W, Q', Kbar, U~, O~, Gamma_C) into `summ`.
// bwd_layout: W, Q' token-contiguous and Kbar channel-contiguous (what the
// backward scan reads); U~ and O~ are then not written.
hipError_t launch_fwd_prep(const ChunkShape& s, const void* q, const void* k, const void* v,
                           const void* log_a, const void* erase, const void* write,
                           const void* gamma, void* summ, bool bwd_layout, hipStream_t stream);

// Sequential over chunks: o (may be NULL), S_chunks (may be NULL), S_T (may be NULL).
hipError_t launch_fwd_scan(const ChunkShape& s, const void* summ, const float* S0, void* o,
                           float* S_chunks, float* S_T, hipStream_t stream);

// Reverse sequential over chunks: dS_chunks[c] = gradient w.r.t. the state at the
// END of chunk c; dS0 (may be NULL).
hipError_t launch_bwd_scan(const ChunkShape& s, const void* summ, const void* dO,
                           const float* dS_T, float* dS_chunks, float* dS0, hipStream_t stream);

// Chunk-parallel: all input gradients of every chunk.  `scratch` holds
// bwd_chunk_scratch_bytes(s) per chunk (the chunk's deltas, their gradients
// and its leaf inverses).
size_t bwd_chunk_scratch_bytes(const ChunkShape& s);
hipError_t launch_bwd_chunk(const ChunkShape& s, const void* q, const void* k, const void* v,
                            const void* log_a, const void* erase, const void* write,
                            const void* gamma, const float* S_chunks, const float* dS_chunks,
                            const void* dO, float* dq, float* dk, float* dv, float* dlog_a,
                            float* derase, float* dwrite, float* dgamma, void* scratch,
                            hipStream_t stream);

}  // namespace muir
