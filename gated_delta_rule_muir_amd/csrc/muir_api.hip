// C ABI of the Muir operator: argument validation, workspace sizing and
// kernel dispatch.  Every entry point checks its arguments before launching
// anything and never allocates, frees or synchronises.
#include <muir.h>

#include <mutex>

#include "kernels.h"

using muir::ChunkShape;
using muir::CI_DOC;
using muir::CI_END;
using muir::CI_START;

// Workspace of the no-allocation forward (muir_chunk_fwd_noalloc): one array
// per GPU, in the library's code object.  Host code never uses this name as
// an address (on the host it is only a stand-in); it takes the device
// address from hipGetSymbolAddress, once per device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[MUIR_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// `bwd`: the sizes of a backward call, whose per-token gradients are fp32 or,
// for bf16 inputs, bf16 (the forward calls ignore grad_dtype).
muir_status_t check_dims(const muir_dims_t* d, ChunkShape* s, bool bwd = false) {
  if (!d) return MUIR_ERR_NULL;
  if (d->dtype != MUIR_F32 && d->dtype != MUIR_BF16) return MUIR_ERR_DTYPE;
  if (bwd && d->grad_dtype != MUIR_F32 && !(d->grad_dtype == MUIR_BF16 && d->dtype == MUIR_BF16))
    return MUIR_ERR_DTYPE;
  if (d->gamma_mode < MUIR_GAMMA_TOKEN || d->gamma_mode > MUIR_GAMMA_NONE) return MUIR_ERR_MODE;
  if (d->B < 0 || d->T < 0 || d->H < 0) return MUIR_ERR_SHAPE;
  if (d->dk != d->dv || (d->dk != 64 && d->dk != 128)) return MUIR_ERR_SHAPE;
  if (d->chunk != 64 && d->chunk != 128 && d->chunk != 256) return MUIR_ERR_SHAPE;
  const long long nc = (static_cast<long long>(d->T) + d->chunk - 1) / d->chunk;
  // keep every flat index inside 32-bit chunk counts and 64-bit element counts
  if (static_cast<long long>(d->B) * d->H * nc > (1LL << 30)) return MUIR_ERR_SHAPE;
  // the kernels address one chunk of a [B, T, H, D] tensor with 32-bit offsets
  if (static_cast<long long>(d->H) * d->dk * d->chunk * 4 >= (1LL << 31)) return MUIR_ERR_SHAPE;
  s->B = d->B;
  s->T = d->T;
  s->H = d->H;
  s->DK = d->dk;
  s->DV = d->dv;
  s->C = d->chunk;
  s->bf16 = d->dtype == MUIR_BF16;
  s->gbf16 = bwd && d->grad_dtype == MUIR_BF16;
  s->gmode = d->gamma_mode;
  return MUIR_OK;
}

// The shape the kernels run on: T rounded up to whole chunks.  A call whose
// T is not a multiple of the chunk (a tail chunk), and every packed
// variable-length call, runs on zero-padded [N, T_padded, H, D] copies of its
// sequences: a zero token (k = q = v = 0, log_a = 0) leaves the state as it
// is, so the padded run's states and every real token's results are those of
// the unpadded sequence.
ChunkShape padded(const ChunkShape& s) {
  ChunkShape p = s;
  p.T = (s.T + s.C - 1) / s.C * s.C;
  return p;
}

// Forward workspace: the chunk summaries, then the split scan's segment
// transitions and starts (when the shape splits its scan).
size_t fwd_ws(const ChunkShape& s) { return s.nchunks() * s.summary_bytes() + s.scan_split_bytes(); }

// Backward workspace: chunk summaries (used when the caller passes none),
// recomputed chunk states (used when the caller passes no S_chunks), the
// chunk-end state gradients, per-chunk scratch for the deltas and their
// gradients, then the split scans' segment area (shared by the recomputed
// forward scan and the reverse scan, which run one after the other) and a
// static readout gate's per-chunk partial gradients.  Every part is always
// reserved, so the size does not depend on which pointers are passed.
size_t bwd_scratch_bytes(const ChunkShape& s) { return round256(muir::bwd_chunk_scratch_bytes(s)); }
size_t gamma_part_bytes(const ChunkShape& s) { return round256(s.nchunks() * s.DK * 4); }
size_t bwd_ws(const ChunkShape& s) {
  return s.nchunks() * (s.summary_bytes() + 2 * s.state_bytes() + bwd_scratch_bytes(s)) + s.scan_split_bytes() +
         gamma_part_bytes(s);
}

// Staging area of a padded call, after the kernels' workspace: one
// [N, T_padded, H, D] copy per staged tensor -- the inputs (the gate only
// when it is per token) and o, or the inputs, dO and the gradients; inputs,
// o and dO in the compute type, gradients in their own type (esize bytes).
size_t staged_bytes(const ChunkShape& p, int D, size_t esize) {
  return round256(static_cast<size_t>(p.B) * p.T * p.H * D * esize);
}
int staged_dk_inputs(const ChunkShape& p) { return p.gmode == MUIR_GAMMA_TOKEN ? 5 : 4; }  // q, k, log_a, erase, [gamma]
size_t fwd_stage_bytes(const ChunkShape& p) {
  return staged_dk_inputs(p) * staged_bytes(p, p.DK, p.tc_bytes()) + 3 * staged_bytes(p, p.DV, p.tc_bytes());  // + v, write, o
}
size_t bwd_stage_bytes(const ChunkShape& p) {
  return staged_dk_inputs(p) * (staged_bytes(p, p.DK, p.tc_bytes()) + staged_bytes(p, p.DK, p.tg_bytes())) +
         3 * staged_bytes(p, p.DV, p.tc_bytes()) + 2 * staged_bytes(p, p.DV, p.tg_bytes());  // + v, write, dO; dv, dwrite
}

// The readout gate's pointer is required (and checked) unless the gate is absent.
muir_status_t check_gate(const ChunkShape& s, const void* p) {
  if (s.gmode == MUIR_GAMMA_NONE) return MUIR_OK;
  if (!p) return MUIR_ERR_NULL;
  return aligned16(p) ? MUIR_OK : MUIR_ERR_ALIGN;
}

// Optional per-kernel timing: when the caller registers an array of HIP
// events, each entry point records the next event before its first kernel
// and after every kernel it launches, on the caller's stream, until the array
// is used up.  No work is skipped or reordered.
thread_local hipEvent_t* g_events = nullptr;
thread_local int g_nevents = 0;
thread_local int g_cursor = 0;

inline void mark(hipStream_t s) {
  if (g_events && g_cursor < g_nevents) (void)hipEventRecord(g_events[g_cursor++], s);
}

// Copy n floats (or write zeros when src is NULL); used for T == 0, where the
// final state is the initial state.  A kernel rather than a memset so that a
// caller may capture the call in a graph.
__global__ void copy_or_zero_kernel(float* __restrict__ dst, const float* __restrict__ src, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

hipError_t copy_or_zero(float* dst, const float* src, size_t n, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3(blocks), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

// Sequence tensors between their caller layout and the padded layout, in
// 16-byte words (WW per token).  Sequence n's tokens are rows
// cu[n] .. cu[n+1]-1 of a packed [T_total, H, D] tensor when cu is given,
// else rows n*Tsrc .. n*Tsrc + Tsrc-1 of a [N, Tsrc, H, D] tensor; in the
// padded [N, Tp, H, D] copy, rows past a sequence's end are zero.  to_padded:
// caller -> padded (every padded row written); else padded -> caller (the
// real rows only).  A block takes whole rows (grid-stride) and copies each
// row's words with consecutive threads, as pack_kernel does.
__global__ __launch_bounds__(256) void stage_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int N,
                                                    int Tsrc, int Tp, int WW, const int32_t* __restrict__ cu,
                                                    int to_padded) {
  const long long rows = static_cast<long long>(N) * Tp;
  for (long long row = blockIdx.x; row < rows; row += gridDim.x) {
    const int n = static_cast<int>(row / Tp);
    const int t = static_cast<int>(row - static_cast<long long>(n) * Tp);
    const long long start = cu ? cu[n] : static_cast<long long>(n) * Tsrc;
    const int len = cu ? cu[n + 1] - cu[n] : Tsrc;
    const bool real = t < len;
    const size_t crow = static_cast<size_t>(start + t);
    if (to_padded) {
      uint4* o = dst + static_cast<size_t>(row) * WW;
      if (real) {
        const uint4* s = src + crow * WW;
        for (int w = threadIdx.x; w < WW; w += blockDim.x) o[w] = s[w];
      } else {
        const uint4 z = {0u, 0u, 0u, 0u};
        for (int w = threadIdx.x; w < WW; w += blockDim.x) o[w] = z;
      }
    } else if (real) {
      const uint4* s = src + static_cast<size_t>(row) * WW;
      uint4* o = dst + crow * WW;
      for (int w = threadIdx.x; w < WW; w += blockDim.x) o[w] = s[w];
    }
  }
}

hipError_t stage(const void* src, void* dst, const ChunkShape& p, int Tsrc, int D, size_t esize, const int32_t* cu,
                 bool to_padded, hipStream_t s) {
  const int WW = static_cast<int>(static_cast<size_t>(p.H) * D * esize / 16);
  const long long rows = static_cast<long long>(p.B) * p.T;
  if (rows == 0 || WW == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(rows < 8192 ? rows : 8192);
  hipLaunchKernelGGL(stage_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), p.B, Tsrc, p.T, WW, cu, to_padded ? 1 : 0);
  return hipGetLastError();
}

// Pointers of one call: the seven inputs in the caller's order (q, k, v,
// log_a, erase, write, gamma) and the seven gradients (dq, dk, dv, dlog_a,
// derase, dwrite, dgamma); which ones have dk (else dv) channels.
struct Inputs {
  const void* x[7];
};
struct Grads {
  void* x[7];
};
constexpr bool kIsDk[7] = {true, true, false, true, true, false, true};

// The kernels of the forward on a shape whose T is a multiple of the chunk.
muir_status_t fwd_core(const ChunkShape& s, const Inputs& in, const float* S0, void* o, float* S_T,
                       void* S_chunks, void* workspace, hipStream_t hs) {
  mark(hs);
  if (muir::launch_fwd_prep(s, in.x[0], in.x[1], in.x[2], in.x[3], in.x[4], in.x[5], in.x[6], workspace, hs) !=
      hipSuccess)
    return MUIR_ERR_HIP;
  mark(hs);
  // a forward that saves its chunk states keeps the deltas for the direct backward
  void* deltas = S_chunks && s.bwd_direct() ? workspace : nullptr;
  float* split = reinterpret_cast<float*>(static_cast<char*>(workspace) + s.nchunks() * s.summary_bytes());
  if (muir::launch_fwd_scan(s, workspace, S0, o, S_chunks, S_T, deltas, split, hs) != hipSuccess)
    return MUIR_ERR_HIP;
  mark(hs);
  return MUIR_OK;
}

// The kernels of the backward on a shape whose T is a multiple of the chunk.
muir_status_t bwd_core(const ChunkShape& s, const Inputs& in, const float* S0, const void* S_chunks,
                       const void* summaries, const void* dO, const float* dS_T, const Grads& gr, float* dS0,
                       void* workspace, hipStream_t hs) {
  char* ws = static_cast<char*>(workspace);
  float* S_rec = reinterpret_cast<float*>(ws + s.nchunks() * s.summary_bytes());
  float* dS_chunks = S_rec + s.nchunks() * static_cast<size_t>(s.DK) * s.DV;
  float* chunk_scratch = dS_chunks + s.nchunks() * static_cast<size_t>(s.DK) * s.DV;
  float* split = reinterpret_cast<float*>(reinterpret_cast<char*>(chunk_scratch) + s.nchunks() * bwd_scratch_bytes(s));
  float* gpart = reinterpret_cast<float*>(reinterpret_cast<char*>(split) + s.scan_split_bytes());
  const void* Sc = S_chunks;
  const void* summ = summaries;
  mark(hs);
  // The direct backward reads the deltas that the forward scan keeps in the
  // summaries when it saves the chunk states: both are taken from one forward
  // call, or both recomputed here.
  if (s.bwd_direct() && !(summ && Sc)) {
    summ = nullptr;
    Sc = nullptr;
  }
  // A split reverse scan takes the forward's segment transitions: from the
  // forward's workspace (after its summaries) when that is given, else from
  // the forward scan rerun here, else formed here on their own.
  const float* ftrans =
      summ ? reinterpret_cast<const float*>(static_cast<const char*>(summ) + s.nchunks() * s.summary_bytes())
           : split;
  if (!summ) {
    // the forward's chunk summaries are not given: recompute them
    if (muir::launch_fwd_prep(s, in.x[0], in.x[1], in.x[2], in.x[3], in.x[4], in.x[5], in.x[6], ws, hs) !=
        hipSuccess)
      return MUIR_ERR_HIP;
    mark(hs);
    summ = ws;
    if (Sc && muir::launch_fwd_trans(s, summ, split, hs) != hipSuccess) return MUIR_ERR_HIP;
  }
  if (!Sc) {
    // chunk-start states are not given: rerun the forward scan (it leaves
    // the segment transitions in `split`)
    void* deltas = s.bwd_direct() ? ws : nullptr;  // summ is ws here
    if (muir::launch_fwd_scan(s, summ, S0, nullptr, S_rec, nullptr, deltas, split, hs) != hipSuccess)
      return MUIR_ERR_HIP;
    mark(hs);
    Sc = S_rec;
    ftrans = split;
  }
  if (muir::launch_bwd_scan(s, summ, dO, dS_T, dS_chunks, dS0, split, ftrans, hs) != hipSuccess)
    return MUIR_ERR_HIP;
  mark(hs);
  if (muir::launch_bwd_chunk(s, in.x[0], in.x[1], in.x[2], in.x[3], in.x[4], in.x[5], in.x[6], summ, Sc,
                             dS_chunks, dO, gr.x[0], gr.x[1], gr.x[2], gr.x[3], gr.x[4], gr.x[5], gr.x[6],
                             chunk_scratch, gpart, hs) != hipSuccess)
    return MUIR_ERR_HIP;
  if (s.gmode == MUIR_GAMMA_STATIC &&
      muir::launch_gamma_sum(s, gpart, static_cast<float*>(gr.x[6]), hs) != hipSuccess)
    return MUIR_ERR_HIP;
  mark(hs);
  return MUIR_OK;
}

// Carves the staged tensors out of the staging area, in call order.
struct StageCursor {
  char* p;
  void* take(const ChunkShape& ps, int D, size_t esize) {
    void* r = p;
    p += staged_bytes(ps, D, esize);
    return r;
  }
};

// Copies the caller's inputs into padded tensors carved from `cur`.
muir_status_t stage_inputs(const ChunkShape& p, int Tsrc, const int32_t* cu, const Inputs& in, Inputs* out,
                           StageCursor* cur, hipStream_t hs) {
  for (int i = 0; i < 7; ++i) {
    if (i == 6 && p.gmode != MUIR_GAMMA_TOKEN) {
      out->x[6] = in.x[6];  // a static gate is [H, dk] and needs no staging; an absent one is not read
      continue;
    }
    const int D = kIsDk[i] ? p.DK : p.DV;
    void* dst = cur->take(p, D, p.tc_bytes());
    if (stage(in.x[i], dst, p, Tsrc, D, p.tc_bytes(), cu, true, hs) != hipSuccess) return MUIR_ERR_HIP;
    out->x[i] = dst;
  }
  return MUIR_OK;
}

// The tensors of a forward call (the workspace is checked by check_workspace).
muir_status_t check_fwd_tensors(const ChunkShape& s, const Inputs& in, const float* S0, const void* o,
                                const float* S_T, const void* S_chunks) {
  muir_status_t st;
  if (s.nchunks() != 0) {
    for (int i = 0; i < 6; ++i)
      if (!in.x[i]) return MUIR_ERR_NULL;
    if (!o) return MUIR_ERR_NULL;
    for (int i = 0; i < 6; ++i)
      if (!aligned16(in.x[i])) return MUIR_ERR_ALIGN;
    if (!aligned16(o)) return MUIR_ERR_ALIGN;
    if ((st = check_gate(s, in.x[6])) != MUIR_OK) return st;
  }
  const void* opt[] = {S0, S_T, S_chunks};
  for (const void* p : opt)
    if (p && !aligned16(p)) return MUIR_ERR_ALIGN;
  return MUIR_OK;
}

// A caller's workspace, needed whenever there are chunks to run.
muir_status_t check_workspace(const ChunkShape& s, const void* workspace, size_t workspace_bytes, size_t need) {
  if (s.nchunks() == 0) return MUIR_OK;
  if (!workspace || workspace_bytes < need) return MUIR_ERR_WORKSPACE;
  return aligned16(workspace) ? MUIR_OK : MUIR_ERR_ALIGN;
}

muir_status_t check_fwd_args(const ChunkShape& s, const Inputs& in, const float* S0, const void* o, const float* S_T,
                             const void* S_chunks, const void* workspace, size_t workspace_bytes, size_t need) {
  const muir_status_t st = check_fwd_tensors(s, in, S0, o, S_T, S_chunks);
  return st != MUIR_OK ? st : check_workspace(s, workspace, workspace_bytes, need);
}

muir_status_t check_bwd_args(const ChunkShape& s, const Inputs& in, const float* S0, const void* S_chunks,
                             const void* summaries, const void* dO, const float* dS_T, const Grads& gr,
                             const float* dS0, const void* workspace, size_t workspace_bytes, size_t need) {
  muir_status_t st;
  if (s.nchunks() != 0) {
    for (int i = 0; i < 6; ++i)
      if (!in.x[i] || !gr.x[i]) return MUIR_ERR_NULL;
    if (!dO) return MUIR_ERR_NULL;
    for (int i = 0; i < 6; ++i)
      if (!aligned16(in.x[i]) || !aligned16(gr.x[i])) return MUIR_ERR_ALIGN;
    if (!aligned16(dO)) return MUIR_ERR_ALIGN;
    if ((st = check_gate(s, in.x[6])) != MUIR_OK) return st;
    if ((st = check_gate(s, gr.x[6])) != MUIR_OK) return st;
    if (!workspace || workspace_bytes < need) return MUIR_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MUIR_ERR_ALIGN;
  }
  const void* opt[] = {S0, S_chunks, summaries, dS_T, dS0};
  for (const void* p : opt)
    if (p && !aligned16(p)) return MUIR_ERR_ALIGN;
  return MUIR_OK;
}

// No tokens (T == 0, or no sequences): the final state is the initial state,
// the initial state's gradient is the final state's, and a static gate's
// gradient is a sum over no tokens.
muir_status_t fwd_empty(const ChunkShape& s, const float* S0, float* S_T, hipStream_t hs) {
  if (S_T && s.B * s.H > 0) {
    const size_t n = static_cast<size_t>(s.B) * s.H * s.DK * s.DV;
    if (copy_or_zero(S_T, S0, n, hs) != hipSuccess) return MUIR_ERR_HIP;
  }
  return MUIR_OK;
}
muir_status_t bwd_empty(const ChunkShape& s, const float* dS_T, void* dgamma, float* dS0, hipStream_t hs) {
  if (dS0 && s.B * s.H > 0) {
    const size_t n = static_cast<size_t>(s.B) * s.H * s.DK * s.DV;
    if (copy_or_zero(dS0, dS_T, n, hs) != hipSuccess) return MUIR_ERR_HIP;
  }
  if (s.gmode == MUIR_GAMMA_STATIC && dgamma && s.H > 0) {
    if (!aligned16(dgamma)) return MUIR_ERR_ALIGN;
    if (copy_or_zero(static_cast<float*>(dgamma), nullptr, static_cast<size_t>(s.H) * s.DK, hs) != hipSuccess)
      return MUIR_ERR_HIP;
  }
  return MUIR_OK;
}

// Forward of batched ([N, T, H, D], cu == NULL) or packed (cu given)
// sequences through the padded layout.
muir_status_t fwd_staged(const ChunkShape& s, const int32_t* cu, const Inputs& in, const float* S0, void* o,
                         float* S_T, void* S_chunks, void* workspace, hipStream_t hs) {
  const ChunkShape p = padded(s);
  StageCursor cur{static_cast<char*>(workspace) + fwd_ws(p)};
  Inputs sin;
  muir_status_t st = stage_inputs(p, s.T, cu, in, &sin, &cur, hs);
  if (st != MUIR_OK) return st;
  void* po = cur.take(p, p.DV, p.tc_bytes());
  if ((st = fwd_core(p, sin, S0, po, S_T, S_chunks, workspace, hs)) != MUIR_OK) return st;
  return stage(po, o, p, s.T, p.DV, p.tc_bytes(), cu, false, hs) == hipSuccess ? MUIR_OK : MUIR_ERR_HIP;
}

muir_status_t bwd_staged(const ChunkShape& s, const int32_t* cu, const Inputs& in, const float* S0,
                         const void* S_chunks, const void* summaries, const void* dO, const float* dS_T,
                         const Grads& gr, float* dS0, void* workspace, hipStream_t hs) {
  const ChunkShape p = padded(s);
  StageCursor cur{static_cast<char*>(workspace) + bwd_ws(p)};
  Inputs sin;
  muir_status_t st = stage_inputs(p, s.T, cu, in, &sin, &cur, hs);
  if (st != MUIR_OK) return st;
  void* pdO = cur.take(p, p.DV, p.tc_bytes());
  if (stage(dO, pdO, p, s.T, p.DV, p.tc_bytes(), cu, true, hs) != hipSuccess) return MUIR_ERR_HIP;
  Grads sg;
  for (int i = 0; i < 7; ++i) {
    if (i == 6 && p.gmode != MUIR_GAMMA_TOKEN) {
      sg.x[6] = gr.x[6];  // a static gate's gradient is [H, dk] fp32; an absent gate has none
      continue;
    }
    sg.x[i] = cur.take(p, kIsDk[i] ? p.DK : p.DV, p.tg_bytes());
  }
  if ((st = bwd_core(p, sin, S0, S_chunks, summaries, pdO, dS_T, sg, dS0, workspace, hs)) != MUIR_OK) return st;
  for (int i = 0; i < 7; ++i) {
    if (i == 6 && p.gmode != MUIR_GAMMA_TOKEN) continue;
    if (stage(sg.x[i], gr.x[i], p, s.T, kIsDk[i] ? p.DK : p.DV, p.tg_bytes(), cu, false, hs) != hipSuccess)
      return MUIR_ERR_HIP;
  }
  return MUIR_OK;
}

// ---- Packed documents (variable-length calls) ----
// The documents run as one sequence (B = 1) in which document n starts at
// chunk c0(n) = the chunks of the documents before it (ceil(L / C) each), so
// the kernels see the documents' own chunks and nothing more; the scans start
// each document from its S0 and end it at its S_T (ChunkShape::cinfo).  The
// launch sizes count N ceil(L_max / C) chunks, the most the documents can
// fill (the padded layout's count, so the workspace is no larger); the
// chunks in use are counted on the device and every kernel skips the rest.

// The packed sequence's shape: s has B = N documents and T = the longest length.
ChunkShape packed_shape(const ChunkShape& s) {
  ChunkShape p = s;
  p.B = 1;
  p.T = s.B * ((s.T + s.C - 1) / s.C) * s.C;
  return p;
}
// Whether a call fits the packed form's 32-bit row and document indices
// (else it takes the padded form).
bool packable(const ChunkShape& s) {
  const long long rows = static_cast<long long>(s.B) * ((s.T + s.C - 1) / s.C) * s.C;
  return s.B < CI_DOC && rows < (1LL << 31) - 256;
}
// The plan: the chunk table (one int32 per chunk), the chunk count and each
// document's first row (int32 each).
size_t plan_bytes(const ChunkShape& p, int N) {
  return round256(static_cast<size_t>(p.NC()) * 4) + 256 + round256(static_cast<size_t>(N) * 4);
}
struct Plan {
  int32_t* cinfo;
  int32_t* ncu;
  int32_t* docoff;
};
Plan carve_plan(char* at, const ChunkShape& p) {
  Plan r;
  r.cinfo = reinterpret_cast<int32_t*>(at);
  r.ncu = reinterpret_cast<int32_t*>(at + round256(static_cast<size_t>(p.NC()) * 4));
  r.docoff = reinterpret_cast<int32_t*>(at + round256(static_cast<size_t>(p.NC()) * 4) + 256);
  return r;
}

// One workgroup: each thread takes a run of consecutive documents, the runs'
// chunk counts are scanned in LDS, and each thread then writes its
// documents' first rows and chunk-table entries.  Nothing is written past
// the NCmax chunks the launch sizes count: a document longer than the
// call's max_len (which must bound every length) is cut there, as the
// padded form would cut it.
__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu, int N, int C, int NCmax,
                                                   int32_t* __restrict__ cinfo, int32_t* __restrict__ ncu,
                                                   int32_t* __restrict__ docoff) {
  __shared__ int run[256];
  const int t = threadIdx.x;
  const int per = (N + 255) / 256;
  const int d0 = min(N, t * per), d1 = min(N, d0 + per);
  int sum = 0;
  for (int d = d0; d < d1; ++d) sum += (cu[d + 1] - cu[d] + C - 1) / C;
  run[t] = sum;
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = run[i];
      run[i] = acc;
      acc += v;
    }
    *ncu = min(acc, NCmax);
  }
  __syncthreads();
  int c0 = run[t];
  for (int d = d0; d < d1; ++d) {
    const int n = (cu[d + 1] - cu[d] + C - 1) / C;
    docoff[d] = c0 * C;
    for (int k = 0; k < n && c0 + k < NCmax; ++k)
      cinfo[c0 + k] = d | (k == 0 ? CI_START : 0) | (k == n - 1 ? CI_END : 0);
    c0 += n;
  }
}

// Sequence tensors between the caller's packed [T_total, H, D] layout and the
// chunk-aligned one, in 16-byte words (WW per token): document d's tokens
// from row docoff[d], zero rows after them to its last chunk's end.  Rows
// past the chunks in use are neither written nor read.  A block takes whole
// rows (grid-stride), looks up the row's document once and copies its words
// with consecutive threads.  (One thread per word, each dividing its 64-bit
// word index and reading the tables, moved these copies at about 3.7 TB/s.)
__global__ __launch_bounds__(256) void pack_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int WW,
                                                   int C, const int32_t* __restrict__ cu,
                                                   const int32_t* __restrict__ cinfo, const int32_t* __restrict__ ncu,
                                                   const int32_t* __restrict__ docoff, int to_packed) {
  const int rows = *ncu * C;
  for (int row = blockIdx.x; row < rows; row += gridDim.x) {
    const int d = cinfo[row / C] & CI_DOC;
    const int t = row - docoff[d];
    const bool real = t < cu[d + 1] - cu[d];
    const size_t crow = static_cast<size_t>(cu[d]) + t;
    if (to_packed) {
      // a padding row (past the document's end) reads nothing: its source
      // row would lie past the document, perhaps past the tensor
      uint4* o = dst + static_cast<size_t>(row) * WW;
      if (real) {
        const uint4* s = src + crow * WW;
        for (int w = threadIdx.x; w < WW; w += blockDim.x) o[w] = s[w];
      } else {
        const uint4 z = {0u, 0u, 0u, 0u};
        for (int w = threadIdx.x; w < WW; w += blockDim.x) o[w] = z;
      }
    } else if (real) {
      const uint4* s = src + static_cast<size_t>(row) * WW;
      uint4* o = dst + crow * WW;
      for (int w = threadIdx.x; w < WW; w += blockDim.x) o[w] = s[w];
    }
  }
}

hipError_t pack(const void* src, void* dst, const ChunkShape& p, int D, size_t esize, const int32_t* cu,
                const Plan& pl, bool to_packed, hipStream_t s) {
  const int WW = static_cast<int>(static_cast<size_t>(p.H) * D * esize / 16);
  if (p.T == 0 || WW == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(p.T < 8192 ? p.T : 8192);  // p.T: the most rows in use
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), WW, p.C, cu, pl.cinfo, pl.ncu, pl.docoff, to_packed ? 1 : 0);
  return hipGetLastError();
}

// Documents without tokens: the final state is the initial state (zero
// without one), and the initial state's gradient is the final state's.  16
// blocks per document, n floats each.
__global__ void empty_docs_kernel(const int32_t* __restrict__ cu, size_t n, const float* __restrict__ src,
                                  float* __restrict__ dst) {
  const int d = blockIdx.x / 16;
  if (cu[d + 1] != cu[d]) return;
  const size_t base = static_cast<size_t>(d) * n;
  for (size_t i = static_cast<size_t>(blockIdx.x % 16) * blockDim.x + threadIdx.x; i < n; i += 16 * blockDim.x)
    dst[base + i] = src ? src[base + i] : 0.f;
}
hipError_t empty_docs(const int32_t* cu, int N, const ChunkShape& s, const float* src, float* dst, hipStream_t hs) {
  if (!dst || N == 0) return hipSuccess;
  hipLaunchKernelGGL(empty_docs_kernel, dim3(static_cast<unsigned>(N) * 16), dim3(256), 0, hs, cu,
                     static_cast<size_t>(s.H) * s.DK * s.DV, src, dst);
  return hipGetLastError();
}

muir_status_t pack_inputs(const ChunkShape& p, const int32_t* cu, const Plan& pl, const Inputs& in, Inputs* out,
                          StageCursor* cur, hipStream_t hs) {
  for (int i = 0; i < 7; ++i) {
    if (i == 6 && p.gmode != MUIR_GAMMA_TOKEN) {
      out->x[6] = in.x[6];  // a static gate is [H, dk] and needs no staging; an absent one is not read
      continue;
    }
    const int D = kIsDk[i] ? p.DK : p.DV;
    void* dst = cur->take(p, D, p.tc_bytes());
    if (pack(in.x[i], dst, p, D, p.tc_bytes(), cu, pl, true, hs) != hipSuccess) return MUIR_ERR_HIP;
    out->x[i] = dst;
  }
  return MUIR_OK;
}

// The chunk-start states a packed forward keeps for its backward (keep), in
// the compute type, after the plan; always reserved.
size_t packed_states_bytes(const ChunkShape& p) {
  return round256(p.nchunks() * static_cast<size_t>(p.DK) * p.DV * p.tc_bytes());
}
size_t packed_fwd_need(const ChunkShape& s) {
  const ChunkShape p = packed_shape(s);
  return fwd_ws(p) + fwd_stage_bytes(p) + plan_bytes(p, s.B) + packed_states_bytes(p);
}
// The packed forward's workspace: its kernels' workspace (the chunk
// summaries, then the split scans' area), the packed inputs and o, the plan,
// the kept chunk-start states.
struct PackedFwd {
  char* ws;
  Plan pl;
  char* staging;
  void* S_chunks;
};
PackedFwd packed_fwd_parts(void* workspace, const ChunkShape& p, int N) {
  char* w = static_cast<char*>(workspace);
  PackedFwd r;
  r.ws = w;
  r.staging = w + fwd_ws(p);
  r.pl = carve_plan(r.staging + fwd_stage_bytes(p), p);
  r.S_chunks = r.staging + fwd_stage_bytes(p) + plan_bytes(p, N);
  return r;
}
size_t packed_bwd_need(const ChunkShape& s) {
  const ChunkShape p = packed_shape(s);
  return bwd_ws(p) + bwd_stage_bytes(p) + plan_bytes(p, s.B);
}

// keep: the chunk-start states (and with them the deltas, in the summaries)
// are saved, and the summaries, packed inputs and plan stay in the workspace
// for muir_chunk_varlen_bwd to reuse.
muir_status_t fwd_packed(const ChunkShape& s, const int32_t* cu, const Inputs& in, const float* S0, void* o,
                         float* S_T, bool keep, void* workspace, hipStream_t hs) {
  ChunkShape p = packed_shape(s);
  const PackedFwd f = packed_fwd_parts(workspace, p, s.B);
  const Plan pl = f.pl;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, hs, cu, s.B, s.C, p.NC(), pl.cinfo, pl.ncu, pl.docoff);
  if (hipGetLastError() != hipSuccess) return MUIR_ERR_HIP;
  p.cinfo = pl.cinfo;
  p.ncu = pl.ncu;
  StageCursor cur{f.staging};
  Inputs sin;
  muir_status_t st = pack_inputs(p, cu, pl, in, &sin, &cur, hs);
  if (st != MUIR_OK) return st;
  void* po = cur.take(p, p.DV, p.tc_bytes());
  if ((st = fwd_core(p, sin, S0, po, S_T, keep ? f.S_chunks : nullptr, workspace, hs)) != MUIR_OK) return st;
  if (pack(po, o, p, p.DV, p.tc_bytes(), cu, pl, false, hs) != hipSuccess) return MUIR_ERR_HIP;
  return empty_docs(cu, s.B, s, S0, S_T, hs) == hipSuccess ? MUIR_OK : MUIR_ERR_HIP;
}

// fwd_workspace: a keeping forward's workspace, whose plan, packed inputs,
// summaries and chunk-start states are reused (else all are formed here).
muir_status_t bwd_packed(const ChunkShape& s, const int32_t* cu, const Inputs& in, const float* S0, const void* dO,
                         const float* dS_T, const Grads& gr, float* dS0, const void* fwd_workspace, void* workspace,
                         hipStream_t hs) {
  ChunkShape p = packed_shape(s);
  char* w = static_cast<char*>(workspace);
  StageCursor cur{w + bwd_ws(p)};
  Inputs sin;
  Plan pl;
  const void* summ = nullptr;
  const void* Sc = nullptr;
  muir_status_t st;
  if (fwd_workspace) {
    // the forward's parts, carved as the forward carved them
    const PackedFwd f = packed_fwd_parts(const_cast<void*>(fwd_workspace), p, s.B);
    pl = f.pl;
    StageCursor fc{f.staging};
    for (int i = 0; i < 7; ++i) {
      if (i == 6 && p.gmode != MUIR_GAMMA_TOKEN) {
        sin.x[6] = in.x[6];
        continue;
      }
      sin.x[i] = fc.take(p, kIsDk[i] ? p.DK : p.DV, p.tc_bytes());
    }
    summ = f.ws;
    Sc = f.S_chunks;  // (this call's own input copies are not needed: dO and the gradients take the staging area)
  } else {
    pl = carve_plan(w + bwd_ws(p) + bwd_stage_bytes(p), p);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, hs, cu, s.B, s.C, p.NC(), pl.cinfo, pl.ncu, pl.docoff);
    if (hipGetLastError() != hipSuccess) return MUIR_ERR_HIP;
  }
  p.cinfo = pl.cinfo;
  p.ncu = pl.ncu;
  if (!fwd_workspace && (st = pack_inputs(p, cu, pl, in, &sin, &cur, hs)) != MUIR_OK) return st;
  void* pdO = cur.take(p, p.DV, p.tc_bytes());
  if (pack(dO, pdO, p, p.DV, p.tc_bytes(), cu, pl, true, hs) != hipSuccess) return MUIR_ERR_HIP;
  // the chunk kernel writes the per-token gradients straight to the caller's
  // tensors when it can (ChunkShape::packed_output), else to copies here
  const bool direct = p.packed_output();
  if (direct) {
    p.cu = cu;
    p.docoff = pl.docoff;
  }
  Grads sg;
  for (int i = 0; i < 7; ++i) {
    if ((i == 6 && p.gmode != MUIR_GAMMA_TOKEN) || direct) {
      sg.x[i] = gr.x[i];  // (a static gate's gradient is [H, dk] fp32; an absent gate has none)
      continue;
    }
    sg.x[i] = cur.take(p, kIsDk[i] ? p.DK : p.DV, p.tg_bytes());
  }
  if ((st = bwd_core(p, sin, S0, Sc, summ, pdO, dS_T, sg, dS0, workspace, hs)) != MUIR_OK) return st;
  for (int i = 0; i < 7 && !direct; ++i) {
    if (i == 6 && p.gmode != MUIR_GAMMA_TOKEN) continue;
    if (pack(sg.x[i], gr.x[i], p, kIsDk[i] ? p.DK : p.DV, p.tg_bytes(), cu, pl, false, hs) != hipSuccess)
      return MUIR_ERR_HIP;
  }
  return empty_docs(cu, s.B, s, dS_T, dS0, hs) == hipSuccess ? MUIR_OK : MUIR_ERR_HIP;
}

size_t fwd_need(const ChunkShape& s) {
  return s.T % s.C == 0 ? fwd_ws(s) : fwd_ws(padded(s)) + fwd_stage_bytes(padded(s));
}
size_t bwd_need(const ChunkShape& s) {
  return s.T % s.C == 0 ? bwd_ws(s) : bwd_ws(padded(s)) + bwd_stage_bytes(padded(s));
}
// Sizes of a gate-prologue call.
muir_status_t check_gate_dims(const muir_gate_dims_t* d, muir::GateShape* s) {
  if (!d) return MUIR_ERR_NULL;
  if (d->dtype != MUIR_F32 && d->dtype != MUIR_BF16) return MUIR_ERR_DTYPE;
  if (d->M < 0 || d->d <= 0 || d->d % 64 != 0 || d->d > (1 << 16) || d->H <= 0) return MUIR_ERR_SHAPE;
  if ((d->dk != 64 && d->dk != 128) || (d->dv != 64 && d->dv != 128)) return MUIR_ERR_SHAPE;
  if (static_cast<long long>(d->H) * (d->dk > d->dv ? d->dk : d->dv) > (1 << 16)) return MUIR_ERR_SHAPE;
  s->M = d->M;
  s->d = d->d;
  s->H = d->H;
  s->dk = d->dk;
  s->dv = d->dv;
  s->bf16 = d->dtype == MUIR_BF16;
  return MUIR_OK;
}

muir_status_t qk_norm_call(int64_t rows, int32_t D, int32_t dtype, const void* u, const void* dy, void* out,
                           void* stream) {
  if (dtype != MUIR_F32 && dtype != MUIR_BF16) return MUIR_ERR_DTYPE;
  if (rows < 0 || (D != 64 && D != 128) || rows > (1LL << 40)) return MUIR_ERR_SHAPE;
  if (rows == 0) return MUIR_OK;
  if (!u || !out) return MUIR_ERR_NULL;
  if (!aligned16(u) || !aligned16(out) || (dy && !aligned16(dy))) return MUIR_ERR_ALIGN;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  mark(hs);
  if (muir::launch_qk_norm(rows, D, dtype == MUIR_BF16, u, dy, out, hs) != hipSuccess) return MUIR_ERR_HIP;
  mark(hs);
  return MUIR_OK;
}

// Device address of the no-allocation scratch array on the current device,
// looked up once per device (each GPU holds its own copy of the array at its
// own address) and kept; NULL if the lookup fails.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Counts the values of x[0..n) that break the inputs' preconditions: NaN or
// infinite (exponent bits all set), and, for a log-decay, finite and above 0
// (sign bit clear, not zero).  Per-lane counts, a wave sum, one atomic add per wave.
template <typename T>
__global__ __launch_bounds__(256) void check_values_kernel(int64_t n, const T* __restrict__ x, int log_decay,
                                                           int32_t* __restrict__ counts) {
  constexpr uint32_t kExp = sizeof(T) == 2 ? 0x7F80u : 0x7F800000u;
  constexpr uint32_t kSign = sizeof(T) == 2 ? 0x8000u : 0x80000000u;
  int bad = 0, pos = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    uint32_t b;
    if constexpr (sizeof(T) == 2) b = x[i];
    else b = __float_as_uint(x[i]);
    bad += (b & kExp) == kExp;
    pos += log_decay && !(b & kSign) && b != 0u && (b & kExp) != kExp;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    bad += __shfl_xor(bad, off, 64);
    pos += __shfl_xor(pos, off, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    if (bad) atomicAdd(&counts[0], bad);
    if (pos) atomicAdd(&counts[1], pos);
  }
}

size_t varlen_fwd_need(const ChunkShape& s) {
  return packable(s) ? packed_fwd_need(s) : fwd_ws(padded(s)) + fwd_stage_bytes(padded(s));
}
size_t varlen_bwd_need(const ChunkShape& s) {
  return packable(s) ? packed_bwd_need(s) : bwd_ws(padded(s)) + bwd_stage_bytes(padded(s));
}

}  // namespace

extern "C" {

int32_t muir_abi_version(void) { return 10; }

int32_t muir_set_profile_events(void** events, int32_t count) {
  if (count < 0 || (count > 0 && !events)) return MUIR_ERR_NULL;
  g_events = reinterpret_cast<hipEvent_t*>(events);
  g_nevents = events ? count : 0;
  g_cursor = 0;
  return MUIR_OK;
}

int32_t muir_profile_events_recorded(void) { return g_cursor; }

const char* muir_status_string(muir_status_t st) {
  switch (st) {
    case MUIR_OK: return "ok";
    case MUIR_ERR_NULL: return "a required pointer is NULL";
    case MUIR_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case MUIR_ERR_DTYPE: return "unknown dtype code";
    case MUIR_ERR_WORKSPACE: return "workspace missing or too small";
    case MUIR_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MUIR_ERR_HIP: return "a HIP kernel launch failed";
    case MUIR_ERR_MODE: return "unknown readout-gate mode";
    case MUIR_ERR_SCRATCH: return "the call needs more than the no-allocation scratch (MUIR_NOALLOC_SCRATCH_BYTES)";
    case MUIR_ERR_NONFINITE: return "an input is NaN or infinite, or a log-decay is above 0";
  }
  return "unknown status";
}

muir_status_t muir_check_values(int64_t n, int32_t dtype, const void* x, int32_t log_decay, int32_t* counts,
                                void* stream) {
  if (dtype != MUIR_F32 && dtype != MUIR_BF16) return MUIR_ERR_DTYPE;
  if (n < 0) return MUIR_ERR_SHAPE;
  if (n == 0) return MUIR_OK;
  if (!x || !counts) return MUIR_ERR_NULL;
  const size_t es = dtype == MUIR_BF16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(x) & (es - 1)) || (reinterpret_cast<uintptr_t>(counts) & 3)) return MUIR_ERR_ALIGN;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const int64_t want = (n + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 4096 ? want : 4096);
  if (dtype == MUIR_BF16)
    hipLaunchKernelGGL(check_values_kernel<uint16_t>, dim3(blocks), dim3(256), 0, hs, n,
                       static_cast<const uint16_t*>(x), log_decay ? 1 : 0, counts);
  else
    hipLaunchKernelGGL(check_values_kernel<float>, dim3(blocks), dim3(256), 0, hs, n, static_cast<const float*>(x),
                       log_decay ? 1 : 0, counts);
  return hipGetLastError() == hipSuccess ? MUIR_OK : MUIR_ERR_HIP;
}

size_t muir_chunk_fwd_workspace(const muir_dims_t* dims) {
  ChunkShape s;
  if (check_dims(dims, &s) != MUIR_OK) return 0;
  return fwd_need(s);
}

muir_status_t muir_chunk_fwd_noalloc(const muir_dims_t* dims, const void* q, const void* k, const void* v,
                                     const void* log_a, const void* erase, const void* write, const void* gamma,
                                     const float* S0, void* o, float* S_T, void* S_chunks, void* stream) {
  ChunkShape s;
  muir_status_t st = check_dims(dims, &s);
  if (st != MUIR_OK) return st;
  const size_t need = fwd_need(s);
  if (need > MUIR_NOALLOC_SCRATCH_BYTES) return MUIR_ERR_SCRATCH;
  const Inputs in{{q, k, v, log_a, erase, write, gamma}};
  if ((st = check_fwd_tensors(s, in, S0, o, S_T, S_chunks)) != MUIR_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (s.nchunks() == 0) return fwd_empty(s, S0, S_T, hs);
  void* ws = noalloc_scratch();
  if (!ws) return MUIR_ERR_HIP;
  if (s.T % s.C == 0) return fwd_core(s, in, S0, o, S_T, S_chunks, ws, hs);
  return fwd_staged(s, nullptr, in, S0, o, S_T, S_chunks, ws, hs);
}

size_t muir_chunk_bwd_workspace(const muir_dims_t* dims) {
  ChunkShape s;
  if (check_dims(dims, &s, true) != MUIR_OK) return 0;
  return bwd_need(s);
}

muir_status_t muir_chunk_fwd(const muir_dims_t* dims, const void* q, const void* k,
                             const void* v, const void* log_a, const void* erase,
                             const void* write, const void* gamma, const float* S0, void* o,
                             float* S_T, void* S_chunks, void* workspace,
                             size_t workspace_bytes, void* stream) {
  ChunkShape s;
  muir_status_t st = check_dims(dims, &s);
  if (st != MUIR_OK) return st;
  const Inputs in{{q, k, v, log_a, erase, write, gamma}};
  if ((st = check_fwd_args(s, in, S0, o, S_T, S_chunks, workspace, workspace_bytes, fwd_need(s))) != MUIR_OK)
    return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (s.nchunks() == 0) return fwd_empty(s, S0, S_T, hs);
  if (s.T % s.C == 0) return fwd_core(s, in, S0, o, S_T, S_chunks, workspace, hs);
  return fwd_staged(s, nullptr, in, S0, o, S_T, S_chunks, workspace, hs);
}

muir_status_t muir_chunk_bwd(const muir_dims_t* dims, const void* q, const void* k,
                             const void* v, const void* log_a, const void* erase,
                             const void* write, const void* gamma, const float* S0,
                             const void* S_chunks, const void* summaries, const void* dO,
                             const float* dS_T, void* dq, void* dk, void* dv, void* dlog_a,
                             void* derase, void* dwrite, void* dgamma, float* dS0,
                             void* workspace, size_t workspace_bytes, void* stream) {
  ChunkShape s;
  muir_status_t st = check_dims(dims, &s, true);
  if (st != MUIR_OK) return st;
  const Inputs in{{q, k, v, log_a, erase, write, gamma}};
  const Grads gr{{dq, dk, dv, dlog_a, derase, dwrite, dgamma}};
  if ((st = check_bwd_args(s, in, S0, S_chunks, summaries, dO, dS_T, gr, dS0, workspace, workspace_bytes,
                           bwd_need(s))) != MUIR_OK)
    return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (s.nchunks() == 0) return bwd_empty(s, dS_T, dgamma, dS0, hs);
  if (s.T % s.C == 0) return bwd_core(s, in, S0, S_chunks, summaries, dO, dS_T, gr, dS0, workspace, hs);
  return bwd_staged(s, nullptr, in, S0, S_chunks, summaries, dO, dS_T, gr, dS0, workspace, hs);
}

size_t muir_chunk_varlen_fwd_workspace(const muir_dims_t* dims) {
  ChunkShape s;
  if (check_dims(dims, &s) != MUIR_OK) return 0;
  return varlen_fwd_need(s);
}

size_t muir_chunk_varlen_bwd_workspace(const muir_dims_t* dims) {
  ChunkShape s;
  if (check_dims(dims, &s, true) != MUIR_OK) return 0;
  return varlen_bwd_need(s);
}

muir_status_t muir_chunk_varlen_fwd(const muir_dims_t* dims, const int32_t* cu_seqlens, const void* q,
                                    const void* k, const void* v, const void* log_a, const void* erase,
                                    const void* write, const void* gamma, const float* S0, void* o,
                                    float* S_T, int32_t keep, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  ChunkShape s;
  muir_status_t st = check_dims(dims, &s);
  if (st != MUIR_OK) return st;
  const Inputs in{{q, k, v, log_a, erase, write, gamma}};
  if ((st = check_fwd_args(s, in, S0, o, S_T, nullptr, workspace, workspace_bytes, varlen_fwd_need(s))) !=
      MUIR_OK)
    return st;
  if (s.nchunks() != 0 && !cu_seqlens) return MUIR_ERR_NULL;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (s.nchunks() == 0) return fwd_empty(s, S0, S_T, hs);
  if (packable(s)) return fwd_packed(s, cu_seqlens, in, S0, o, S_T, keep != 0, workspace, hs);
  return fwd_staged(s, cu_seqlens, in, S0, o, S_T, nullptr, workspace, hs);
}

muir_status_t muir_chunk_varlen_bwd(const muir_dims_t* dims, const int32_t* cu_seqlens, const void* q,
                                    const void* k, const void* v, const void* log_a, const void* erase,
                                    const void* write, const void* gamma, const float* S0, const void* dO,
                                    const float* dS_T, void* dq, void* dk, void* dv, void* dlog_a, void* derase,
                                    void* dwrite, void* dgamma, float* dS0, const void* fwd_workspace,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  ChunkShape s;
  muir_status_t st = check_dims(dims, &s, true);
  if (st != MUIR_OK) return st;
  const Inputs in{{q, k, v, log_a, erase, write, gamma}};
  const Grads gr{{dq, dk, dv, dlog_a, derase, dwrite, dgamma}};
  if ((st = check_bwd_args(s, in, S0, nullptr, nullptr, dO, dS_T, gr, dS0, workspace, workspace_bytes,
                           varlen_bwd_need(s))) != MUIR_OK)
    return st;
  if (s.nchunks() != 0 && !cu_seqlens) return MUIR_ERR_NULL;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (s.nchunks() == 0) return bwd_empty(s, dS_T, dgamma, dS0, hs);
  if (fwd_workspace && !aligned16(fwd_workspace)) return MUIR_ERR_ALIGN;
  if (packable(s)) return bwd_packed(s, cu_seqlens, in, S0, dO, dS_T, gr, dS0, fwd_workspace, workspace, hs);
  return bwd_staged(s, cu_seqlens, in, S0, nullptr, nullptr, dO, dS_T, gr, dS0, workspace, hs);
}

size_t muir_gate_proj_bwd_workspace(const muir_gate_dims_t* dims) {
  muir::GateShape s;
  if (check_gate_dims(dims, &s) != MUIR_OK) return 0;
  return muir::gate_workspace(s).bytes;
}

muir_status_t muir_gate_proj_fwd(const muir_gate_dims_t* dims, const void* x, const void* W_down,
                                 const void* W_up, const void* bias, void* z, void* log_a, void* erase,
                                 void* g, void* write, void* gamma, void* stream) {
  muir::GateShape s;
  muir_status_t st = check_gate_dims(dims, &s);
  if (st != MUIR_OK) return st;
  if (s.M == 0) return MUIR_OK;
  const void* req[] = {x, W_down, W_up, bias, z, log_a, erase, g, write, gamma};
  for (const void* p : req)
    if (!p) return MUIR_ERR_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return MUIR_ERR_ALIGN;
  void* const gates[5] = {log_a, erase, g, write, gamma};
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  mark(hs);
  if (muir::launch_gate_fwd(s, x, W_down, W_up, bias, z, gates, hs) != hipSuccess) return MUIR_ERR_HIP;
  mark(hs);
  return MUIR_OK;
}

muir_status_t muir_gate_proj_bwd(const muir_gate_dims_t* dims, const void* x, const void* W_down,
                                 const void* W_up, const void* bias, const void* z, const void* dlog_a,
                                 const void* derase, const void* dg, const void* dwrite, const void* dgamma,
                                 void* dx, float* dW_down, float* dW_up, float* dbias, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  muir::GateShape s;
  muir_status_t st = check_gate_dims(dims, &s);
  if (st != MUIR_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (s.M == 0) {
    // no tokens: the weight gradients are sums over nothing
    float* outs[] = {dW_down, dW_up, dbias};
    for (float* p : outs)
      if (!p) return MUIR_ERR_NULL;
    for (float* p : outs)
      if (!aligned16(p)) return MUIR_ERR_ALIGN;
    const muir::GateWorkspace w = muir::gate_workspace(s);
    const size_t n[] = {static_cast<size_t>(s.d) * muir::GATE_RTOT,
                        muir::gate_up_numel(s),
                        static_cast<size_t>(w.colsum_ld)};
    for (int i = 0; i < 3; ++i)
      if (copy_or_zero(outs[i], nullptr, n[i], hs) != hipSuccess) return MUIR_ERR_HIP;
    return MUIR_OK;
  }
  const void* req[] = {x, W_down, W_up, bias, dlog_a, derase, dg, dwrite, dgamma, dx, dW_down, dW_up, dbias};
  for (const void* p : req)
    if (!p) return MUIR_ERR_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return MUIR_ERR_ALIGN;
  if (z && !aligned16(z)) return MUIR_ERR_ALIGN;
  const muir::GateWorkspace w = muir::gate_workspace(s);
  if (!workspace || workspace_bytes < w.bytes) return MUIR_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MUIR_ERR_ALIGN;
  mark(hs);
  const void* const dgates[5] = {dlog_a, derase, dg, dwrite, dgamma};
  if (muir::launch_gate_bwd(s, x, W_down, W_up, bias, z, dgates, dx, dW_down, dW_up, dbias, workspace, hs) !=
      hipSuccess)
    return MUIR_ERR_HIP;
  mark(hs);
  return MUIR_OK;
}

muir_status_t muir_qk_norm_fwd(int64_t rows, int32_t D, int32_t dtype, const void* u, void* y, void* stream) {
  return qk_norm_call(rows, D, dtype, u, nullptr, y, stream);
}

muir_status_t muir_qk_norm_bwd(int64_t rows, int32_t D, int32_t dtype, const void* u, const void* dy, void* du,
                               void* stream) {
  if (rows > 0 && !dy) return MUIR_ERR_NULL;
  return qk_norm_call(rows, D, dtype, u, dy, du, stream);
}

muir_status_t muir_step(int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t dtype,
                        int32_t gamma_mode, const void* q, const void* k, const void* v,
                        const void* log_a, const void* erase, const void* write, const void* gamma,
                        float* S, void* o, void* stream) {
  if (dtype != MUIR_F32 && dtype != MUIR_BF16) return MUIR_ERR_DTYPE;
  if (gamma_mode < MUIR_GAMMA_TOKEN || gamma_mode > MUIR_GAMMA_NONE) return MUIR_ERR_MODE;
  if (N < 0 || H < 0 || (dk != 64 && dk != 128) || dv <= 0 || dv % 64 != 0 || dv > 4096)
    return MUIR_ERR_SHAPE;
  if (static_cast<long long>(N) * H * (dv / 64) > (1LL << 30)) return MUIR_ERR_SHAPE;
  if (static_cast<long long>(N) * H == 0) return MUIR_OK;
  const void* req[] = {q, k, v, log_a, erase, write, S, o};
  for (const void* p : req)
    if (!p) return MUIR_ERR_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return MUIR_ERR_ALIGN;
  if (gamma_mode != MUIR_GAMMA_NONE) {
    if (!gamma) return MUIR_ERR_NULL;
    if (!aligned16(gamma)) return MUIR_ERR_ALIGN;
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  mark(hs);
  if (muir::launch_step(N, H, dk, dv, dtype == MUIR_BF16, gamma_mode, q, k, v, log_a, erase, write, gamma,
                        S, o, hs) != hipSuccess)
    return MUIR_ERR_HIP;
  mark(hs);
  return MUIR_OK;
}

}  // extern "C"
