// C ABI of the Muir operator: argument validation, workspace sizing and
// kernel dispatch.  Every entry point checks its arguments before launching
// anything and never allocates, frees or synchronises.
#include <muir.h>

#include "kernels.h"

using muir::ChunkShape;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

muir_status_t check_dims(const muir_dims_t* d, ChunkShape* s) {
  if (!d) return MUIR_ERR_NULL;
  if (d->dtype != MUIR_F32 && d->dtype != MUIR_BF16) return MUIR_ERR_DTYPE;
  if (d->gamma_mode < MUIR_GAMMA_TOKEN || d->gamma_mode > MUIR_GAMMA_NONE) return MUIR_ERR_MODE;
  if (d->B < 0 || d->T < 0 || d->H < 0) return MUIR_ERR_SHAPE;
  if (d->dk != d->dv || (d->dk != 64 && d->dk != 128)) return MUIR_ERR_SHAPE;
  if (d->chunk != 64 && d->chunk != 128 && d->chunk != 256) return MUIR_ERR_SHAPE;
  if (d->T % d->chunk != 0) return MUIR_ERR_SHAPE;
  // keep every flat index inside 32-bit chunk counts and 64-bit element counts
  if (static_cast<long long>(d->B) * d->H * (d->T / d->chunk) > (1LL << 30)) return MUIR_ERR_SHAPE;
  // the kernels address one chunk of a [B, T, H, D] tensor with 32-bit offsets
  if (static_cast<long long>(d->H) * d->dk * d->chunk * 4 >= (1LL << 31)) return MUIR_ERR_SHAPE;
  s->B = d->B;
  s->T = d->T;
  s->H = d->H;
  s->DK = d->dk;
  s->DV = d->dv;
  s->C = d->chunk;
  s->bf16 = d->dtype == MUIR_BF16;
  s->gmode = d->gamma_mode;
  return MUIR_OK;
}

// Forward workspace: the chunk summaries, then the split scan's segment
// transitions and starts (when the shape splits its scan).
size_t fwd_ws(const ChunkShape& s) { return s.nchunks() * s.summary_bytes() + s.scan_split_bytes(); }

// Backward workspace: chunk summaries (used when the caller passes none),
// recomputed chunk states (used when the caller passes no S_chunks), the
// chunk-end state gradients, per-chunk scratch for the deltas and their
// gradients, then the split scans' segment area (shared by the recomputed
// forward scan and the reverse scan, which run one after the other).  Every
// part is always reserved, so the size does not depend on which pointers are
// passed.
size_t bwd_scratch_bytes(const ChunkShape& s) {
  return (muir::bwd_chunk_scratch_bytes(s) + 255) & ~static_cast<size_t>(255);
}
// per-chunk partial sums of a static readout gate's gradient, [nchunks][dk] fp32
size_t gamma_part_bytes(const ChunkShape& s) {
  return (s.nchunks() * s.DK * 4 + 255) & ~static_cast<size_t>(255);
}
size_t bwd_ws(const ChunkShape& s) {
  return s.nchunks() * (s.summary_bytes() + 2 * s.state_bytes() + bwd_scratch_bytes(s)) + s.scan_split_bytes() +
         gamma_part_bytes(s);
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

}  // namespace

extern "C" {

int32_t muir_abi_version(void) { return 4; }

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
  }
  return "unknown status";
}

size_t muir_chunk_fwd_workspace(const muir_dims_t* dims) {
  ChunkShape s;
  if (check_dims(dims, &s) != MUIR_OK) return 0;
  return fwd_ws(s);
}

size_t muir_chunk_bwd_workspace(const muir_dims_t* dims) {
  ChunkShape s;
  if (check_dims(dims, &s) != MUIR_OK) return 0;
  return bwd_ws(s);
}

muir_status_t muir_chunk_fwd(const muir_dims_t* dims, const void* q, const void* k,
                             const void* v, const void* log_a, const void* erase,
                             const void* write, const void* gamma, const float* S0, void* o,
                             float* S_T, float* S_chunks, void* workspace,
                             size_t workspace_bytes, void* stream) {
  ChunkShape s;
  muir_status_t st = check_dims(dims, &s);
  if (st != MUIR_OK) return st;
  const bool empty = s.nchunks() == 0;
  if (!empty) {
    const void* req[] = {q, k, v, log_a, erase, write, o};
    for (const void* p : req)
      if (!p) return MUIR_ERR_NULL;
    for (const void* p : req)
      if (!aligned16(p)) return MUIR_ERR_ALIGN;
    if ((st = check_gate(s, gamma)) != MUIR_OK) return st;
    if (!workspace || workspace_bytes < fwd_ws(s)) return MUIR_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MUIR_ERR_ALIGN;
  }
  const void* opt[] = {S0, S_T, S_chunks};
  for (const void* p : opt)
    if (p && !aligned16(p)) return MUIR_ERR_ALIGN;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (empty) {
    // T == 0: the final state is the initial state
    if (S_T && s.B * s.H > 0) {
      const size_t n = static_cast<size_t>(s.B) * s.H * s.DK * s.DV;
      if (copy_or_zero(S_T, S0, n, hs) != hipSuccess) return MUIR_ERR_HIP;
    }
    return MUIR_OK;
  }
  mark(hs);
  if (muir::launch_fwd_prep(s, q, k, v, log_a, erase, write, gamma, workspace, hs) != hipSuccess)
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

muir_status_t muir_chunk_bwd(const muir_dims_t* dims, const void* q, const void* k,
                             const void* v, const void* log_a, const void* erase,
                             const void* write, const void* gamma, const float* S0,
                             const float* S_chunks, const void* summaries, const void* dO,
                             const float* dS_T, void* dq, void* dk, void* dv, void* dlog_a,
                             void* derase, void* dwrite, void* dgamma, float* dS0,
                             void* workspace, size_t workspace_bytes, void* stream) {
  ChunkShape s;
  muir_status_t st = check_dims(dims, &s);
  if (st != MUIR_OK) return st;
  const bool empty = s.nchunks() == 0;
  if (!empty) {
    const void* req[] = {q, k, v, log_a, erase, write, dO, dq, dk, dv, dlog_a, derase, dwrite};
    for (const void* p : req)
      if (!p) return MUIR_ERR_NULL;
    for (const void* p : req)
      if (!aligned16(p)) return MUIR_ERR_ALIGN;
    if ((st = check_gate(s, gamma)) != MUIR_OK) return st;
    if ((st = check_gate(s, dgamma)) != MUIR_OK) return st;
    if (!workspace || workspace_bytes < bwd_ws(s)) return MUIR_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MUIR_ERR_ALIGN;
  }
  const void* opt[] = {S0, S_chunks, summaries, dS_T, dS0};
  for (const void* p : opt)
    if (p && !aligned16(p)) return MUIR_ERR_ALIGN;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (empty) {
    if (dS0 && s.B * s.H > 0) {
      const size_t n = static_cast<size_t>(s.B) * s.H * s.DK * s.DV;
      if (copy_or_zero(dS0, dS_T, n, hs) != hipSuccess) return MUIR_ERR_HIP;
    }
    // a static gate's gradient is a sum over no tokens
    if (s.gmode == MUIR_GAMMA_STATIC && dgamma && s.H > 0) {
      if ((st = check_gate(s, dgamma)) != MUIR_OK) return st;
      if (copy_or_zero(static_cast<float*>(dgamma), nullptr, static_cast<size_t>(s.H) * s.DK, hs) != hipSuccess)
        return MUIR_ERR_HIP;
    }
    return MUIR_OK;
  }
  char* ws = static_cast<char*>(workspace);
  float* S_rec = reinterpret_cast<float*>(ws + s.nchunks() * s.summary_bytes());
  float* dS_chunks = S_rec + s.nchunks() * static_cast<size_t>(s.DK) * s.DV;
  float* scratch = dS_chunks + s.nchunks() * static_cast<size_t>(s.DK) * s.DV;
  float* split = reinterpret_cast<float*>(reinterpret_cast<char*>(scratch) + s.nchunks() * bwd_scratch_bytes(s));
  float* gpart = reinterpret_cast<float*>(reinterpret_cast<char*>(split) + s.scan_split_bytes());
  const float* Sc = S_chunks;
  const void* summ = summaries;
  mark(hs);
  // The direct backward reads the deltas that the forward scan keeps in the
  // summaries when it saves the chunk states: both are taken from one forward
  // call, or both recomputed here.
  if (s.bwd_direct() && !(summ && Sc)) {
    summ = nullptr;
    Sc = nullptr;
  }
  if (!summ) {
    // the forward's chunk summaries are not given: recompute them
    if (muir::launch_fwd_prep(s, q, k, v, log_a, erase, write, gamma, ws, hs) != hipSuccess)
      return MUIR_ERR_HIP;
    mark(hs);
    summ = ws;
  }
  if (!Sc) {
    // chunk-start states are not given: rerun the forward scan
    void* deltas = s.bwd_direct() ? ws : nullptr;  // summ is ws here
    if (muir::launch_fwd_scan(s, summ, S0, nullptr, S_rec, nullptr, deltas, split, hs) != hipSuccess)
      return MUIR_ERR_HIP;
    mark(hs);
    Sc = S_rec;
  }
  if (muir::launch_bwd_scan(s, summ, dO, dS_T, dS_chunks, dS0, split, hs) != hipSuccess)
    return MUIR_ERR_HIP;
  mark(hs);
  if (muir::launch_bwd_chunk(s, q, k, v, log_a, erase, write, gamma, summ, Sc, dS_chunks, dO, dq,
                             dk, dv, dlog_a, derase, dwrite, dgamma, scratch, gpart, hs) != hipSuccess)
    return MUIR_ERR_HIP;
  if (s.gmode == MUIR_GAMMA_STATIC &&
      muir::launch_gamma_sum(s, gpart, static_cast<float*>(dgamma), hs) != hipSuccess)
    return MUIR_ERR_HIP;
  mark(hs);
  return MUIR_OK;
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
