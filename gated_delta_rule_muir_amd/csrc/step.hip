// Decode step of the Muir gated delta rule: one token for N streams x H heads.
//
// Per (stream, head), with the fp32 state S (dk x dv, rows = key channels):
//   S' = diag(exp(log_a)) S
//   r  = S'^T (gamma*q)          p = S'^T (erase*k)       (two column reductions)
//   d  = write*v - p
//   o  = r + (gamma*q . k) d     (the readout of S' + k d^T, without re-reading it)
//   S  = S' + k d^T
// (arXiv 2611.08376: abstract -- decay, erase the key's prediction, write;
// Methodology -- row-wise decay and the readout gate on the query.)
//
// The step is bound by HBM: one read and one write of S.  Each workgroup owns
// one head and a 64-column slice of S; every thread keeps its part of the
// slice (DK/16 rows x 4 columns) in registers between the reductions and the
// write-back, so S is streamed exactly once each way with 16-byte accesses.
#include "device_common.h"
#include "kernels.h"

namespace muir {

constexpr int STEP_THREADS = 256;
constexpr int STEP_COLS = 64;  // state columns per workgroup

// NT: the state is streamed with non-temporal loads and stores (chosen for
// states larger than the 256 MB Infinity Cache; smaller ones stay cacheable
// across steps).
template <typename Tin, int DK, bool NT>
__global__ __launch_bounds__(STEP_THREADS) void step_kernel(
    int H, int DV, const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ log_a, const Tin* __restrict__ erase, const Tin* __restrict__ write,
    const Tin* __restrict__ gamma, float* __restrict__ S, Tin* __restrict__ o, int gmode) {
  constexpr int RP = DK / 16;  // rows per thread
  const int nslices = DV / STEP_COLS;
  const int head = blockIdx.x / nslices;  // flattened (n, h)
  const int slice = blockIdx.x % nslices;
  const int tid = threadIdx.x;
  const int cg = tid & 15;   // column group: columns 4*cg .. 4*cg+3 of the slice
  const int rg = tid >> 4;   // row group: rows rg + 16*p

  __shared__ float s_alpha[DK], s_ek[DK], s_qt[DK], s_k[DK];
  __shared__ float s_red[2][STEP_THREADS / 64][4][STEP_COLS];  // [r|p][wave][row-group in wave][col]
  __shared__ float s_qk;

  // Every global read is issued before the first wait, in the order it is
  // needed: the per-head vectors, this thread's part of the state slice, and
  // its write and v words (kept raw until used).  Loads complete in order, so
  // the wait for the vectors does not wait for the state.
  const size_t vk = static_cast<size_t>(head) * DK;
  constexpr int VPT = (DK + STEP_THREADS - 1) / STEP_THREADS;  // vector elements per thread
  float xk[VPT], xl[VPT], xe[VPT], xg[VPT], xq[VPT];
  // readout gate per token, static per (head, channel), or none (its address
  // then points into q and the value is not used)
  const Tin* gsrc = gmode == GAMMA_NONE ? q : gamma;
#pragma unroll
  for (int e = 0; e < VPT; ++e) {
    const int j = min(tid + e * STEP_THREADS, DK - 1);
    xk[e] = Elem<Tin>::load(k, vk + j);
    xl[e] = Elem<Tin>::load(log_a, vk + j);
    xe[e] = Elem<Tin>::load(erase, vk + j);
    xg[e] = Elem<Tin>::load(gsrc, gmode == GAMMA_STATIC ? static_cast<size_t>(head % H) * DK + j : vk + j);
    xq[e] = Elem<Tin>::load(q, vk + j);
  }
  const int col0 = slice * STEP_COLS + 4 * cg;
  float* Sh = S + static_cast<size_t>(head) * DK * DV;
  f32x4 st[RP];
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    const float* src = Sh + static_cast<size_t>(rg + 16 * p) * DV + col0;
    if constexpr (NT) st[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
    else st[p] = load4(src);
  }
  const size_t vv = static_cast<size_t>(head) * DV + col0;
  const typename Raw4<Tin>::type wraw = *reinterpret_cast<const typename Raw4<Tin>::type*>(write + vv);
  const typename Raw4<Tin>::type vraw = *reinterpret_cast<const typename Raw4<Tin>::type*>(v + vv);

  // (threads past DK repeat element DK-1 with the same values: no branch, so
  // the compiler does not drain the state loads at a join)
#pragma unroll
  for (int e = 0; e < VPT; ++e) {
    const int j = min(tid + e * STEP_THREADS, DK - 1);
    s_alpha[j] = __expf(xl[e]);
    s_ek[j] = xe[e] * xk[e];
    s_qt[j] = (gmode == GAMMA_NONE ? 1.f : xg[e]) * xq[e];
    s_k[j] = xk[e];
  }
  __syncthreads();

  // q~ . k : one wave reduces it while the others go on with the state.
  if (tid < 64) {
    float acc = 0.f;
    for (int j = tid; j < DK; j += 64) acc += s_qt[j] * s_k[j];
    acc = wave_sum(acc);
    if (tid == 0) s_qk = acc;
  }

  f32x4 racc = zero4(), pacc = zero4();
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    const int row = rg + 16 * p;
    const float a = s_alpha[row];
    st[p] = st[p] * a;
    racc += st[p] * s_qt[row];
    pacc += st[p] * s_ek[row];
  }
  // reduce over the 4 row groups inside the wave (lanes l, l^16, l^32, l^48)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    racc[i] += __shfl_xor(racc[i], 16, 64);
    racc[i] += __shfl_xor(racc[i], 32, 64);
    pacc[i] += __shfl_xor(pacc[i], 16, 64);
    pacc[i] += __shfl_xor(pacc[i], 32, 64);
  }
  const int wave = tid >> 6;
  const int lane = tid & 63;
  if (lane < 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s_red[0][wave][0][4 * cg + i] = racc[i];
      s_red[1][wave][0][4 * cg + i] = pacc[i];
    }
  }
  __syncthreads();
  // every thread needs d for its 4 columns: sum the per-wave partials
  f32x4 rr = zero4(), pp = zero4();
#pragma unroll
  for (int w = 0; w < STEP_THREADS / 64; ++w)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rr[i] += s_red[0][w][0][4 * cg + i];
      pp[i] += s_red[1][w][0][4 * cg + i];
    }
  const f32x4 u = load4(reinterpret_cast<const Tin*>(&wraw)) * load4(reinterpret_cast<const Tin*>(&vraw));
  f32x4 d = u - pp;
  if (tid < 16) {
    f32x4 ov = rr + s_qk * d;
    store4(o + vv, ov);
  }
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    const int row = rg + 16 * p;
    float* dst = Sh + static_cast<size_t>(row) * DV + col0;
    if constexpr (NT) __builtin_nontemporal_store(st[p] + s_k[row] * d, reinterpret_cast<f32x4*>(dst));
    else store4(dst, st[p] + s_k[row] * d);
  }
}

hipError_t launch_step(int N, int H, int dk, int dv, bool bf16, int gmode, const void* q,
                       const void* k, const void* v, const void* log_a, const void* erase,
                       const void* write, const void* gamma, float* S, void* o, hipStream_t stream) {
  const int grid = N * H * (dv / STEP_COLS);
  if (grid == 0) return hipSuccess;
  // states beyond the Infinity Cache (256 MB) are streamed non-temporally
  const bool nt = static_cast<size_t>(N) * H * dk * dv * sizeof(float) >= (static_cast<size_t>(256) << 20);
#define MUIR_STEP_LAUNCH1(TT, DD, NTV)                                                                  \
  hipLaunchKernelGGL((step_kernel<TT, DD, NTV>), dim3(grid), dim3(STEP_THREADS), 0, stream, H, dv,     \
                     (const TT*)q, (const TT*)k, (const TT*)v, (const TT*)log_a, (const TT*)erase,      \
                     (const TT*)write, (const TT*)gamma, S, (TT*)o, gmode)
#define MUIR_STEP_LAUNCH(TT, DD)                    \
  do {                                              \
    if (nt) MUIR_STEP_LAUNCH1(TT, DD, true);        \
    else MUIR_STEP_LAUNCH1(TT, DD, false);          \
  } while (0)
  if (bf16) {
    if (dk == 128) MUIR_STEP_LAUNCH(uint16_t, 128);
    else MUIR_STEP_LAUNCH(uint16_t, 64);
  } else {
    if (dk == 128) MUIR_STEP_LAUNCH(float, 128);
    else MUIR_STEP_LAUNCH(float, 64);
  }
#undef MUIR_STEP_LAUNCH
#undef MUIR_STEP_LAUNCH1
  return hipGetLastError();
}

}  // namespace muir
