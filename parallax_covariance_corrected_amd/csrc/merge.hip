// Split-K merge and epilogue for Parallax decode.
//
// Each split of a (sequence, query head) holds a partial online state
// (m, l, S, A, P) relative to its own running max m (log2 domain). The merge
// rescales every split by exp2(m_i - M), M = max_i m_i, sums them and applies
// the epilogue out = A/l - (P/l - (A/l)(S/l)), i.e. softmax attention minus the
// softmax-weighted KV covariance times the probe (zubnet.ai (pt), "Parallax
// mantém softmax ...", second paragraph). Only the splits that cover
// [0, seq_lens[b]) are read; sequences that fit in one chunk (length 0
// included) were finished by the decode kernel and are skipped.
//
// One workgroup per (sequence, query head): its 4 waves take interleaved
// splits (loads of several splits in flight per wave), lanes own D/64 dims,
// and the waves' sums are combined through LDS in a fixed order.
#include "common.h"

namespace parallax {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
  constexpr int DPL = D / 64;   // dims per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t bh = blockIdx.x;
  const int b = (int)(bh / a.Hq);
  const int n = min(max(a.seq_lens[b], 0), a.max_ctx);
  if (single_chunk(a, n)) return;   // written by the decode kernel
  const int ns = (n + a.chunk - 1) / a.chunk;
  const float4* ml = a.ml + bh * a.splits;
  const float* ap = a.ap + bh * a.splits * 2 * D;

  __shared__ float sred[4];
  __shared__ float sacc[4][2 * D + 2];

  float mloc = kNegInf;
  for (int s = threadIdx.x; s < ns; s += 256) mloc = fmaxf(mloc, ml[s].x);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
  if (lane == 0) sred[wave] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(sred[0], sred[1]), fmaxf(sred[2], sred[3]));

  float l = 0.f, S = 0.f, A[DPL], P[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) { A[k] = 0.f; P[k] = 0.f; }
#pragma unroll 4
  for (int s = wave; s < ns; s += 4) {
    const float4 st = ml[s];
    const float* p = ap + (size_t)s * 2 * D + lane * DPL;
    float av[DPL], pv[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) { av[k] = p[k]; pv[k] = p[D + k]; }
    const float c = rescale(st.x, M);
    l = fmaf(c, st.y, l);
    S = fmaf(c, st.z, S);
#pragma unroll
    for (int k = 0; k < DPL; ++k) { A[k] = fmaf(c, av[k], A[k]); P[k] = fmaf(c, pv[k], P[k]); }
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    sacc[wave][lane * DPL + k] = A[k];
    sacc[wave][D + lane * DPL + k] = P[k];
  }
  if (lane == 0) { sacc[wave][2 * D] = l; sacc[wave][2 * D + 1] = S; }
  __syncthreads();
  if (wave == 0) {
    const float lt = sacc[0][2 * D] + sacc[1][2 * D] + sacc[2][2 * D] + sacc[3][2 * D];
    const float St = sacc[0][2 * D + 1] + sacc[1][2 * D + 1] + sacc[2][2 * D + 1] + sacc[3][2 * D + 1];
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int i = lane * DPL + k;
      const float At = sacc[0][i] + sacc[1][i] + sacc[2][i] + sacc[3][i];
      const float Pt = sacc[0][D + i] + sacc[1][D + i] + sacc[2][D + i] + sacc[3][D + i];
      store_output(a, bh * D + i, parallax_out(At, Pt, lt, St));
    }
  }
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, int d, LaunchEvents ev, hipStream_t s) {
  const size_t grid = (size_t)a.B * a.Hq;
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if (d == 64) hipExtLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, ev.start, ev.stop, 0, a);
  else hipExtLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

}  // namespace parallax
