// Split-K merge and epilogue for Parallax decode.
//
// Each split of a (sequence, query head) holds a partial online state
// (m, l, S, A, P) relative to its own running max m (log2 domain). The merge
// rescales every split by exp2(m_i - M), M = max_i m_i, sums them and applies
// the epilogue out = A/l - (P/l - (A/l)(S/l)), i.e. softmax attention minus the
// softmax-weighted KV covariance times the probe (zubnet.ai (pt), "Parallax
// mantém softmax ...", second paragraph). Only the splits that cover
// [0, seq_lens[b]) are read; a sequence of length 0 gets out = 0.
#include "common.h"

namespace parallax {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
  constexpr int HPW = 256 / D;   // (sequence, head) pairs per workgroup
  const int hl = threadIdx.x / D, i = threadIdx.x % D;
  const size_t bh = (size_t)blockIdx.x * HPW + hl;
  if (bh >= (size_t)a.B * a.Hq) return;
  const int b = (int)(bh / a.Hq);
  const int n = min(max(a.seq_lens[b], 0), a.max_ctx);
  const int ns = (n + a.chunk - 1) / a.chunk;
  const float4* ml = a.ml + bh * a.splits;
  const float* ap = a.ap + bh * a.splits * 2 * D;

  float M = kNegInf;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[s].x);
  float l = 0.f, S = 0.f, A = 0.f, P = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float4 st = ml[s];
    const float c = rescale(st.x, M);
    l = fmaf(c, st.y, l);
    S = fmaf(c, st.z, S);
    A = fmaf(c, ap[(size_t)s * 2 * D + i], A);
    P = fmaf(c, ap[(size_t)s * 2 * D + D + i], P);
  }
  const float o = parallax_out(A, P, l, S);
  if (a.out_f32) store_out<float>((float*)a.out + bh * D + i, o);
  else store_out<uint16_t>((uint16_t*)a.out + bh * D + i, o);
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, int d, hipStream_t s) {
  const size_t pairs = (size_t)a.B * a.Hq;
  const int hpw = 256 / d;
  const size_t grid = (pairs + hpw - 1) / hpw;
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if (d == 64) hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace parallax
