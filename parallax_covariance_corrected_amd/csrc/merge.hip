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
// splits, lanes own D/64 dims. Each wave folds its splits with a running max
// (so the state and partial-sum loads of all its splits are issued together:
// one memory round trip), then the four wave states are combined through LDS
// in a fixed order.
#include "common.h"

namespace parallax {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(PARALLAX_DECODE_HEAD_PARAMS, DecodeArgs args) {
  DecodeArgs a = args;
  PARALLAX_DECODE_HEAD_APPLY(a);
  constexpr int DPL = D / 64;   // dims per lane
  constexpr int U = 4;          // splits per wave whose loads are in flight together
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t bh = blockIdx.x;
  const int b = (int)(bh / a.Hq);
  const int n = min(max(a.seq_lens[b], 0), a.max_ctx);
  if (single_chunk(a, n)) return;   // written by the decode kernel
  const int ns = (n + a.chunk - 1) / a.chunk;
  const float4* ml = a.ml + bh * a.splits;
  const float* ap = a.ap + bh * a.splits * 2 * D;

  __shared__ float4 sst[4];
  __shared__ float sacc[4][2 * D];

  // Running state of this wave: max m, and l, S, A, P relative to it.
  float m = kNegInf, l = 0.f, S = 0.f, A[DPL], P[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) { A[k] = 0.f; P[k] = 0.f; }
  for (int s0 = wave; s0 < ns; s0 += 4 * U) {
    float4 st[U];
    float av[U][DPL], pv[U][DPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + 4 * u;
      st[u] = s < ns ? ml[s] : make_float4(kNegInf, 0.f, 0.f, 0.f);
      const float* p = ap + (size_t)min(s, ns - 1) * 2 * D + lane * DPL;
#pragma unroll
      for (int k = 0; k < DPL; ++k) { av[u][k] = p[k]; pv[u][k] = p[D + k]; }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + 4 * u >= ns) break;
      const float mn = fmaxf(m, st[u].x);
      const float cold = rescale(m, mn), cnew = rescale(st[u].x, mn);
      m = mn;
      l = l * cold + cnew * st[u].y;
      S = S * cold + cnew * st[u].z;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        A[k] = A[k] * cold + cnew * av[u][k];
        P[k] = P[k] * cold + cnew * pv[u][k];
      }
    }
  }
  if (lane == 0) sst[wave] = make_float4(m, l, S, 0.f);
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    sacc[wave][lane * DPL + k] = A[k];
    sacc[wave][D + lane * DPL + k] = P[k];
  }
  __syncthreads();
  if (wave == 0) {
    const float M = fmaxf(fmaxf(sst[0].x, sst[1].x), fmaxf(sst[2].x, sst[3].x));
    float c[4], lt = 0.f, St = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      c[w] = rescale(sst[w].x, M);
      lt += c[w] * sst[w].y;
      St += c[w] * sst[w].z;
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int i = lane * DPL + k;
      float At = 0.f, Pt = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        At += c[w] * sacc[w][i];
        Pt += c[w] * sacc[w][D + i];
      }
      store_output(a, bh * D + i, parallax_out(At, Pt, lt, St));
    }
  }
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, int d, LaunchEvents ev, hipStream_t s) {
  const size_t grid = (size_t)a.B * a.Hq;
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if (d == 64) hipExtLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, ev.start, ev.stop, 0,
                                        PARALLAX_DECODE_HEAD_ARGS(a), a);
  else hipExtLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, ev.start, ev.stop, 0,
                                        PARALLAX_DECODE_HEAD_ARGS(a), a);
  return hipGetLastError();
}

}  // namespace parallax
