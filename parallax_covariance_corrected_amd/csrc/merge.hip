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
// (the state and partial-sum loads of a batch of its splits are issued
// together, the first batch before the sequence's length is known: one memory
// round trip for up to 16 splits), then the four wave states are combined
// through LDS in a fixed order.
#include "common.h"

namespace parallax {
namespace {

// The fields the merge needs first arrive as preloaded leading arguments.
// SPEC: the first batch of splits is requested before the length (small
// grids, where the merge's latency is what costs); otherwise a sequence that
// fits in one chunk leaves at once and no split is read speculatively.
template <int D, bool SPEC>
__global__ __launch_bounds__(256) void merge_kernel(const int* pk_seq_lens, float4* pk_ml,
                                                    float* pk_ap, void* pk_out, int pk_Hq,
                                                    int pk_max_ctx, int pk_chunk, int pk_splits,
                                                    int pk_out_f32, DecodeArgs args) {
  DecodeArgs a = args;
  a.out = pk_out;
  a.out_f32 = pk_out_f32;
  a.seq_lens = pk_seq_lens;
  a.ml = pk_ml;
  a.ap = pk_ap;
  a.Hq = pk_Hq;
  a.max_ctx = pk_max_ctx;
  a.chunk = pk_chunk;
  a.splits = pk_splits;
  constexpr int DPL = D / 64;   // dims per lane
  constexpr int U = 4;          // splits per wave whose loads are in flight together
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t bh = blockIdx.x;
  const int b = (int)(bh / a.Hq);
  // This (sequence, head)'s split states, read through buffer resources over
  // exactly its own records.
  const __amdgpu_buffer_rsrc_t mrs = make_rsrc(a.ml + bh * a.splits, (unsigned)a.splits * 16u);
  const __amdgpu_buffer_rsrc_t ars =
      make_rsrc(a.ap + bh * a.splits * 2 * D, (unsigned)a.splits * 2u * D * 4u);

  __shared__ float4 sst[4];
  __shared__ float sacc[4][2 * D];

  // A wave takes splits wave, wave + 4, ... in batches of U whose loads are all
  // in flight at once; the fold has no branch: a split past the sequence's
  // split count is weighted by zero. With SPEC the first batch is requested
  // before the length arrives (it may read stale records of splits the
  // sequence does not have); otherwise batches stop at the sequence's last
  // split, re-reading it.
  f32x4 st[U];
  float av[U][DPL], pv[U][DPL];
  auto fetch = [&](int s0, int limit) {   // splits past `limit` re-read its last one
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const unsigned s = (unsigned)min(s0 + 4 * u, limit - 1);
      st[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(mrs, s * 16u, 0, 0));
      const unsigned off = (s * 2u * D + lane * DPL) * 4u;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        av[u][k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ars, off + 4u * k, 0, 0));
        pv[u][k] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(ars, off + 4u * (D + k), 0, 0));
      }
    }
  };
  // Running state of this wave: max m, and l, S, A, P relative to it.
  float m = kNegInf, l = 0.f, S = 0.f, A[DPL], P[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) { A[k] = 0.f; P[k] = 0.f; }
  auto fold = [&](int s0, int ns) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = s0 + 4 * u < ns;
      const float mu = ok ? st[u][0] : kNegInf;
      const float mn = fmaxf(m, mu);
      const float cold = rescale(m, mn), cnew = rescale(mu, mn);
      m = mn;
      l = l * cold + (ok ? cnew * st[u][1] : 0.f);
      S = S * cold + (ok ? cnew * st[u][2] : 0.f);
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        A[k] = A[k] * cold + (ok ? cnew * av[u][k] : 0.f);
        P[k] = P[k] * cold + (ok ? cnew * pv[u][k] : 0.f);
      }
    }
  };
  if constexpr (SPEC) fetch(wave, a.splits);
  const int n = min(max(a.seq_lens[b], 0), a.max_ctx);
  // A sequence that fits in one chunk was finished by the decode kernel. With
  // SPEC the workgroup then folds nothing (ns = 0) and writes nothing: no
  // early exit, so that the first batch's loads stay ahead of the length.
  const bool single = single_chunk(a, n);
  if constexpr (!SPEC) {
    if (single) return;
  }
  const int ns = single ? 0 : (n + a.chunk - 1) / a.chunk;
  if constexpr (!SPEC) fetch(wave, ns);
  fold(wave, ns);
  for (int s0 = wave + 4 * U; s0 < ns; s0 += 4 * U) {
    fetch(s0, ns);
    fold(s0, ns);
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
      if (!single) store_output(a, bh * D + i, parallax_out(At, Pt, lt, St));
    }
  }
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, int d, LaunchEvents ev, hipStream_t s) {
  const size_t grid = (size_t)a.B * a.Hq;
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  // Speculative first batch for grids of up to one workgroup per compute unit.
  const bool spec = grid <= 256;
#define PARALLAX_LAUNCH_MERGE(DD, SP)                                                      \
  hipExtLaunchKernelGGL((merge_kernel<DD, SP>), dim3((unsigned)grid), dim3(256), 0, s,     \
                        ev.start, ev.stop, 0, a.seq_lens, a.ml, a.ap, a.out, a.Hq,         \
                        a.max_ctx, a.chunk, a.splits, a.out_f32, a)
  if (d == 64) {
    if (spec) PARALLAX_LAUNCH_MERGE(64, true);
    else PARALLAX_LAUNCH_MERGE(64, false);
  } else {
    if (spec) PARALLAX_LAUNCH_MERGE(128, true);
    else PARALLAX_LAUNCH_MERGE(128, false);
  }
#undef PARALLAX_LAUNCH_MERGE
  return hipGetLastError();
}

}  // namespace parallax
