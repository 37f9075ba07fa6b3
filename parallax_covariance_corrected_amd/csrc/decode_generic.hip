// Generic vector-ALU Parallax decode kernel (fp32 or bf16 storage, d in {64, 128},
// any GQA group). Serves the fp32 path (decode, and prefill with one "sequence"
// per token) and cross-checks the matrix-core kernel.
//
// One workgroup (4 waves) per (split, sequence, KV head, head block). With the
// probe fused in, the workgroup first computes rho of its head block from W_R
// and x into LDS (rho never goes through memory). Each key
// is read by LPK lanes with one 16-byte load of K and one of V; the lanes of a
// key reduce the score s = q.k and the probe p = k.rho with xor shuffles and
// keep their own exact online state (m, l, S, A, P). States are merged across
// key groups (shuffles) and waves (LDS) by their running maxima; the merge
// kernel combines the splits of a long sequence. Both
// branches read the same K/V rows (zubnet.ai (pt), "Parallax mantém softmax
// ...", second paragraph: one KV stream feeds softmax and correction).
#include "common.h"

namespace parallax {
namespace {

template <bool F32IN>
struct Elem;
template <>
struct Elem<true> {
  static constexpr int kSize = 4;
  static constexpr int kPerLoad = 4;
  __device__ static void unpack(const u32x4& w, float* f) {
    f[0] = __uint_as_float(w[0]); f[1] = __uint_as_float(w[1]);
    f[2] = __uint_as_float(w[2]); f[3] = __uint_as_float(w[3]);
  }
};
template <>
struct Elem<false> {
  static constexpr int kSize = 2;
  static constexpr int kPerLoad = 8;
  __device__ static void unpack(const u32x4& w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(w[i]); f[2 * i + 1] = bf16_hi(w[i]); }
  }
};

__device__ __forceinline__ void combine(float& m, float& l, float& S, float* A, float* P,
                                        float m2, float l2, float S2, const float* A2,
                                        const float* P2, int n) {
  float M = fmaxf(m, m2);
  float c1 = rescale(m, M), c2 = rescale(m2, M);
  l = c1 * l + c2 * l2;
  S = c1 * S + c2 * S2;
  for (int i = 0; i < n; ++i) {
    A[i] = c1 * A[i] + c2 * A2[i];
    P[i] = c1 * P[i] + c2 * P2[i];
  }
  m = M;
}

template <bool F32IN, int D, int GB, bool FUSED>
__global__ __launch_bounds__(256) void decode_generic_kernel(PARALLAX_DECODE_HEAD_PARAMS,
                                                             DecodeArgs args) {
  DecodeArgs a = args;
  PARALLAX_DECODE_HEAD_APPLY(a);
  using E = Elem<F32IN>;
  constexpr int EPL = E::kPerLoad;   // elements per lane
  constexpr int LPK = D / EPL;       // lanes per key
  constexpr int KPW = 64 / LPK;      // keys per wave per step
  constexpr int ROW = D * E::kSize;  // bytes per cache row

  const int G = a.Hq / a.Hkv;
  const int hblocks = G / GB;
  // Split-major numbering: consecutive workgroups (dealt round-robin to the
  // XCDs) take different sequences of the same split.
  const int units = a.B * a.Hkv * hblocks;
  const int split = blockIdx.x / units;
  const int unit_id = blockIdx.x - split * units;
  const int hb = unit_id % hblocks;
  const int kvh = (unit_id / hblocks) % a.Hkv;
  const int b = unit_id / hblocks / a.Hkv;
  // Cache sequence and number of keys: decode reads seq_lens; the many-query
  // form maps sequence b to token b % T of cache sequence b / T.
  int cb = b, n;
  if (a.T > 0) {
    cb = b / a.T;
    const int pre = min(max(a.prefix ? a.prefix[cb] : 0, 0), a.max_ctx - a.T);
    n = pre + b % a.T + 1;
  } else {
    n = min(max(a.seq_lens[b], 0), a.max_ctx);
  }
  const int c0 = split * a.chunk;
  if (split > 0 && c0 >= n) return;   // empty split (split 0 always runs: n = 0 -> out = 0)
  const int c1 = min(c0 + a.chunk, n);
  const bool direct = single_chunk(a, n);   // split 0 writes the output itself

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kg = lane / LPK, sub = lane % LPK;
  const int h0 = kvh * G + hb * GB;

  // Keys are taken in batches of U per lane whose K/V loads are in flight
  // together; the first batch and q are requested before the probe, so that
  // their memory round trips overlap the probe's.
  constexpr int U = 4;
  constexpr int STEP = 4 * KPW;      // keys between a lane's consecutive keys
  const size_t seq = ((size_t)cb * a.Hkv + kvh) * (size_t)a.max_ctx;
  const char* kb = (const char*)a.k + seq * ROW + sub * 16;
  const char* vb = (const char*)a.v + seq * ROW + sub * 16;
  u32x4 kw[U], vw[U];
  auto fetch = [&](int jb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = jb + u * STEP;
        kw[u] = j < c1 ? *(const u32x4*)(kb + (size_t)j * ROW) : (u32x4){0u, 0u, 0u, 0u};
        vw[u] = j < c1 ? *(const u32x4*)(vb + (size_t)j * ROW) : (u32x4){0u, 0u, 0u, 0u};
      }
    };
    const int j0 = c0 + wave * KPW + kg;
    u32x4 qw[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h)
      qw[h] = *(const u32x4*)((const char*)a.q + (((size_t)b * a.Hq + h0 + h) * D + sub * EPL) * E::kSize);
    fetch(j0);

    const float* rsrc = a.rho;   // null: softmax only
    if constexpr (FUSED) {
      __shared__ float sR[GB * D];
      probe_rows<F32IN, 256>(a.W_R, (const char*)a.x + (size_t)b * a.d_model * E::kSize, a.d_model,
                             (size_t)h0 * D, GB * D, sR);
      __syncthreads();
      rsrc = sR;
    }
    float qf[GB][EPL], rf[GB][EPL];
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      E::unpack(qw[h], qf[h]);
      const size_t rbase = FUSED ? (size_t)h * D + sub * EPL : ((size_t)b * a.Hq + h0 + h) * D + sub * EPL;
#pragma unroll
      for (int i = 0; i < EPL; ++i) rf[h][i] = rsrc ? rsrc[rbase + i] : 0.f;
    }

    float m[GB], l[GB], S[GB], A[GB][EPL], P[GB][EPL];
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      m[h] = kNegInf; l[h] = 0.f; S[h] = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) { A[h][i] = 0.f; P[h][i] = 0.f; }
    }

    for (int jb = j0; jb < c1; jb += U * STEP) {
      u32x4 kc[U], vc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) { kc[u] = kw[u]; vc[u] = vw[u]; }
      if (jb + U * STEP < c1) fetch(jb + U * STEP);   // the next batch in flight
#pragma unroll
      for (int u = 0; u < U; ++u) {
      const int j = jb + u * STEP;
      if (j >= c1) break;
      float kf[EPL], vf[EPL];
      E::unpack(kc[u], kf);
      E::unpack(vc[u], vf);
#pragma unroll
      for (int h = 0; h < GB; ++h) {
        float s = 0.f, p = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) { s = fmaf(qf[h][i], kf[i], s); p = fmaf(rf[h][i], kf[i], p); }
#pragma unroll
        for (int o = 1; o < LPK; o <<= 1) { s += __shfl_xor(s, o); p += __shfl_xor(p, o); }
        s *= a.scale_log2;
        const float mn = fmaxf(m[h], s);
        const float al = rescale(m[h], mn);
        const float e = fast_exp2(s - mn);
        const float ep = e * p;
        l[h] = fmaf(l[h], al, e);
        S[h] = fmaf(S[h], al, ep);
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          A[h][i] = fmaf(A[h][i], al, e * vf[i]);
          P[h][i] = fmaf(P[h][i], al, ep * vf[i]);
        }
        m[h] = mn;
      }
    }
  }

  // Merge the key groups of this wave.
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) {
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      float A2[EPL], P2[EPL];
      const float m2 = __shfl_xor(m[h], o), l2 = __shfl_xor(l[h], o), S2 = __shfl_xor(S[h], o);
#pragma unroll
      for (int i = 0; i < EPL; ++i) { A2[i] = __shfl_xor(A[h][i], o); P2[i] = __shfl_xor(P[h][i], o); }
      combine(m[h], l[h], S[h], A[h], P[h], m2, l2, S2, A2, P2, EPL);
    }
  }

  // Merge the four waves through LDS.
  __shared__ float sA[4][GB][D], sP[4][GB][D], sM[4][GB], sL[4][GB], sS[4][GB];
  if (kg == 0) {
#pragma unroll
    for (int h = 0; h < GB; ++h) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) { sA[wave][h][sub * EPL + i] = A[h][i]; sP[wave][h][sub * EPL + i] = P[h][i]; }
      if (sub == 0) { sM[wave][h] = m[h]; sL[wave][h] = l[h]; sS[wave][h] = S[h]; }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < GB * D; idx += 256) {
    const int h = idx / D, i = idx % D;
    float M = sM[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sM[w][h]);
    float lt = 0.f, St = 0.f, At = 0.f, Pt = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float c = rescale(sM[w][h], M);
      lt = fmaf(c, sL[w][h], lt); St = fmaf(c, sS[w][h], St);
      At = fmaf(c, sA[w][h][i], At); Pt = fmaf(c, sP[w][h][i], Pt);
    }
    const size_t bh = (size_t)b * a.Hq + h0 + h;
    if (direct) {
      store_output(a, bh * D + i, parallax_out(At, Pt, lt, St));
    } else {
      const size_t ps = bh * a.splits + split;
      a.ap[ps * 2 * D + i] = At;
      a.ap[ps * 2 * D + D + i] = Pt;
      if (i == 0) a.ml[ps] = make_float4(M, lt, St, 0.f);
    }
  }
}

template <bool F32IN, int D, bool FUSED>
hipError_t launch_d(const DecodeArgs& a, LaunchEvents ev, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int GB = (G % 4 == 0) ? 4 : (G % 3 == 0) ? 3 : (G % 2 == 0) ? 2 : 1;
  const size_t grid = (size_t)a.B * a.Hkv * (G / GB) * a.splits;
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), blk(256);
  switch (GB) {
    case 4: hipExtLaunchKernelGGL((decode_generic_kernel<F32IN, D, 4, FUSED>), g, blk, 0, s, ev.start, ev.stop, 0, PARALLAX_DECODE_HEAD_ARGS(a), a); break;
    case 3: hipExtLaunchKernelGGL((decode_generic_kernel<F32IN, D, 3, FUSED>), g, blk, 0, s, ev.start, ev.stop, 0, PARALLAX_DECODE_HEAD_ARGS(a), a); break;
    case 2: hipExtLaunchKernelGGL((decode_generic_kernel<F32IN, D, 2, FUSED>), g, blk, 0, s, ev.start, ev.stop, 0, PARALLAX_DECODE_HEAD_ARGS(a), a); break;
    default: hipExtLaunchKernelGGL((decode_generic_kernel<F32IN, D, 1, FUSED>), g, blk, 0, s, ev.start, ev.stop, 0, PARALLAX_DECODE_HEAD_ARGS(a), a); break;
  }
  return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_f(const DecodeArgs& a, int d, int f32_inputs, LaunchEvents ev, hipStream_t s) {
  if (f32_inputs)
    return d == 64 ? launch_d<true, 64, FUSED>(a, ev, s) : launch_d<true, 128, FUSED>(a, ev, s);
  return d == 64 ? launch_d<false, 64, FUSED>(a, ev, s) : launch_d<false, 128, FUSED>(a, ev, s);
}

}  // namespace

hipError_t launch_decode_generic(const DecodeArgs& a, int d, int f32_inputs, int fused,
                                 LaunchEvents ev, hipStream_t s) {
  if (fused && (a.T > 0 || !a.W_R || !a.x)) return hipErrorInvalidValue;
  return fused ? launch_f<true>(a, d, f32_inputs, ev, s) : launch_f<false>(a, d, f32_inputs, ev, s);
}

}  // namespace parallax
