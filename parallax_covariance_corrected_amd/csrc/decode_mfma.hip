// Matrix-core Parallax decode kernel for gfx950 (bf16 K/V cache, d in {64, 128}).
//
// What it computes (zubnet.ai (pt), "Parallax mantém softmax ...", second
// paragraph): per query head, softmax attention minus the softmax-weighted KV
// covariance times the probe rho, in the one-pass form
//   out = A/l - (P/l - (A/l)(S/l)),  l = sum e, S = sum e p, A = sum e v,
//   P = sum e p v,  e = exp(s - m),  s = q.k/sqrt(d),  p = k.rho,
// with both branches fed by one read of each K/V row (same paragraph: the KV
// stream is shared, which is what doubles the arithmetic intensity).
//
// Work items. An item is (split of `chunk` keys, sequence, KV head, head block
// of GH query heads), numbered split-major so that consecutive workgroups —
// which the dispatcher deals round-robin to the 8 XCDs — take different
// sequences of the same split: the non-empty items of a ragged or sparsely
// filled cache then spread over every XCD. Two decompositions share the tile
// code:
//  * workgroup items (long contexts): the 4 waves of a workgroup take
//    interleaved 16-key tiles of one item and merge their states in LDS;
//  * wave items (short contexts, many sequences): every wave owns one item.
// With a ragged batch in a large cache many split-major items are empty (the
// split starts past the sequence's end). In the compacted numbering
// (workgroup items, up to 256 sequences) workgroup i takes the i-th non-empty
// item of the split-major order instead, so the workgroups that find nothing
// form one run at the end of the grid rather than being interleaved with
// working ones.
// With the probe fused in (workgroup items only), the workgroup computes rho
// of its head block from W_R and x into LDS while its first K/V tiles load.
// A sequence that fits in one chunk gets its output written directly;
// otherwise each non-empty split writes its partial state (m, l, S, A, P)
// and the merge kernel combines them.
//
// Per wave, 16-key tiles stream through a 3-deep register ring: the loads of
// tiles t+1 and t+2 are in flight while tile t is computed. K/V rows are read
// with raw buffer loads whose range ends at the last key of the item, so the
// ragged tail reads zeros without touching memory and nothing past seq_lens is
// ever read.
//
// Per tile:
//  * scores and probes: one bf16 16x16x32 MFMA product K_tile (16 keys x 32
//    dims) . X^T (32 dims x 16 columns) per 32 dims; the columns of X are q of
//    each head (exact: bf16 x bf16 products are exact in fp32) and rho of each
//    head split as rho_hi + rho_lo in two further columns (summed after the
//    product, so rho keeps ~16 significant bits). Lane l receives keys
//    4*(l/16) + r, r = 0..3, of column l % 16. X lives in LDS.
//  * online softmax with a lazy rescale: the running max moves only when a
//    score exceeds it by more than 8 (log2 units), so e <= 2^8 between
//    rescales; the common path needs no cross-lane reduction.
//  * weights: e and e*p formed in the lanes of the score columns, the probe
//    halves fetched with DPP row shifts.
//  * weighted value sums: fp32 4x4x1 MFMA blocks with the A operand broadcast
//    from one block (the weight rows (e_h, e_h p_h) of one key) to all 16
//    blocks, whose B operands are 64 consecutive value dims of that key (one
//    32-bit load of 2 bf16 dims per lane). Weights stay fp32 (a bf16 weight
//    would cost about 1e-3 relative error), V needs no transpose, and each
//    lane accumulates only its own dims.
#include <type_traits>
#include <utility>

#include "common.h"

namespace parallax {
namespace {

constexpr float kRescaleThreshold = 8.0f;   // log2 units
// K/V rows are read exactly once: non-temporal loads keep them from displacing
// reused lines in the caches.
constexpr int kStreamLoad = 2;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int kDppRowShl4 = 0x104;   // lane i reads lane i+4 of its 16-lane row
constexpr int kDppRowShl8 = 0x108;   // lane i reads lane i+8 of its 16-lane row

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

template <int GH, bool CORR>
struct Layout {
  // Weight row r of MFMA set `set` -> query head of the block (-1: unused row)
  // and whether it accumulates A (e v) or P (e p v). Without the correction
  // branch (plain softmax attention) only the A rows are accumulated.
  static constexpr int NSET = (GH <= 2 || !CORR) ? 1 : 2;
  __device__ static constexpr int head(int set, int r) {
    return GH <= 2 ? (r < GH ? r : (r < 2 * GH ? r - GH : -1)) : (r < GH ? r : -1);
  }
  __device__ static constexpr bool is_A(int set, int r) {
    return GH <= 2 ? (r < GH) : (set == 0);
  }
};

template <int D>
struct KV {
  static constexpr int NC = D / 32;    // 32-dim chunks of the score product
  static constexpr int TPL = D / 64;   // value dims per lane (per key)
  static constexpr int ROW = 2 * D;    // bytes per cache row
  using VE = typename std::conditional<D == 128, unsigned, unsigned short>::type;
  struct Tile {
    u32x4 k[NC];
    VE v[16];
  };
  __device__ static VE vload(__amdgpu_buffer_rsrc_t r, unsigned off) {
    if constexpr (D == 128) return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kStreamLoad);
    else return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kStreamLoad);
  }
  __device__ static float velem(VE w, int t) {
    if constexpr (D == 128) return t ? bf16_hi(w) : bf16_lo(w);
    else return bf16_bits_to_f32(w);
  }
};

// Weighted value sums of key KK of a tile: broadcast block 4*(KK/4) (the lanes
// holding that key's weight rows) to every block.
template <int D, int NSET, int KK>
__device__ __forceinline__ void pv_key(const typename KV<D>::Tile& tl, const float (&w0)[4],
                                       const float (&w1)[4], f32x4 (&acc)[NSET][KV<D>::TPL]) {
  constexpr int ABID = 4 * (KK >> 2), R = KK & 3;
#pragma unroll
  for (int t = 0; t < KV<D>::TPL; ++t) {
    const float vf = KV<D>::velem(tl.v[KK], t);
    acc[0][t] = __builtin_amdgcn_mfma_f32_4x4x1f32(w0[R], vf, acc[0][t], 4, ABID, 0);
    if constexpr (NSET > 1)
      acc[1][t] = __builtin_amdgcn_mfma_f32_4x4x1f32(w1[R], vf, acc[1][t], 4, ABID, 0);
  }
}
template <int D, int NSET, int... KK>
__device__ __forceinline__ void pv_tile(const typename KV<D>::Tile& tl, const float (&w0)[4],
                                        const float (&w1)[4], f32x4 (&acc)[NSET][KV<D>::TPL],
                                        std::integer_sequence<int, KK...>) {
  (pv_key<D, NSET, KK>(tl, w0, w1, acc), ...);
}

// Compacted numbering: item `item` of the call is the item-th non-empty
// (split, unit) pair in split-major order, where a unit is one of the `ups`
// (KV head, head block) pairs of a sequence and split s >= 1 of sequence b is
// non-empty when it starts before the sequence's end (split 0 always runs).
// Every wave of the workgroup computes the same answer from the B lengths
// (B <= 64 * kCompactGroups); returns false when the item does not exist.
constexpr int kCompactGroups = 4;
__device__ __forceinline__ bool compact_item(const DecodeArgs& a, int item, int ups, int& split,
                                             int& unit_id) {
  const int lane = threadIdx.x & 63;
  const int groups = (a.B + 63) >> 6;
  int n[kCompactGroups];
  int mine = 0;   // non-empty splits of this lane's sequences
#pragma unroll
  for (int g = 0; g < kCompactGroups; ++g) {
    const int b = 64 * g + lane;
    n[g] = b < a.B ? min(max(a.seq_lens[b], 0), a.max_ctx) : -1;
    if (n[g] >= 0) mine += max(1, (n[g] + a.chunk - 1) / a.chunk);
  }
  // Workgroups past the last non-empty item leave at once.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mine += __shfl_xor(mine, o);
  if (item >= mine * ups) return false;
  int base = 0;
  for (int s = 0; s < a.splits; ++s) {
    const int lo = s * a.chunk;
    unsigned long long m[kCompactGroups];
    int cnt = 0;
#pragma unroll
    for (int g = 0; g < kCompactGroups; ++g) {
      m[g] = g < groups ? __ballot(s == 0 ? n[g] >= 0 : n[g] > lo) : 0ull;
      cnt += __popcll(m[g]);
    }
    const int span = cnt * ups;
    if (item < base + span) {
      int r = (item - base) / ups;
      const int within = (item - base) - r * ups;
#pragma unroll
      for (int g = 0; g < kCompactGroups; ++g) {
        const int c = __popcll(m[g]);
        if (r < c) {
          // the lane holding the r-th set bit of m[g]
          const unsigned below = __builtin_amdgcn_mbcnt_hi(
              (unsigned)(m[g] >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m[g], 0u));
          const unsigned long long hit = __ballot(((m[g] >> lane) & 1ull) && (int)below == r);
          const int b = 64 * g + __builtin_ctzll(hit);
          split = __builtin_amdgcn_readfirstlane(s);
          unit_id = __builtin_amdgcn_readfirstlane(b * ups + within);
          return true;
        }
        r -= c;
      }
    }
    base += span;
  }
  return false;
}

template <int D, int GH, bool WAVE_ITEM, int NW, bool CORR, bool COMPACT, bool FUSED>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(!FUSED || (CORR && !WAVE_ITEM), "the fused probe serves workgroup items");
  using L = Layout<GH, CORR>;
  using C = KV<D>;
  constexpr int NC = C::NC, TPL = C::TPL, ROW = C::ROW, NSET = L::NSET;
  constexpr int STRIDE = WAVE_ITEM ? 16 : 16 * NW;   // keys between a wave's tiles

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int G = a.Hq / a.Hkv;
  const int hblocks = G / GH;
  const int units = a.B * a.Hkv * hblocks;
  int item = WAVE_ITEM ? blockIdx.x * NW + wave : blockIdx.x;
  if (WAVE_ITEM && item >= units * a.splits) return;
  int split, unit_id;
  if constexpr (COMPACT) {
    static_assert(!WAVE_ITEM, "compacted numbering is for workgroup items");
    if (!compact_item(a, item, units / a.B, split, unit_id)) return;
  } else {
    split = item / units;
    unit_id = item - split * units;
  }
  const int hb = unit_id % hblocks;
  const int kvh = (unit_id / hblocks) % a.Hkv;
  const int b = unit_id / hblocks / a.Hkv;
  const int n = min(max(a.seq_lens[b], 0), a.max_ctx);
  const int c0 = split * a.chunk;
  if (split > 0 && c0 >= n) return;   // empty split (split 0 always runs: n = 0 -> out = 0)
  const int c1 = min(c0 + a.chunk, n);
  const bool direct = single_chunk(a, n);   // split 0 writes the output itself

  const int grp = lane >> 4, quad = (lane & 15) >> 2, qi = lane & 3;
  const int h0 = kvh * G + hb * GH;

  // K/V streams of this (sequence, KV head), ranged to [0, c1).
  const size_t seq = ((size_t)b * a.Hkv + kvh) * (size_t)a.max_ctx;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc((const char*)a.k + seq * ROW, (unsigned)c1 * ROW);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const char*)a.v + seq * ROW, (unsigned)c1 * ROW);
  const unsigned koff = (lane & 15) * ROW + 16 * grp;
  const unsigned voff = lane * (ROW / 64);
  auto load = [&](typename C::Tile& t, int j) {
    const unsigned base = (unsigned)j * ROW;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      t.k[c] = __builtin_amdgcn_raw_buffer_load_b128(krs, base + koff + 64 * c, 0, kStreamLoad);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) t.v[kk] = C::vload(vrs, base + voff + kk * ROW);
  };

  // Start streaming before the q/rho prologue so the latencies overlap.
  typename C::Tile t0, t1, t2;
  int j = c0 + (WAVE_ITEM ? 0 : 16 * wave);
  load(t0, j);
  load(t1, j + STRIDE);

  // Column role of this lane in the score/probe product: quad 0 holds q of
  // head qi, quad 1 the high and quad 2 the low bf16 half of rho of head qi
  // (quad 3 and heads >= GH are zero). The value MFMA broadcasts its weight
  // rows from quad 0 of each 16-lane group, so only quad-0 lanes carry state.
  const bool is_s = quad == 0 && qi < GH;

  // B operand at dims 32c + 8*grp + t, staged in LDS and re-read per tile: one
  // copy per wave for wave items, one per workgroup (written by wave 0) for
  // workgroup items.
  constexpr int NBS = WAVE_ITEM ? NW : 1;
  const int bslot = WAVE_ITEM ? wave : 0;
  __shared__ u32x4 sB[NBS][NC][64];
  const float* rsrc = a.rho;
  if constexpr (FUSED) {
    __shared__ __attribute__((aligned(16))) float sR[GH * D];
    probe_rows<false, NW * 64>(a.W_R, (const uint16_t*)a.x + (size_t)b * a.d_model, a.d_model,
                               (size_t)h0 * D, GH * D, sR);
    __syncthreads();
    rsrc = sR;
  }
  if (WAVE_ITEM || wave == 0) {
    const size_t bh = (size_t)b * a.Hq + h0 + (qi < GH ? qi : 0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      const size_t off = bh * D + 32 * c + 8 * grp;
      if (qi < GH && quad == 0) {
        v = *(const u32x4*)((const uint16_t*)a.q + off);
      } else if (CORR && qi < GH && (quad == 1 || quad == 2)) {
        const size_t roff = FUSED ? (size_t)qi * D + 32 * c + 8 * grp : off;
        const float4 r0 = *(const float4*)(rsrc + roff);
        const float4 r1 = *(const float4*)(rsrc + roff + 4);
        const float r[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const unsigned hi = pack_bf16x2(r[2 * w], r[2 * w + 1]);
          v[w] = quad == 1 ? hi : pack_bf16x2(r[2 * w] - bf16_lo(hi), r[2 * w + 1] - bf16_hi(hi));
        }
      }
      sB[bslot][c][lane] = v;
    }
  }
  if constexpr (!WAVE_ITEM) __syncthreads();

  float m_run = kNegInf;      // running max (log2 domain), score lanes
  float lsum = 0.f, ssum = 0.f;
  f32x4 acc[NSET][TPL];
#pragma unroll
  for (int s = 0; s < NSET; ++s)
#pragma unroll
    for (int t = 0; t < TPL; ++t) acc[s][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const typename C::Tile& tl, int jt) {
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tl.k[c]),
                                                     as_bf16x8(sB[bslot][c][lane]), sacc, 0, 0, 0);
    float x[4];
    float lmax = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = is_s ? sacc[r] * a.scale_log2 : kNegInf;
      lmax = fmaxf(lmax, x[r]);
    }
    if (jt + 16 > c1) {   // last tile of the item: mask keys past its end
      lmax = kNegInf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (jt + 4 * grp + r >= c1) x[r] = kNegInf;
        lmax = fmaxf(lmax, x[r]);
      }
    }
    if (__any(is_s && lmax > m_run + kRescaleThreshold)) {
      float tmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const bool need = is_s && tmax > m_run + kRescaleThreshold;
      const float mnew = need ? tmax : m_run;
      const float alpha = need ? rescale(m_run, mnew) : 1.f;
      if (is_s) m_run = mnew;
      float ah[GH];
#pragma unroll
      for (int h = 0; h < GH; ++h) ah[h] = readlane_f(alpha, h);
#pragma unroll
      for (int s = 0; s < NSET; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = L::head(s, r);
          if (h < 0) continue;
#pragma unroll
          for (int t = 0; t < TPL; ++t) acc[s][t][r] *= ah[h];
        }
      float a0 = 1.f, a1 = 1.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (qi == r && L::head(0, r) >= 0) a0 = ah[L::head(0, r)];
        if (NSET > 1 && qi == r && L::head(1, r) >= 0) a1 = ah[L::head(1, r)];
      }
      lsum *= a0;
      ssum *= a1;
    }
    float w0[4], w1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = is_s ? fast_exp2(x[r] - m_run) : 0.f;
      // p = k . (rho_hi + rho_lo): the two halves sit 4 and 8 lanes up.
      const float p = CORR ? dpp<kDppRowShl4>(sacc[r]) + dpp<kDppRowShl8>(sacc[r]) : 0.f;
      const float ep = e * p;
      if constexpr (GH <= 2) {
        // weight rows (e_0 .. e_{GH-1}, ep_0 .. ep_{GH-1}): lane qi >= GH takes
        // ep of head qi - GH from its quad.
        constexpr int kQuadPerm = GH == 2 ? 0x44 : 0x00;
        const float eps = dpp<kQuadPerm>(ep);
        w0[r] = qi < GH ? e : (qi < 2 * GH ? eps : 0.f);
        w1[r] = 0.f;
        lsum += w0[r];
      } else {
        w0[r] = e;
        w1[r] = ep;
        lsum += w0[r];
        if constexpr (CORR) ssum += w1[r];
      }
    }
    pv_tile<D, NSET>(tl, w0, w1, acc, std::make_integer_sequence<int, 16>{});
  };

  // Three-deep ring: compute tile t while tiles t+1, t+2 are loading (deeper
  // rings and 8-wave workgroups measured slower).
  while (j < c1) {
    load(t2, j + 2 * STRIDE);
    compute(t0, j);
    j += STRIDE;
    if (j >= c1) break;
    load(t0, j + 2 * STRIDE);
    compute(t1, j);
    j += STRIDE;
    if (j >= c1) break;
    load(t1, j + 2 * STRIDE);
    compute(t2, j);
    j += STRIDE;
  }

  // Sum the per-lane weight sums over the four key slots (lane groups of 16).
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if constexpr (NSET > 1) {
    ssum += __shfl_xor(ssum, 16);
    ssum += __shfl_xor(ssum, 32);
  }
  // Lane l holds A and P of every head of the block at dims TPL*l + t.
  if constexpr (WAVE_ITEM) {
    float mh[GH], lh[GH], sh[GH];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      mh[h] = readlane_f(m_run, h);
      lh[h] = readlane_f(lsum, h);
      sh[h] = (GH <= 2) ? readlane_f(lsum, GH + h) : readlane_f(ssum, h);
    }
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      const size_t bh = (size_t)b * a.Hq + h0 + h;
#pragma unroll
      for (int t = 0; t < TPL; ++t) {
        float Av = 0.f, Pv = 0.f;
#pragma unroll
        for (int s = 0; s < NSET; ++s)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (L::head(s, r) != h) continue;
            if (L::is_A(s, r)) Av = acc[s][t][r];
            else Pv = acc[s][t][r];
          }
        const int i = TPL * lane + t;
        if (direct) {
          store_output(a, bh * D + i, parallax_out(Av, Pv, lh[h], sh[h]));
        } else {
          const size_t ps = bh * a.splits + split;
          a.ap[ps * 2 * D + i] = Av;
          a.ap[ps * 2 * D + D + i] = Pv;
        }
      }
      if (!direct && lane == 0)
        a.ml[bh * a.splits + split] = make_float4(mh[h], lh[h], sh[h], 0.f);
    }
    return;
  } else {
    __shared__ float sA[NW][GH][D], sP[NW][GH][D], sM[NW][GH], sL[NW][GH], sS[NW][GH];
    if constexpr (!CORR) {   // no P rows are accumulated: the P sums are zero
#pragma unroll
      for (int h = 0; h < GH; ++h)
#pragma unroll
        for (int t = 0; t < TPL; ++t) sP[wave][h][TPL * lane + t] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < NSET; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = L::head(s, r);
        if (h < 0) continue;
#pragma unroll
        for (int t = 0; t < TPL; ++t) {
          if (L::is_A(s, r)) sA[wave][h][TPL * lane + t] = acc[s][t][r];
          else sP[wave][h][TPL * lane + t] = acc[s][t][r];
        }
      }
    if (lane < GH) sM[wave][lane] = m_run;
    if constexpr (GH <= 2) {
      if (lane < GH) sL[wave][lane] = lsum;
      else if (lane < 2 * GH) sS[wave][lane - GH] = lsum;
    } else {
      if (lane < GH) { sL[wave][lane] = lsum; sS[wave][lane] = ssum; }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < GH * D; idx += NW * 64) {
      const int h = idx / D, i = idx % D;
      float M = sM[0][h];
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, sM[w][h]);
      float lt = 0.f, St = 0.f, At = 0.f, Pt = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
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
}

int head_block(int G) {
  if (G <= 4) return G;
  if (G % 4 == 0) return 4;
  if (G % 3 == 0) return 3;
  if (G % 2 == 0) return 2;
  return 1;
}

template <int D, bool WI, int NW, bool CORR, bool CP, bool FU = false>
hipError_t launch_dw(const DecodeArgs& a, LaunchEvents ev, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int GH = head_block(G);
  const size_t items = (size_t)a.B * a.Hkv * (G / GH) * a.splits;
  const size_t grid = WI ? (items + NW - 1) / NW : items;
  if (grid > 0x7fffffffu || items > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), blk(NW * 64);
  switch (GH) {
    case 4: hipExtLaunchKernelGGL((decode_mfma_kernel<D, 4, WI, NW, CORR, CP, FU>), g, blk, 0, s, ev.start, ev.stop, 0, a); break;
    case 3: hipExtLaunchKernelGGL((decode_mfma_kernel<D, 3, WI, NW, CORR, CP, FU>), g, blk, 0, s, ev.start, ev.stop, 0, a); break;
    case 2: hipExtLaunchKernelGGL((decode_mfma_kernel<D, 2, WI, NW, CORR, CP, FU>), g, blk, 0, s, ev.start, ev.stop, 0, a); break;
    default: hipExtLaunchKernelGGL((decode_mfma_kernel<D, 1, WI, NW, CORR, CP, FU>), g, blk, 0, s, ev.start, ev.stop, 0, a); break;
  }
  return hipGetLastError();
}

template <bool CORR>
hipError_t launch_d(const DecodeArgs& a, int d, int wave_items, int compact, LaunchEvents ev,
                    hipStream_t s) {
  if constexpr (CORR) {
    if (a.W_R)
      return d == 64 ? launch_dw<64, false, 4, true, false, true>(a, ev, s)
                     : launch_dw<128, false, 4, true, false, true>(a, ev, s);
  }
  if (wave_items)
    return d == 64 ? launch_dw<64, true, 4, CORR, false>(a, ev, s)
                   : launch_dw<128, true, 4, CORR, false>(a, ev, s);
  if (compact)
    return d == 64 ? launch_dw<64, false, 4, CORR, true>(a, ev, s)
                   : launch_dw<128, false, 4, CORR, true>(a, ev, s);
  return d == 64 ? launch_dw<64, false, 4, CORR, false>(a, ev, s)
                 : launch_dw<128, false, 4, CORR, false>(a, ev, s);
}

}  // namespace

bool decode_mfma_supported(int d, int G) { return (d == 64 || d == 128) && G >= 1; }

hipError_t launch_decode_mfma(const DecodeArgs& a, int d, int wave_items, int compact, int fused,
                              LaunchEvents ev, hipStream_t s) {
  if (compact && (wave_items || a.B > 64 * kCompactGroups)) return hipErrorInvalidValue;
  if (fused) {
    if (wave_items || compact || !a.W_R || !a.x) return hipErrorInvalidValue;
    DecodeArgs f = a;
    f.rho = nullptr;
    return launch_d<true>(f, d, 0, 0, ev, s);
  }
  // rho == nullptr selects plain softmax attention (no correction branch).
  DecodeArgs u = a;
  u.W_R = nullptr;
  return u.rho ? launch_d<true>(u, d, wave_items, compact, ev, s)
               : launch_d<false>(u, d, wave_items, compact, ev, s);
}

}  // namespace parallax
