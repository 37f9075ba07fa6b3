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
// of GH <= 8 query heads: the whole GQA group when it has at most 8 heads, so
// every K/V row is read once per group), numbered split-major so that
// consecutive workgroups —
// which the dispatcher deals round-robin to the 8 XCDs — take different
// sequences of the same split: the non-empty items of a ragged or sparsely
// filled cache then spread over every XCD. Two decompositions share the tile
// code:
//  * workgroup items (long contexts): the 4 waves of a workgroup (8 for head
//    blocks of 5 to 8 heads, whose value sums cost 2-4x the MFMAs of a small
//    block) take interleaved 16-key tiles of one item and merge their states
//    in LDS;
//  * wave items (short contexts, many sequences): every wave owns one item.
// With a ragged batch in a large cache many split-major items are empty (the
// split starts past the sequence's end). In the compacted numbering
// (workgroup items, up to 256 sequences) workgroup i takes the i-th non-empty
// item instead, longest first, so the workgroups that find nothing form one
// run at the end of the grid rather than being interleaved with working ones
// and the shortest items fill the end of the launch.
// With the probe fused in (workgroup items only), the workgroup computes rho
// of its head block from W_R and x into LDS while its first K/V tiles load.
// A sequence that fits in one chunk gets its output written directly;
// otherwise each non-empty split writes its partial state (m, l, S, A, P)
// and the merge kernel combines them.
//
// Per wave, 16-key tiles stream through a 3-deep register ring: the loads of
// tiles t+1 and t+2 are in flight while tile t is computed. K/V rows are read
// with raw buffer loads whose range ends at the last key of the item, so the
// ragged tail reads zeros without touching memory. With the prefetch flag the
// wave's first tile is requested before the sequence's length is known
// (ranged to the split's chunk instead), which takes one memory round trip
// off the start of every item; rows past the length never reach the sums.
//
// Per tile:
//  * scores and probes: one bf16 16x16x32 MFMA product K_tile (16 keys x 32
//    dims) . X^T (32 dims x 16 columns) per 32 dims and group of four heads,
//    all groups multiplying the same K registers; the columns of X are q of
//    each head (exact: bf16 x bf16 products are exact in fp32) and rho of each
//    head split as rho_hi + rho_lo in two further columns (summed after the
//    product, so rho keeps ~16 significant bits). Lane l receives keys
//    4*(l/16) + r, r = 0..3, of column l % 16. Each wave keeps its own copy
//    of X in LDS.
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

// Head block of GH <= 8 query heads (one work item), in groups of four: group
// g holds heads 4g .. 4g + hg(g) - 1 and has a score product of its own (its
// q, rho_hi and rho_lo columns fill quads 0, 1 and 2 of one 16-column MFMA
// operand). Its weight rows feed the value-sum MFMAs in one or two "sets" of
// four rows: a group of one or two heads packs (e_0 .., e p_0 ..) into one set;
// a group of three or four heads has set A (e_h) and, with the correction,
// set P (e_h p_h). Without the correction branch (plain softmax attention)
// only the e rows are accumulated.
template <int GH, bool CORR>
struct Layout {
  static_assert(GH >= 1 && GH <= 8, "head blocks of 1 to 8 query heads");
  static constexpr int NHG = (GH + 3) / 4;
  __host__ __device__ static constexpr int hg(int g) { return GH - 4 * g < 4 ? GH - 4 * g : 4; }
  __host__ __device__ static constexpr bool packed(int g) { return hg(g) <= 2; }
  __host__ __device__ static constexpr int ns(int g) { return (packed(g) || !CORR) ? 1 : 2; }
  __host__ __device__ static constexpr int base(int g) {
    int b = 0;
    for (int i = 0; i < g; ++i) b += ns(i);
    return b;
  }
  static constexpr int NSET = base(NHG);
  __host__ __device__ static constexpr int group(int set) {
    int g = 0;
    while (g + 1 < NHG && base(g + 1) <= set) ++g;
    return g;
  }
  // Weight row r of set `set` -> query head of the block (-1: unused row) and
  // whether it accumulates A (e v) or P (e p v).
  __host__ __device__ static constexpr int head(int set, int r) {
    const int g = group(set), h = hg(g);
    if (packed(g)) return r < h ? 4 * g + r : (CORR && r < 2 * h ? 4 * g + r - h : -1);
    return r < h ? 4 * g + r : -1;
  }
  __host__ __device__ static constexpr bool is_A(int set, int r) {
    const int g = group(set);
    return packed(g) ? r < hg(g) : set == base(g);
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
// holding that key's weight rows) to every block. Set s takes its rows from
// w0 of its group (packed or A set) or w1 (P set).
template <int D, int GH, bool CORR, int KK>
__device__ __forceinline__ void pv_key(const typename KV<D>::Tile& tl,
                                       const float (&w0)[Layout<GH, CORR>::NHG][4],
                                       const float (&w1)[Layout<GH, CORR>::NHG][4],
                                       f32x4 (&acc)[Layout<GH, CORR>::NSET][KV<D>::TPL]) {
  using L = Layout<GH, CORR>;
  constexpr int ABID = 4 * (KK >> 2), R = KK & 3;
#pragma unroll
  for (int t = 0; t < KV<D>::TPL; ++t) {
    const float vf = KV<D>::velem(tl.v[KK], t);
#pragma unroll
    for (int s = 0; s < L::NSET; ++s) {
      const int g = L::group(s);
      const float w = s == L::base(g) ? w0[g][R] : w1[g][R];
      acc[s][t] = __builtin_amdgcn_mfma_f32_4x4x1f32(w, vf, acc[s][t], 4, ABID, 0);
    }
  }
}
template <int D, int GH, bool CORR, int... KK>
__device__ __forceinline__ void pv_tile(const typename KV<D>::Tile& tl,
                                        const float (&w0)[Layout<GH, CORR>::NHG][4],
                                        const float (&w1)[Layout<GH, CORR>::NHG][4],
                                        f32x4 (&acc)[Layout<GH, CORR>::NSET][KV<D>::TPL],
                                        std::integer_sequence<int, KK...>) {
  (pv_key<D, GH, CORR, KK>(tl, w0, w1, acc), ...);
}

// Compacted numbering: the call's items are the non-empty (split, unit)
// pairs, where a unit is one of the `ups` (KV head, head block) pairs of a
// sequence and split s >= 1 of sequence b is non-empty when it starts before
// the sequence's end (split 0 always runs). They are numbered longest first,
// so that the short ones fill the end of the launch: every full chunk in
// split-major order, then the sequences' shorter last chunks in
// kTailClasses classes of remaining length, longest class first (a
// zero-length sequence's one item falls in the last class). Every wave of the
// workgroup computes the same answer from the B lengths
// (B <= 64 * kCompactGroups); returns false when the item does not exist.
constexpr int kCompactGroups = 4;
constexpr int kTailClasses = 8;
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
  // Rounds 0 .. splits-1 take the full chunks of split s; the following
  // kTailClasses rounds take the partial last chunks, class by class.
  for (int s = 0; s < a.splits + kTailClasses; ++s) {
    const bool tail = s >= a.splits;
    const int cls = kTailClasses - 1 - (s - a.splits);
    unsigned long long m[kCompactGroups];
    int cnt = 0;
#pragma unroll
    for (int g = 0; g < kCompactGroups; ++g) {
      const int rem = n[g] % a.chunk;   // keys in the last chunk when partial
      const bool partial = n[g] == 0 || rem > 0;
      const bool have = tail ? n[g] >= 0 && partial && (kTailClasses * rem) / a.chunk == cls
                             : n[g] >= (s + 1) * a.chunk;
      m[g] = g < groups ? __ballot(have) : 0ull;
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
          const int l = __builtin_ctzll(hit);
          const int b = 64 * g + l;
          // a partial chunk is its sequence's last split
          split = tail ? __builtin_amdgcn_readlane(n[g], l) / a.chunk
                       : __builtin_amdgcn_readfirstlane(s);
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
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(PARALLAX_DECODE_HEAD_PARAMS,
                                                             DecodeArgs args) {
  DecodeArgs a = args;
  PARALLAX_DECODE_HEAD_APPLY(a);
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
  const int c0 = split * a.chunk;
  const int len = a.seq_lens[b];

  const int grp = lane >> 4, quad = (lane & 15) >> 2, qi = lane & 3;
  const int h0 = kvh * G + hb * GH;

  // K/V streams of this (sequence, KV head), ranged to the item's keys.
  const size_t seq = ((size_t)b * a.Hkv + kvh) * (size_t)a.max_ctx;
  const char* kbase = (const char*)a.k + seq * ROW;
  const char* vbase = (const char*)a.v + seq * ROW;
  __amdgpu_buffer_rsrc_t krs, vrs;
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

  // Column role of this lane in the score/probe product of head group g:
  // quad 0 holds q of head 4g + qi, quad 1 the high and quad 2 the low bf16
  // half of rho of that head (quad 3 and heads past the group are zero). The
  // value MFMA broadcasts its weight rows from quad 0 of each 16-lane group,
  // so only quad-0 lanes carry state.
  constexpr int NHG = L::NHG;
  // Every wave builds its own copy of the q/rho operand (so no wave waits at
  // a workgroup barrier for another's loads) and requests its q and rho
  // pieces first, all at once: vector loads complete in order, so issued
  // before the K/V tiles they are waited for without waiting for the tiles,
  // and issued together (two 16-byte loads per lane and chunk, from an address
  // chosen per lane, with no branch whose results would have to be merged
  // before the next load) they cost one memory round trip. A q lane loads its
  // piece twice; lanes without a piece load their head's q and ignore it. The
  // fused probe's rho is read from LDS.
  u32x4 opc[NHG][NC][2];
  {
#pragma unroll
    for (int g = 0; g < NHG; ++g) {
      const bool valid = qi < L::hg(g);
      const size_t off = ((size_t)b * a.Hq + h0 + 4 * g + (valid ? qi : 0)) * D + 8 * grp;
      const bool from_rho = CORR && !FUSED && valid && (quad == 1 || quad == 2);
      const char* p0 = from_rho ? (const char*)(a.rho + off) : (const char*)((const uint16_t*)a.q + off);
      const char* p1 = from_rho ? p0 + 16 : p0;
      const size_t cstep = from_rho ? 32 * sizeof(float) : 32 * sizeof(uint16_t);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        opc[g][c][0] = *(const u32x4*)(p0 + c * cstep);
        opc[g][c][1] = *(const u32x4*)(p1 + c * cstep);
      }
    }
  }

  // The wave's first tile starts loading before its q/rho operand is built,
  // and the second once the sequence's length is known. With a.prefetch the
  // first is issued even before the length has arrived, ranged to the split's
  // chunk: rows past the length that it brings in are zeroed before use (in
  // compute), and an empty split waits for it and leaves. Otherwise the
  // item's range is known first. (Requesting more before the q/rho operand
  // and the length arrive measured slower: every wave of the launch does so
  // at once, and those requests queue ahead of the operand's.)
  typename C::Tile t0, t1, t2;
  int j = c0 + (WAVE_ITEM ? 0 : 16 * wave);
  const bool prefetch = !COMPACT && a.prefetch;
  if (prefetch) {
    const int cs = min(c0 + a.chunk, a.max_ctx);
    krs = make_rsrc(kbase, (unsigned)cs * ROW);
    vrs = make_rsrc(vbase, (unsigned)cs * ROW);
    load(t0, j);
  }
  // The other fields the item needs (the score scale, the epilogue's split
  // count and output type) come from the argument block; an opaque use here
  // makes the compiler load them now, under the length's wait, rather than
  // just before their first use (a round trip before the first tile's
  // scores, and one more at the end of the item).
  {
    int sp = a.splits, of = a.out_f32;
    float sc = a.scale_log2;
    asm volatile("" : "+s"(sp), "+s"(of), "+s"(sc));
    a.splits = sp;
    a.out_f32 = of;
    a.scale_log2 = sc;
  }
  const int n = min(max(len, 0), a.max_ctx);
  if (split > 0 && c0 >= n) {   // empty split (split 0 always runs: n = 0 -> out = 0)
    if (prefetch) __builtin_amdgcn_s_waitcnt(0);   // no loads in flight at exit
    return;
  }
  const int c1 = min(c0 + a.chunk, n);
  const bool direct = single_chunk(a, n);   // split 0 writes the output itself
  krs = make_rsrc(kbase, (unsigned)c1 * ROW);
  vrs = make_rsrc(vbase, (unsigned)c1 * ROW);
  if (!prefetch) load(t0, j);
  load(t1, j + STRIDE);

  // B operands at dims 32c + 8*grp + t, staged in LDS (one copy per wave,
  // written and read by that wave only) and re-read per tile.
  __shared__ u32x4 sB[NW][NHG][NC][64];
  const int bslot = wave;
  // With the probe fused in, rho of the block's heads is computed into LDS.
  __shared__ __attribute__((aligned(16))) float sR[FUSED ? GH * D : 1];
  if constexpr (FUSED) {
    probe_rows<false, NW * 64>(a.W_R, (const uint16_t*)a.x + (size_t)b * a.d_model, a.d_model,
                               (size_t)h0 * D, GH * D, sR);
    __syncthreads();
  }
  {
#pragma unroll
    for (int g = 0; g < NHG; ++g) {
      const bool valid = qi < L::hg(g);
      const int hh = 4 * g + (valid ? qi : 0);   // head within the block
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (valid && quad == 0) {
          v = opc[g][c][0];
        } else if (CORR && valid && (quad == 1 || quad == 2)) {
          u32x4 w0 = opc[g][c][0], w1 = opc[g][c][1];
          if constexpr (FUSED) {
            const float* rl = sR + (size_t)hh * D + 32 * c + 8 * grp;
            w0 = *(const u32x4*)rl;
            w1 = *(const u32x4*)(rl + 4);
          }
          const float r[8] = {__uint_as_float(w0[0]), __uint_as_float(w0[1]),
                              __uint_as_float(w0[2]), __uint_as_float(w0[3]),
                              __uint_as_float(w1[0]), __uint_as_float(w1[1]),
                              __uint_as_float(w1[2]), __uint_as_float(w1[3])};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const unsigned hi = pack_bf16x2(r[2 * w], r[2 * w + 1]);
            v[w] = quad == 1 ? hi : pack_bf16x2(r[2 * w] - bf16_lo(hi), r[2 * w + 1] - bf16_hi(hi));
          }
        }
        sB[bslot][g][c][lane] = v;
      }
    }
  }

  // Online state per head group, in the quad-0 lanes of the score columns:
  // running max (log2 domain), weight sum l and probe-weight sum S (a packed
  // group keeps S of head h in lane hg + h of lsum).
  float m_run[NHG], lsum[NHG], ssum[NHG];
#pragma unroll
  for (int g = 0; g < NHG; ++g) {
    m_run[g] = kNegInf;
    lsum[g] = 0.f;
    ssum[g] = 0.f;
  }
  f32x4 acc[NSET][TPL];
#pragma unroll
  for (int s = 0; s < NSET; ++s)
#pragma unroll
    for (int t = 0; t < TPL; ++t) acc[s][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](typename C::Tile& tl, int jt) {
    if (jt + 16 > c1) {   // last tile of the item: zero the rows past its end
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (jt + (lane & 15) >= c1) tl.k[c] = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int kk = 0; kk < 16; ++kk)
        if (jt + kk >= c1) tl.v[kk] = 0;
    }
    f32x4 sacc[NHG];
#pragma unroll
    for (int g = 0; g < NHG; ++g) sacc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int g = 0; g < NHG; ++g)
        sacc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(tl.k[c]), as_bf16x8(sB[bslot][g][c][lane]), sacc[g], 0, 0, 0);
    float w0[NHG][4], w1[NHG][4];
#pragma unroll
    for (int g = 0; g < NHG; ++g) {
      const int hgn = L::hg(g);
      const bool is_s = quad == 0 && qi < hgn;
      float x[4];
      float lmax = kNegInf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = is_s ? sacc[g][r] * a.scale_log2 : kNegInf;
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
      if (__any(is_s && lmax > m_run[g] + kRescaleThreshold)) {
        float tmax = fmaxf(lmax, __shfl_xor(lmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const bool need = is_s && tmax > m_run[g] + kRescaleThreshold;
        const float mnew = need ? tmax : m_run[g];
        const float alpha = need ? rescale(m_run[g], mnew) : 1.f;
        if (is_s) m_run[g] = mnew;
        float ah[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) ah[h] = h < hgn ? readlane_f(alpha, h) : 1.f;
#pragma unroll
        for (int s = L::base(g); s < L::base(g) + L::ns(g); ++s)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int h = L::head(s, r);
            if (h < 0) continue;
#pragma unroll
            for (int t = 0; t < TPL; ++t) acc[s][t][r] *= ah[h - 4 * g];
          }
        float a0 = 1.f, a1 = 1.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h0r = L::head(L::base(g), r);
          if (qi == r && h0r >= 0) a0 = ah[h0r - 4 * g];
          if (L::ns(g) > 1) {
            const int h1r = L::head(L::base(g) + 1, r);
            if (qi == r && h1r >= 0) a1 = ah[h1r - 4 * g];
          }
        }
        lsum[g] *= a0;
        ssum[g] *= a1;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = is_s ? fast_exp2(x[r] - m_run[g]) : 0.f;
        // p = k . (rho_hi + rho_lo): the two halves sit 4 and 8 lanes up.
        const float p = CORR ? dpp<kDppRowShl4>(sacc[g][r]) + dpp<kDppRowShl8>(sacc[g][r]) : 0.f;
        const float ep = e * p;
        if (L::packed(g)) {
          // weight rows (e_0 .. e_{hg-1}, ep_0 .. ep_{hg-1}): lane qi >= hg
          // takes ep of head qi - hg from its quad.
          const float eps = hgn == 2 ? dpp<0x44>(ep) : dpp<0x00>(ep);
          w0[g][r] = qi < hgn ? e : (qi < 2 * hgn ? eps : 0.f);
          w1[g][r] = 0.f;
          lsum[g] += w0[g][r];
        } else {
          w0[g][r] = e;
          w1[g][r] = ep;
          lsum[g] += e;
          if constexpr (CORR) ssum[g] += ep;
        }
      }
    }
    pv_tile<D, GH, CORR>(tl, w0, w1, acc, std::make_integer_sequence<int, 16>{});
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
#pragma unroll
  for (int g = 0; g < NHG; ++g) {
    lsum[g] += __shfl_xor(lsum[g], 16);
    lsum[g] += __shfl_xor(lsum[g], 32);
    if (!L::packed(g) && CORR) {
      ssum[g] += __shfl_xor(ssum[g], 16);
      ssum[g] += __shfl_xor(ssum[g], 32);
    }
  }
  // Lane l holds A and P of every head of the block at dims TPL*l + t.
  if constexpr (WAVE_ITEM) {
    float mh[GH], lh[GH], sh[GH];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      const int g = h / 4, qh = h % 4;
      mh[h] = readlane_f(m_run[g], qh);
      lh[h] = readlane_f(lsum[g], qh);
      sh[h] = L::packed(g) ? readlane_f(lsum[g], L::hg(g) + qh) : readlane_f(ssum[g], qh);
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
#pragma unroll
    for (int g = 0; g < NHG; ++g) {
      const int hgn = L::hg(g);
      if (lane < hgn) sM[wave][4 * g + lane] = m_run[g];
      if (L::packed(g)) {
        if (lane < hgn) sL[wave][4 * g + lane] = lsum[g];
        else if (lane < 2 * hgn) sS[wave][4 * g + lane - hgn] = CORR ? lsum[g] : 0.f;
      } else {
        if (lane < hgn) {
          sL[wave][4 * g + lane] = lsum[g];
          sS[wave][4 * g + lane] = ssum[g];
        }
      }
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

// Query heads per work item: the whole GQA group up to 8 heads (one read of
// each K/V row per group); larger groups in blocks of the largest divisor <= 8.
int head_block(int G) {
  for (int gh = 8; gh > 1; --gh)
    if (G % gh == 0) return gh;
  return 1;
}

template <int D, bool WI, int NW, bool CORR, bool CP, bool FU = false>
hipError_t launch_dw(const DecodeArgs& a, LaunchEvents ev, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int GH = head_block(G);
  const size_t items = (size_t)a.B * a.Hkv * (G / GH) * a.splits;
  const size_t grid = WI ? (items + NW - 1) / NW : items;
  if (grid > 0x7fffffffu || items > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid);
#define PARALLAX_LAUNCH_GH(N)                                                              \
  case N: {                                                                                \
    /* head blocks of 5-8 heads: 8-wave workgroup items (two waves per SIMD) */            \
    constexpr int NWX = (!WI && N >= 5) ? 8 : NW;                                          \
    hipExtLaunchKernelGGL((decode_mfma_kernel<D, N, WI, NWX, CORR, CP, FU>), g,            \
                          dim3(NWX * 64), 0, s,                                            \
                          ev.start, ev.stop, 0, PARALLAX_DECODE_HEAD_ARGS(a), a);          \
    break;                                                                                 \
  }
  switch (GH) {
    PARALLAX_LAUNCH_GH(8)
    PARALLAX_LAUNCH_GH(7)
    PARALLAX_LAUNCH_GH(6)
    PARALLAX_LAUNCH_GH(5)
    PARALLAX_LAUNCH_GH(4)
    PARALLAX_LAUNCH_GH(3)
    PARALLAX_LAUNCH_GH(2)
    PARALLAX_LAUNCH_GH(1)
    default: return hipErrorInvalidValue;
  }
#undef PARALLAX_LAUNCH_GH
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
  // One-wave items go two to a workgroup: a finished wave's slot is refilled
  // without waiting for three others (4 per workgroup measured 1.5% slower on
  // the large batch, 1 per workgroup the same as 2).
  if (wave_items)
    return d == 64 ? launch_dw<64, true, 2, CORR, false>(a, ev, s)
                   : launch_dw<128, true, 2, CORR, false>(a, ev, s);
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
