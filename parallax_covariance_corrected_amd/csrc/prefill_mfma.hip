// Causal many-query Parallax forward (prefill) on the bf16 matrix cores.
//
// Token t of sequence b sits at cache position prefix[b] + t and attends to
// cache rows 0 .. prefix[b] + t; its output is softmax attention minus the
// softmax-weighted KV covariance times its own probe (zubnet.ai (pt),
// "Parallax mantém softmax ...", second paragraph), in the one-pass form
//   out = A/l - (P/l - (A/l)(S/l)),  l = sum e, S = sum e p, A = sum e v,
//   P = sum e p v,  e = exp(s - m),  s = q.k/sqrt(d),  p = k.rho.
//
// Work: a workgroup owns 64 rows of one (sequence, KV head): rows are the
// flattened (token, query head of the group) pairs, so the G query heads that
// share a KV head share every K/V tile. Four waves of 16 rows. Keys advance in
// blocks of 64 through double-buffered LDS, up to the last key any row of the
// workgroup may see; a wave skips the blocks that lie entirely after its own
// rows. K and V tiles go from memory straight into LDS (buffer loads with an
// LDS destination: no staging registers, no LDS store instructions), both
// row-major (a row per key) with their 16-byte chunks permuted per row so that
// the operand reads below hit distinct LDS banks; the permutation is applied
// by choosing which global chunk each lane fetches, since lane L of such a
// load always writes the 16 bytes at the piece's base + 16 L.
//
// Everything is computed transposed (keys x rows), which keeps every step in
// the lane that produced it:
//  * S^T = K Q^T and Pr^T = K R^T with bf16 16x16x32 MFMAs (K tile as the A
//    operand from LDS, q and rho of the wave's rows as B operands in
//    registers). q.k products of bf16 are exact in fp32; rho enters as two bf16
//    terms hi + lo accumulated into the same product (16 significant bits).
//    Lane l receives keys 4*(l/16) + r of row l % 16.
//  * online softmax per row (lane's row = l % 16) with a lazy rescale: the
//    running max moves only when a block max exceeds it by more than 8 (log2
//    units).
//  * weights e and e*p in fp32, split into bf16 hi + lo (a bf16 weight alone
//    would cost ~1e-3 relative error), become the B operand of O^T = V^T E^T
//    directly from the registers that hold them: the MFMA's k slots are bound
//    to keys (4*(l/16) + t of two 16-key sub-tiles), and the A operand V^T
//    gets the same keys from the row-major V tile through the gfx950
//    transposing LDS read (ds_read_b64_tr_b16: in each 16-lane group, lane j
//    receives element j % 4 of the 4-element reads of lanes 4c + j / 4,
//    c = 0..3, so a lane ends up with one dim of four keys).
#include "common.h"

namespace parallax {
namespace {

constexpr int kPfRows = 64;        // rows per workgroup
constexpr int kPfKeys = 64;        // keys per block
constexpr int kPfThreads = 256;
constexpr float kPfRescale = 8.0f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// Tiles: row = key, D*2 bytes; 16-byte chunk c of row r sits at slot
// c ^ swz(r). K: the 16 rows one score-operand read touches (one chunk each)
// fall in distinct bank groups. V: a transposing read touches 16 rows x 2
// adjacent chunks (2 dt, 2 dt + 1); an even swizzle keeps the pair adjacent
// and spreads the rows over the banks.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) { return (2 * row) & (D / 8 - 1); }

template <int D>
struct PfSmem {
  unsigned char k[2][kPfKeys * D * 2];
  unsigned char v[2][kPfKeys * D * 2];
};
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ unsigned pk2(float lo, float hi) { return pack_bf16x2(lo, hi); }

// A row's four lanes are l16 + 16*grp, grp = 0..3. The permlane swaps (gfx950)
// hand every lane the value of the lane 16 apart and then 32 apart, in
// registers (no LDS round trip): after a swap each lane holds its own value
// and its partner's.
__device__ __forceinline__ float row_max4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// CORR = false: plain softmax attention (no probe products, no e*p sums).
// Two waves per SIMD (at most 256 registers per lane) is part of the design:
// the second wave's MFMAs cover the first one's softmax and LDS staging. The
// attribute keeps the register allocator from trading that occupancy away (a
// build at one wave per SIMD measured 1.4x slower).
template <int D, bool F32_OUT, bool CORR>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int NKS = D / 32;            // 32-dim k-steps of the score product
  constexpr int NDT = D / 16;            // 16-dim output tiles
  constexpr int ROW = D * 2;             // bytes per K/V cache row
  constexpr int PIECES = kPfKeys * ROW / 1024;        // 1 KB pieces per tile
  static_assert(PIECES % 4 == 0, "every wave loads the same number of pieces");
  __shared__ __attribute__((aligned(16))) PfSmem<D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  const int G = a.Hq / a.Hkv;
  const int TG = a.T * G;
  const int nrb = (TG + kPfRows - 1) / kPfRows;
  const int rb = nrb - 1 - (int)blockIdx.x;          // heaviest row blocks first
  const int g = blockIdx.y, b = blockIdx.z;
  const int F0 = rb * kPfRows;
  int prefix = a.prefix ? a.prefix[b] : 0;
  prefix = min(max(prefix, 0), a.max_ctx - a.T);
  const int nvalid = prefix + a.T;                   // cache rows that exist

  // Rows of this lane (column of the transposed products) and of the wave.
  const int F = F0 + 16 * wave + l16;
  const bool row_ok = F < TG;
  const int tok = row_ok ? F / G : 0;
  const int head = g * G + (row_ok ? F % G : 0);
  const int pos = row_ok ? prefix + tok : -1;        // last key this row sees
  const int Fw_last = min(F0 + 16 * wave + 15, TG - 1);
  const int wave_last_key = F0 + 16 * wave < TG ? prefix + Fw_last / G : -1;
  // Smallest position of the wave's rows (-1 when it holds rows past the end):
  // key blocks that end at or before it need no causal mask.
  const int wave_first_key = Fw_last == F0 + 16 * wave + 15 ? prefix + (F0 + 16 * wave) / G : -1;
  const int wg_last_key = prefix + (min(F0 + kPfRows, TG) - 1) / G;
  const int nkb = wg_last_key / kPfKeys + 1;

  // K/V of (b, g): rows past nvalid read as zero (buffer range).
  const size_t kv_base = ((size_t)b * a.Hkv + g) * (size_t)a.max_ctx * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc((const uint16_t*)a.k + kv_base, (unsigned)nvalid * ROW);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const uint16_t*)a.v + kv_base, (unsigned)nvalid * ROW);

  // Key block kb -> LDS stage buf: wave w fills the 1 KB pieces w, w + 4, ...
  // of each tile; lane L's 16 bytes land at byte 16 L of the piece, i.e. at
  // slot (row, sc), which holds global chunk sc ^ swz(row).
  auto stage = [&](int kb, int buf) {
#pragma unroll
    for (int pc = 0; pc < PIECES / 4; ++pc) {
      const int piece = 4 * pc + wave;
      const int byte = piece * 1024 + 16 * lane;
      const int row = byte / ROW, sc = (byte % ROW) / 16;
      const unsigned grow = (unsigned)(kb * kPfKeys + row) * ROW;
      // (offsets in variables: with a device-function call inside the builtin's
      // arguments the host compilation pass silently drops the kernel)
      const unsigned ko = grow + 16u * (sc ^ k_swz<D>(row));
      const unsigned vo = grow + 16u * (sc ^ v_swz<D>(row));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&sm.k[buf][piece * 1024], 16, ko, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&sm.v[buf][piece * 1024], 16, vo, 0, 0, 0);
    }
  };

  stage(0, 0);   // start streaming before the q/rho prologue

  // q and rho of this lane's row as B operands: dims 32*ks + 8*grp .. +7.
  u32x4 qb[NKS], rh[NKS], rl[NKS];
  {
    const size_t off = (((size_t)b * a.T + tok) * a.Hq + head) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 qv = {0u, 0u, 0u, 0u}, hv = {0u, 0u, 0u, 0u}, lv = {0u, 0u, 0u, 0u};
      if (row_ok) {
        qv = *(const u32x4*)((const uint16_t*)a.q + off + 32 * ks);
      }
      if (CORR && row_ok) {
        const float4 r0 = *(const float4*)(a.rho + off + 32 * ks);
        const float4 r1 = *(const float4*)(a.rho + off + 32 * ks + 4);
        const float r[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const unsigned hi = pk2(r[2 * w], r[2 * w + 1]);
          hv[w] = hi;
          lv[w] = pk2(r[2 * w] - bf16_lo(hi), r[2 * w + 1] - bf16_hi(hi));
        }
      }
      qb[ks] = qv;
      rh[ks] = hv;
      rl[ks] = lv;
    }
  }

  f32x4 oa[NDT], op[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) {
    oa[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    op[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  float m_run = kNegInf, lpart = 0.f, spart = 0.f;

  // Each wave waits for its own LDS-destination loads; the barrier then
  // publishes the whole stage.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    // stage cur ^ 1 was last read before the previous barrier
    if (kb + 1 < nkb) stage(kb + 1, cur ^ 1);
    if (kb * kPfKeys <= wave_last_key) {
      // ---- scores and probes, 4 sub-tiles of 16 keys. k-steps outside,
      // sub-tiles inside: eight independent accumulators between dependent
      // MFMAs; the K operands of the next k-step are read ahead.
      f32x4 s[4], pr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        pr[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
      u32x4 kcur[4], knext[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        kcur[j] = *(const u32x4*)&sm.k[cur][(16 * j + l16) * ROW + 16 * (grp ^ k_swz<D>(16 * j + l16))];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks + 1 < NKS) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            knext[j] = *(const u32x4*)&sm.k[cur][(16 * j + l16) * ROW +
                                                 16 * ((4 * (ks + 1) + grp) ^ k_swz<D>(16 * j + l16))];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kcur[j]), as_bf16x8(qb[ks]), s[j], 0, 0, 0);
          if constexpr (CORR)
            pr[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kcur[j]), as_bf16x8(rh[ks]), pr[j], 0, 0, 0);
        }
        if constexpr (CORR) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            pr[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kcur[j]), as_bf16x8(rl[ks]), pr[j], 0, 0, 0);
        }
        if (ks + 1 < NKS) {
#pragma unroll
          for (int j = 0; j < 4; ++j) kcur[j] = knext[j];
        }
      }
      // ---- causal mask (only blocks that reach past a row of the wave), block
      // max of this lane's row on the raw scores
      if (kb * kPfKeys + kPfKeys - 1 > wave_first_key) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kb * kPfKeys + 16 * j + 4 * grp + r > pos) s[j][r] = kNegInf;
      }
      float bmax = kNegInf;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) bmax = fmaxf(bmax, s[j][r]);
      bmax = row_max4(bmax) * a.scale_log2;   // log2 domain
      // Lazy rescale: the running max moves only when the block max exceeds it
      // by a margin; the branch is taken by the whole wave, rarely.
      const bool moves = bmax > m_run + kPfRescale;
      if (__any(moves)) {
        const float c = moves ? rescale(m_run, bmax) : 1.f;
        m_run = moves ? bmax : m_run;
        lpart *= c;
        spart *= c;
#pragma unroll
        for (int i = 0; i < NDT; ++i) {
          oa[i] *= c;
          op[i] *= c;
        }
      }
      // A row with no key yet keeps m = -inf; its scores are all -inf, and
      // exp2(-inf - 0) = 0.
      const float neg_m = m_run == kNegInf ? 0.f : -m_run;
      // ---- weights, then O^T += V^T (e, e*p)^T per 32-key step
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        float e[8], ep[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int j = 2 * h2 + (t >> 2), r = t & 3;
          e[t] = fast_exp2(fmaf(s[j][r], a.scale_log2, neg_m));
          ep[t] = CORR ? e[t] * pr[j][r] : 0.f;
          lpart += e[t];
          if constexpr (CORR) spart += ep[t];
        }
        u32x4 eh, el, ph, pl;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          eh[w] = pk2(e[2 * w], e[2 * w + 1]);
          el[w] = pk2(e[2 * w] - bf16_lo(eh[w]), e[2 * w + 1] - bf16_hi(eh[w]));
          if constexpr (CORR) {
            ph[w] = pk2(ep[2 * w], ep[2 * w + 1]);
            pl[w] = pk2(ep[2 * w] - bf16_lo(ph[w]), ep[2 * w + 1] - bf16_hi(ph[w]));
          }
        }
        // A operand: dims 16*dt + l16 of keys 32*h2 + 4*grp .. +3 and
        // 32*h2 + 16 + 4*grp .. +3 (the keys bound to k slots t = 0..7), by two
        // transposing reads: lane 4c + q of a 16-lane group reads dims
        // 16*dt + 4q .. +3 of key 32*h2 + 4*grp + c (+ 16).
        const int vkey = 32 * h2 + 4 * grp + (l16 >> 2);
        const unsigned char* vb = &sm.v[cur][vkey * ROW + 8 * (lane & 3)];
        const int vsw = v_swz<D>(vkey);   // the same for vkey + 16
        auto vload = [&](int dt) {
          const int o = 16 * ((2 * dt) ^ vsw);
          const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(vb + o));
          const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(vb + 16 * ROW + o));
          const u32x2 a0 = __builtin_bit_cast(u32x2, r0), a1 = __builtin_bit_cast(u32x2, r1);
          return (u32x4){a0[0], a0[1], a1[0], a1[1]};
        };
        // hi terms of tile dt, then lo terms of tile dt - 1: no accumulator is
        // hit by two MFMAs in a row.
        u32x4 vprev = vload(0);
        u32x4 vcur = vprev;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const u32x4 vnext = dt + 1 < NDT ? vload(dt + 1) : vcur;
          oa[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vcur), as_bf16x8(eh), oa[dt], 0, 0, 0);
          if constexpr (CORR)
            op[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vcur), as_bf16x8(ph), op[dt], 0, 0, 0);
          if (dt > 0) {
            oa[dt - 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vprev), as_bf16x8(el), oa[dt - 1], 0, 0, 0);
            if constexpr (CORR)
              op[dt - 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vprev), as_bf16x8(pl), op[dt - 1], 0, 0, 0);
          }
          vprev = vcur;
          vcur = vnext;
        }
        oa[NDT - 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vprev), as_bf16x8(el), oa[NDT - 1], 0, 0, 0);
        if constexpr (CORR)
          op[NDT - 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vprev), as_bf16x8(pl), op[NDT - 1], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: row sums over the 4 lanes of the row, then out
  lpart = row_sum4(lpart);
  if constexpr (CORR) spart = row_sum4(spart);
  if (!row_ok) return;
  const size_t obase = (((size_t)b * a.T + tok) * a.Hq + head) * D + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    float o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = parallax_out(oa[dt][r], op[dt][r], lpart, spart);
    if constexpr (F32_OUT) {
      *(float4*)((float*)a.out + obase + 16 * dt) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
      *(u32x2*)((uint16_t*)a.out + obase + 16 * dt) = (u32x2){pk2(o[0], o[1]), pk2(o[2], o[3])};
    }
  }
}

}  // namespace

template <int D, bool CORR>
void launch_pf(const PrefillArgs& a, dim3 grid, LaunchEvents ev, hipStream_t s) {
  if (a.out_f32)
    hipExtLaunchKernelGGL((prefill_mfma_kernel<D, true, CORR>), grid, dim3(kPfThreads), 0, s, ev.start, ev.stop, 0, a);
  else
    hipExtLaunchKernelGGL((prefill_mfma_kernel<D, false, CORR>), grid, dim3(kPfThreads), 0, s, ev.start, ev.stop, 0, a);
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, int d, LaunchEvents ev, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const long long rows = (long long)a.T * G;
  const long long nrb = (rows + kPfRows - 1) / kPfRows;
  if (nrb > 0x7fffffffLL || a.Hkv > 65535 || a.B > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nrb, (unsigned)a.Hkv, (unsigned)a.B);
  // rho == nullptr selects plain softmax attention (no correction branch).
  if (d == 128) {
    if (a.rho) launch_pf<128, true>(a, grid, ev, s);
    else launch_pf<128, false>(a, grid, ev, s);
  } else {
    if (a.rho) launch_pf<64, true>(a, grid, ev, s);
    else launch_pf<64, false>(a, grid, ev, s);
  }
  return hipGetLastError();
}

}  // namespace parallax
