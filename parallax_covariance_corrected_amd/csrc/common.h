// Shared device helpers and internal launcher declarations for libparallax.
// gfx950 (CDNA4) only: 64-lane wavefronts, bf16 matrix cores, raw buffer loads.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace parallax {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

// bf16 storage is handled as raw 16-bit patterns; the value of a bf16 is the
// fp32 with the same top 16 bits.
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((unsigned)b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even, in
// one v_cvt_pk_bf16_f32.
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Raw buffer resource over [base, base + bytes): loads at byte offsets past
// `bytes` return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

// exp2 on the hardware transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Scale factor that moves a running sum from reference max m_old to m_new
// (log2 domain); an empty state (m_old = -inf) contributes nothing.
__device__ __forceinline__ float rescale(float m_old, float m_new) {
  return m_old == kNegInf ? 0.f : fast_exp2(m_old - m_new);
}

// Final epilogue: out = A/l - (P/l - (A/l)(S/l)); l == 0 (no keys) gives 0.
__device__ __forceinline__ float parallax_out(float A, float P, float l, float S) {
  if (!(l > 0.f)) return 0.f;
  float inv = 1.f / l;
  float vbar = A * inv;
  return vbar - (P * inv - vbar * (S * inv));
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float v) {
  *p = f32_to_bf16_rne(v);
}

// Kernel arguments in SGPRs. The library is built with kernarg preloading: the
// leading scalar arguments of a kernel (up to 14 SGPRs) are in SGPRs when its
// waves start, so a wave does not wait for a load of its argument block before
// it can address memory. The decode kernels take the fields of DecodeArgs that
// a work item needs first (K/V, length, q and rho pointers, shape, chunk) as
// such leading arguments, Hq and Hkv packed into one word (both < 2^16) and
// the prefetch flag in the top bit of the chunk; the struct, passed after
// them, supplies the rest. On entry the kernel writes them back into its copy
// of the struct. (The merge kernel has a head of its own.)
#define PARALLAX_DECODE_HEAD_PARAMS                                                        \
  const void *pk_k, const void *pk_v, const int *pk_seq_lens, const void *pk_q,            \
      const float *pk_rho, int pk_B, int pk_max_ctx, unsigned pk_heads, unsigned pk_chunk
#define PARALLAX_DECODE_HEAD_ARGS(a)                                                       \
  (a).k, (a).v, (a).seq_lens, (a).q, (a).rho, (a).B, (a).max_ctx,                          \
      (unsigned)(a).Hq | ((unsigned)(a).Hkv << 16),                                        \
      (unsigned)(a).chunk | ((a).prefetch ? 0x80000000u : 0u)
#define PARALLAX_DECODE_HEAD_APPLY(a)                                                      \
  do {                                                                                     \
    (a).k = pk_k;                                                                          \
    (a).v = pk_v;                                                                          \
    (a).seq_lens = pk_seq_lens;                                                            \
    (a).q = pk_q;                                                                          \
    (a).rho = pk_rho;                                                                      \
    (a).B = pk_B;                                                                          \
    (a).max_ctx = pk_max_ctx;                                                              \
    (a).Hq = (int)(pk_heads & 0xffffu);                                                    \
    (a).Hkv = (int)(pk_heads >> 16);                                                       \
    (a).chunk = (int)(pk_chunk & 0x7fffffffu);                                             \
    (a).prefetch = (int)(pk_chunk >> 31);                                                  \
  } while (0)

// Split-K partial state of one (sequence, query head, split), fp32:
//   ml[(b*Hq + h)*splits + s] = {m (log2 domain), l, S, 0}
//   ap[((b*Hq + h)*splits + s)*2*d + {0: A, d: P} + i]
// The fields a decode work item needs first (item numbering, its length and
// K/V addresses) come first; the kernels also receive them as preloaded
// leading arguments (PARALLAX_DECODE_HEAD_PARAMS).
struct DecodeArgs {
  const void* k;
  const void* v;
  const int* seq_lens;
  int B, Hq, Hkv, max_ctx;
  int chunk;       // keys per split
  int splits;      // splits per (sequence, KV head)
  int prefetch = 0;  // matrix-core kernel: first tiles requested before the length arrives
  int out_f32;     // 1: out is fp32, 0: bf16
  const void* q;
  const float* rho;
  void* out;
  float4* ml;
  float* ap;
  float scale_log2;  // log2(e) / sqrt(d)
  // Many-query (prefill) form of the generic kernel: when T > 0, sequence b of
  // this call is token b % T of cache sequence b / T and attends to cache rows
  // 0 .. prefix[b / T] + b % T (prefix may be null: 0); seq_lens is unused.
  int T = 0;
  const int* prefix = nullptr;
  // Probe fused into the decode (kernels launched with the fused flag): rho is
  // not read from memory; each work item computes the rho of its query heads
  // from W_R [Hq*d, d_model] and x [B, d_model] (storage type of q) in its
  // prologue. d_model is a multiple of 16 / element size.
  const void* W_R = nullptr;
  const void* x = nullptr;
  int d_model = 0;
};

// The probe fused into a decode work item: dst[r] = sum_c W[row0 + r][c] * xb[c]
// for r < nrows (rows of d_model elements; xb = x of the item's sequence), fp32
// accumulation, computed by the NT threads of the workgroup into LDS. A row
// takes a group of LPR lanes (the power of two <= 16 that covers its 16-byte
// pieces), lane i of the group reading pieces i, i + LPR, ...; each group
// takes kProbeRowBatch rows at a time and issues their loads together (one
// memory round trip per batch and piece step), then sums its lanes with xor
// shuffles. The caller synchronises the workgroup before dst is read.
constexpr int kProbeRowBatch = 8;
template <bool F32IN, int NT>
__device__ __forceinline__ void probe_rows(const void* W, const void* xb, int d_model,
                                           size_t row0, int nrows, float* dst) {
  constexpr int ESZ = F32IN ? 4 : 2;
  constexpr int RB = kProbeRowBatch;
  const int pieces = d_model * ESZ / 16;
  int lpr = 16;
  while (lpr > 1 && lpr / 2 >= pieces) lpr >>= 1;
  const int ngroup = NT / lpr;
  const int li = threadIdx.x & (lpr - 1), group = threadIdx.x / lpr;
  const char* x8 = (const char*)xb;
  const char* w8 = (const char*)W + row0 * (size_t)d_model * ESZ;
  const size_t wrow = (size_t)d_model * ESZ;
  for (int r0 = 0; r0 < nrows; r0 += ngroup * RB) {
    float acc[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) acc[k] = 0.f;
    for (int pc = li; pc < pieces; pc += lpr) {
      const u32x4 xv = *(const u32x4*)(x8 + (size_t)pc * 16);
      u32x4 wv[RB];
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        const int r = r0 + group + ngroup * k;
        wv[k] = r < nrows ? *(const u32x4*)(w8 + r * wrow + (size_t)pc * 16)
                          : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int k = 0; k < RB; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (F32IN) {
            acc[k] = fmaf(__uint_as_float(wv[k][i]), __uint_as_float(xv[i]), acc[k]);
          } else {
            acc[k] = fmaf(bf16_lo(wv[k][i]), bf16_lo(xv[i]), acc[k]);
            acc[k] = fmaf(bf16_hi(wv[k][i]), bf16_hi(xv[i]), acc[k]);
          }
        }
    }
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      float a = acc[k];
      for (int o = lpr >> 1; o >= 1; o >>= 1) a += __shfl_xor(a, o);
      const int r = r0 + group + ngroup * k;
      if (r < nrows && li == 0) dst[r] = a;
    }
  }
}

// Causal many-query forward: token t of sequence b is at cache position
// prefix[b] + t and attends to cache rows 0 .. prefix[b] + t.
struct PrefillArgs {
  const void* q;        // [B, T, Hq, d] bf16
  const float* rho;     // [B, T, Hq, d] fp32
  const void* k;        // [B, Hkv, max_ctx, d] bf16
  const void* v;
  const int* prefix;    // [B] device, or null (all 0)
  void* out;            // [B, T, Hq, d] bf16 or fp32
  int B, T, Hq, Hkv, max_ctx;
  int out_f32;
  float scale_log2;
};

__device__ __forceinline__ void store_output(const DecodeArgs& a, size_t idx, float o) {
  if (a.out_f32) store_out<float>((float*)a.out + idx, o);
  else store_out<uint16_t>((uint16_t*)a.out + idx, o);
}

// A sequence that fits in one chunk (including length 0) is finished by its
// split 0, which writes the output; longer ones leave one partial state per
// non-empty split for the merge kernel.
__device__ __forceinline__ bool single_chunk(const DecodeArgs& a, int n) { return n <= a.chunk; }

// Optional start/stop events stamped by the dispatch packet (profiling).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Internal launchers (one translation unit each). Return hipError_t.
// fused = 1: the probe runs in each work item's prologue (DecodeArgs W_R, x,
// d_model; rho unused).
hipError_t launch_decode_generic(const DecodeArgs& a, int d, int f32_inputs, int fused,
                                 LaunchEvents ev, hipStream_t s);
// compact = 1: compacted item numbering (workgroup items, B <= 256 only).
// fused = 1: workgroup items without compaction only.
hipError_t launch_decode_mfma(const DecodeArgs& a, int d, int wave_items, int compact, int fused,
                              LaunchEvents ev, hipStream_t s);
hipError_t launch_merge(const DecodeArgs& a, int d, LaunchEvents ev, hipStream_t s);
hipError_t launch_prefill_mfma(const PrefillArgs& a, int d, LaunchEvents ev, hipStream_t s);
bool decode_mfma_supported(int d, int G);
// path (bf16): 0 = automatic, 1 = the small-batch kernel (row blocks of at
// most 64), 2 = the LDS-tiled GEMM.
hipError_t launch_probe(const void* W, const void* x, float* rho, int B, int N, int K,
                        int f32_inputs, int path, LaunchEvents ev, hipStream_t s);

}  // namespace parallax
