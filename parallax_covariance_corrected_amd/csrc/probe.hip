// Probe rho = W_R x for every sequence and query head (zubnet.ai (pt),
// "Parallax mantém softmax ...", second paragraph: rho_i = W_R x_i from the
// layer input).
//
// As a matrix product: rho[B, N] = x[B, K] . W_R[N, K]^T with N = Hq*d and
// K = d_model; both operands have K contiguous, which is exactly the operand
// layout of the bf16 MFMA (8 consecutive K values per lane), so neither needs
// a transpose. Products of bf16 values are exact in fp32 and the accumulation
// is fp32.
//
// bf16, small batch (B <= 64): a workgroup of NW waves owns a (16*MT rows) x
// 16 columns tile and loads its operands straight from memory into MFMA
// registers; its waves split K NW ways, each issuing the loads of U k-steps
// before their MFMAs, and reduce through LDS in a fixed order. Rows past B
// read zeros (buffer range); B up to 128 runs as row blocks of this kernel.
// Larger batches (B > 128): an LDS-tiled GEMM with 128 x 128 tiles (below),
// where operand reuse across waves pays for staging.
// fp32 kernel: one wave per output, a plain dot product.
#include <type_traits>
#include <utility>

#include "common.h"

namespace parallax {
namespace {

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }
typedef __attribute__((address_space(3))) void lds_void;

// rho is written with streaming (non-temporal) stores: the decode kernel that
// follows reads it once. Written normally, its dirty lines (16.8 MB at
// B = 2048) are flushed to HBM while that decode streams the K/V cache
// (measured on the large-batch step: decode 193 -> 182 us, step 217 -> 207 us;
// streaming the decode's own outputs as well changed nothing).
__device__ __forceinline__ void store_stream(float* p, float v) { __builtin_nontemporal_store(v, p); }

// COLS < 16 (with NT = 1): the workgroup owns only COLS output columns (the
// other MFMA columns read zeros), so twice as many workgroups share the W_R
// stream (measured 8% faster at B = 16, d_model = 2048).
template <int MT, int NT, int NW, int U, int COLS = 16 * NT>
__global__ __launch_bounds__(NW * 64) void probe_mfma_kernel(const uint16_t* __restrict__ W,
                                                             const uint16_t* __restrict__ x,
                                                             float* __restrict__ rho, int B, int N,
                                                             int K) {
  static_assert(COLS == 16 * NT || (NT == 1 && COLS < 16), "narrow tiles are single MFMA tiles");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * COLS;
  const int m0 = blockIdx.y * 16 * MT;
  const unsigned rowb = (unsigned)K * 2;
  // x rows m0.. (rows >= B read as zero), W rows n0.. n0 + COLS - 1
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (size_t)m0 * K,
                                              (unsigned)(min(B - m0, 16 * MT)) * rowb);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(W + (size_t)n0 * K,
                                              (unsigned)(min(N - n0, COLS)) * rowb);
  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int jn = 0; jn < NT; ++jn) acc[i][jn] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // The NW waves split K into 32-wide steps (wave w takes steps w, w + NW, ...);
  // each wave issues the loads of U steps before their MFMAs.
  for (int k0 = 32 * wave; k0 < K; k0 += 32 * NW * U) {
    u32x4 xa[U][MT], wb[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k0 + u * 32 * NW + 8 * grp;
      // K % 8 == 0: an 8-wide group is entirely inside or past the row; a group
      // past the row gets an offset beyond the buffer range and reads 0.
      const unsigned koff = kk < K ? (unsigned)kk * 2 : 0x80000000u;
#pragma unroll
      for (int i = 0; i < MT; ++i) xa[u][i] = buf_load16(xr, (unsigned)(16 * i + l16) * rowb + koff);
#pragma unroll
      for (int jn = 0; jn < NT; ++jn)
        wb[u][jn] = buf_load16(wr, 16 * jn + l16 < COLS ? (unsigned)(16 * jn + l16) * rowb + koff
                                                        : 0x80000000u);
    }
    // Keep every load above in flight together: left alone, the scheduler
    // interleaves them with the MFMAs below to save registers, and the wave
    // then waits out several memory round trips per U steps instead of one.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int jn = 0; jn < NT; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[u][i]), as_bf16x8(wb[u][jn]),
                                                                acc[i][jn], 0, 0, 0);
  }

  __shared__ f32x4 red[NW - 1][MT * NT][64];
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int jn = 0; jn < NT; ++jn) red[wave - 1][i * NT + jn][lane] = acc[i][jn];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int jn = 0; jn < NT; ++jn) {
        f32x4 v = acc[i][jn];
#pragma unroll
        for (int w = 0; w < NW - 1; ++w) {
          const f32x4 o = red[w][i * NT + jn][lane];
          v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
        }
        const int col = n0 + 16 * jn + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + 16 * i + 4 * grp + r;
          if (16 * jn + l16 < COLS && row < B && col < N) store_stream(rho + (size_t)row * N + col, v[r]);
        }
      }
  }
}

// Large-batch probe: a 128 x 128 tile of rho per workgroup, eight waves in a
// 4 x 2 arrangement each owning 32 x 64 (2 x 4 MFMA tiles). K advances in
// steps of 128 through double-buffered LDS (2 x 64 KB), so every workgroup
// reads its x and W_R panels from the caches once. The panels go from memory
// straight into LDS (buffer loads with an LDS destination: lane L of a load
// writes the 16 bytes at the piece's base + 16 L), so no registers hold them
// in transit and no LDS store instructions are issued. LDS rows are 256 bytes
// (sixteen 16-byte chunks); chunk c of row r sits at slot c ^ (r & 15), chosen
// by the global chunk each lane fetches, which puts the 16 rows of one MFMA
// operand read in distinct bank groups. The four LDS buffers are separate
// arrays and each loop half names its own: with one array indexed by a
// run-time stage, the compiler could not tell that the operand reads of one
// stage never touch the stage being loaded and waited for the loads first.
constexpr int kGM = 128, kGN = 128, kGK = 128;
constexpr int kGWM = 4, kGWN = 2;                  // wave grid
constexpr int kGTI = kGM / 16 / kGWM;              // MFMA tiles per wave, rows
constexpr int kGTJ = kGN / 16 / kGWN;              // MFMA tiles per wave, columns
constexpr int kGWaves = kGWM * kGWN;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kLdsRow = kGK * 2;                   // bytes per LDS row (16 chunks)
constexpr int kPieces = kGM * kLdsRow / 1024;      // 1 KB pieces per operand panel
static_assert(kGM == kGN && kPieces % kGWaves == 0, "every wave loads the same pieces");

__device__ __forceinline__ int lds_slot(int row, int chunk) {
  return row * kLdsRow + 16 * (chunk ^ (row & 15));
}

__global__ __launch_bounds__(kGThreads) void probe_gemm_kernel(const uint16_t* __restrict__ W,
                                                               const uint16_t* __restrict__ x,
                                                               float* __restrict__ rho, int B,
                                                               int N, int K) {
  __shared__ __attribute__((aligned(16))) unsigned char sA0[kGM * kLdsRow], sA1[kGM * kLdsRow];
  __shared__ __attribute__((aligned(16))) unsigned char sB0[kGN * kLdsRow], sB1[kGN * kLdsRow];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  const int wm = wave / kGWN, wn = wave % kGWN;
  const int m0 = blockIdx.y * kGM, n0 = blockIdx.x * kGN;
  const unsigned rowb = (unsigned)K * 2;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (size_t)m0 * K, (unsigned)min(B - m0, kGM) * rowb);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(W + (size_t)n0 * K, (unsigned)min(N - n0, kGN) * rowb);

  // Panels of k0 .. k0 + kGK - 1 -> stage BUF: wave w loads pieces w, w + 8, ...
  // of each panel. Rows past B (or N) and columns past K read as zero.
  auto stage = [&](int k0, auto BUF) {
    unsigned char* a = decltype(BUF)::value ? sA1 : sA0;
    unsigned char* b = decltype(BUF)::value ? sB1 : sB0;
#pragma unroll
    for (int pc = 0; pc < kPieces / kGWaves; ++pc) {
      const int piece = pc * kGWaves + wave;
      const int byte = piece * 1024 + 16 * lane;
      const int row = byte / kLdsRow, sc = (byte % kLdsRow) / 16;
      const int kk = k0 + 8 * (sc ^ (row & 15));
      const unsigned off = kk < K ? (unsigned)row * rowb + (unsigned)kk * 2 : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)&a[piece * 1024], 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)&b[piece * 1024], 16, off, 0, 0, 0);
    }
  };

  f32x4 acc[kGTI][kGTJ];
#pragma unroll
  for (int i = 0; i < kGTI; ++i)
#pragma unroll
    for (int jn = 0; jn < kGTJ; ++jn) acc[i][jn] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int nk = (K + kGK - 1) / kGK;
  // One K step on stage CUR while the next one loads into the other stage
  // (last read before the previous barrier).
  auto step = [&](int kt, auto CUR) {
    constexpr int cur = decltype(CUR)::value;
    const unsigned char* a = cur ? sA1 : sA0;
    const unsigned char* b = cur ? sB1 : sB0;
    if (kt + 1 < nk) stage((kt + 1) * kGK, std::integral_constant<int, cur ^ 1>{});
#pragma unroll
    for (int ks = 0; ks < kGK / 32; ++ks) {
      u32x4 av[kGTI], bv[kGTJ];
#pragma unroll
      for (int i = 0; i < kGTI; ++i)
        av[i] = *(const u32x4*)&a[lds_slot(wm * 16 * kGTI + 16 * i + l16, 4 * ks + grp)];
#pragma unroll
      for (int jn = 0; jn < kGTJ; ++jn)
        bv[jn] = *(const u32x4*)&b[lds_slot(wn * 16 * kGTJ + 16 * jn + l16, 4 * ks + grp)];
#pragma unroll
      for (int i = 0; i < kGTI; ++i)
#pragma unroll
        for (int jn = 0; jn < kGTJ; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[i]), as_bf16x8(bv[jn]),
                                                                acc[i][jn], 0, 0, 0);
    }
    // each wave waits for its own LDS-destination loads; the barrier then
    // publishes the whole stage
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  stage(0, std::integral_constant<int, 0>{});
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
  }

#pragma unroll
  for (int i = 0; i < kGTI; ++i)
#pragma unroll
    for (int jn = 0; jn < kGTJ; ++jn) {
      const int col = n0 + wn * 16 * kGTJ + 16 * jn + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 16 * kGTI + 16 * i + 4 * grp + r;
        if (row < B && col < N) store_stream(rho + (size_t)row * N + col, acc[i][jn][r]);
      }
    }
}

// The same 128 x 128 tile product for the common K = 64 * NK, unrolled over K:
// 64-deep K steps through a four-stage LDS ring (4 x 32 KB), steps k + 1 ..
// k + 3 in flight while step k is multiplied. Unrolled, every step names its
// stage and its wait at compile time (in a loop the compiler's tracking of the
// LDS-destination loads loses the stages at the loop header and waits for all
// of them). LDS rows are 128 bytes (eight 16-byte chunks); chunk c of row r
// sits at slot c ^ ((r >> 1) & 7), so the 16 rows of one operand read cover
// the 64 banks once per row pair.
constexpr int kDK = 64;
constexpr int kDRow = kDK * 2;
constexpr int kDPieces = kGM * kDRow / 1024;             // 1 KB pieces per panel
constexpr int kDLoads = 2 * kDPieces / kGWaves;          // per wave and stage
static_assert(kDPieces % kGWaves == 0, "every wave loads the same pieces");

__device__ __forceinline__ int deep_slot(int row, int chunk) {
  return row * kDRow + 16 * (chunk ^ ((row >> 1) & 7));
}

// Wait until at most N of this wave's vector memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <typename F, int... KT>
__device__ __forceinline__ void each_step(F& f, std::integer_sequence<int, KT...>) {
  (f(std::integral_constant<int, KT>{}), ...);
}

template <int NK>
__global__ __launch_bounds__(kGThreads) void probe_gemm_deep_kernel(const uint16_t* __restrict__ W,
                                                                    const uint16_t* __restrict__ x,
                                                                    float* __restrict__ rho, int B,
                                                                    int N) {
  constexpr int K = NK * kDK;
  __shared__ __attribute__((aligned(16))) unsigned char sA0[kGM * kDRow], sA1[kGM * kDRow],
      sA2[kGM * kDRow], sA3[kGM * kDRow];
  __shared__ __attribute__((aligned(16))) unsigned char sB0[kGN * kDRow], sB1[kGN * kDRow],
      sB2[kGN * kDRow], sB3[kGN * kDRow];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  const int wm = wave / kGWN, wn = wave % kGWN;
  const int m0 = blockIdx.y * kGM, n0 = blockIdx.x * kGN;
  constexpr unsigned rowb = (unsigned)K * 2;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (size_t)m0 * K, (unsigned)min(B - m0, kGM) * rowb);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(W + (size_t)n0 * K, (unsigned)min(N - n0, kGN) * rowb);

  auto stage = [&](auto KT) {
    constexpr int kt = decltype(KT)::value, st = kt % 4;
    unsigned char* a = st == 0 ? sA0 : st == 1 ? sA1 : st == 2 ? sA2 : sA3;
    unsigned char* b = st == 0 ? sB0 : st == 1 ? sB1 : st == 2 ? sB2 : sB3;
#pragma unroll
    for (int pc = 0; pc < kDPieces / kGWaves; ++pc) {
      const int piece = pc * kGWaves + wave;
      const int byte = piece * 1024 + 16 * lane;
      const int row = byte / kDRow, sc = (byte % kDRow) / 16;
      const unsigned off = (unsigned)row * rowb + (unsigned)(kt * kDK + 8 * (sc ^ ((row >> 1) & 7))) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)&a[piece * 1024], 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)&b[piece * 1024], 16, off, 0, 0, 0);
    }
  };

  f32x4 acc[kGTI][kGTJ];
#pragma unroll
  for (int i = 0; i < kGTI; ++i)
#pragma unroll
    for (int jn = 0; jn < kGTJ; ++jn) acc[i][jn] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto step = [&](auto KT) {
    constexpr int kt = decltype(KT)::value, st = kt % 4;
    const unsigned char* a = st == 0 ? sA0 : st == 1 ? sA1 : st == 2 ? sA2 : sA3;
    const unsigned char* b = st == 0 ? sB0 : st == 1 ? sB1 : st == 2 ? sB2 : sB3;
    // this wave's loads of step kt done (those of kt + 1, kt + 2 may not be)
    wait_vm<(kt + 2 < NK ? 2 : kt + 1 < NK ? 1 : 0) * kDLoads>();
    // A bare barrier: __syncthreads() would also wait for the later stages'
    // loads. After it every wave's part of stage kt is in LDS, and every wave
    // has finished reading the stage of step kt - 1, which step kt + 3 reuses.
    // The empty asm statements keep the compiler from moving memory accesses
    // across the barrier.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (kt + 3 < NK) stage(std::integral_constant<int, kt + 3>{});
#pragma unroll
    for (int ks = 0; ks < kDK / 32; ++ks) {
      u32x4 av[kGTI], bv[kGTJ];
#pragma unroll
      for (int i = 0; i < kGTI; ++i)
        av[i] = *(const u32x4*)&a[deep_slot(wm * 16 * kGTI + 16 * i + l16, 4 * ks + grp)];
#pragma unroll
      for (int jn = 0; jn < kGTJ; ++jn)
        bv[jn] = *(const u32x4*)&b[deep_slot(wn * 16 * kGTJ + 16 * jn + l16, 4 * ks + grp)];
#pragma unroll
      for (int i = 0; i < kGTI; ++i)
#pragma unroll
        for (int jn = 0; jn < kGTJ; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[i]), as_bf16x8(bv[jn]),
                                                                acc[i][jn], 0, 0, 0);
    }
  };
  stage(std::integral_constant<int, 0>{});
  if constexpr (NK > 1) stage(std::integral_constant<int, 1>{});
  if constexpr (NK > 2) stage(std::integral_constant<int, 2>{});
  each_step(step, std::make_integer_sequence<int, NK>{});

#pragma unroll
  for (int i = 0; i < kGTI; ++i)
#pragma unroll
    for (int jn = 0; jn < kGTJ; ++jn) {
      const int col = n0 + wn * 16 * kGTJ + 16 * jn + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 16 * kGTI + 16 * i + 4 * grp + r;
        if (row < B && col < N) store_stream(rho + (size_t)row * N + col, acc[i][jn][r]);
      }
    }
}

// fp32: one wave per output rho[row][col]; lane l takes elements l, l + 64, ...
// of the dot product (each load instruction reads 256 contiguous bytes of the
// W_R row and of x), four accumulators, then a wave sum.
__global__ __launch_bounds__(256) void probe_f32_kernel(const float* __restrict__ W,
                                                        const float* __restrict__ x,
                                                        float* __restrict__ rho, int B, int N,
                                                        int K) {
  const int lane = threadIdx.x & 63;
  const size_t idx = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= (size_t)B * N) return;   // whole waves
  const int row = (int)(idx / N), col = (int)(idx % N);
  const float* w = W + (size_t)col * K;
  const float* xr = x + (size_t)row * K;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  int k = lane;
  for (; k + 192 < K; k += 256) {
    s0 = fmaf(w[k], xr[k], s0);
    s1 = fmaf(w[k + 64], xr[k + 64], s1);
    s2 = fmaf(w[k + 128], xr[k + 128], s2);
    s3 = fmaf(w[k + 192], xr[k + 192], s3);
  }
  for (; k < K; k += 64) s0 = fmaf(w[k], xr[k], s0);
  float s = (s0 + s1) + (s2 + s3);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) store_stream(rho + idx, s);
}

}  // namespace

hipError_t launch_probe(const void* W, const void* x, float* rho, int B, int N, int K,
                        int f32_inputs, int path, LaunchEvents ev, hipStream_t s) {
  if (f32_inputs) {
    const size_t total = (size_t)B * N;
    const size_t grid = (total + 3) / 4;
    if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
    hipExtLaunchKernelGGL(probe_f32_kernel, dim3(grid), dim3(256), 0, s, ev.start, ev.stop, 0,
                          (const float*)W, (const float*)x, rho, B, N, K);
    return hipGetLastError();
  }
  const uint16_t* Wb = (const uint16_t*)W;
  const uint16_t* xb = (const uint16_t*)x;
  // The tiled GEMM has few workgroups below a few hundred rows (one per 128 x
  // 128 tile), each waiting out a memory round trip per K step: 19-21 us at
  // B = 64-256 for a cold 2048 x 2048 W_R, against 7.4 / 12.8 / 23.5 us for
  // the small-batch kernel at B = 64 / 128 / 256, whose cost grows with the
  // row blocks (4096 x 2560: 15.6 / 27.3 / 51 against 28-32 us).
  const bool gemm = path == 2 || (path == 0 && B > 128);
  if (gemm) {
    dim3 grid((N + kGN - 1) / kGN, (B + kGM - 1) / kGM);
    if (grid.y > 65535u) return hipErrorInvalidConfiguration;
#define PARALLAX_DEEP(NK)                                                                   \
  case NK * kDK:                                                                            \
    hipExtLaunchKernelGGL(probe_gemm_deep_kernel<NK>, grid, dim3(kGThreads), 0, s, ev.start, \
                          ev.stop, 0, Wb, xb, rho, B, N);                                   \
    return hipGetLastError();
    switch (K) {
      PARALLAX_DEEP(16)
      PARALLAX_DEEP(32)
      PARALLAX_DEEP(40)
      PARALLAX_DEEP(48)
      PARALLAX_DEEP(64)
      default: break;
    }
#undef PARALLAX_DEEP
    hipExtLaunchKernelGGL(probe_gemm_kernel, grid, dim3(kGThreads), 0, s, ev.start, ev.stop, 0, Wb, xb, rho, B, N, K);
  } else {
    // Shapes picked by a sweep over cold W_R (tiles of 8 / 16 columns, 4-16
    // waves, 2-8 k-steps in flight): aim for at least 256 workgroups, since a
    // workgroup's read of its W_R rows is latency-bound. Batches above 64 rows
    // take row blocks of 64 (32 with few column tiles) on grid.y.
    const int mt = min((B + 15) / 16, 4);
    dim3 grid((N + 15) / 16, (unsigned)((B + 16 * mt - 1) / (16 * mt)));
    if ((B + 31) / 32 > 65535) return hipErrorInvalidConfiguration;
    if (mt == 1) {
      grid.x = (N + 7) / 8;
      hipExtLaunchKernelGGL((probe_mfma_kernel<1, 1, 16, 4, 8>), grid, dim3(1024), 0, s, ev.start, ev.stop, 0, Wb, xb, rho, B, N, K);
    } else if (mt == 2) {
      grid.x = (N + 7) / 8;
      hipExtLaunchKernelGGL((probe_mfma_kernel<2, 1, 8, 8, 8>), grid, dim3(512), 0, s, ev.start, ev.stop, 0, Wb, xb, rho, B, N, K);
    } else if (grid.x < 256) {
      // few column tiles: two workgroups of 32 rows each per tile
      grid.y = (B + 31) / 32;
      hipExtLaunchKernelGGL((probe_mfma_kernel<2, 1, 8, 8>), grid, dim3(512), 0, s, ev.start, ev.stop, 0, Wb, xb, rho, B, N, K);
    } else if (mt == 3) {
      hipExtLaunchKernelGGL((probe_mfma_kernel<3, 1, 8, 4>), grid, dim3(512), 0, s, ev.start, ev.stop, 0, Wb, xb, rho, B, N, K);
    } else if ((long long)((N + 31) / 32) * grid.y >= 256) {
      // 32-column tiles of 16 waves wherever they still make 256 workgroups:
      // x is read by half as many workgroups (B = 128, 4096 columns: 27.5 ->
      // 19.4 us; 8192 columns, B = 64: 22.1 -> 15.9 us; with fewer workgroups,
      // as at B = 64 over 4096 columns, the 16-column tiles stay faster).
      grid.x = (N + 31) / 32;
      hipExtLaunchKernelGGL((probe_mfma_kernel<4, 2, 16, 2>), grid, dim3(1024), 0, s, ev.start, ev.stop, 0, Wb, xb, rho, B, N, K);
    } else {
      hipExtLaunchKernelGGL((probe_mfma_kernel<4, 1, 8, 4>), grid, dim3(512), 0, s, ev.start, ev.stop, 0, Wb, xb, rho, B, N, K);
    }
  }
  return hipGetLastError();
}

}  // namespace parallax
