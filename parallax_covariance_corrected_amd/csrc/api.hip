// Host side of the libparallax C ABI (declared in include/parallax.h):
// argument checks, the split-K plan, the per-stream workspace, kernel
// launches, error reporting and optional per-kernel event timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <iterator>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/parallax.h"
#include "common.h"

namespace parallax {
hipError_t launch_read_stream(const void* buf, size_t bytes, int grid, unsigned* sink,
                              LaunchEvents ev, hipStream_t s);
}

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PARALLAX_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ---------------------------------------------------------------- options
// Process-wide; atomics so that a call on one thread may overlap
// parallax_set_option on another (the call then sees the old or the new value).
std::atomic<int> g_opt_chunk{0};
std::atomic<int> g_opt_kernel{0};
std::atomic<int> g_opt_profile{0};
std::atomic<int> g_opt_items{0};
std::atomic<int> g_opt_order{0};
std::atomic<int> g_opt_fuse{0};
std::atomic<int> g_opt_prefetch{0};
std::atomic<int> g_opt_probe{0};

// ---------------------------------------------------------------- profiling
// Start/stop events are handed to hipExtLaunchKernel, which stamps them from
// the kernel's own dispatch packet (no extra packets between kernels).
struct Timing {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
  double total_ms = 0.0;
  long long launches = 0;
};
std::mutex g_prof_mu;
Timing g_prof[5];   // probe, decode, merge, prefill, read reference
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

parallax::LaunchEvents profile_events() {
  parallax::LaunchEvents ev;
  if (!g_opt_profile) return ev;
  std::lock_guard<std::mutex> g(g_prof_mu);
  ev.start = take_event();
  ev.stop = take_event();
  if (!ev.start || !ev.stop) {
    if (ev.start) g_event_pool.push_back(ev.start);
    if (ev.stop) g_event_pool.push_back(ev.stop);
    ev.start = ev.stop = nullptr;
  }
  return ev;
}

void profile_record(int kind, parallax::LaunchEvents ev, bool launched) {
  if (!ev.start) return;
  std::lock_guard<std::mutex> g(g_prof_mu);
  if (launched) {
    g_prof[kind].pending.emplace_back(ev.start, ev.stop);
  } else {
    g_event_pool.push_back(ev.start);
    g_event_pool.push_back(ev.stop);
  }
}

// ---------------------------------------------------------------- workspace
// Split-K partial states, cached per (device, stream): calls on one stream are
// ordered, so they can share one buffer; calls on different streams never do.
// A buffer only grows (at least doubling, so retired buffers add up to less
// than the current one); growing is stream-ordered and is refused while the
// stream is being captured into a graph. A retired buffer is never freed: a
// graph captured earlier on the stream still holds its address, and a replay
// of that graph must not write freed memory.
struct Workspace {
  void* base = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<void*> g_ws_retired;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int get_workspace(hipStream_t stream, size_t bytes, void** base) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> g(g_ws_mu);
  Workspace& w = g_ws[std::make_pair(dev, stream)];
  if (w.base == nullptr || w.bytes < bytes) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cap != hipStreamCaptureStatusNone)
      return fail(PARALLAX_ERR_NO_MEMORY,
                  "the split-K workspace of this stream must grow, which cannot happen during "
                  "graph capture: run one call of this size on the stream before capturing");
    Workspace nw;
    nw.bytes = round_up(std::max(bytes, 2 * w.bytes), 1 << 20);
    e = hipMallocAsync(&nw.base, nw.bytes, stream);
    if (e != hipSuccess || !nw.base) return fail(PARALLAX_ERR_NO_MEMORY, "workspace allocation failed");
    if (w.base) g_ws_retired.push_back(w.base);
    w = nw;
  }
  *base = w.base;
  return PARALLAX_OK;
}

// ---------------------------------------------------------------- static scratch
// parallax_probe_decode_noalloc keeps the probe's rho and the split states in
// this file-scope device array instead of the per-stream workspace, so that it
// never allocates. Each device holds its own copy (kScratchBytes) from the
// library's first use on it until the process ends. In host code `scratch`
// only names the symbol: its device address comes from hipGetSymbolAddress,
// looked up once per device and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;   // device -> address of its scratch array

int scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> g(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(PARALLAX_ERR_HIP, "hipGetSymbolAddress(scratch) gave null");
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return PARALLAX_OK;
}

// ---------------------------------------------------------------- planning
struct Plan {
  int chunk;
  int splits;
  int kernel;   // 1 generic, 2 matrix-core workgroup items, 3 matrix-core wave items
  int compact;  // 1: compacted item numbering (kernel 2 only)
  int prefetch; // 1: first tiles requested before the sequence length (kernels 2, 3)
};

// Probe fused into the decode prologue (parallax_probe_decode): every work item
// recomputes rho of its head block from W_R (GH*d rows of d_model elements), so
// W_R is read once per work item instead of once per call — from the caches
// after the first time, but still through each compute unit. That replaces the
// probe launch (a few microseconds whatever its size) only where the reads per
// item and in total stay small. Limits from timing whole steps both ways over
// batch 1-64 x d_model 64-2048 x context 128-4096 (Hq 16, Hkv 8, d 128, bf16;
// and fp32 shapes): on the matrix-core kernel the fused step took 0.73-1.01x
// the separate one at 32 KiB of W_R per item (up to 16 MiB in all),
// 0.78-0.86x at 64 KiB per item up to 8 MiB in all (0.84-1.20x beyond),
// 0.86-0.91x at 128 KiB per item up to 4 MiB in all (0.93-1.23x beyond), and
// more at larger rows (up to 2.3x at 1 MiB per item); on the generic kernel,
// whose decode is slower and hides more of the prologue, 0.75-0.94x up to
// 128 KiB per item.
struct FuseLimit {
  long long item_bytes, total_bytes;
};
constexpr FuseLimit kFuseMfma[] = {{32LL << 10, 16LL << 20}, {64LL << 10, 8LL << 20},
                                   {128LL << 10, 4LL << 20}};
constexpr FuseLimit kFuseGeneric[] = {{128LL << 10, 8LL << 20}};

int esize(int dtype) { return dtype == PARALLAX_F32 ? 4 : 2; }

int check_decode_shape(int B, int Hq, int Hkv, int d, int max_ctx, int dtype) {
  if (dtype != PARALLAX_F32 && dtype != PARALLAX_BF16 && dtype != PARALLAX_BF16_F32OUT)
    return fail(PARALLAX_ERR_UNSUPPORTED, "unknown dtype " + std::to_string(dtype));
  if (B < 1 || Hq < 1 || Hkv < 1 || max_ctx < 1)
    return fail(PARALLAX_ERR_INVALID_ARG, "B, Hq, Hkv and max_ctx must be >= 1");
  if (Hq % Hkv != 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
  if (d != 64 && d != 128)
    return fail(PARALLAX_ERR_UNSUPPORTED, "head dim d must be 64 or 128");
  // Buffer offsets inside one (sequence, KV head) stream are 32-bit.
  if ((long long)max_ctx * d * esize(dtype) + 256LL * d * esize(dtype) >= (1LL << 31))
    return fail(PARALLAX_ERR_UNSUPPORTED, "max_ctx too large for one KV stream (2 GiB)");
  if ((long long)B * Hq > (1LL << 30))
    return fail(PARALLAX_ERR_UNSUPPORTED, "B * Hq too large");
  if (Hq > 65535) return fail(PARALLAX_ERR_UNSUPPORTED, "Hq too large (at most 65535)");
  return PARALLAX_OK;
}

// Query heads per work item (each item reads its K/V rows once). Matrix-core
// kernel: the whole GQA group up to 8 heads, larger groups in blocks of the
// largest divisor <= 8; generic kernel: blocks of up to 4.
int head_block(int G, bool mfma) {
  for (int gh = mfma ? 8 : 4; gh > 1; --gh)
    if (G % gh == 0) return gh;
  return 1;
}

Plan make_plan(int B, int Hq, int Hkv, int d, int max_ctx, int dtype) {
  Plan p;
  const int G = Hq / Hkv;
  const bool mfma_ok = dtype != PARALLAX_F32 && parallax::decode_mfma_supported(d, G);
  bool mfma = mfma_ok;
  if (g_opt_kernel == 1) mfma = false;
  const long long units = (long long)B * Hkv * (G / head_block(G, mfma));
  // Wave items (one wave per item) suit many short sequences; workgroup items
  // (four or eight waves per item) suit long ones.
  bool wave_items = mfma && units >= 1024 && max_ctx <= 1024;
  if (mfma && g_opt_items == 1) wave_items = false;
  if (mfma && g_opt_items == 2) wave_items = true;
  p.kernel = !mfma ? 1 : (wave_items ? 3 : 2);
  int chunk = g_opt_chunk;
  if (chunk <= 0) {
    // About one busy workgroup per compute unit (256; 2048 waves for wave
    // items): fewer, longer items amortise each item's prologue and epilogue,
    // which measured faster than more, shorter ones. Chunks stay within
    // 64 (wave items) / 128 (workgroup items) .. 2048 keys so that a ragged
    // batch stays balanced.
    const long long target = wave_items ? 2048 : 256;
    const long long want = units >= target ? 1 : (target + units - 1) / units;
    long long c = (max_ctx + want - 1) / want;
    c = (c + 63) / 64 * 64;
    const long long lo = wave_items ? 64 : 128;
    if (c < lo) c = lo;
    if (c > 2048) c = 2048;
    // Short caches: one split. The merge launch costs a few microseconds
    // whatever its size, more than the longer items cost here (measured: up
    // to 22% faster at 256-512 keys and B <= 8; from 1024 keys on, splitting
    // wins).
    if (max_ctx <= 512) c = std::max<long long>(lo, (max_ctx + 63) / 64 * 64);
    chunk = (int)c;
  }
  p.chunk = chunk;
  p.splits = (max_ctx + chunk - 1) / chunk;
  // Several sequences in a cache of many chunks: lengths may differ, leaving
  // empty items among the working ones; number only the non-empty ones (the
  // kernel reads the lengths; up to 256 sequences and 64 splits). Measured on
  // a log-uniform ragged batch (64 sequences, 32768-key cache): 9-25% faster
  // decode. Each workgroup then finds its item from all the lengths before its
  // first load, about 1 us that only pays off when the grid has several
  // workgroups per compute unit.
  const bool can_compact = p.kernel == 2 && B <= 256 && p.splits <= 64;
  p.compact = can_compact && B >= 2 && p.splits >= 3 && units * p.splits >= 1024;
  if (g_opt_order == 1) p.compact = 0;
  if (g_opt_order == 2) p.compact = can_compact;
  // Each item's first two tiles per wave are requested before its sequence's
  // length arrives (one memory round trip less before the first tile; about
  // 2 us under load). An empty split then fetches those tiles for nothing, so
  // the prefetch is left off where many empty splits are possible: the
  // compacted numbering (which reads all lengths first anyway) and large
  // batches over several splits.
  p.prefetch = p.kernel >= 2 && !p.compact && (p.splits <= 2 || B <= 256);
  if (g_opt_prefetch == 1) p.prefetch = 0;
  if (g_opt_prefetch == 2) p.prefetch = p.kernel >= 2 && !p.compact;
  return p;
}

// Whether parallax_probe_decode runs the probe inside the decode kernel for
// this plan (shapes already checked).
bool fuse_probe(const Plan& p, int B, int Hq, int Hkv, int d, int d_model, int dtype) {
  const int es = esize(dtype);
  const bool can = (p.kernel == 1 || (p.kernel == 2 && !p.compact)) && (d_model * es) % 16 == 0;
  if (!can || g_opt_fuse == 1) return false;
  if (g_opt_fuse == 2) return true;
  const int G = Hq / Hkv;
  const int GH = head_block(G, p.kernel >= 2);
  const long long item_bytes = (long long)GH * d * d_model * es;   // > 0
  const long long items = (long long)B * Hkv * (G / GH) * p.splits;
  auto within = [&](const FuseLimit& f) {
    return item_bytes <= f.item_bytes && items <= f.total_bytes / item_bytes;
  };
  if (p.kernel >= 2) return std::any_of(std::begin(kFuseMfma), std::end(kFuseMfma), within);
  return std::any_of(std::begin(kFuseGeneric), std::end(kFuseGeneric), within);
}

int check_probe(const void* W_R, const void* x, int B, int Hq, int d, int d_model, int dtype) {
  if (dtype != PARALLAX_F32 && dtype != PARALLAX_BF16 && dtype != PARALLAX_BF16_F32OUT)
    return fail(PARALLAX_ERR_UNSUPPORTED, "unknown dtype " + std::to_string(dtype));
  if (!W_R || !x) return fail(PARALLAX_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(W_R, 16) || !aligned(x, 16))
    return fail(PARALLAX_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (B < 1 || Hq < 1 || d_model < 1)
    return fail(PARALLAX_ERR_INVALID_ARG, "B, Hq and d_model must be >= 1");
  if (d != 64 && d != 128) return fail(PARALLAX_ERR_UNSUPPORTED, "head dim d must be 64 or 128");
  if (dtype != PARALLAX_F32 && d_model % 8 != 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "d_model must be a multiple of 8 for bf16");
  if ((long long)d_model * 2 * 64 >= (1LL << 30) || (long long)Hq * d > (1LL << 28) ||
      (long long)B > (1LL << 22))
    return fail(PARALLAX_ERR_UNSUPPORTED, "probe size out of range");
  return PARALLAX_OK;
}

}  // namespace

extern "C" {

const char* parallax_last_error(void) { return g_last_error.c_str(); }

int parallax_set_option(int option, int value) {
  switch (option) {
    case PARALLAX_OPT_CHUNK:
      if (value < 0 || value % 64 != 0)
        return fail(PARALLAX_ERR_INVALID_ARG, "chunk must be 0 or a positive multiple of 64");
      g_opt_chunk = value;
      return PARALLAX_OK;
    case PARALLAX_OPT_KERNEL:
      if (value < 0 || value > 2) return fail(PARALLAX_ERR_INVALID_ARG, "kernel must be 0, 1 or 2");
      g_opt_kernel = value;
      return PARALLAX_OK;
    case PARALLAX_OPT_PROFILE:
      if (value != 0 && value != 1) return fail(PARALLAX_ERR_INVALID_ARG, "profile must be 0 or 1");
      g_opt_profile = value;
      return PARALLAX_OK;
    case PARALLAX_OPT_ITEMS:
      if (value < 0 || value > 2) return fail(PARALLAX_ERR_INVALID_ARG, "items must be 0, 1 or 2");
      g_opt_items = value;
      return PARALLAX_OK;
    case PARALLAX_OPT_ORDER:
      if (value < 0 || value > 2) return fail(PARALLAX_ERR_INVALID_ARG, "order must be 0, 1 or 2");
      g_opt_order = value;
      return PARALLAX_OK;
    case PARALLAX_OPT_FUSE:
      if (value < 0 || value > 2) return fail(PARALLAX_ERR_INVALID_ARG, "fuse must be 0, 1 or 2");
      g_opt_fuse = value;
      return PARALLAX_OK;
    case PARALLAX_OPT_PREFETCH:
      if (value < 0 || value > 2)
        return fail(PARALLAX_ERR_INVALID_ARG, "prefetch must be 0, 1 or 2");
      g_opt_prefetch = value;
      return PARALLAX_OK;
    case PARALLAX_OPT_PROBE:
      if (value < 0 || value > 2) return fail(PARALLAX_ERR_INVALID_ARG, "probe must be 0, 1 or 2");
      g_opt_probe = value;
      return PARALLAX_OK;

    default:
      return fail(PARALLAX_ERR_INVALID_ARG, "unknown option " + std::to_string(option));
  }
}

int parallax_get_option(int option, int* value) {
  if (!value) return fail(PARALLAX_ERR_INVALID_ARG, "value is null");
  switch (option) {
    case PARALLAX_OPT_CHUNK: *value = g_opt_chunk; return PARALLAX_OK;
    case PARALLAX_OPT_KERNEL: *value = g_opt_kernel; return PARALLAX_OK;
    case PARALLAX_OPT_PROFILE: *value = g_opt_profile; return PARALLAX_OK;
    case PARALLAX_OPT_ITEMS: *value = g_opt_items; return PARALLAX_OK;
    case PARALLAX_OPT_ORDER: *value = g_opt_order; return PARALLAX_OK;
    case PARALLAX_OPT_FUSE: *value = g_opt_fuse; return PARALLAX_OK;
    case PARALLAX_OPT_PREFETCH: *value = g_opt_prefetch; return PARALLAX_OK;
    case PARALLAX_OPT_PROBE: *value = g_opt_probe; return PARALLAX_OK;
    default: return fail(PARALLAX_ERR_INVALID_ARG, "unknown option " + std::to_string(option));
  }
}

int parallax_profile_reset(void) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  for (auto& t : g_prof) {
    for (auto& pr : t.pending) {
      (void)hipEventSynchronize(pr.second);
      g_event_pool.push_back(pr.first);
      g_event_pool.push_back(pr.second);
    }
    t.pending.clear();
    t.total_ms = 0.0;
    t.launches = 0;
  }
  return PARALLAX_OK;
}

int parallax_profile_read(int kernel, double* total_ms, long long* launches) {
  if (kernel < 0 || kernel > 4) return fail(PARALLAX_ERR_INVALID_ARG, "kernel must be 0 .. 4");
  if (!total_ms || !launches) return fail(PARALLAX_ERR_INVALID_ARG, "null output pointer");
  std::lock_guard<std::mutex> g(g_prof_mu);
  Timing& t = g_prof[kernel];
  for (auto& pr : t.pending) {
    hipError_t e = hipEventSynchronize(pr.second);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    t.total_ms += ms;
    t.launches += 1;
    g_event_pool.push_back(pr.first);
    g_event_pool.push_back(pr.second);
  }
  t.pending.clear();
  *total_ms = t.total_ms;
  *launches = t.launches;
  return PARALLAX_OK;
}

int parallax_probe(const void* W_R, const void* x, float* rho, int B, int Hq, int d,
                   int d_model, int dtype, hipStream_t stream) {
  int rc = check_probe(W_R, x, B, Hq, d, d_model, dtype);
  if (rc != PARALLAX_OK) return rc;
  if (!rho) return fail(PARALLAX_ERR_INVALID_ARG, "null pointer argument (rho)");
  if (!aligned(rho, 16)) return fail(PARALLAX_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const parallax::LaunchEvents ev = profile_events();
  hipError_t e = parallax::launch_probe(W_R, x, rho, B, Hq * d, d_model,
                                        dtype == PARALLAX_F32 ? 1 : 0, g_opt_probe, ev, stream);
  profile_record(0, ev, e == hipSuccess);
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return PARALLAX_OK;
}

int parallax_decode_plan(int B, int Hq, int Hkv, int d, int max_ctx, int dtype, int* chunk,
                         int* splits, int* kernel) {
  int rc = check_decode_shape(B, Hq, Hkv, d, max_ctx, dtype);
  if (rc != PARALLAX_OK) return rc;
  if (!chunk || !splits || !kernel) return fail(PARALLAX_ERR_INVALID_ARG, "null output pointer");
  const Plan p = make_plan(B, Hq, Hkv, d, max_ctx, dtype);
  *chunk = p.chunk;
  *splits = p.splits;
  *kernel = p.kernel;
  return PARALLAX_OK;
}

int parallax_probe_decode_plan(int B, int Hq, int Hkv, int d, int d_model, int max_ctx, int dtype,
                               int* fused) {
  int rc = check_decode_shape(B, Hq, Hkv, d, max_ctx, dtype);
  if (rc != PARALLAX_OK) return rc;
  if (d_model < 1) return fail(PARALLAX_ERR_INVALID_ARG, "d_model must be >= 1");
  if (!fused) return fail(PARALLAX_ERR_INVALID_ARG, "null output pointer");
  const Plan p = make_plan(B, Hq, Hkv, d, max_ctx, dtype);
  *fused = fuse_probe(p, B, Hq, Hkv, d, d_model, dtype) ? 1 : 0;
  return PARALLAX_OK;
}

}  // extern "C"

namespace {

// A checked and planned decode call. The workspace holds `front` bytes for the
// caller (the probe's rho in parallax_probe_decode), then the split states.
struct DecodeCall {
  parallax::DecodeArgs a;
  Plan p;
  void* front = nullptr;
};

// Workspace bytes of a planned decode call: `front` bytes for the caller
// (rounded up to 256), then one (m, l, S) record and the A, P sums per
// (sequence, query head, split) when there is more than one split.
size_t decode_ws_bytes(const Plan& p, int B, int Hq, int d, size_t front_bytes) {
  const size_t states = p.splits > 1 ? (size_t)B * Hq * p.splits : 0;
  return round_up(front_bytes, 256) + states * sizeof(float4) + states * 2 * d * sizeof(float);
}

// use_scratch: take the workspace from the static scratch array (rejecting
// plans that need more) instead of the per-stream workspace; no allocation.
int setup_decode(const void* q, const float* rho, const void* k_cache, const void* v_cache,
                 const int* seq_lens, void* out, int B, int Hq, int Hkv, int d, int max_ctx,
                 int dtype, size_t front_bytes, hipStream_t stream, DecodeCall& c,
                 bool use_scratch = false) {
  int rc = check_decode_shape(B, Hq, Hkv, d, max_ctx, dtype);
  if (rc != PARALLAX_OK) return rc;
  if (!q || !k_cache || !v_cache || !seq_lens || !out)
    return fail(PARALLAX_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(q, 16) || (rho && !aligned(rho, 16)) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(out, 16) || !aligned(seq_lens, 4))
    return fail(PARALLAX_ERR_INVALID_ARG, "pointers must be 16-byte aligned (seq_lens 4-byte)");

  const Plan p = make_plan(B, Hq, Hkv, d, max_ctx, dtype);
  c.p = p;
  parallax::DecodeArgs& a = c.a;
  a.q = q;
  a.rho = rho;
  a.k = k_cache;
  a.v = v_cache;
  a.seq_lens = seq_lens;
  a.out = out;
  a.ml = nullptr;
  a.ap = nullptr;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_ctx = max_ctx;
  a.chunk = p.chunk;
  a.splits = p.splits;
  a.out_f32 = (dtype == PARALLAX_BF16) ? 0 : 1;
  a.prefetch = p.prefetch;
  a.scale_log2 = parallax::kLog2e / sqrtf((float)d);

  const size_t front = round_up(front_bytes, 256);
  const size_t states = p.splits > 1 ? (size_t)B * Hq * p.splits : 0;
  if (front + states > 0) {
    const size_t need = decode_ws_bytes(p, B, Hq, d, front_bytes);
    void* ws = nullptr;
    if (use_scratch) {
      if (need > kScratchBytes)
        return fail(PARALLAX_ERR_UNSUPPORTED,
                    "this shape needs " + std::to_string(need) + " bytes of scratch (rho and "
                    "split states), more than the " + std::to_string(kScratchBytes) +
                    " bytes of the static scratch array of the allocation-free call");
      rc = scratch_address(&ws);
    } else {
      rc = get_workspace(stream, need, &ws);
    }
    if (rc != PARALLAX_OK) return rc;
    c.front = front ? ws : nullptr;
    if (states) {
      a.ml = (float4*)((char*)ws + front);
      a.ap = (float*)((char*)ws + front + states * sizeof(float4));
    }
  }
  return PARALLAX_OK;
}

// Decode (split-K pass) and, for split sequences, the merge.
int launch_decode_call(const DecodeCall& c, int d, int dtype, int fused, hipStream_t stream,
                       bool timed = true) {
  const parallax::DecodeArgs& a = c.a;
  parallax::LaunchEvents ev = timed ? profile_events() : parallax::LaunchEvents{};
  hipError_t e =
      (c.p.kernel >= 2)
          ? parallax::launch_decode_mfma(a, d, c.p.kernel == 3 ? 1 : 0, c.p.compact, fused, ev,
                                         stream)
          : parallax::launch_decode_generic(a, d, dtype == PARALLAX_F32 ? 1 : 0, fused, ev, stream);
  profile_record(1, ev, e == hipSuccess);
  if (e == hipSuccess && c.p.splits > 1) {
    ev = timed ? profile_events() : parallax::LaunchEvents{};
    e = parallax::launch_merge(a, d, ev, stream);
    profile_record(2, ev, e == hipSuccess);
  }
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return PARALLAX_OK;
}

// Shared by parallax_decode and parallax_softmax_decode (rho == nullptr).
int decode_impl(const void* q, const float* rho, const void* k_cache, const void* v_cache,
                const int* seq_lens, void* out, int B, int Hq, int Hkv, int d, int max_ctx,
                int dtype, hipStream_t stream) {
  DecodeCall c;
  int rc = setup_decode(q, rho, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, d, max_ctx, dtype, 0,
                        stream, c);
  if (rc != PARALLAX_OK) return rc;
  return launch_decode_call(c, d, dtype, 0, stream);
}

// parallax_probe_decode and its allocation-free variant (noalloc: rho and the
// split states go to the static scratch array; no allocation and no profiling
// events; shapes whose plan needs more than the array are rejected).
int probe_decode_impl(const void* W_R, const void* x, const void* q, const void* k_cache,
                      const void* v_cache, const int* seq_lens, void* out, int B, int Hq, int Hkv,
                      int d, int d_model, int max_ctx, int dtype, hipStream_t stream,
                      bool noalloc) {
  int rc = check_probe(W_R, x, B, Hq, d, d_model, dtype);
  if (rc != PARALLAX_OK) return rc;
  rc = check_decode_shape(B, Hq, Hkv, d, max_ctx, dtype);
  if (rc != PARALLAX_OK) return rc;
  const bool fused = fuse_probe(make_plan(B, Hq, Hkv, d, max_ctx, dtype), B, Hq, Hkv, d, d_model,
                                dtype);
  DecodeCall c;
  rc = setup_decode(q, nullptr, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, d, max_ctx, dtype,
                    fused ? 0 : (size_t)B * Hq * d * sizeof(float), stream, c, noalloc);
  if (rc != PARALLAX_OK) return rc;
  if (fused) {
    c.a.W_R = W_R;
    c.a.x = x;
    c.a.d_model = d_model;
    return launch_decode_call(c, d, dtype, 1, stream, !noalloc);
  }
  float* rho = (float*)c.front;
  const parallax::LaunchEvents ev = noalloc ? parallax::LaunchEvents{} : profile_events();
  hipError_t e = parallax::launch_probe(W_R, x, rho, B, Hq * d, d_model,
                                        dtype == PARALLAX_F32 ? 1 : 0, g_opt_probe, ev, stream);
  profile_record(0, ev, e == hipSuccess);
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  c.a.rho = rho;
  return launch_decode_call(c, d, dtype, 0, stream, !noalloc);
}

}  // namespace

extern "C" {

int parallax_decode(const void* q, const float* rho, const void* k_cache, const void* v_cache,
                    const int* seq_lens, void* out, int B, int Hq, int Hkv, int d, int max_ctx,
                    int dtype, hipStream_t stream) {
  if (!rho) return fail(PARALLAX_ERR_INVALID_ARG, "null pointer argument (rho)");
  return decode_impl(q, rho, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, d, max_ctx, dtype,
                     stream);
}

int parallax_softmax_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int* seq_lens, void* out, int B, int Hq, int Hkv, int d,
                            int max_ctx, int dtype, hipStream_t stream) {
  return decode_impl(q, nullptr, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, d, max_ctx, dtype,
                     stream);
}

int parallax_probe_decode(const void* W_R, const void* x, const void* q, const void* k_cache,
                          const void* v_cache, const int* seq_lens, void* out, int B, int Hq,
                          int Hkv, int d, int d_model, int max_ctx, int dtype, hipStream_t stream) {
  return probe_decode_impl(W_R, x, q, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, d, d_model,
                           max_ctx, dtype, stream, false);
}

int parallax_probe_decode_noalloc(const void* W_R, const void* x, const void* q,
                                  const void* k_cache, const void* v_cache, const int* seq_lens,
                                  void* out, int B, int Hq, int Hkv, int d, int d_model,
                                  int max_ctx, int dtype, hipStream_t stream) {
  return probe_decode_impl(W_R, x, q, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, d, d_model,
                           max_ctx, dtype, stream, true);
}

long long parallax_noalloc_scratch_bytes(void) { return (long long)kScratchBytes; }

}  // extern "C"

namespace {

// Shared by parallax_prefill and parallax_softmax_prefill (rho == nullptr).
int prefill_impl(const void* q, const float* rho, const void* k_cache, const void* v_cache,
                 const int* prefix_lens, void* out, int B, int T, int Hq, int Hkv, int d,
                 int max_ctx, int dtype, hipStream_t stream) {
  int rc = check_decode_shape(B, Hq, Hkv, d, max_ctx, dtype);
  if (rc != PARALLAX_OK) return rc;
  if (T < 1 || T > max_ctx) return fail(PARALLAX_ERR_INVALID_ARG, "T must be in 1 .. max_ctx");
  if (!q || !k_cache || !v_cache || !out)
    return fail(PARALLAX_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(q, 16) || (rho && !aligned(rho, 16)) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, 16) || (prefix_lens && !aligned(prefix_lens, 4)))
    return fail(PARALLAX_ERR_INVALID_ARG, "pointers must be 16-byte aligned (prefix_lens 4-byte)");
  if (B > 65535 || Hkv > 65535 || (long long)T * (Hq / Hkv) > (1LL << 30) ||
      (long long)B * T * Hq > (1LL << 40))
    return fail(PARALLAX_ERR_UNSUPPORTED, "prefill size out of range");
  if (dtype == PARALLAX_F32) {
    // fp32: the vector-ALU decode kernel over B*T single-token "sequences"
    // (token t of sequence b attends to rows 0 .. P_b + t), one split each.
    if ((long long)B * T * Hkv * (Hq / Hkv) > 0x7fffffffLL)
      return fail(PARALLAX_ERR_UNSUPPORTED, "prefill size out of range");
    parallax::DecodeArgs g;
    g.q = q;
    g.rho = rho;
    g.k = k_cache;
    g.v = v_cache;
    g.seq_lens = nullptr;
    g.out = out;
    g.ml = nullptr;
    g.ap = nullptr;
    g.B = B * T;
    g.Hq = Hq;
    g.Hkv = Hkv;
    g.max_ctx = max_ctx;
    g.chunk = max_ctx;
    g.splits = 1;
    g.out_f32 = 1;
    g.scale_log2 = parallax::kLog2e / sqrtf((float)d);
    g.T = T;
    g.prefix = prefix_lens;
    const parallax::LaunchEvents ev = profile_events();
    hipError_t e = parallax::launch_decode_generic(g, d, 1, 0, ev, stream);
    profile_record(3, ev, e == hipSuccess);
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return PARALLAX_OK;
  }
  parallax::PrefillArgs a;
  a.q = q;
  a.rho = rho;
  a.k = k_cache;
  a.v = v_cache;
  a.prefix = prefix_lens;
  a.out = out;
  a.B = B;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_ctx = max_ctx;
  a.out_f32 = dtype == PARALLAX_BF16 ? 0 : 1;
  a.scale_log2 = parallax::kLog2e / sqrtf((float)d);
  const parallax::LaunchEvents ev = profile_events();
  hipError_t e = parallax::launch_prefill_mfma(a, d, ev, stream);
  profile_record(3, ev, e == hipSuccess);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return PARALLAX_OK;
}

}  // namespace

extern "C" {

int parallax_prefill(const void* q, const float* rho, const void* k_cache, const void* v_cache,
                     const int* prefix_lens, void* out, int B, int T, int Hq, int Hkv, int d,
                     int max_ctx, int dtype, hipStream_t stream) {
  if (!rho) return fail(PARALLAX_ERR_INVALID_ARG, "null pointer argument (rho)");
  return prefill_impl(q, rho, k_cache, v_cache, prefix_lens, out, B, T, Hq, Hkv, d, max_ctx,
                      dtype, stream);
}

int parallax_softmax_prefill(const void* q, const void* k_cache, const void* v_cache,
                             const int* prefix_lens, void* out, int B, int T, int Hq, int Hkv,
                             int d, int max_ctx, int dtype, hipStream_t stream) {
  return prefill_impl(q, nullptr, k_cache, v_cache, prefix_lens, out, B, T, Hq, Hkv, d, max_ctx,
                      dtype, stream);
}

}  // extern "C"

extern "C" {

int parallax_read_bandwidth(const void* buf, long long bytes, unsigned* sink, hipStream_t stream) {
  constexpr int kGrid = 256;
  if (!buf || !sink) return fail(PARALLAX_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(buf, 16) || !aligned(sink, 4))
    return fail(PARALLAX_ERR_INVALID_ARG, "buf must be 16-byte aligned (sink 4-byte)");
  if (bytes <= 0 || bytes % ((long long)kGrid * 4096) != 0 || bytes / kGrid >= (1LL << 31))
    return fail(PARALLAX_ERR_INVALID_ARG,
                "bytes must be a positive multiple of 1 MiB and below 512 GiB");
  const parallax::LaunchEvents ev = profile_events();
  hipError_t e = parallax::launch_read_stream(buf, (size_t)bytes, kGrid, sink, ev, stream);
  profile_record(4, ev, e == hipSuccess);
  if (e != hipSuccess) return hip_fail(e, "read launch");
  return PARALLAX_OK;
}

}  // extern "C"
