/*
 * parallax.h — C ABI of libparallax.so: Parallax decode attention on AMD
 * Instinct MI355X (gfx950).
 *
 * Parallax keeps softmax attention and subtracts a learned covariance
 * correction: the output for query i is softmax attention minus the
 * softmax-weighted KV covariance multiplied by a probe rho_i = W_R x_i, where
 * W_R is a learned projection of the layer input x_i; W_R = 0 gives plain
 * softmax attention exactly (zubnet.ai (pt), "Parallax mantém softmax ...",
 * second paragraph; zubnet.ai (fr), "Parallax garde softmax ...", second
 * paragraph; encorp.ai (de), sections "Parallax behält Softmax bei" and "Warum
 * das Entfernen des konjugierten Gradienten-Solvers ..."). The setting is
 * decoding with a KV cache: one query token per sequence (same paragraph:
 * the method still needs a KV cache and is not linear-complexity attention).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller. The library
 *   never frees caller memory and keeps no pointer after a call returns.
 * - Calls only enqueue work on `stream` (0 = the null stream) and return; the
 *   results are valid once the caller synchronises that stream.
 * - Arguments are checked on the host before any HIP call. On failure the call
 *   returns a non-zero parallax_status, enqueues nothing and leaves a message
 *   in parallax_last_error(). No C++ exception crosses this ABI.
 * - All tensors are dense, row-major (last index fastest), 16-byte aligned.
 * - dtype selects the storage type (see parallax_dtype). rho is passed as
 *   fp32 and all accumulation is fp32. Precision of rho inside the kernels:
 *   PARALLAX_F32 uses rho as given. The bf16 dtypes run on the matrix cores,
 *   which carry each component of rho as two bf16 terms, hi = bf16(rho) and
 *   lo = bf16(rho - hi) (round to nearest even): |rho_i - (hi_i + lo_i)| <=
 *   2^-16 |rho_i|, about 16 significant bits. The probes p_j = k_j . rho then
 *   differ from their fp32 value by at most 2^-16 sum_i |k_ji rho_i|, and the
 *   output by at most 2^-16 sum_j w_j (sum_i |k_ji rho_i|) |v_j - vbar| per
 *   component (w: the softmax weights), beyond fp32 rounding. This is far
 *   below the bf16 output's rounding; it matters only when rho is an exact
 *   solve (local linear attention) read through an fp32 output.
 * - Calls may be made from several threads at once: options are atomic, the
 *   workspace cache and the profiling records are locked, and the error
 *   message is per thread. Calls that share output buffers, or that run on
 *   one stream (they share that stream's workspace), must be ordered by the
 *   caller, as stream order does.
 */
#ifndef PARALLAX_H_
#define PARALLAX_H_

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PARALLAX_OK = 0,
  PARALLAX_ERR_INVALID_ARG = 1,   /* bad size, null or misaligned pointer, Hq % Hkv != 0 */
  PARALLAX_ERR_UNSUPPORTED = 2,   /* valid but unsupported: d not in {64, 128}, unknown dtype */
  PARALLAX_ERR_HIP = 3,           /* a HIP runtime call or kernel launch failed */
  PARALLAX_ERR_NO_MEMORY = 4      /* the split-K workspace could not be allocated or grown */
} parallax_status;

typedef enum {
  PARALLAX_F32 = 0,          /* x, W_R, q, K, V, out: fp32                              */
  PARALLAX_BF16 = 1,         /* x, W_R, q, K, V, out: bf16 (out rounded to nearest even) */
  PARALLAX_BF16_F32OUT = 2   /* x, W_R, q, K, V: bf16; out: fp32 (same arithmetic as
                                PARALLAX_BF16 up to the final rounding)                  */
} parallax_dtype;

/*
 * parallax_probe — the layer-input probe rho = W_R x (zubnet.ai (pt),
 * "Parallax mantém softmax ...", second paragraph: the learned projection W_R
 * probes the KV covariance directly from the layer input).
 *
 *   W_R : [Hq*d, d_model], dtype storage (bf16 for both bf16 dtypes)
 *   x   : [B, d_model],    dtype storage
 *   rho : [B, Hq, d] fp32 output; rho[b][h][i] = sum_c W_R[h*d + i][c] * x[b][c]
 *
 * Row h*d + i of W_R produces component i of query head h's probe (one probe
 * per query head). Requires B >= 1, Hq >= 1, d in {64, 128}, d_model >= 1, and
 * d_model % 8 == 0 for the bf16 dtypes.
 */
int parallax_probe(const void* W_R, const void* x, float* rho,
                   int B, int Hq, int d, int d_model, int dtype, hipStream_t stream);

/*
 * parallax_decode — one decode step of Parallax attention (zubnet.ai (pt),
 * second paragraph: softmax attention minus the KV covariance times the probe;
 * both branches read the same KV stream — same paragraph and encorp.ai (de),
 * section "Wie Parallax die Hardware-Geschichte auf Hopper-GPUs verändert").
 *
 * For every sequence b and query head h, with g = h / (Hq / Hkv) and
 * n = seq_lens[b], over cached tokens j = 0 .. n-1:
 *   s_j  = q[b][h] . K[b][g][j] / sqrt(d),   w = softmax(s)
 *   kbar = sum_j w_j K[b][g][j],   vbar = sum_j w_j V[b][g][j]
 *   C    = sum_j w_j (V[b][g][j] - vbar)(K[b][g][j] - kbar)^T      (d x d)
 *   out[b][h] = vbar - C rho[b][h]
 * computed in one pass as out = A/l - (P/l - (A/l)(S/l)) from the running sums
 * l = sum e_j, S = sum e_j p_j, A = sum e_j v_j, P = sum e_j p_j v_j with
 * e_j = exp(s_j - max s) and p_j = K[b][g][j] . rho[b][h].
 *
 *   q        : [B, Hq, d]               dtype storage (bf16 for both bf16 dtypes)
 *   rho      : [B, Hq, d]               fp32 (from parallax_probe)
 *   k_cache  : [B, Hkv, max_ctx, d]     dtype storage; rows j >= seq_lens[b] never
 *                                       reach the output (the matrix-core kernel may fetch
 *                                       up to 128 of them per split and discard them)
 *   v_cache  : [B, Hkv, max_ctx, d]     same layout as k_cache
 *   seq_lens : [B] int32, device memory; 0 <= seq_lens[b] <= max_ctx
 *   out      : [B, Hq, d]               fp32 or bf16 per dtype
 *
 * Requires B, Hq, Hkv, max_ctx >= 1, Hq % Hkv == 0, d in {64, 128}; Hq above
 * 65535 is PARALLAX_ERR_UNSUPPORTED (also for the prefill calls). A sequence
 * with seq_lens[b] == 0 gets out = 0 (a convention). seq_lens[b] > max_ctx is
 * clamped to max_ctx and seq_lens[b] < 0 to 0 on the device (memory safety; a
 * caller error).
 *
 * Long sequences are split into chunks processed in parallel and a second
 * kernel merges the chunks' states by their running maxima (sequences that fit
 * in one chunk are finished by the first kernel). The chunk states live in a
 * workspace the library owns, cached per (device, stream) and kept until the
 * process ends; it grows stream-ordered on `stream` (hipMallocAsync, at least
 * doubling; the old buffer is kept). Growing is refused (PARALLAX_ERR_NO_MEMORY) while
 * `stream` is being captured into a graph: make one call of the largest shape
 * on that stream before capturing. A graph captured on a stream uses that
 * stream's workspace at the address it had during capture (a buffer the
 * workspace grows out of is kept, never freed, so the address stays valid):
 * replays of such a graph, eager calls on the capture stream and other graphs
 * captured on it all write the same partial states, so they must not run
 * concurrently with each other. The cache is keyed by the stream handle: a
 * stream with library work still pending must be synchronised before it is
 * destroyed, since a stream created afterwards may receive the same handle and
 * would share the workspace.
 */
int parallax_decode(const void* q, const float* rho, const void* k_cache,
                    const void* v_cache, const int* seq_lens, void* out,
                    int B, int Hq, int Hkv, int d, int max_ctx, int dtype,
                    hipStream_t stream);

/*
 * parallax_softmax_decode — the same decode kernel without the correction
 * branch: plain softmax attention out[b][h] = sum_j w_j V[b][g][j], which is
 * what Parallax reduces to when W_R = 0 (encorp.ai (de), section "Parallax
 * behält Softmax bei"). It reads the same KV stream and does half the
 * arithmetic per key, so timing it beside parallax_decode gives the cost of
 * the correction at equal bytes (and, with twice the query heads, at equal
 * arithmetic). Arguments, layouts and errors as parallax_decode, without rho.
 */
int parallax_softmax_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int* seq_lens, void* out, int B, int Hq, int Hkv, int d,
                            int max_ctx, int dtype, hipStream_t stream);

/*
 * parallax_probe_decode — one whole decode step: the probe rho = W_R x of every
 * query head and the Parallax decode that uses it, in one call. The probe is
 * computed from the layer input as part of the attention step (zubnet.ai (pt),
 * "Parallax mantém softmax ...", second paragraph: the probe comes from the
 * layer input through the learned W_R, and the correction reuses the KV stream
 * of softmax attention).
 *
 *   W_R, x   : as parallax_probe (W_R [Hq*d, d_model], x [B, d_model])
 *   q, k_cache, v_cache, seq_lens, out : as parallax_decode
 *
 * The result equals parallax_probe followed by parallax_decode on the same
 * inputs, up to fp32 rounding of rho. Two plans (parallax_probe_decode_plan
 * tells which one a shape gets):
 *   - fused: the decode kernel computes rho of each work item's query heads
 *     from W_R and x in its prologue, into on-chip memory; rho is never
 *     written to device memory and the step is one launch (plus the merge of
 *     split sequences). Each work item then reads G*d rows of W_R, so this is
 *     chosen only where those reads are small per item and in total (small
 *     d_model and few work items): there they cost less than a launch.
 *   - separate: the probe kernel writes rho into the library's workspace (the
 *     same per-stream workspace as the split states, grown the same way), then
 *     the decode runs as parallax_decode.
 * Requires the argument rules of both parallax_probe and parallax_decode;
 * errors as theirs. Enqueue-only on `stream`.
 */
int parallax_probe_decode(const void* W_R, const void* x, const void* q, const void* k_cache,
                          const void* v_cache, const int* seq_lens, void* out,
                          int B, int Hq, int Hkv, int d, int d_model, int max_ctx, int dtype,
                          hipStream_t stream);

/*
 * parallax_probe_decode_noalloc — parallax_probe_decode for callers that must
 * not allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid allocation. Same arguments, plan,
 * kernels and results as parallax_probe_decode (bit for bit); it never calls
 * an allocator and records no profiling events.
 *
 * The probe's rho (separate-probe plan) and the split-K states live in a
 * static device array of parallax_noalloc_scratch_bytes() bytes (64 MiB),
 * one per device, held from the first call on that device until the process
 * ends (that first call looks up the array's address; make it before any
 * capture). A shape whose plan needs more — B*Hq*d*4 bytes for rho unless the
 * probe is fused, plus B*Hq*splits*(16 + 8*d) bytes when sequences are split
 * — returns PARALLAX_ERR_UNSUPPORTED with the sizes in the message (all five
 * benchmark workloads fit). Nothing in the array needs clearing between calls.
 * Every call on one device shares that device's array: calls that may overlap
 * on one device (different streams, threads or graph replays) race on it and
 * must be ordered by the caller. Errors otherwise as parallax_probe_decode.
 */
int parallax_probe_decode_noalloc(const void* W_R, const void* x, const void* q,
                                  const void* k_cache, const void* v_cache, const int* seq_lens,
                                  void* out, int B, int Hq, int Hkv, int d, int d_model,
                                  int max_ctx, int dtype, hipStream_t stream);

/* Size in bytes of the static scratch array of parallax_probe_decode_noalloc. */
long long parallax_noalloc_scratch_bytes(void);

/*
 * parallax_probe_decode_plan — writes 1 to *fused when parallax_probe_decode
 * would compute the probe inside the decode kernel for this shape, else 0.
 * Same shape checks as parallax_decode; d_model >= 1.
 */
int parallax_probe_decode_plan(int B, int Hq, int Hkv, int d, int d_model, int max_ctx, int dtype,
                               int* fused);

/*
 * parallax_prefill — the causal many-query forward (prefill or chunked
 * prefill): T new tokens per sequence, each attending to the cache up to and
 * including its own position. The layer is pretrained as language-model
 * attention (encorp.ai (de), section "Die Pretraining-Gewinne sind real ...");
 * the causal prefix is the reading taken, and each token's output is the
 * Parallax output of parallax_decode over its prefix with its own query and
 * probe (zubnet.ai (pt), second paragraph).
 *
 * Token t (0 <= t < T) of sequence b sits at cache position P_b + t, with
 * P_b = prefix_lens[b] (0 when prefix_lens is null), and attends to cache rows
 * 0 .. P_b + t of KV head g = h / (Hq / Hkv). The caller has written the K/V
 * rows of the new tokens into the cache at P_b .. P_b + T - 1.
 *
 *   q           : [B, T, Hq, d]            dtype storage (bf16 for both bf16 dtypes)
 *   rho         : [B, T, Hq, d]            fp32 (from parallax_probe on the B*T tokens)
 *   k_cache     : [B, Hkv, max_ctx, d]     dtype storage; rows >= P_b + T are never read
 *   v_cache     : [B, Hkv, max_ctx, d]     same layout as k_cache
 *   prefix_lens : [B] int32, device memory, or null; 0 <= P_b <= max_ctx - T
 *   out         : [B, T, Hq, d]            bf16 (PARALLAX_BF16) or fp32 (the other dtypes)
 *
 * Requires 1 <= T <= max_ctx and the decode shape rules. The bf16 dtypes run
 * on the matrix cores; PARALLAX_F32 runs the vector-ALU decode kernel with one
 * single-token sequence per token (a correctness path, not a fast one). P_b
 * outside 0 .. max_ctx - T is clamped on the device (memory safety; a caller
 * error). No workspace; enqueue-only on `stream`.
 */
int parallax_prefill(const void* q, const float* rho, const void* k_cache, const void* v_cache,
                     const int* prefix_lens, void* out, int B, int T, int Hq, int Hkv, int d,
                     int max_ctx, int dtype, hipStream_t stream);

/*
 * parallax_softmax_prefill — the same causal forward without the correction
 * branch (plain softmax attention, the W_R = 0 reduction; encorp.ai (de),
 * section "Parallax behält Softmax bei"): the baseline that prices the
 * correction in the compute-bound regime. Arguments, layouts and errors as
 * parallax_prefill, without rho.
 */
int parallax_softmax_prefill(const void* q, const void* k_cache, const void* v_cache,
                             const int* prefix_lens, void* out, int B, int T, int Hq, int Hkv,
                             int d, int max_ctx, int dtype, hipStream_t stream);

/* Message of the last non-OK status returned on the calling thread ("" if none). */
const char* parallax_last_error(void);

/*
 * parallax_decode_plan — the launch plan parallax_decode would use (for tests
 * and measurement). Writes the chunk length in keys, the number of splits per
 * (sequence, KV head) and the decode kernel (1 = generic vector-ALU kernel,
 * 2 = matrix-core kernel with four waves per work item, 3 = matrix-core
 * kernel with one wave per work item). Same argument checks as
 * parallax_decode.
 */
int parallax_decode_plan(int B, int Hq, int Hkv, int d, int max_ctx, int dtype,
                         int* chunk, int* splits, int* kernel);

/*
 * Process-wide tuning options (for tests and measurement). Not to be changed
 * while other threads call the library.
 *   PARALLAX_OPT_CHUNK   : 0 = automatic, else keys per split (multiple of 64)
 *   PARALLAX_OPT_KERNEL  : 0 = automatic, 1 = force the generic kernel,
 *                          2 = force the matrix-core kernel (where supported)
 *   PARALLAX_OPT_PROFILE : 1 = record HIP events around every kernel launch
 *   PARALLAX_OPT_ITEMS   : matrix-core work items: 0 = automatic,
 *                          1 = four waves per item, 2 = one wave per item
 *   PARALLAX_OPT_ORDER   : numbering of four-wave work items: 0 = automatic,
 *                          1 = every (split, sequence, head) item, split-major,
 *                          2 = only the non-empty ones (up to 256 sequences and
 *                          64 splits; otherwise as 1)
 *   PARALLAX_OPT_FUSE    : probe placement in parallax_probe_decode:
 *                          0 = automatic, 1 = always a separate probe launch,
 *                          2 = inside the decode kernel wherever its plan
 *                          allows it (generic kernel, or four-wave items
 *                          without the compacted numbering; d_model * element
 *                          size a multiple of 16 bytes)
 *   PARALLAX_OPT_PREFETCH: matrix-core kernel, first K/V tile of each wave of a
 *                          work item requested before the sequence length
 *                          arrives:
 *                          0 = automatic, 1 = never, 2 = wherever the item
 *                          numbering is not compacted
 *   PARALLAX_OPT_PROBE   : bf16 probe kernel (parallax_probe and the separate
 *                          probe of parallax_probe_decode): 0 = automatic,
 *                          1 = the small-batch matrix-core kernel (row blocks
 *                          of at most 64 rows), 2 = the LDS-tiled GEMM
 */
typedef enum {
  PARALLAX_OPT_CHUNK = 1,
  PARALLAX_OPT_KERNEL = 2,
  PARALLAX_OPT_PROFILE = 3,
  PARALLAX_OPT_ITEMS = 4,
  PARALLAX_OPT_ORDER = 5,
  PARALLAX_OPT_FUSE = 6,
  PARALLAX_OPT_PREFETCH = 7,
  PARALLAX_OPT_PROBE = 8
} parallax_option;

int parallax_set_option(int option, int value);
int parallax_get_option(int option, int* value);

/*
 * Kernel timing when PARALLAX_OPT_PROFILE is 1: every launch carries start and
 * stop HIP events stamped by its own dispatch (hipExtLaunchKernel), so the
 * timing adds no work between kernels. kernel: 0 = probe, 1 = decode
 * (split-K pass), 2 = merge, 3 = prefill, 4 = the read reference below.
 * parallax_profile_read waits for the recorded events and returns the summed
 * duration (ms) and the number of launches since the last reset.
 */
int parallax_profile_read(int kernel, double* total_ms, long long* launches);
int parallax_profile_reset(void);

/*
 * parallax_read_bandwidth — a measurement hook, not part of the method: reads
 * `bytes` of device memory at `buf` once, with the load shape the decode kernel
 * uses for K (non-temporal 16-byte loads, eight in flight per lane, 256
 * workgroups each streaming a contiguous share), so that the decode's HBM rate
 * can be stated against a rate this machine reaches as well as the nominal
 * peak. bytes: a positive multiple of 1 MiB, below 512 GiB; buf 16-byte
 * aligned; sink: 4 bytes of device memory the kernel may write (it keeps the
 * loads from being optimised away). Enqueue-only on `stream`; time it with
 * PARALLAX_OPT_PROFILE (kernel 4).
 */
int parallax_read_bandwidth(const void* buf, long long bytes, unsigned* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif  /* PARALLAX_H_ */
