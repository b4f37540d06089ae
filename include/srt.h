/*
 * srt.h - C ABI of the scaled-RoPE tiled attention library (libsrt.so, gfx950).
 *
 * RoPE with PI / NTK-aware / YaRN frequency scaling applied to Q and K, fused
 * into tiled online-softmax causal attention that never forms the N x N score
 * matrix; a log-sum-exp merge of partial attention states (one device's ring
 * step); split-K decode over a rotated KV cache.
 *
 * Sources, cited by page title and section:
 *   [LC]  "Long Context: RoPE / YaRN / NTK / MLA" (mathieu0905.github.io)
 *   [BK]  "8.3 长上下文技术" (LLM full-stack book, paper.xwysyy.cn)
 *   [NB]  "长上下文外推" notebook (doc.minddiy.top)
 *   [PL]  "长上下文推理：RoPE 扩展、位置插值与 Ring Attention" (plumephp.com)
 *
 * Conventions shared by every entry point
 *   - Tensors are row-major [B][H][N][D] with D innermost.  Each (b, h) slice
 *     is N rows of D contiguous elements; consecutive heads of a tensor are
 *     `*_hstride` elements apart (N*D for a contiguous tensor; larger for a
 *     slice along N of a bigger tensor).  Batch b, head h starts at element
 *     (b*H + h) * hstride.
 *   - dtype codes: SRT_F32 (float) or SRT_BF16 (bfloat16, round-to-nearest-even).
 *     Arithmetic is fp32 inside every kernel; bf16 is a storage type.
 *   - Pairing is interleaved by default: pair i is (x[2i], x[2i+1]) ([LC] §2.1,
 *     [NB] §5.1).  Half-split pairing, pair i = (x[i], x[i + D/2]) ([LC] §2.4
 *     code), is selected per call (SRT_PAIR_HALF); the table is the same.
 *   - The cos/sin table (srt_rope_cos_sin) holds, for position p and pair i,
 *     the two floats mscale*cos(p*theta'_i), mscale*sin(p*theta'_i) at
 *     table[(p*(D/2) + i)*2 + {0,1}].  A row at absolute position p uses table
 *     row p, so positions must lie in [0, table_npos).
 *   - GQA: query head h reads KV head h / (Hq / Hkv).
 *   - lse is the natural-log log-sum-exp of the scaled scores of a row.  A row
 *     with no visible key has O = 0 and lse = -inf.
 *   - Device pointers are caller-owned device memory (e.g. torch tensors);
 *     host pointers are marked _host.  The library allocates no device memory
 *     and keeps no state across calls except a thread-local error message.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it; a call returns before the work finishes.
 *   - Errors: every function returns an srt_status.  Arguments are checked on
 *     the host before anything is enqueued; a failed check returns
 *     SRT_ERR_INVALID (or SRT_ERR_UNSUPPORTED for a valid shape with no kernel)
 *     and has no side effect.  A launch failure returns SRT_ERR_HIP.  Faults
 *     inside a kernel surface at the caller's next synchronisation.  NaN/Inf in
 *     the inputs are not checked and propagate.  srt_last_error() gives the
 *     reason of the last failure on the calling thread.
 */
#ifndef SRT_H
#define SRT_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SRT_OK = 0,
  SRT_ERR_INVALID = 1,      /* bad argument: null pointer, bad size, bad method ... */
  SRT_ERR_UNSUPPORTED = 2,  /* valid arguments without a kernel (e.g. D or dtype)   */
  SRT_ERR_HIP = 3,          /* the HIP runtime refused a launch                     */
  SRT_ERR_WORKSPACE = 4     /* caller workspace smaller than required               */
} srt_status;

typedef enum { SRT_ROPE_NONE = 0, SRT_ROPE_PI = 1, SRT_ROPE_NTK = 2, SRT_ROPE_YARN = 3 } srt_rope_method;
typedef enum { SRT_F32 = 0, SRT_BF16 = 1 } srt_dtype;

/* rope_flags of srt_attn_prefill */
#define SRT_ROTATE_Q 1      /* rotate q rows on load with table rows q_pos0 + r */
#define SRT_ROTATE_K 2      /* rotate k rows on load with table rows k_pos0 + c */
#define SRT_PAIR_HALF 4     /* half-split pairs (x[i], x[i + D/2]) instead of interleaved */

/* Bytes of the scheduling block of srt_attn_prefill (see there). */
#define SRT_PREFILL_SCHED_BYTES 128

/* pairing argument of srt_rope_apply and srt_attn_decode_splitk */
#define SRT_PAIRING_INTERLEAVED 0
#define SRT_PAIRING_HALF 1

/* band labels written by srt_rope_inv_freq ([BK] §8.3.3) */
#define SRT_BAND_LOW 0      /* r(d) <  alpha : gamma = 1/s (interpolated)  */
#define SRT_BAND_MID 1      /* alpha <= r(d) <= beta : linear ramp         */
#define SRT_BAND_HIGH 2     /* r(d) >  beta  : gamma = 1 (kept)            */

/* Version of this ABI (incremented on any incompatible change). */
int srt_abi_version(void);

/* Static text for a status code.  Never NULL. */
const char* srt_status_string(int status);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char* srt_last_error(void);

/*
 * srt_rope_inv_freq - frequency step (host only, fp64, no GPU call).
 *
 * theta_d = base^(-2d/D), d = 0..D/2-1 ([LC] §2.1, [BK] §8.3.1), then by method:
 *   NONE: theta' = theta.
 *   PI:   theta' = theta / s                     ([LC] §4.2, [BK] §8.3.2).
 *   NTK:  theta' = b'^(-2d/D), b' = base * s^(D/(D-2))   ([LC] §5.2; needs D > 2).
 *   YARN: r_d = L*theta_d/(2 pi) (original base), w = clip((r_d-alpha)/(beta-alpha),0,1),
 *         theta' = (1-w)*theta/s + w*theta          ([LC] §6.2, [BK] §8.3.3);
 *         mscale = 0.1 ln s + 1 if s > 1, else 1   ([LC] §6.3-6.4).
 * mscale is 1 for the other methods.  band_out: YARN labels pair d LOW if
 * r_d < alpha, HIGH if r_d > beta, MID otherwise ([BK] §8.3.3); NONE labels
 * every pair HIGH, PI every pair LOW, NTK every pair MID.
 *
 * Arguments: method (srt_rope_method); base > 0; s > 0 (PI, NTK, YARN);
 * L > 0 (YARN); alpha < beta (YARN); D even, 2 <= D <= 256.
 * inv_freq_out_host: caller-owned host array of D/2 doubles (required).
 * mscale_out_host, band_out_host (D/2 entries): optional, may be NULL.
 */
int srt_rope_inv_freq(int method, double base, double s, double L, double alpha, double beta, int D,
                      double* inv_freq_out_host, double* mscale_out_host, signed char* band_out_host);

/*
 * srt_rope_inv_freq_dynamic_ntk - NTK-aware frequencies with the scale taken
 * from the actual sequence length (host only, fp64).
 *
 * Dynamic NTK adjusts the base from the length seen at inference ("AI Day 9:
 * 长上下文技术", Dynamic NTK).  Reading: s = max(1, seq_len / L), then
 * theta'_d = b'^(-2d/D) with b' = base * s^(D/(D-2)) as in srt_rope_inv_freq
 * (NTK); a sequence no longer than L keeps the original frequencies.
 * base > 0; seq_len >= 0; L > 0; D even, 4 <= D <= 256.  inv_freq_out_host:
 * D/2 doubles (required); s_out_host: optional.
 */
int srt_rope_inv_freq_dynamic_ntk(double base, long long seq_len, double L, int D, double* inv_freq_out_host,
                                  double* s_out_host);

/*
 * srt_rope_inv_freq_factors - per-pair factors: theta'_d = base^(-2d/D) / lambda_d
 * ([LC] §7.3, the LongRoPE search space; the search itself is out of scope).
 * lambda_host: D/2 positive finite doubles.  inv_freq_out_host: D/2 doubles.
 */
int srt_rope_inv_freq_factors(double base, const double* lambda_host, int D, double* inv_freq_out_host);

/*
 * srt_rope_cos_sin - cos/sin table for positions [0, npos) (GPU kernel).
 *
 * table_dev[(p*(D/2) + i)*2 + 0] = mscale*cos(p*theta'_i),
 * table_dev[(p*(D/2) + i)*2 + 1] = mscale*sin(p*theta'_i).
 * The angle p*theta'_i is formed and reduced in fp64, the result rounded to
 * fp32 once ([LC] §A.1: compute cos/sin in fp32 or better, then cast).
 * Folding mscale into the table is [LC] §6.4's attention-scale form of the
 * YaRN temperature.
 * inv_freq_host: host array of D/2 doubles (e.g. from srt_rope_inv_freq).
 * table_dev: device buffer of npos*D floats.  1 <= npos <= 2^31, D even <= 256.
 */
int srt_rope_cos_sin(const double* inv_freq_host, int D, double mscale, long long npos,
                     float* table_dev, void* stream);

/*
 * srt_rope_apply - rotate rows of a [B][H][N][D] tensor (GPU kernel).
 *
 * y_{2i} = x_{2i} c - x_{2i+1} s,  y_{2i+1} = x_{2i} s + x_{2i+1} c with (c, s)
 * the table entry of row r's position pos0 + r ([LC] §2.2, [NB] §4.2); the
 * table already carries mscale.  With pairing = SRT_PAIRING_HALF the pair is
 * (x_i, x_{i+D/2}) instead ([LC] §2.4).  Used to build a rotated KV cache and
 * to pre-rotate K.  x, y: device, contiguous, 16-byte aligned, dtype; y may
 * equal x (in place).  D a multiple of 8 (of 16 for half-split).
 * Requires 0 <= pos0 and pos0 + N <= table_npos.
 */
int srt_rope_apply(const void* x, void* y, int dtype, int B, int H, int N, int D, long long pos0,
                   const float* table_dev, long long table_npos, int pairing, void* stream);

/*
 * srt_attn_prefill - tiled online-softmax attention with rotate-on-load RoPE.
 *
 * For each batch b, query head h and query row r (absolute position
 * q_pos0 + r):  s_c = sm_scale * <q~_r, k~_c> over the keys c whose absolute
 * position k_pos0 + c <= q_pos0 + r (all keys if causal == 0);
 * O_r = softmax(s) V, lse_r = log sum exp(s) ([LC] §2.4).  q~ / k~ are the
 * rows rotated with the table (carrying the YaRN mscale) when rope_flags has
 * SRT_ROTATE_Q / SRT_ROTATE_K, else used as given; SRT_PAIR_HALF selects the
 * half-split pairing for both.  Scores are produced tile by
 * tile with the online softmax (running max and sum, rescaled accumulator:
 * [BK] §8.3.4 (1)-(2)); tiles wholly above the causal diagonal are skipped.
 *
 * Sliding window and sinks ([LC] §10.1-10.2): with window > 0 (causal only)
 * a key at absolute position j stays visible to the query at position i only
 * if i - j < window (the window counts the query's own position) or j < sink
 * (the first `sink` positions of the sequence are attention sinks).  Tiles
 * outside both are skipped, so the work is O(Nq * (window + sink)).
 * window = 0 means no window (sink is then irrelevant); both must be >= 0.
 *
 * q: [B][Hq][Nq][D] with head stride q_hstride; k, v: [B][Hkv][Nk][D] with head
 * stride kv_hstride; dtype for q, k, v.  out: [B][Hq][Nq][D] in out_dtype with
 * head stride o_hstride (SRT_F32 keeps a partial state exact for merging).
 * lse: [B][Hq][Nq] fp32 with head stride lse_hstride, or NULL.  All device
 * pointers (q, k, v, out, table_dev) must be 16-byte aligned and the head
 * strides q_hstride, kv_hstride, o_hstride multiples of 8 elements (rows are
 * moved in 16-byte vectors), else SRT_ERR_INVALID.  The table is
 * [table_npos][D/2][2] fp32 for this D; a narrower table is read past its end.
 * Kernels: dtype BF16 with D = 128 (matrix cores), dtype F32 with D in {64, 128}.
 * table_dev may be NULL only when rope_flags == 0.  Without SRT_ROTATE_Q the
 * bf16 kernel uses q exactly as given and scales the scores in fp32; with it,
 * the rotated q carries one bf16 rounding (the MFMA operand).
 *
 * sched: NULL, or a device block of SRT_PREFILL_SCHED_BYTES bytes, 8-byte
 * aligned (else SRT_ERR_INVALID), owned by the caller and zero-filled before
 * its first use.  With it the bf16 kernel hands its (head, query tile) work
 * items to workgroups at run time: each XCD first takes the heavy query tiles
 * of its own KV heads (its L2 keeps their K/V), then the light last quarter
 * of the tiles from a pool shared by all XCDs, so XCDs that run faster take
 * more of it.  The results are bit-identical either way; only the finishing
 * times of the XCDs change.  The launch's last workgroup zero-fills the block
 * again, so one block serves any number of calls issued one after another
 * (one stream); calls that may run at the same time each need their own
 * block.  Launches of at most two workgroups per compute unit, and the fp32
 * kernel, ignore it.  NULL keeps a fixed assignment.
 */
int srt_attn_prefill(const void* q, const void* k, const void* v, int dtype,
                     int B, int Hq, int Hkv, int Nq, int Nk, int D,
                     long long q_hstride, long long kv_hstride,
                     long long q_pos0, long long k_pos0, int causal, int window, int sink, float sm_scale,
                     const float* table_dev, long long table_npos, int rope_flags,
                     void* out, int out_dtype, long long o_hstride,
                     float* lse, long long lse_hstride, void* sched, void* stream);

/*
 * srt_attn_merge_states - combine two partial attention states over disjoint keys.
 *
 * lse = log(e^lse_a + e^lse_b);  O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b:
 * the rescaling step of the online softmax that each Ring Attention step
 * applies to a newly received K/V block ([BK] §8.3.5 step 3, §8.3.4 (2)).  A
 * state with lse = -inf is the identity; two of them give (0, -inf).
 * o_a, o_b: [B][H][N][D] in in_dtype (head stride in_hstride for both);
 * lse_a, lse_b: [B][H][N] fp32 (head stride N).  o_out: out_dtype with head
 * stride out_hstride; lse_out: fp32 with head stride lse_out_hstride (may be
 * NULL).  o_out may alias o_a (same dtype and stride), lse_out may alias lse_a.
 */
int srt_attn_merge_states(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                          int in_dtype, long long in_hstride,
                          void* o_out, int out_dtype, long long out_hstride,
                          float* lse_out, long long lse_out_hstride,
                          int B, int H, int N, int D, void* stream);

/*
 * srt_attn_decode_workspace_size - bytes of workspace srt_attn_decode_splitk needs.
 */
int srt_attn_decode_workspace_size(int B, int Hq, int D, int num_splits, size_t* bytes_out_host);

/*
 * srt_attn_decode_splitk - one new query per sequence against a rotated KV cache.
 *
 * Every decode step reads the whole K/V cache ([LC] §12.3; [PL] KV-cache
 * notes).  Query q[b][h] (raw, [B][Hq][D]) is rotated at position
 * seq_len_b - 1 with the table (skipped if table_dev is NULL), pairs chosen by
 * `pairing` (SRT_PAIRING_INTERLEAVED or SRT_PAIRING_HALF); the cache holds
 * keys already rotated at their positions (built with srt_rope_apply).  The
 * visible keys are cut into num_splits blocks: all of [0, seq_len_b) without
 * a window; with window > 0 only [max(0, seq_len_b - window), seq_len_b) plus
 * the sinks [0, min(sink, seq_len_b)) ([LC] §10.1-10.2, same rule as
 * srt_attn_prefill at query position seq_len_b - 1), so a windowed step reads
 * O(window + sink) cache rows.  Blocks hold ceil(span/num_splits) keys, span =
 * Nk without a window, min(Nk, window + sink) with one;
 * a first kernel computes each block's partial (O, lse) into the workspace,
 * a second merges the partials with the log-sum-exp rule ([BK] §8.3.6 query
 * phase: partial results combined by online softmax).
 * k_cache, v_cache: [B][Hkv][Nk][D] contiguous, dtype BF16, D = 128.
 * seq_lens_dev: device int32[B] with 0 <= seq_len <= Nk, or NULL (all Nk).
 * workspace: device, >= srt_attn_decode_workspace_size bytes, 16-byte aligned.
 * out: [B][Hq][D] in dtype; lse: [B][Hq] fp32 or NULL.
 * 1 <= num_splits <= 1024.
 */
int srt_attn_decode_splitk(const void* q, const void* k_cache, const void* v_cache, int dtype,
                           int B, int Hq, int Hkv, int Nk, int D, const int* seq_lens_dev,
                           int num_splits, float sm_scale, const float* table_dev, long long table_npos,
                           int pairing, int window, int sink, void* workspace, size_t workspace_bytes,
                           void* out, float* lse, void* stream);

/*
 * srt_attn_decode_splitk_noalloc - srt_attn_decode_splitk for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, meaning, layouts
 * and results as srt_attn_decode_splitk, without the workspace: the split
 * partials go to a static device array of the library (one per GPU, kept until
 * the process ends) of srt_attn_decode_noalloc_max_workspace() bytes
 * (32 MiB).  Calls whose partials need more,
 * B * Hq * num_splits * (D + 1) * 4 bytes, return SRT_ERR_WORKSPACE with no
 * side effects.  The call makes no allocation (no hipMalloc, hipFree or
 * allocating library routine).  All calls on one GPU share that GPU's array:
 * calls that overlap on one GPU (e.g. on two streams) race and must be
 * ordered by the caller.
 */
int srt_attn_decode_splitk_noalloc(const void* q, const void* k_cache, const void* v_cache, int dtype,
                                   int B, int Hq, int Hkv, int Nk, int D, const int* seq_lens_dev,
                                   int num_splits, float sm_scale, const float* table_dev, long long table_npos,
                                   int pairing, int window, int sink, void* out, float* lse, void* stream);

/* Bytes of the static scratch of srt_attn_decode_splitk_noalloc (its size limit). */
size_t srt_attn_decode_noalloc_max_workspace(void);

/*
 * srt_attn_backward_workspace_size - bytes of workspace srt_attn_backward
 * needs for these arguments: delta = rowsum(dO * O), fp32 [B][Hq][Nq], and
 * for BF16 room for a copy of q ([B][Hq][Nq][D]: with SRT_ROTATE_Q, or a zero
 * sm_scale, q rotated, multiplied by sm_scale log2(e) and rounded once exactly
 * as the forward kernel forms its q; otherwise q is used as given, as the
 * forward uses it, and the room stays unused), so the recomputed scores equal
 * the forward's, and a
 * rotated copy of k ([B][Hkv][Nk][D], with SRT_ROTATE_K) and two scheduling
 * blocks (the run-time work assignment of srt_attn_prefill, for the dk/dv and
 * the dq kernel, zero-filled by each call), each region 256-byte aligned.  The
 * copies are made once per call, so the kernels stage tiles that need no
 * rotation.  Returns SRT_ERR_INVALID for a bad dtype, negative sizes or
 * unknown flags.
 */
int srt_attn_backward_workspace_size(int dtype, int B, int Hq, int Hkv, int Nq, int Nk, int D, int rope_flags,
                                     size_t* bytes_out_host);

/*
 * srt_attn_backward - gradients of srt_attn_prefill with respect to q, k, v.
 *
 * For upstream dO and the forward's out and lse, with P = exp(S - lse) the
 * recomputed attention matrix ([BK] §8.3.4 (3): recompute from Q, K, V and
 * the saved softmax statistics instead of storing P):
 *   dv = P^T dO;  dS = P * (dO V^T - delta), delta = rowsum(dO * out);
 *   dq~ = sm_scale dS k~;  dk~ = sm_scale dS^T q~;
 * and, for inputs rotated on load (SRT_ROTATE_Q / SRT_ROTATE_K), the gradient
 * turned back by the transposed rotation, the rotation by the opposite angle
 * with the same table ([NB] §4: R^T = R(-a)), so dq, dk are gradients with
 * respect to the raw q, k.  Without the flag the input is taken as given and
 * so is its gradient.  GQA: dk, dv sum over the query heads of a group.
 * The arguments mean what they mean for srt_attn_prefill (same mask: causal,
 * window, sink; same table and flags); lse must be the forward's lse of
 * exactly these inputs.
 *
 * q, out, dout: [B][Hq][Nq][D]; k, v: [B][Hkv][Nk][D]; all contiguous, dtype
 * (BF16 with D = 128 on the matrix cores, F32 with D = 64).  lse: [B][Hq][Nq]
 * fp32.  dq: [B][Hq][Nq][D], dk, dv: [B][Hkv][Nk][D], fp32 device buffers,
 * overwritten.  workspace: >= srt_attn_backward_workspace_size bytes for the
 * same dtype, sizes and flags, 16-byte aligned (SRT_ERR_WORKSPACE if smaller).
 */
int srt_attn_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, int dtype, int B, int Hq, int Hkv, int Nq, int Nk, int D,
                      long long q_pos0, long long k_pos0, int causal, int window, int sink, float sm_scale,
                      const float* table_dev, long long table_npos, int rope_flags,
                      void* workspace, size_t workspace_bytes,
                      float* dq, float* dk, float* dv, void* stream);

/* partition argument of srt_attn_ring_prefill ([BK] §8.3.5, causal load balance) */
#define SRT_PART_CONTIGUOUS 0   /* shard r = positions [r C, (r+1) C), C = N / P              */
#define SRT_PART_STRIPED 1      /* shard r = positions r, r + P, r + 2P, ...                  */
#define SRT_PART_ZIGZAG 2       /* shard r = chunk r then chunk 2P-1-r of 2P chunks of N/(2P) */

/*
 * srt_attn_ring_workspace_size - bytes of workspace srt_attn_ring_prefill needs:
 * the fp32 running state of one query run (O [B][Hq][R][D] and lse
 * [B][Hq][R], R = N/P, or N/(2P) for zigzag), the scheduling block of its
 * prefill launches (zero-filled by each call) and, when rope_flags has
 * SRT_ROTATE_K, a rotated copy of K ([B][Hkv][N][D] in dtype).
 */
int srt_attn_ring_workspace_size(int B, int Hq, int Hkv, int N, int D, int dtype, int num_devices, int partition,
                                 int rope_flags, size_t* bytes_out_host);

/*
 * srt_attn_ring_prefill - causal Ring Attention over num_devices = P devices,
 * every device's work run on this GPU ([BK] §8.3.5).
 *
 * Device r holds query shard r and K/V shard r.  It attends its own K/V shard,
 * then at ring step s = 1 .. P-1 the shard of device (r - s) mod P, and folds
 * each partial state into its running one with the log-sum-exp rule (the
 * online-softmax rescaling; same rule as srt_attn_merge_states).  The result
 * equals srt_attn_prefill over the whole sequence (causal, same window and
 * sinks).  `partition` chooses the positions of a shard (SRT_PART_*: Striped
 * and Zig-Zag balance the causal work across devices); tensors are stored
 * shard-major: row r*(N/P) + t holds row t of shard r, at the position the
 * partition gives it.  device = -1 runs every device; 0 <= device < P runs
 * only that device's share (writes only its N/P rows of out and lse).
 *
 * q: [B][Hq][N][D], k, v: [B][Hkv][N][D], contiguous, dtype (BF16 with
 * D = 128, or F32 with D in {64, 128}); out: [B][Hq][N][D] in dtype; lse:
 * [B][Hq][N] fp32 or NULL.  rope_flags as srt_attn_prefill: with SRT_ROTATE_K
 * the keys are rotated once into the workspace at their positions, and
 * without it k must already be rotated.  N a multiple of P (of 2P for
 * zigzag); window and sink as srt_attn_prefill (window with STRIPED is
 * unsupported).  workspace: device, >= srt_attn_ring_workspace_size bytes,
 * 256-byte aligned.  Launches run in order on `stream`.
 */
int srt_attn_ring_prefill(const void* q, const void* k, const void* v, int dtype,
                          int B, int Hq, int Hkv, int N, int D,
                          int num_devices, int partition, int device,
                          int window, int sink, float sm_scale,
                          const float* table_dev, long long table_npos, int rope_flags,
                          void* workspace, size_t workspace_bytes,
                          void* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SRT_H */
