// C-ABI layer of libsrt: argument checks on the host, the fp64 frequency step,
// and dispatch to the kernel launchers.  No exception crosses the ABI.
#include "../../include/srt.h"
#include "srt_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return SRT_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SRT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool valid_dtype(int d) { return d == SRT_F32 || d == SRT_BF16; }

bool misaligned16(const void* p) { return ((uintptr_t)p & 15u) != 0; }

constexpr double kTwoPi = 6.283185307179586476925286766559;

}  // namespace

extern "C" {

int srt_abi_version(void) { return 2; }

const char* srt_status_string(int status) {
  switch (status) {
    case SRT_OK: return "ok";
    case SRT_ERR_INVALID: return "invalid argument";
    case SRT_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SRT_ERR_HIP: return "HIP runtime error";
    case SRT_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* srt_last_error(void) { return g_err; }

// Frequency step: "Long Context: RoPE / YaRN / NTK / MLA" §2.1 (base
// frequencies), §4.2 (PI), §5.2 (NTK-aware base), §6.2-6.4 (NTK-by-parts ramp
// and temperature); band labels from "8.3 长上下文技术" §8.3.3.
int srt_rope_inv_freq(int method, double base, double s, double L, double alpha, double beta, int D,
                      double* inv_freq_out, double* mscale_out, signed char* band_out) {
  if (!inv_freq_out) return fail(SRT_ERR_INVALID, "rope_inv_freq: inv_freq_out is NULL");
  if (D < 2 || D > 2 * srt::kMaxHalf || (D & 1))
    return fail(SRT_ERR_INVALID, "rope_inv_freq: D=%d must be even and in [2, %d]", D, 2 * srt::kMaxHalf);
  if (!(base > 0.0) || !std::isfinite(base)) return fail(SRT_ERR_INVALID, "rope_inv_freq: base must be > 0");
  if (method < SRT_ROPE_NONE || method > SRT_ROPE_YARN)
    return fail(SRT_ERR_INVALID, "rope_inv_freq: unknown method %d", method);
  if (method != SRT_ROPE_NONE && (!(s > 0.0) || !std::isfinite(s)))
    return fail(SRT_ERR_INVALID, "rope_inv_freq: scale s must be > 0");
  if (method == SRT_ROPE_NTK && D <= 2) return fail(SRT_ERR_INVALID, "rope_inv_freq: NTK needs D > 2");
  if (method == SRT_ROPE_YARN) {
    if (!(L > 0.0) || !std::isfinite(L)) return fail(SRT_ERR_INVALID, "rope_inv_freq: YaRN needs L > 0");
    if (!(beta > alpha)) return fail(SRT_ERR_INVALID, "rope_inv_freq: YaRN needs beta > alpha");
  }
  const int half = D / 2;
  double mscale = 1.0;
  // NTK-aware: new base b' = b * s^(D/(D-2)), exponent formed in fp64.
  const double b_eff = (method == SRT_ROPE_NTK) ? base * std::pow(s, (double)D / (double)(D - 2)) : base;
  for (int d = 0; d < half; ++d) {
    const double th = std::pow(b_eff, -2.0 * (double)d / (double)D);
    double out = th;
    signed char band = SRT_BAND_HIGH;
    switch (method) {
      case SRT_ROPE_NONE: break;
      case SRT_ROPE_PI: out = th / s; band = SRT_BAND_LOW; break;
      case SRT_ROPE_NTK: band = SRT_BAND_MID; break;
      case SRT_ROPE_YARN: {
        const double r = L * th / kTwoPi;                 // turns within the training length
        double w = (r - alpha) / (beta - alpha);          // ramp, clipped to [0, 1]
        w = w < 0.0 ? 0.0 : (w > 1.0 ? 1.0 : w);
        out = (1.0 - w) * (th / s) + w * th;
        band = r > beta ? SRT_BAND_HIGH : (r < alpha ? SRT_BAND_LOW : SRT_BAND_MID);
        break;
      }
    }
    inv_freq_out[d] = out;
    if (band_out) band_out[d] = band;
  }
  if (method == SRT_ROPE_YARN && s > 1.0) mscale = 0.1 * std::log(s) + 1.0;
  if (mscale_out) *mscale_out = mscale;
  return ok();
}

int srt_rope_inv_freq_dynamic_ntk(double base, long long seq_len, double L, int D, double* inv_freq_out,
                                  double* s_out) {
  if (!inv_freq_out) return fail(SRT_ERR_INVALID, "rope_inv_freq_dynamic_ntk: inv_freq_out is NULL");
  if (seq_len < 0) return fail(SRT_ERR_INVALID, "rope_inv_freq_dynamic_ntk: seq_len < 0");
  if (!(L > 0.0) || !std::isfinite(L)) return fail(SRT_ERR_INVALID, "rope_inv_freq_dynamic_ntk: L must be > 0");
  if (D < 4) return fail(SRT_ERR_INVALID, "rope_inv_freq_dynamic_ntk: D must be >= 4");
  // Dynamic NTK: the scale follows the length actually seen, never below 1.
  const double s = (double)seq_len > L ? (double)seq_len / L : 1.0;
  if (s_out) *s_out = s;
  return srt_rope_inv_freq(SRT_ROPE_NTK, base, s, 0.0, 1.0, 2.0, D, inv_freq_out, nullptr, nullptr);
}

int srt_rope_inv_freq_factors(double base, const double* lambda, int D, double* inv_freq_out) {
  if (!lambda || !inv_freq_out) return fail(SRT_ERR_INVALID, "rope_inv_freq_factors: NULL pointer");
  if (D < 2 || D > 2 * srt::kMaxHalf || (D & 1))
    return fail(SRT_ERR_INVALID, "rope_inv_freq_factors: D=%d must be even and in [2, %d]", D, 2 * srt::kMaxHalf);
  if (!(base > 0.0) || !std::isfinite(base)) return fail(SRT_ERR_INVALID, "rope_inv_freq_factors: base must be > 0");
  for (int d = 0; d < D / 2; ++d)
    if (!(lambda[d] > 0.0) || !std::isfinite(lambda[d]))
      return fail(SRT_ERR_INVALID, "rope_inv_freq_factors: lambda[%d] must be positive and finite", d);
  for (int d = 0; d < D / 2; ++d) inv_freq_out[d] = std::pow(base, -2.0 * (double)d / (double)D) / lambda[d];
  return ok();
}

int srt_rope_cos_sin(const double* inv_freq_host, int D, double mscale, long long npos, float* table_dev,
                     void* stream) {
  if (!inv_freq_host || !table_dev) return fail(SRT_ERR_INVALID, "rope_cos_sin: NULL pointer");
  if (D < 2 || D > 2 * srt::kMaxHalf || (D & 1)) return fail(SRT_ERR_INVALID, "rope_cos_sin: bad D=%d", D);
  if (npos < 1 || npos > (1LL << 31)) return fail(SRT_ERR_INVALID, "rope_cos_sin: npos=%lld out of range", npos);
  if (!std::isfinite(mscale)) return fail(SRT_ERR_INVALID, "rope_cos_sin: mscale not finite");
  srt::Theta th{};
  for (int i = 0; i < D / 2; ++i) {
    if (!std::isfinite(inv_freq_host[i])) return fail(SRT_ERR_INVALID, "rope_cos_sin: theta[%d] not finite", i);
    th.v[i] = inv_freq_host[i];
  }
  return hip_status(srt::launch_rope_table(th, D / 2, mscale, npos, table_dev, (hipStream_t)stream),
                    "rope_cos_sin launch");
}

int srt_rope_apply(const void* x, void* y, int dtype, int B, int H, int N, int D, long long pos0,
                   const float* table_dev, long long table_npos, int pairing, void* stream) {
  if (!valid_dtype(dtype)) return fail(SRT_ERR_INVALID, "rope_apply: bad dtype %d", dtype);
  if (B < 0 || H < 0 || N < 0) return fail(SRT_ERR_INVALID, "rope_apply: negative size");
  if ((long long)B * H * N == 0) return ok();   // nothing to rotate: pointers may be NULL
  if (!x || !y || !table_dev) return fail(SRT_ERR_INVALID, "rope_apply: NULL pointer");
  if (D < 2 || (D & 1) || D > 2 * srt::kMaxHalf) return fail(SRT_ERR_INVALID, "rope_apply: bad D=%d", D);
  if (pairing != SRT_PAIRING_INTERLEAVED && pairing != SRT_PAIRING_HALF)
    return fail(SRT_ERR_INVALID, "rope_apply: bad pairing %d", pairing);
  if (D % 8) return fail(SRT_ERR_UNSUPPORTED, "rope_apply: D=%d must be a multiple of 8", D);
  if (pairing == SRT_PAIRING_HALF && D % 16)
    return fail(SRT_ERR_UNSUPPORTED, "rope_apply: half-split pairing needs D a multiple of 16 (D=%d)", D);
  if (pos0 < 0 || pos0 + N > table_npos)
    return fail(SRT_ERR_INVALID, "rope_apply: positions [%lld, %lld) outside table [0, %lld)", pos0,
                pos0 + N, table_npos);
  if (misaligned16(x) || misaligned16(y) || misaligned16(table_dev))
    return fail(SRT_ERR_INVALID, "rope_apply: pointers must be 16-byte aligned");
  const srt::PosMap map{pos0, srt::kContiguous, 1, N};
  return hip_status(srt::launch_rope_apply(x, y, dtype == SRT_BF16, pairing == SRT_PAIRING_HALF, (long long)B * H,
                                           N, D, map, table_dev, (hipStream_t)stream),
                    "rope_apply launch");
}

int srt_attn_prefill(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv, int Nq,
                     int Nk, int D, long long q_hstride, long long kv_hstride, long long q_pos0,
                     long long k_pos0, int causal, int window, int sink, float sm_scale, const float* table_dev,
                     long long table_npos, int rope_flags, void* out, int out_dtype, long long o_hstride,
                     float* lse, long long lse_hstride, void* sched, void* stream) {
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return fail(SRT_ERR_INVALID, "attn_prefill: bad dtype");
  if (B < 0 || Hq < 1 || Hkv < 1 || Nq < 0 || Nk < 0) return fail(SRT_ERR_INVALID, "attn_prefill: bad sizes");
  if ((long long)B * Nq == 0) return ok();     // no query row: nothing to write, pointers may be NULL
  if (!q || !out) return fail(SRT_ERR_INVALID, "attn_prefill: NULL q or out");
  if (Nk > 0 && (!k || !v)) return fail(SRT_ERR_INVALID, "attn_prefill: NULL k or v");
  if (Hq % Hkv) return fail(SRT_ERR_INVALID, "attn_prefill: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (D < 2 || (D & 1)) return fail(SRT_ERR_INVALID, "attn_prefill: D=%d must be even", D);
  if (q_hstride < (long long)Nq * D || kv_hstride < (long long)Nk * D || o_hstride < (long long)Nq * D)
    return fail(SRT_ERR_INVALID, "attn_prefill: head stride smaller than N*D");
  if (lse && lse_hstride < Nq) return fail(SRT_ERR_INVALID, "attn_prefill: lse head stride smaller than Nq");
  if (rope_flags & ~(SRT_ROTATE_Q | SRT_ROTATE_K | SRT_PAIR_HALF))
    return fail(SRT_ERR_INVALID, "attn_prefill: bad rope_flags");
  if ((rope_flags & (SRT_ROTATE_Q | SRT_ROTATE_K)) && !table_dev)
    return fail(SRT_ERR_INVALID, "attn_prefill: rope_flags set without a table");
  if (q_pos0 < 0 || k_pos0 < 0) return fail(SRT_ERR_INVALID, "attn_prefill: negative position offset");
  if ((rope_flags & SRT_ROTATE_Q) && q_pos0 + Nq > table_npos)
    return fail(SRT_ERR_INVALID, "attn_prefill: q positions [%lld, %lld) outside table [0, %lld)", q_pos0,
                q_pos0 + Nq, table_npos);
  if ((rope_flags & SRT_ROTATE_K) && k_pos0 + Nk > table_npos)
    return fail(SRT_ERR_INVALID, "attn_prefill: k positions [%lld, %lld) outside table [0, %lld)", k_pos0,
                k_pos0 + Nk, table_npos);
  if (!std::isfinite(sm_scale)) return fail(SRT_ERR_INVALID, "attn_prefill: sm_scale not finite");
  if (window < 0 || sink < 0) return fail(SRT_ERR_INVALID, "attn_prefill: window and sink must be >= 0");
  if (window > 0 && !causal) return fail(SRT_ERR_INVALID, "attn_prefill: a sliding window needs causal = 1");
  if (Nq > (1 << 30) || Nk > (1 << 30)) return fail(SRT_ERR_UNSUPPORTED, "attn_prefill: N above 2^30");
  // the kernels move rows in 16-byte vectors (q, k, v rows and table entries
  // in, 8- or 16-byte groups of out rows out): every row must start on a
  // 16-byte boundary, so the base pointers are 16-byte aligned and the head
  // strides whole multiples of 8 elements
  if (misaligned16(q) || misaligned16(out) || (Nk > 0 && (misaligned16(k) || misaligned16(v))) ||
      misaligned16(table_dev))
    return fail(SRT_ERR_INVALID, "attn_prefill: q, k, v, out and the table must be 16-byte aligned");
  if ((q_hstride % 8) || (kv_hstride % 8) || (o_hstride % 8))
    return fail(SRT_ERR_INVALID, "attn_prefill: head strides must be multiples of 8 elements");
  srt::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.table = table_dev;
  a.q_hstride = q_hstride; a.kv_hstride = kv_hstride; a.o_hstride = o_hstride; a.lse_hstride = lse_hstride;
  a.q_pos0 = q_pos0; a.k_pos0 = k_pos0;
  a.q_rope0 = q_pos0; a.k_rope0 = k_pos0; a.rope_step = 1;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.D = D;
  a.causal = causal ? 1 : 0; a.rope_flags = rope_flags; a.out_bf16 = out_dtype == SRT_BF16;
  a.window = window; a.sink = window > 0 ? sink : 0;
  a.sm_scale = sm_scale;
  if (sched && (reinterpret_cast<uintptr_t>(sched) & 7))
    return fail(SRT_ERR_INVALID, "attn_prefill: sched must be 8-byte aligned");
  a.sched = static_cast<unsigned long long*>(sched);
  if (dtype == SRT_BF16) {
    if (D != 128) return fail(SRT_ERR_UNSUPPORTED, "attn_prefill: bf16 kernel needs D = 128 (got %d)", D);
    const int g = Hq / Hkv;
    if (!(g == 1 || g == 2 || g % 4 == 0))
      return fail(SRT_ERR_UNSUPPORTED, "attn_prefill: bf16 kernel needs Hq/Hkv in {1, 2} or a multiple of 4");
    return hip_status(srt::launch_prefill_bf16_d128(a, (hipStream_t)stream), "attn_prefill bf16 launch");
  }
  if (D != 64 && D != 128) return fail(SRT_ERR_UNSUPPORTED, "attn_prefill: fp32 kernel needs D in {64,128}");
  return hip_status(srt::launch_prefill_f32(a, (hipStream_t)stream), "attn_prefill fp32 launch");
}

int srt_attn_merge_states(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                          int in_dtype, long long in_hstride, void* o_out, int out_dtype, long long out_hstride,
                          float* lse_out, long long lse_out_hstride, int B, int H, int N, int D, void* stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(SRT_ERR_INVALID, "attn_merge_states: bad dtype");
  if (B < 0 || H < 0 || N < 0) return fail(SRT_ERR_INVALID, "attn_merge_states: negative size");
  if ((long long)B * H * N == 0) return ok();  // nothing to merge: pointers may be NULL
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out) return fail(SRT_ERR_INVALID, "attn_merge_states: NULL pointer");
  if (D < 8 || D > 512 || (D & (D - 1)))
    return fail(SRT_ERR_UNSUPPORTED, "attn_merge_states: D=%d must be a power of two in [8, 512]", D);
  if (in_hstride < (long long)N * D || out_hstride < (long long)N * D)
    return fail(SRT_ERR_INVALID, "attn_merge_states: head stride smaller than N*D");
  if (lse_out && lse_out_hstride < N) return fail(SRT_ERR_INVALID, "attn_merge_states: lse_out stride < N");
  if (o_out == o_a && (out_dtype != in_dtype || out_hstride != in_hstride))
    return fail(SRT_ERR_INVALID, "attn_merge_states: in-place merge needs equal dtype and stride");
  if (misaligned16(o_a) || misaligned16(o_b) || misaligned16(o_out))
    return fail(SRT_ERR_INVALID, "attn_merge_states: tensors must be 16-byte aligned");
  if ((in_hstride % 8) || (out_hstride % 8))
    return fail(SRT_ERR_INVALID, "attn_merge_states: head strides must be multiples of 8 elements");
  srt::MergeArgs a{};
  a.oa = o_a; a.la = lse_a; a.ob = o_b; a.lb = lse_b; a.oo = o_out; a.lo = lse_out;
  a.in_hstride = in_hstride; a.out_hstride = out_hstride; a.lse_out_hstride = lse_out_hstride;
  a.BH = B * H; a.N = N; a.D = D; a.in_bf16 = in_dtype == SRT_BF16; a.out_bf16 = out_dtype == SRT_BF16;
  return hip_status(srt::launch_merge(a, (hipStream_t)stream), "attn_merge_states launch");
}

int srt_attn_decode_workspace_size(int B, int Hq, int D, int num_splits, size_t* bytes_out) {
  if (!bytes_out) return fail(SRT_ERR_INVALID, "attn_decode_workspace_size: NULL output");
  if (B < 0 || Hq < 1 || D < 2 || num_splits < 1 || num_splits > 1024)
    return fail(SRT_ERR_INVALID, "attn_decode_workspace_size: bad sizes");
  *bytes_out = srt::decode_workspace_bytes(B, Hq, D, num_splits);
  return ok();
}

}  // extern "C"

namespace {

// Checks shared by the two decode entry points; fills everything of `a` but
// the workspace pointers.
int decode_args(const void* q, const void* k_cache, const void* v_cache, int dtype, int B, int Hq, int Hkv, int Nk,
                int D, const int* seq_lens_dev, int num_splits, float sm_scale, const float* table_dev,
                long long table_npos, int pairing, int window, int sink, void* out, float* lse, srt::DecodeArgs& a) {
  if (!valid_dtype(dtype)) return fail(SRT_ERR_INVALID, "attn_decode_splitk: bad dtype");
  if (B < 0 || Hq < 1 || Hkv < 1 || Nk < 0) return fail(SRT_ERR_INVALID, "attn_decode_splitk: bad sizes");
  if (B == 0) return SRT_OK;                   // no sequence: pointers may be NULL
  if (!q || !out) return fail(SRT_ERR_INVALID, "attn_decode_splitk: NULL q or out");
  if (Nk > 0 && (!k_cache || !v_cache)) return fail(SRT_ERR_INVALID, "attn_decode_splitk: NULL cache pointer");
  if (Hq % Hkv) return fail(SRT_ERR_INVALID, "attn_decode_splitk: Hq not a multiple of Hkv");
  if (num_splits < 1 || num_splits > 1024) return fail(SRT_ERR_INVALID, "attn_decode_splitk: num_splits out of [1,1024]");
  if (D < 2 || (D & 1)) return fail(SRT_ERR_INVALID, "attn_decode_splitk: D must be even");
  if (pairing != SRT_PAIRING_INTERLEAVED && pairing != SRT_PAIRING_HALF)
    return fail(SRT_ERR_INVALID, "attn_decode_splitk: bad pairing %d", pairing);
  if (table_dev && table_npos < Nk)
    return fail(SRT_ERR_INVALID, "attn_decode_splitk: table has %lld positions, query may sit at %d", table_npos, Nk - 1);
  if (!std::isfinite(sm_scale)) return fail(SRT_ERR_INVALID, "attn_decode_splitk: sm_scale not finite");
  if (window < 0 || sink < 0) return fail(SRT_ERR_INVALID, "attn_decode_splitk: window and sink must be >= 0");
  if (dtype != SRT_BF16 || D != 128)
    return fail(SRT_ERR_UNSUPPORTED, "attn_decode_splitk: kernel needs bf16 and D = 128");
  {
    const int g = Hq / Hkv;
    if (g != 1 && g != 2 && g != 4 && g != 8)
      return fail(SRT_ERR_UNSUPPORTED, "attn_decode_splitk: Hq/Hkv=%d must be 1, 2, 4 or 8", g);
  }
  if (misaligned16(q) || misaligned16(k_cache) || misaligned16(v_cache) || misaligned16(table_dev))
    return fail(SRT_ERR_INVALID, "attn_decode_splitk: tensors must be 16-byte aligned");
  a = srt::DecodeArgs{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.seq_lens = seq_lens_dev; a.table = table_dev;
  a.half_pairs = pairing == SRT_PAIRING_HALF;
  a.out = out; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nk = Nk; a.D = D; a.splits = num_splits;
  a.window = window; a.sink = window > 0 ? sink : 0;
  {
    // keys a sequence can see: the whole cache, or its window plus the sinks
    const long long span = window > 0 ? std::min<long long>(Nk, (long long)window + a.sink) : Nk;
    a.split_len = (int)((span + num_splits - 1) / num_splits);
  }
  a.sm_scale = sm_scale;
  return SRT_OK;
}

}  // namespace

extern "C" {

int srt_attn_decode_splitk(const void* q, const void* k_cache, const void* v_cache, int dtype, int B, int Hq,
                           int Hkv, int Nk, int D, const int* seq_lens_dev, int num_splits, float sm_scale,
                           const float* table_dev, long long table_npos, int pairing, int window, int sink,
                           void* workspace,
                           size_t workspace_bytes, void* out, float* lse, void* stream) {
  srt::DecodeArgs a;
  const int st = decode_args(q, k_cache, v_cache, dtype, B, Hq, Hkv, Nk, D, seq_lens_dev, num_splits, sm_scale,
                             table_dev, table_npos, pairing, window, sink, out, lse, a);
  if (st != SRT_OK) return st;
  if (B == 0) return ok();
  const size_t need = srt::decode_workspace_bytes(B, Hq, D, num_splits);
  if (!workspace || workspace_bytes < need)
    return fail(SRT_ERR_WORKSPACE, "attn_decode_splitk: workspace %zu bytes, need %zu", workspace_bytes, need);
  if (((uintptr_t)workspace) & 15) return fail(SRT_ERR_INVALID, "attn_decode_splitk: workspace not 16-byte aligned");
  a.ws_o = (float*)workspace;
  a.ws_lse = (float*)((char*)workspace + (size_t)B * Hq * num_splits * D * sizeof(float));
  return hip_status(srt::launch_decode(a, (hipStream_t)stream), "attn_decode_splitk launch");
}

size_t srt_attn_decode_noalloc_max_workspace(void) { return srt::kDecodeScratchBytes; }

int srt_attn_decode_splitk_noalloc(const void* q, const void* k_cache, const void* v_cache, int dtype, int B, int Hq,
                                   int Hkv, int Nk, int D, const int* seq_lens_dev, int num_splits, float sm_scale,
                                   const float* table_dev, long long table_npos, int pairing, int window, int sink,
                                   void* out, float* lse, void* stream) {
  srt::DecodeArgs a;
  const int st = decode_args(q, k_cache, v_cache, dtype, B, Hq, Hkv, Nk, D, seq_lens_dev, num_splits, sm_scale,
                             table_dev, table_npos, pairing, window, sink, out, lse, a);
  if (st != SRT_OK) return st;
  if (B == 0) return ok();
  const size_t need = srt::decode_workspace_bytes(B, Hq, D, num_splits);
  if (need > srt::kDecodeScratchBytes)
    return fail(SRT_ERR_WORKSPACE,
                "attn_decode_splitk_noalloc: the split partials need %zu bytes, above the %zu-byte static scratch "
                "(B * Hq * num_splits * (D + 1) * 4 bytes); use fewer splits or srt_attn_decode_splitk", need,
                srt::kDecodeScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = srt::decode_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "attn_decode_splitk_noalloc: scratch address");
  a.ws_o = (float*)scratch;
  a.ws_lse = (float*)((char*)scratch + (size_t)B * Hq * num_splits * D * sizeof(float));
  return hip_status(srt::launch_decode(a, (hipStream_t)stream), "attn_decode_splitk_noalloc launch");
}

namespace {
// Backward workspace: delta, then (bf16 only) the scaled, rotated q copy, the rotated k copy and the two
// scheduling blocks of the dk/dv and dq kernels, each 256-byte aligned.
struct BwdWorkspace {
  size_t delta, q_rot, k_rot, sched, total;   // offsets of the regions (0 when absent) and the size
};
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
BwdWorkspace bwd_workspace(int dtype, int B, int Hq, int Hkv, int Nq, int Nk, int D, int rope_flags) {
  BwdWorkspace w{0, 0, 0, 0, 0};
  size_t off = round256((size_t)B * Hq * Nq * sizeof(float));
  if (dtype == SRT_BF16 && (size_t)B * Nq > 0) {
    w.q_rot = off;
    off += round256((size_t)B * Hq * Nq * D * 2);
  }
  if (dtype == SRT_BF16 && (rope_flags & SRT_ROTATE_K) && (size_t)B * Nk > 0) {
    w.k_rot = off;
    off += round256((size_t)B * Hkv * Nk * D * 2);
  }
  if (dtype == SRT_BF16 && (size_t)B * Nq > 0) {
    w.sched = off;
    off += round256(2 * srt::kSchedBlockWords * sizeof(unsigned long long));
  }
  w.total = off;
  return w;
}
}  // namespace

int srt_attn_backward_workspace_size(int dtype, int B, int Hq, int Hkv, int Nq, int Nk, int D, int rope_flags,
                                     size_t* bytes_out) {
  if (!bytes_out) return fail(SRT_ERR_INVALID, "attn_backward_workspace_size: NULL output");
  if (!valid_dtype(dtype)) return fail(SRT_ERR_INVALID, "attn_backward_workspace_size: bad dtype");
  if (B < 0 || Hq < 1 || Hkv < 1 || Nq < 0 || Nk < 0 || D < 2)
    return fail(SRT_ERR_INVALID, "attn_backward_workspace_size: bad sizes");
  if (rope_flags & ~(SRT_ROTATE_Q | SRT_ROTATE_K | SRT_PAIR_HALF))
    return fail(SRT_ERR_INVALID, "attn_backward_workspace_size: bad rope_flags");
  *bytes_out = bwd_workspace(dtype, B, Hq, Hkv, Nq, Nk, D, rope_flags).total;
  return ok();
}

int srt_attn_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, int dtype, int B, int Hq, int Hkv, int Nq, int Nk, int D, long long q_pos0,
                      long long k_pos0, int causal, int window, int sink, float sm_scale, const float* table_dev,
                      long long table_npos, int rope_flags, void* workspace, size_t workspace_bytes, float* dq,
                      float* dk, float* dv, void* stream) {
  if (!valid_dtype(dtype)) return fail(SRT_ERR_INVALID, "attn_backward: bad dtype");
  if (B < 0 || Hq < 1 || Hkv < 1 || Nq < 0 || Nk < 0) return fail(SRT_ERR_INVALID, "attn_backward: bad sizes");
  if (Hq % Hkv) return fail(SRT_ERR_INVALID, "attn_backward: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (rope_flags & ~(SRT_ROTATE_Q | SRT_ROTATE_K | SRT_PAIR_HALF))
    return fail(SRT_ERR_INVALID, "attn_backward: bad rope_flags");
  if (window < 0 || sink < 0) return fail(SRT_ERR_INVALID, "attn_backward: window and sink must be >= 0");
  if (window > 0 && !causal) return fail(SRT_ERR_INVALID, "attn_backward: a sliding window needs causal = 1");
  if (q_pos0 < 0 || k_pos0 < 0) return fail(SRT_ERR_INVALID, "attn_backward: negative position offset");
  if (!std::isfinite(sm_scale)) return fail(SRT_ERR_INVALID, "attn_backward: sm_scale not finite");
  if (dtype == SRT_BF16) {
    if (D != 128) return fail(SRT_ERR_UNSUPPORTED, "attn_backward: bf16 kernels need D = 128 (got %d)", D);
    const int g = Hq / Hkv;
    if (!(g == 1 || g == 2 || g % 4 == 0))
      return fail(SRT_ERR_UNSUPPORTED, "attn_backward: bf16 kernels need Hq/Hkv in {1, 2} or a multiple of 4");
  } else if (D != 64) {
    return fail(SRT_ERR_UNSUPPORTED, "attn_backward: fp32 kernels need D = 64 (got %d)", D);
  }
  if ((long long)B * (Nq + (long long)Nk) == 0) return ok();   // nothing to compute: pointers may be NULL
  if (Nq > (1 << 30) || Nk > (1 << 30)) return fail(SRT_ERR_UNSUPPORTED, "attn_backward: N above 2^30");
  if ((rope_flags & SRT_ROTATE_Q) && (!table_dev || q_pos0 + Nq > table_npos))
    return fail(SRT_ERR_INVALID, "attn_backward: q positions [%lld, %lld) outside table [0, %lld)", q_pos0,
                q_pos0 + Nq, table_npos);
  if ((rope_flags & SRT_ROTATE_K) && (!table_dev || k_pos0 + Nk > table_npos))
    return fail(SRT_ERR_INVALID, "attn_backward: k positions [%lld, %lld) outside table [0, %lld)", k_pos0,
                k_pos0 + Nk, table_npos);
  if ((Nq > 0 && (!q || !out || !dout || !lse || !dq)) || (Nk > 0 && (!k || !v || !dk || !dv)))
    return fail(SRT_ERR_INVALID, "attn_backward: NULL pointer");
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(out) || misaligned16(dout) ||
      misaligned16(dq) || misaligned16(dk) || misaligned16(dv) || misaligned16(lse) || misaligned16(table_dev))
    return fail(SRT_ERR_INVALID, "attn_backward: tensors must be 16-byte aligned");
  const BwdWorkspace ws = bwd_workspace(dtype, B, Hq, Hkv, Nq, Nk, D, rope_flags);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total))
    return fail(SRT_ERR_WORKSPACE, "attn_backward: workspace %zu bytes, need %zu", workspace_bytes, ws.total);
  if (misaligned16(workspace)) return fail(SRT_ERR_INVALID, "attn_backward: workspace not 16-byte aligned");
  srt::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse; a.delta = (float*)workspace;
  // rotate q and k once into the workspace ([LC] §2.4: each row by its own position)
  const bool half_pairs = (rope_flags & SRT_PAIR_HALF) != 0;
  if (ws.q_rot && !(rope_flags & SRT_ROTATE_Q) && sm_scale != 0.f) {
    // q not rotated: the kernels use it exactly as the forward kernel does (unscaled; the scores are scaled
    // in fp32), so no copy is made
    a.q_rot = q;
  } else if (ws.q_rot) {
    // q~ = bf16(rotated q * sm_scale log2(e)), rounded once exactly as the forward kernel forms it, so the
    // backward's scores (and P = exp2(S - lse)) are those the forward normalised
    void* qr = (char*)workspace + ws.q_rot;
    const srt::PosMap map{q_pos0, srt::kContiguous, 1, Nq};
    const bool rot_q = (rope_flags & SRT_ROTATE_Q) != 0;
    const hipError_t e = srt::launch_rope_apply(q, qr, true, half_pairs && rot_q, (long long)B * Hq, Nq, D, map,
                                                rot_q ? table_dev : nullptr, (hipStream_t)stream,
                                                sm_scale * 1.44269504f);   // fp32 product, as the kernel forms it
    if (e != hipSuccess) return hip_status(e, "attn_backward: rotating q");
    a.q_rot = qr;
  }
  if (ws.k_rot) {
    void* kr = (char*)workspace + ws.k_rot;
    const srt::PosMap map{k_pos0, srt::kContiguous, 1, Nk};
    const hipError_t e = srt::launch_rope_apply(k, kr, true, half_pairs, (long long)B * Hkv, Nk, D, map, table_dev,
                                                (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "attn_backward: rotating k");
    a.k_rot = kr;
  }
  if (ws.sched) a.sched = reinterpret_cast<unsigned long long*>((char*)workspace + ws.sched);
  a.table = table_dev; a.dq = dq; a.dk = dk; a.dv = dv;
  a.q_pos0 = q_pos0; a.k_pos0 = k_pos0;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.D = D;
  a.causal = causal ? 1 : 0; a.window = window; a.sink = window > 0 ? sink : 0;
  a.rope_flags = rope_flags; a.bf16 = dtype == SRT_BF16; a.sm_scale = sm_scale;
  return hip_status(srt::launch_backward(a, (hipStream_t)stream), "attn_backward launch");
}

namespace {

// Shared checks of the ring entry points; fills `a` on success.
int ring_args(int dtype, int B, int Hq, int Hkv, int N, int D, int P, int partition, int rope_flags,
              srt::RingArgs& a) {
  if (!valid_dtype(dtype)) return fail(SRT_ERR_INVALID, "attn_ring: bad dtype");
  if (B < 0 || Hq < 1 || Hkv < 1 || N < 0) return fail(SRT_ERR_INVALID, "attn_ring: bad sizes");
  if (Hq % Hkv) return fail(SRT_ERR_INVALID, "attn_ring: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (P < 1 || P > 4096) return fail(SRT_ERR_INVALID, "attn_ring: num_devices=%d out of [1, 4096]", P);
  if (partition != SRT_PART_CONTIGUOUS && partition != SRT_PART_STRIPED && partition != SRT_PART_ZIGZAG)
    return fail(SRT_ERR_INVALID, "attn_ring: bad partition %d", partition);
  const int parts = partition == SRT_PART_ZIGZAG ? 2 * P : P;
  if (N % parts) return fail(SRT_ERR_INVALID, "attn_ring: N=%d must be a multiple of %d", N, parts);
  if (rope_flags & ~(SRT_ROTATE_Q | SRT_ROTATE_K | SRT_PAIR_HALF))
    return fail(SRT_ERR_INVALID, "attn_ring: bad rope_flags");
  if (dtype == SRT_BF16) {
    if (D != 128) return fail(SRT_ERR_UNSUPPORTED, "attn_ring: bf16 kernel needs D = 128 (got %d)", D);
    const int g = Hq / Hkv;
    if (!(g == 1 || g == 2 || g % 4 == 0))
      return fail(SRT_ERR_UNSUPPORTED, "attn_ring: bf16 kernel needs Hq/Hkv in {1, 2} or a multiple of 4");
  } else if (D != 64 && D != 128) {
    return fail(SRT_ERR_UNSUPPORTED, "attn_ring: fp32 kernel needs D in {64, 128}");
  }
  a = srt::RingArgs{};
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.D = D; a.P = P;
  a.mode = partition == SRT_PART_STRIPED ? srt::kStriped : (partition == SRT_PART_ZIGZAG ? srt::kZigzag : srt::kContiguous);
  a.rope_flags = rope_flags; a.bf16 = dtype == SRT_BF16;
  return SRT_OK;
}

}  // namespace

int srt_attn_ring_workspace_size(int B, int Hq, int Hkv, int N, int D, int dtype, int num_devices, int partition,
                                 int rope_flags, size_t* bytes_out) {
  if (!bytes_out) return fail(SRT_ERR_INVALID, "attn_ring_workspace_size: NULL output");
  srt::RingArgs a;
  const int st = ring_args(dtype, B, Hq, Hkv, N, D, num_devices, partition, rope_flags, a);
  if (st != SRT_OK) return st;
  *bytes_out = srt::ring_workspace_bytes(a);
  return ok();
}

int srt_attn_ring_prefill(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv, int N,
                          int D, int num_devices, int partition, int device, int window, int sink, float sm_scale,
                          const float* table_dev, long long table_npos, int rope_flags, void* workspace,
                          size_t workspace_bytes, void* out, float* lse, void* stream) {
  srt::RingArgs a;
  const int st = ring_args(dtype, B, Hq, Hkv, N, D, num_devices, partition, rope_flags, a);
  if (st != SRT_OK) return st;
  if (device < -1 || device >= num_devices) return fail(SRT_ERR_INVALID, "attn_ring: device=%d out of range", device);
  if (window < 0 || sink < 0) return fail(SRT_ERR_INVALID, "attn_ring: window and sink must be >= 0");
  if (window > 0 && partition == SRT_PART_STRIPED)
    return fail(SRT_ERR_UNSUPPORTED, "attn_ring: a sliding window with the striped partition is not supported");
  if (!std::isfinite(sm_scale)) return fail(SRT_ERR_INVALID, "attn_ring: sm_scale not finite");
  if ((long long)B * N == 0) return ok();      // nothing to compute: pointers may be NULL
  if (!q || !k || !v || !out) return fail(SRT_ERR_INVALID, "attn_ring: NULL q, k, v or out");
  if ((rope_flags & (SRT_ROTATE_Q | SRT_ROTATE_K)) && (!table_dev || table_npos < N))
    return fail(SRT_ERR_INVALID, "attn_ring: rotation needs a table covering positions [0, %d)", N);
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(out) || misaligned16(table_dev))
    return fail(SRT_ERR_INVALID, "attn_ring: tensors must be 16-byte aligned");
  const size_t need = srt::ring_workspace_bytes(a);
  if (!workspace || workspace_bytes < need)
    return fail(SRT_ERR_WORKSPACE, "attn_ring: workspace %zu bytes, need %zu", workspace_bytes, need);
  if (((uintptr_t)workspace) & 255) return fail(SRT_ERR_INVALID, "attn_ring: workspace not 256-byte aligned");
  a.q = q; a.k = k; a.v = v; a.table = table_dev; a.workspace = workspace; a.out = out; a.lse = lse;
  a.device = device; a.window = window; a.sink = window > 0 ? sink : 0; a.sm_scale = sm_scale;
  return hip_status(srt::ring_prefill(a, (hipStream_t)stream), "attn_ring_prefill launch");
}

}  // extern "C"
