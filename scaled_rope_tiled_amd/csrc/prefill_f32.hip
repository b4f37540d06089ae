// fp32 tiled online-softmax attention with rotate-on-load RoPE (D = 64 or 128).
//
// The fp32 path keeps every product in fp32 (no bf16 rounding), for small
// problems where fp32 accuracy is the point.  One wave owns 64 query rows of
// one head; each lane holds its row of rotated q and its output accumulator
// in registers.  K/V tiles of 32 keys are staged in LDS (K rotated on the way
// in) and read back as broadcasts.  Per tile the lane computes its 32 scores,
// then applies the online softmax: new running max, rescale of the earlier
// accumulator and sum, exponentials of this tile ("8.3 长上下文技术" §8.3.4
// (1)-(2)); the N x N score matrix never exists.  Key tiles wholly above the
// causal diagonal of the wave's rows, or wholly before its sliding window
// (sinks aside, "Long Context..." §10.1-10.2), are never visited.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "srt_internal.h"

namespace srt {
namespace {

constexpr int kRows = 64;   // query rows per workgroup (one wave)
constexpr int kKeys = 32;   // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
__global__ void __launch_bounds__(64) prefill_f32_kernel(PrefillArgs a) {
  __shared__ float ks[kKeys][D + 1];
  __shared__ float vs[kKeys][D];

  const int lane = threadIdx.x;
  const int qtile = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int group = a.Hq / a.Hkv;
  const int hk = h / group;
  const int r = qtile * kRows + lane;
  const bool row_ok = r < a.Nq;
  const long long qpos = a.q_pos0 + r;                          // mask position
  const long long qrope = a.q_rope0 + (long long)r * a.rope_step;  // RoPE position

  const float* qg = reinterpret_cast<const float*>(a.q) + ((long long)b * a.Hq + h) * a.q_hstride;
  const float* kg = reinterpret_cast<const float*>(a.k) + ((long long)b * a.Hkv + hk) * a.kv_hstride;
  const float* vg = reinterpret_cast<const float*>(a.v) + ((long long)b * a.Hkv + hk) * a.kv_hstride;
  const float2* tab = reinterpret_cast<const float2*>(a.table);

  // q row, rotated on load, pre-multiplied by sm_scale * log2(e) so that the
  // softmax runs on base-2 exponentials.
  const float qscale = a.sm_scale * kLog2e;
  float q[D];
  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { q[d] = row_ok ? qg[(long long)r * D + d] : 0.f; o[d] = 0.f; }
  // pair i is (2i, 2i+1) (interleaved) or (i, i + D/2) (half-split)
  const bool half_pairs = (a.rope_flags & 4) != 0;
  // (two loops with compile-time indices keep q in registers)
  if ((a.rope_flags & 1) && row_ok) {
    if (half_pairs) {
#pragma unroll
      for (int i = 0; i < D / 2; ++i) {
        const float2 cs = tab[qrope * (D / 2) + i];
        const float x0 = q[i], x1 = q[i + D / 2];
        q[i] = x0 * cs.x - x1 * cs.y;
        q[i + D / 2] = x0 * cs.y + x1 * cs.x;
      }
    } else {
#pragma unroll
      for (int i = 0; i < D / 2; ++i) {
        const float2 cs = tab[qrope * (D / 2) + i];
        const float x0 = q[2 * i], x1 = q[2 * i + 1];
        q[2 * i] = x0 * cs.x - x1 * cs.y;
        q[2 * i + 1] = x0 * cs.y + x1 * cs.x;
      }
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] *= qscale;

  // keys this workgroup may see: k_pos0 + c <= max query position
  int kend = a.Nk;
  if (a.causal) {
    const long long last_q = a.q_pos0 + min(a.Nq, (qtile + 1) * kRows) - 1;
    const long long lim = last_q - a.k_pos0 + 1;
    kend = (int)max(0LL, min((long long)a.Nk, lim));
  }

  // Sliding window: keys before (first query position - window + 1) are
  // invisible to every row here except the sinks (positions < sink).  Tiles
  // run over [0, sink tiles) and then [window start, kend); each tile is
  // visited once and the per-key mask below is exact, so the two ranges may
  // touch.
  int nsk = 0, shift = 0, ntiles = (kend + kKeys - 1) / kKeys;
  if (a.window > 0) {
    const long long lo = a.q_pos0 + (long long)qtile * kRows - a.window + 1 - a.k_pos0;
    const long long cs = min((long long)kend, max(0LL, (long long)a.sink - a.k_pos0));
    nsk = (int)((cs + kKeys - 1) / kKeys);
    const int tstart = lo >= kend ? ntiles : max(nsk, (int)(max(0LL, lo) / kKeys));
    shift = tstart - nsk;
    ntiles = nsk + max(0, ntiles - tstart);
  }

  float m = -INFINITY, l = 0.f;
  for (int ti = 0; ti < ntiles; ++ti) {
    const int c0 = (ti < nsk ? ti : ti + shift) * kKeys;
    __syncthreads();
    // stage 32 key rows (rotated) and value rows; lane handles pair columns
    for (int e = lane; e < kKeys * (D / 2); e += 64) {
      const int c = e / (D / 2), i = e % (D / 2);
      const int i0 = half_pairs ? i : 2 * i, i1 = half_pairs ? i + D / 2 : 2 * i + 1;
      float k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
      if (c0 + c < a.Nk) {
        const long long off = (long long)(c0 + c) * D;
        k0 = kg[off + i0]; k1 = kg[off + i1]; v0 = vg[off + i0]; v1 = vg[off + i1];
        if (a.rope_flags & 2) {
          const float2 cs = tab[(a.k_rope0 + (long long)(c0 + c) * a.rope_step) * (D / 2) + i];
          const float t0 = k0 * cs.x - k1 * cs.y, t1 = k0 * cs.y + k1 * cs.x;
          k0 = t0; k1 = t1;
        }
      }
      ks[c][i0] = k0; ks[c][i1] = k1;
      vs[c][i0] = v0; vs[c][i1] = v1;
    }
    __syncthreads();
    float s[kKeys];
    float tmax = -INFINITY;
#pragma unroll
    for (int c = 0; c < kKeys; ++c) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], ks[c][d], acc);
      const long long kpos = a.k_pos0 + c0 + c;
      const bool vis = (c0 + c < kend) && (!a.causal || kpos <= qpos) &&
                       (a.window <= 0 || qpos - kpos < a.window || kpos < a.sink);
      s[c] = vis ? acc : -INFINITY;
      tmax = fmaxf(tmax, s[c]);
    }
    const float mnew = fmaxf(m, tmax);
    if (mnew == -INFINITY) continue;     // nothing visible yet for this row
    const float alpha = exp2f(m - mnew); // m = -inf gives 0
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int c = 0; c < kKeys; ++c) {
      const float p = exp2f(s[c] - mnew);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, vs[c][d], o[d]);
    }
    m = mnew;
  }
  if (!row_ok) return;
  float inv = l > 0.f ? 1.0f / l : 0.f;
  float lse_row = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  if (a.acc_o) {
    // one ring step: fold (O, lse) into the running state by the log-sum-exp
    // rule ("8.3 长上下文技术" §8.3.5), in place when out is the state itself
    const float la = a.acc_lse[((long long)b * a.Hq + h) * a.acc_lse_hstride + r];
    const float mx = fmaxf(la, lse_row);
    float wa = 0.f;
    if (mx == -INFINITY) {
      inv = 0.f;
    } else {
      const float ea = expf(la - mx), eb = expf(lse_row - mx);
      wa = ea / (ea + eb);
      inv *= eb / (ea + eb);
      lse_row = mx + logf(ea + eb);
    }
    const float* ap = a.acc_o + ((long long)b * a.Hq + h) * a.acc_hstride + (long long)r * D;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = fmaf(wa, ap[d], o[d] * inv);
    inv = 1.0f;
  }
  if (a.out_bf16) {
    __hip_bfloat16* og = reinterpret_cast<__hip_bfloat16*>(a.out) + ((long long)b * a.Hq + h) * a.o_hstride +
                         (long long)r * D;
#pragma unroll
    for (int d = 0; d < D; ++d) og[d] = __float2bfloat16(o[d] * inv);
  } else {
    float* og = reinterpret_cast<float*>(a.out) + ((long long)b * a.Hq + h) * a.o_hstride + (long long)r * D;
#pragma unroll
    for (int d = 0; d < D; ++d) og[d] = o[d] * inv;
  }
  if (a.lse) a.lse[((long long)b * a.Hq + h) * a.lse_hstride + r] = lse_row;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  const dim3 grid((a.Nq + kRows - 1) / kRows, a.Hq, a.B), block(64);
  if (a.D == 64) hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, 0, stream, a);
  else if (a.D == 128) hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, block, 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace srt
