// Split-K decode: one new query token per sequence against a rotated bf16
// KV cache [B][Hkv][Nk][128].
//
// Every decode step streams the whole K/V cache from HBM ("Long Context: RoPE
// / YaRN / NTK / MLA" §12.3), so the kernel is bound by HBM bandwidth.  The
// cache rows [0, seq_len) of a sequence (with a sliding window, only the
// window's rows and the sinks, §10.1-10.2) are cut into `splits` blocks; one
// workgroup reads one block of one KV head exactly once (K and V in the same
// pass) and serves all query heads of that GQA group from registers.  The
// partial results (O_s, lse_s) are merged by a second, tiny kernel with the
// log-sum-exp rule, the same online-softmax combination the pages use for
// Ring / Star Attention partial results ("8.3 长上下文技术" §8.3.5-8.3.6).
//
// Lane layout: 8 lanes share one cache row.  Lane `sub` of a row loads the
// 16-byte chunks sub and sub+8 (dims 8*sub..8*sub+7 and 64+8*sub..), so each
// load instruction of a wave reads 8 whole 128-byte row halves.  The q.k dot
// is 4 bf16 dot2 instructions per chunk and head, finished by three DPP adds
// inside the 8 lanes (no matrix cores run here, so the dot instructions
// compete with nothing).  Each lane keeps a private online softmax over
// its rows (running max m, sum l, accumulator of its 16 dims per head) and only
// rescales when a score exceeds its running max by more than 2^8 (the result is
// exact for any choice of m; the bound only keeps e^(s-m) <= 2^8).  Partial
// states are merged across lanes and waves once at the end.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "srt_internal.h"

#include <mutex>

namespace srt {
namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;
constexpr int kLanesPerRow = 8;
constexpr int kRowsPerIter = kThreads / kLanesPerRow;   // 32
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;                           // rescale threshold in log2 units

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ inline float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline uint32_t pack2(float a, float b) {
  // one v_cvt_pk_bf16_f32: both values rounded to nearest even
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a, b}, b2_t));
}

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Sum over the 8 lanes of a row group with DPP moves (no LDS traffic): swap
// neighbours, swap pairs within the quad, then the half-row mirror pairs every
// lane with one of the other quad.
__device__ inline float sum8_dpp(float t) {
  t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t), 0xB1, 0xF, 0xF, false));
  t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t), 0x4E, 0xF, 0xF, false));
  t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t), 0x141, 0xF, 0xF, false));
  return t;
}

// Streaming load of the KV cache: every byte is read once per decode step, so
// the loads are marked non-temporal (they bypass cache retention).  Measured
// on the 128K cache: 6.39 TB/s against 5.91 TB/s with ordinary loads.
__device__ inline uint4 ntload(const uint4* p) {
  typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
  const u4_t v = __builtin_nontemporal_load(reinterpret_cast<const u4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int G>
__global__ void __launch_bounds__(kThreads, 2) decode_split_kernel(DecodeArgs a) {
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = tid & (kLanesPerRow - 1);
  const int rgroup = tid / kLanesPerRow;                 // 0..31
  int seq = a.seq_lens ? a.seq_lens[b] : a.Nk;
  seq = seq < 0 ? 0 : (seq > a.Nk ? a.Nk : seq);
  // Visible keys, numbered u = 0 .. nvis-1: without a window the rows [0, seq);
  // with one, the sinks [0, ns) that are not already in the window, then the
  // window [wlo, seq).  Key u sits at cache row u (u < ns) or u + (wlo - ns).
  int ns = 0, wshift = 0, nvis = seq;
  if (a.window > 0) {
    const int wlo = max(0, seq - a.window);
    ns = min(a.sink, wlo);
    wshift = wlo - ns;
    nvis = ns + (seq - wlo);
  }
  const int lo = split * a.split_len;
  const int hi = min(nvis, lo + a.split_len);
  const int h0 = hk * G;
  float* ws_o = a.ws_o + (((long long)b * a.Hq + h0) * a.splits + split) * kD;
  float* ws_l = a.ws_lse + ((long long)b * a.Hq + h0) * a.splits + split;

  __shared__ float red_m[4][G];
  __shared__ float red_l[4][G];
  __shared__ float red_o[4][G][kD];

  if (lo >= hi) {   // empty block of this sequence: identity state
    for (int e = tid; e < G * kD; e += kThreads) ws_o[(long long)(e / kD) * a.splits * kD + e % kD] = 0.f;
    if (tid < G) ws_l[(long long)tid * a.splits] = -INFINITY;
    return;
  }

  // ---- q of the G heads: rotate at position seq-1, fold sm_scale*log2(e), pack to bf16 pairs.
  // A q that is not rotated stays exact (as the prefill kernel keeps it): it is
  // packed as given and the dot products are scaled in fp32 instead, since a
  // rounding of q * sm_scale*log2(e) would move each score by up to 2^-9 of it.
  const long long qpos = seq - 1;
  const float qs_pre = a.table ? a.sm_scale * kLog2e : 1.f;
  const float qs_post = a.table ? 1.f : a.sm_scale * kLog2e;
  uint32_t qp[G][8];       // [head][chunk c (0: dims 8sub.., 1: dims 64+8sub..) * 4 + pair-in-chunk]
  const uint4* qg = reinterpret_cast<const uint4*>(a.q);
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint4 w0 = qg[((long long)b * a.Hq + h0 + j) * (kD / 8) + sub];
    const uint4 w1 = qg[((long long)b * a.Hq + h0 + j) * (kD / 8) + sub + 8];
    const uint32_t ww[2][4] = {{w0.x, w0.y, w0.z, w0.w}, {w1.x, w1.y, w1.z, w1.w}};
    float x[2][8];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int p = 0; p < 4; ++p) { x[c][2 * p] = lo_f(ww[c][p]); x[c][2 * p + 1] = hi_f(ww[c][p]); }
    if (a.table) {
      const float2* tab = reinterpret_cast<const float2*>(a.table) + qpos * (kD / 2);
      if (a.half_pairs) {
        // pair 8*sub + e is (element e of chunk sub, element e of chunk sub + 8)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 cs = tab[8 * sub + e];
          const float t0 = x[0][e] * cs.x - x[1][e] * cs.y, t1 = x[0][e] * cs.y + x[1][e] * cs.x;
          x[0][e] = t0; x[1][e] = t1;
        }
      } else {
        // pair (chunk * 4 + p) is elements 2p, 2p+1 of one chunk
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float2 cs = tab[(sub + 8 * c) * 4 + p];
            const float x0 = x[c][2 * p], x1 = x[c][2 * p + 1];
            x[c][2 * p] = x0 * cs.x - x1 * cs.y;
            x[c][2 * p + 1] = x0 * cs.y + x1 * cs.x;
          }
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int p = 0; p < 4; ++p) qp[j][c * 4 + p] = pack2(x[c][2 * p] * qs_pre, x[c][2 * p + 1] * qs_pre);
  }

  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY; l[j] = 0.f;
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[j][d] = 0.f;
  }

  const long long row_base = ((long long)b * a.Hkv + hk) * a.Nk;
  const uint4* kg = reinterpret_cast<const uint4*>(a.k) + row_base * (kD / 8);
  const uint4* vg = reinterpret_cast<const uint4*>(a.v) + row_base * (kD / 8);

  constexpr int kUnroll = G >= 8 ? 1 : 4;   // rows per lane in flight (G = 8 keeps 8 heads of state)
  for (int r0 = lo; r0 < hi; r0 += kRowsPerIter * kUnroll) {
    uint4 kw[kUnroll][2], vw[kUnroll][2];
    bool valid[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int row = r0 + u * kRowsPerIter + rgroup;
      valid[u] = row < hi;
      const int vrow = valid[u] ? row : lo;
      const long long off = (long long)(vrow < ns ? vrow : vrow + wshift) * (kD / 8);
      kw[u][0] = ntload(kg + off + sub);
      kw[u][1] = ntload(kg + off + sub + 8);
      vw[u][0] = ntload(vg + off + sub);
      vw[u][1] = ntload(vg + off + sub + 8);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t kk[8] = {kw[u][0].x, kw[u][0].y, kw[u][0].z, kw[u][0].w,
                              kw[u][1].x, kw[u][1].y, kw[u][1].z, kw[u][1].w};
      float s[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float t = 0.f;
#pragma unroll
        for (int p = 0; p < 8; ++p) t = dot2(qp[j][p], kk[p], t);
        t = sum8_dpp(t) * qs_post;
        s[j] = valid[u] ? t : -INFINITY;
      }
      const uint32_t vv[8] = {vw[u][0].x, vw[u][0].y, vw[u][0].z, vw[u][0].w,
                              vw[u][1].x, vw[u][1].y, vw[u][1].z, vw[u][1].w};
      float vf[16];
#pragma unroll
      for (int p = 0; p < 8; ++p) { vf[2 * p] = lo_f(vv[p]); vf[2 * p + 1] = hi_f(vv[p]); }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (s[j] > m[j] + kLazy) {          // rare: raise the running max
          const float sc = __builtin_amdgcn_exp2f(m[j] - s[j]);
          l[j] *= sc;
#pragma unroll
          for (int d = 0; d < 16; ++d) acc[j][d] *= sc;
          m[j] = s[j];
        }
        const float p = valid[u] ? __builtin_amdgcn_exp2f(s[j] - m[j]) : 0.f;
        l[j] += p;
#pragma unroll
        for (int d = 0; d < 16; ++d) acc[j][d] = fmaf(p, vf[d], acc[j][d]);
      }
    }
  }

  // ---- merge the per-lane states: lanes of one row group hold the same (m, l);
  // reduce over the 8 row groups of a wave, then over the 4 waves.
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float M = m[j];
    M = fmaxf(M, __shfl_xor(M, 8));
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float sc = (m[j] == -INFINITY) ? 0.f : exp2f(m[j] - M);
    float L = l[j] * sc;
    L += __shfl_xor(L, 8);
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      float x = acc[j][d] * sc;
      x += __shfl_xor(x, 8);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[j][d] = x;
    }
    if (lane < kLanesPerRow) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        red_o[wave][j][8 * sub + d] = acc[j][d];
        red_o[wave][j][64 + 8 * sub + d] = acc[j][8 + d];
      }
    }
    if (lane == 0) { red_m[wave][j] = M; red_l[wave][j] = L; }
  }
  __syncthreads();
  for (int e = tid; e < G * kD; e += kThreads) {
    const int j = e / kD, d = e % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][j]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = red_m[w][j] == -INFINITY ? 0.f : exp2f(red_m[w][j] - M);
      L += red_l[w][j] * sc;
      O += red_o[w][j][d] * sc;
    }
    ws_o[(long long)j * a.splits * kD + d] = L > 0.f ? O / L : 0.f;
    if (d == 0) ws_l[(long long)j * a.splits] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
}

// Merge the `splits` partial states of one (b, h): lse-weighted average.
// Thread (d, part) folds the splits s = part, part + kCombineParts, ... of
// dimension d into a running (m, l, o) state, with eight splits' loads in
// flight at a time, and the kCombineParts states of each d are merged through
// LDS: the splits are read in a few round trips instead of one loop
// iteration after another.
constexpr int kCombineParts = 4;
__global__ void __launch_bounds__(kD * kCombineParts) decode_combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int d = tid % kD, part = tid / kD;
  const long long bh = (long long)b * a.Hq + h;
  const float* pl = a.ws_lse + bh * a.splits;
  const float* po = a.ws_o + bh * a.splits * kD;
  float m = -INFINITY, l = 0.f, o = 0.f;
  for (int s0 = part; s0 < a.splits; s0 += 8 * kCombineParts) {
    float ls[8], os[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u * kCombineParts;
      ls[u] = s < a.splits ? pl[s] : -INFINITY;
      os[u] = s < a.splits ? po[(long long)s * kD + d] : 0.f;
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < 8; ++u) mn = fmaxf(mn, ls[u]);
    if (mn != -INFINITY) {
      const float sc = __expf(m - mn);                  // m = -inf: exp(-inf) = 0, and l = o = 0 anyway
      l *= sc;
      o *= sc;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = __expf(ls[u] - mn);             // an empty split (lse = -inf) weighs 0
        l += w;
        o = fmaf(w, os[u], o);
      }
      m = mn;
    }
  }
  __shared__ float sm_m[kCombineParts], sm_l[kCombineParts], sm_o[kCombineParts][kD];
  if (d == 0) { sm_m[part] = m; sm_l[part] = l; }
  sm_o[part][d] = o;
  __syncthreads();
  if (part != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < kCombineParts; ++p) M = fmaxf(M, sm_m[p]);
  float L = 0.f, O = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int p = 0; p < kCombineParts; ++p) {
      const float w = __expf(sm_m[p] - M);
      L += w * sm_l[p];
      O = fmaf(w, sm_o[p][d], O);
    }
  }
  reinterpret_cast<__hip_bfloat16*>(a.out)[bh * kD + d] = __float2bfloat16(L > 0.f ? O / L : 0.f);
  if (a.lse && d == 0) a.lse[bh] = L > 0.f ? M + __logf(L) : -INFINITY;
}

}  // namespace

// Scratch of srt_attn_decode_splitk_noalloc: the split partials (fp32 O and
// lse of every split) live in this file-scope device array instead of a
// caller workspace, for callers that cannot allocate.  Each GPU holds its own
// copy for the life of the process, at its own address; in host code the
// array's name is only a stand-in, so its device address is looked up once
// per device with hipGetSymbolAddress and the kernels receive that address.
// Every call on a GPU shares that GPU's copy (calls that overlap on one GPU
// race); nothing in it needs clearing, as the split kernel writes every slot
// the combine kernel reads.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));     // with device `dev` current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t decode_workspace_bytes(int B, int Hq, int D, int splits) {
  return (size_t)B * Hq * splits * (size_t)(D + 1) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.D != kD) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv;
  const dim3 grid(a.splits, a.Hkv, a.B), block(kThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(decode_split_kernel<4>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(decode_split_kernel<8>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.Hq, a.B), dim3(kD * kCombineParts), 0, stream, a);
  return hipGetLastError();
}

}  // namespace srt
