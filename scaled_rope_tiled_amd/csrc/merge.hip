// Log-sum-exp merge of two partial attention states over disjoint key sets:
//   lse = log(e^{lse_a} + e^{lse_b}),  O = e^{lse_a - lse} O_a + e^{lse_b - lse} O_b,
// the online-softmax rescaling that a Ring Attention step applies to the
// result of a newly received K/V block ("8.3 长上下文技术" §8.3.5 step 3 and
// §8.3.4 (2)).  A state with lse = -inf is the identity.
//
// HBM-bound: per row it reads 2 lse + 2*D outputs and writes D + 1 values.
// One thread handles 8 consecutive elements of one row (32-byte fp32 or
// 16-byte bf16 vectors); the two weights are recomputed per thread from the
// row's lse pair (cached in L1/L2), which is cheaper than a second pass.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "srt_internal.h"

namespace srt {
namespace {

__device__ inline void load8(const void* base, long long off, bool bf16, float v[8]) {
  if (bf16) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const __hip_bfloat16*>(base) + off);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(ww[i] << 16);
      v[2 * i + 1] = __uint_as_float(ww[i] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ inline uint32_t pack2(float a, float b) {
  // one v_cvt_pk_bf16_f32: both values rounded to nearest even
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a, b}, b2_t));
}

__device__ inline void store8(void* base, long long off, bool bf16, const float v[8]) {
  if (bf16) {
    uint4 w;
    w.x = pack2(v[0], v[1]); w.y = pack2(v[2], v[3]); w.z = pack2(v[4], v[5]); w.w = pack2(v[6], v[7]);
    *reinterpret_cast<uint4*>(reinterpret_cast<__hip_bfloat16*>(base) + off) = w;
  } else {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <bool IN_BF16, bool OUT_BF16>
__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
  const int vpr = a.D / 8;
  const long long total = (long long)a.BH * a.N * vpr;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long row = e / vpr;
    const int j = (int)(e - row * vpr);
    const long long bh = row / a.N;
    const int n = (int)(row - bh * a.N);
    const float la = a.la[bh * a.N + n], lb = a.lb[bh * a.N + n];
    const float m = fmaxf(la, lb);
    float wa = 0.f, wb = 0.f, lse = -INFINITY;
    if (m != -INFINITY) {
      const float ea = __expf(la - m), eb = __expf(lb - m);   // exp(-inf) = 0
      const float inv = 1.0f / (ea + eb);
      wa = ea * inv;
      wb = eb * inv;
      lse = m + __logf(ea + eb);
    }
    const long long in_off = bh * a.in_hstride + (long long)n * a.D + 8 * j;
    float va[8], vb[8], vo[8];
    load8(a.oa, in_off, IN_BF16, va);
    load8(a.ob, in_off, IN_BF16, vb);
#pragma unroll
    for (int i = 0; i < 8; ++i) vo[i] = wa * va[i] + wb * vb[i];
    store8(a.oo, bh * a.out_hstride + (long long)n * a.D + 8 * j, OUT_BF16, vo);
    if (a.lo && j == 0) a.lo[bh * a.lse_out_hstride + n] = lse;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.D % 8) return hipErrorInvalidValue;
  const long long work = (long long)a.BH * a.N * (a.D / 8);
  long long g = (work + 255) / 256;
  if (g > 256LL * 64) g = 256LL * 64;
  const dim3 grid((unsigned)(g < 1 ? 1 : g)), block(256);
  if (a.in_bf16 && a.out_bf16) hipLaunchKernelGGL((merge_kernel<true, true>), grid, block, 0, stream, a);
  else if (a.in_bf16) hipLaunchKernelGGL((merge_kernel<true, false>), grid, block, 0, stream, a);
  else if (a.out_bf16) hipLaunchKernelGGL((merge_kernel<false, true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((merge_kernel<false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace srt
