// RoPE kernels: the cos/sin table and the standalone rotation.
//
// Table: entry (p, i) = mscale * (cos, sin)(p * theta'_i).  The angle is formed
// and the trigonometric functions evaluated in fp64, then rounded to fp32 once,
// so positions up to 2^31 keep full fp32 accuracy ("Long Context: RoPE / YaRN /
// NTK / MLA" §A.1 recommends computing cos/sin in fp32 or better and casting;
// §6.4 folds the YaRN temperature into the cached cos/sin).
//
// Rotation: interleaved pairs (x_{2i}, x_{2i+1}) turned counter-clockwise by
// the table angle ("Long Context..." §2.2; "长上下文外推" §4.2), or half-split
// pairs (x_i, x_{i+D/2}) ("Long Context..." §2.4 code).  HBM-bound:
// each thread moves 8 elements (one 16-byte bf16 vector or two fp32 vectors)
// and reads the matching 4 table entries (32 bytes, L2-resident across heads).
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "srt_internal.h"

namespace srt {
namespace {

__global__ void __launch_bounds__(256) rope_table_kernel(Theta th, int half, double mscale, long long npos,
                                                          float2* __restrict__ table) {
  const long long total = npos * half;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long p = e / half;
    const int i = (int)(e - p * half);
    double s, c;
    sincos((double)p * th.v[i], &s, &c);
    table[e] = make_float2((float)(mscale * c), (float)(mscale * s));
  }
}

// Position of row n of a group (see PosMap).
__device__ inline long long row_pos(const PosMap& m, long long n) {
  if (m.mode == kContiguous) return m.pos0 + n;
  const long long j = n / m.C, t = n - j * m.C;
  if (m.mode == kStriped) return m.pos0 + j + (long long)m.P * t;
  const long long h = m.C / 2;
  return m.pos0 + (t < h ? j * h + t : (2LL * m.P - 1 - j) * h + (t - h));
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 pair -> packed bf16 pair (lo = a, hi = b), round to nearest even
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  // one v_cvt_pk_bf16_f32: both values rounded to nearest even
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a, b}, b2_t));
}

// One thread = 8 consecutive elements of one row = 4 pairs.
// With a null table the rotation is the identity.  Every output is
// multiplied by `scale` (through the table entries, one rounding to bf16).
template <bool BF16>
__global__ void __launch_bounds__(256) rope_apply_kernel(const void* __restrict__ x, void* y, long long groups,
                                                         int N, int D, PosMap map,
                                                         const float4* __restrict__ table, float scale) {
  const int vec_per_row = D / 8;
  const long long total = groups * (long long)N * vec_per_row;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long row = e / vec_per_row;
    const int j = (int)(e - row * vec_per_row);        // which 8-element chunk of the row
    const long long p = row_pos(map, row % N);
    // table row p, pairs 4j .. 4j+3 = two float4 of (cos, sin, cos, sin)
    float4 t0 = make_float4(1.f, 0.f, 1.f, 0.f), t1 = t0;
    if (table) {
      const float4* trow = table + (p * (D / 2) + 4 * j) / 2;
      t0 = trow[0];
      t1 = trow[1];
    }
    const float c[4] = {t0.x * scale, t0.z * scale, t1.x * scale, t1.z * scale};
    const float s[4] = {t0.y * scale, t0.w * scale, t1.y * scale, t1.w * scale};
    float v[8];
    if (BF16) {
      const uint4 w = reinterpret_cast<const uint4*>(x)[e];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(ww[i]); v[2 * i + 1] = bf16_hi(ww[i]); }
    } else {
      const float4 a = reinterpret_cast<const float4*>(x)[2 * e];
      const float4 b = reinterpret_cast<const float4*>(x)[2 * e + 1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    float o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = v[2 * i] * c[i] - v[2 * i + 1] * s[i];
      o[2 * i + 1] = v[2 * i] * s[i] + v[2 * i + 1] * c[i];
    }
    if (BF16) {
      uint4 w;
      w.x = pack_bf16x2(o[0], o[1]); w.y = pack_bf16x2(o[2], o[3]);
      w.z = pack_bf16x2(o[4], o[5]); w.w = pack_bf16x2(o[6], o[7]);
      reinterpret_cast<uint4*>(y)[e] = w;
    } else {
      reinterpret_cast<float4*>(y)[2 * e] = make_float4(o[0], o[1], o[2], o[3]);
      reinterpret_cast<float4*>(y)[2 * e + 1] = make_float4(o[4], o[5], o[6], o[7]);
    }
  }
}

__device__ inline void load8(const void* base, long long idx8, bool bf16, float v[8]) {
  if (bf16) {
    const uint4 w = reinterpret_cast<const uint4*>(base)[idx8];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(ww[i]); v[2 * i + 1] = bf16_hi(ww[i]); }
  } else {
    const float4 a = reinterpret_cast<const float4*>(base)[2 * idx8];
    const float4 b = reinterpret_cast<const float4*>(base)[2 * idx8 + 1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ inline void store8(void* base, long long idx8, bool bf16, const float o[8]) {
  if (bf16) {
    uint4 w;
    w.x = pack_bf16x2(o[0], o[1]); w.y = pack_bf16x2(o[2], o[3]);
    w.z = pack_bf16x2(o[4], o[5]); w.w = pack_bf16x2(o[6], o[7]);
    reinterpret_cast<uint4*>(base)[idx8] = w;
  } else {
    reinterpret_cast<float4*>(base)[2 * idx8] = make_float4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<float4*>(base)[2 * idx8 + 1] = make_float4(o[4], o[5], o[6], o[7]);
  }
}

// Half-split pairs ("Long Context..." §2.4 apply_rope): pair i is
// (x_i, x_{i+D/2}).  One thread = 8 pairs = elements [8j, 8j+8) of the first
// half and the same 8 of the second half.
template <bool BF16>
__global__ void __launch_bounds__(256) rope_apply_half_kernel(const void* __restrict__ x, void* y, long long groups,
                                                              int N, int D, PosMap map,
                                                              const float4* __restrict__ table, float scale) {
  const int per_row = D / 16;
  const long long total = groups * (long long)N * per_row;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long row = e / per_row;
    const int j = (int)(e - row * per_row);
    const long long p = row_pos(map, row % N);
    const float4* trow = table + (p * (D / 2) + 8 * j) / 2;      // pairs 8j .. 8j+7
    const long long i1 = row * (D / 8) + j, i2 = i1 + D / 16;     // 8-element chunks of the two halves
    float a[8], b[8], o1[8], o2[8];
    load8(x, i1, BF16, a);
    load8(x, i2, BF16, b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 tq = trow[q];
      const float4 t = make_float4(tq.x * scale, tq.y * scale, tq.z * scale, tq.w * scale);
      // pairs 2q and 2q+1 of this thread: (cos, sin) = (t.x, t.y), (t.z, t.w)
      o1[2 * q] = a[2 * q] * t.x - b[2 * q] * t.y;
      o2[2 * q] = a[2 * q] * t.y + b[2 * q] * t.x;
      o1[2 * q + 1] = a[2 * q + 1] * t.z - b[2 * q + 1] * t.w;
      o2[2 * q + 1] = a[2 * q + 1] * t.w + b[2 * q + 1] * t.z;
    }
    store8(y, i1, BF16, o1);
    store8(y, i2, BF16, o2);
  }
}

inline unsigned grid_for(long long work, int block) {
  long long g = (work + block - 1) / block;
  const long long cap = 256LL * 64;   // enough waves in flight on 256 CUs; the loops stride beyond
  return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_rope_table(const Theta& th, int half, double mscale, long long npos, float* table,
                             hipStream_t stream) {
  const long long work = npos * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(work, 256)), dim3(256), 0, stream, th, half, mscale, npos,
                     reinterpret_cast<float2*>(table));
  return hipGetLastError();
}

hipError_t launch_rope_apply(const void* x, void* y, bool bf16, bool half_pairs, long long groups, int N, int D,
                             const PosMap& map, const float* table, hipStream_t stream, float scale) {
  const float4* t = reinterpret_cast<const float4*>(table);
  if (half_pairs && table) {
    const long long work = groups * (long long)N * (D / 16);
    if (bf16)
      hipLaunchKernelGGL(rope_apply_half_kernel<true>, dim3(grid_for(work, 256)), dim3(256), 0, stream, x, y, groups,
                         N, D, map, t, scale);
    else
      hipLaunchKernelGGL(rope_apply_half_kernel<false>, dim3(grid_for(work, 256)), dim3(256), 0, stream, x, y,
                         groups, N, D, map, t, scale);
    return hipGetLastError();
  }
  const long long work = groups * (long long)N * (D / 8);
  if (bf16)
    hipLaunchKernelGGL(rope_apply_kernel<true>, dim3(grid_for(work, 256)), dim3(256), 0, stream, x, y, groups, N,
                       D, map, t, scale);
  else
    hipLaunchKernelGGL(rope_apply_kernel<false>, dim3(grid_for(work, 256)), dim3(256), 0, stream, x, y, groups,
                       N, D, map, t, scale);
  return hipGetLastError();
}

}  // namespace srt
