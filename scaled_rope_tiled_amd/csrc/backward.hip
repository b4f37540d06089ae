// Backward pass of RoPE-scaled softmax attention (dq, dk, dv).
//
// The attention matrix is recomputed tile by tile from q, k, v and the lse the
// forward pass saved, never stored ("8.3 长上下文技术" §8.3.4 (3)).  With
// P = exp(S - lse), S = sm_scale q~ k~^T (q~, k~ rotated, mscale in the table):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),  delta = rowsum(dO * O),
//   dq~ = sm_scale dS k~,  dk~ = sm_scale dS^T q~,
// and the gradient of a rotated input is turned back by the transposed
// rotation (the rotation by the opposite angle): dq = R^T dq~ with the same
// (mscale cos, mscale sin) table entries.
//
// Three launches: delta (HBM-bound), dk/dv (a workgroup owns a block of keys
// of one KV head and walks the query tiles of every query head of its GQA
// group that can see them; half its waves produce P and dV, the other half
// dS and dK, exchanging P through LDS) and dq (a workgroup owns query rows,
// like the forward kernel, and walks the visible key tiles; 8 waves, one
// workgroup per CU, every staged k/v tile serving all of them).
// The entry point rotates q and k once into its workspace, so the tiles the
// kernels stage need no rotation (every key block would otherwise rotate each
// q tile again, and every query block each k tile).  bf16 kernels (D = 128)
// use v_mfma_f32_32x32x16_bf16 for all five products; fp32 kernels (D = 64)
// keep every product in fp32 on the vector ALUs.  Gradients are written in
// fp32.
#include "mfma_common.h"
#include "item_queue.h"

#include <type_traits>

namespace srt {
namespace {

using namespace mc;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline void load8f(const void* base, long long idx8, bool bf16, float v[8]) {
  if (bf16) {
    const uint4 w = reinterpret_cast<const uint4*>(base)[idx8];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = bf_lo(ww[i]); v[2 * i + 1] = bf_hi(ww[i]); }
  } else {
    const float4 x = reinterpret_cast<const float4*>(base)[2 * idx8];
    const float4 y = reinterpret_cast<const float4*>(base)[2 * idx8 + 1];
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  }
}

// ------------------------------------------------------------------ delta
// delta[row] = sum_d dO[row][d] O[row][d] in fp32; D/8 lanes per row.
template <bool BF16>
__global__ void __launch_bounds__(256) bwd_delta_kernel(const void* __restrict__ o, const void* __restrict__ dout,
                                                        float* __restrict__ delta, long long rows, int D) {
  const int per_row = D / 8;                    // 8 or 16: divides the wave
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = e / per_row;
  float acc = 0.f;
  if (row < rows) {
    float x[8], y[8];
    load8f(o, e, BF16, x);
    load8f(dout, e, BF16, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(x[i], y[i], acc);
  }
  for (int m = per_row / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, per_row);
  if (row < rows && (e % per_row) == 0) delta[row] = acc;
}

// Visibility of key position kp to query position qp (causal, window, sinks).
__device__ inline bool visible(const BwdArgs& a, long long qp, long long kp) {
  if (!a.causal) return true;
  if (kp > qp) return false;
  return a.window <= 0 || qp - kp < a.window || kp < a.sink;
}

// Turn a gradient pair back: (g0, g1) -> R^T (g0, g1) with (c, s) = mscale (cos, sin).
__device__ inline void rotate_back(float& g0, float& g1, float2 cs) {
  const float y0 = cs.x * g0 + cs.y * g1, y1 = -cs.y * g0 + cs.x * g1;
  g0 = y0;
  g1 = y1;
}

// ------------------------------------------------------------------ fp32 (D = 64)
template <int D>
__global__ void __launch_bounds__(64) bwd_dq_f32_kernel(BwdArgs a) {
  __shared__ float ks[32][D + 1];
  __shared__ float vs[32][D + 1];
  const int lane = threadIdx.x, qtile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (a.Hq / a.Hkv);
  const int r = qtile * 64 + lane;
  const bool row_ok = r < a.Nq;
  const long long qpos = a.q_pos0 + r;
  const bool half = (a.rope_flags & 4) != 0;
  const long long qrow = ((long long)b * a.Hq + h) * a.Nq + r;
  const float* qg = reinterpret_cast<const float*>(a.q);
  const float* dog = reinterpret_cast<const float*>(a.dout);
  const float* kg = reinterpret_cast<const float*>(a.k) + ((long long)b * a.Hkv + hk) * a.Nk * D;
  const float* vg = reinterpret_cast<const float*>(a.v) + ((long long)b * a.Hkv + hk) * a.Nk * D;
  const float2* tab = reinterpret_cast<const float2*>(a.table);

  float q[D], dov[D], dq[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = row_ok ? qg[qrow * D + d] : 0.f;
    dov[d] = row_ok ? dog[qrow * D + d] : 0.f;
    dq[d] = 0.f;
  }
  if ((a.rope_flags & 1) && row_ok) {
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      const int i0 = half ? i : 2 * i, i1 = half ? i + D / 2 : 2 * i + 1;
      const float2 cs = tab[qpos * (D / 2) + i];
      const float x0 = q[i0], x1 = q[i1];
      q[i0] = x0 * cs.x - x1 * cs.y;
      q[i1] = x0 * cs.y + x1 * cs.x;
    }
  }
  const float c2 = a.sm_scale * kLog2e;
  const float lse2 = row_ok ? a.lse[qrow] * kLog2e : 0.f;
  const float dl = row_ok ? a.delta[qrow] : 0.f;

  int kend = a.Nk;
  if (a.causal) {
    const long long last_q = a.q_pos0 + min(a.Nq, (qtile + 1) * 64) - 1;
    kend = (int)max(0LL, min((long long)a.Nk, last_q - a.k_pos0 + 1));
  }
  int kbeg = 0;
  if (a.causal && a.window > 0 && a.sink <= a.k_pos0) {   // no sink in this K: skip keys before every window
    const long long lo = a.q_pos0 + (long long)qtile * 64 - a.window + 1 - a.k_pos0;
    kbeg = (int)max(0LL, min((long long)kend, lo)) / 32 * 32;
  }
  for (int c0 = kbeg; c0 < kend; c0 += 32) {
    __syncthreads();
    for (int e = lane; e < 32 * (D / 2); e += 64) {
      const int c = e / (D / 2), i = e % (D / 2);
      const int i0 = half ? i : 2 * i, i1 = half ? i + D / 2 : 2 * i + 1;
      float k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
      if (c0 + c < a.Nk) {
        const long long off = (long long)(c0 + c) * D;
        k0 = kg[off + i0]; k1 = kg[off + i1]; v0 = vg[off + i0]; v1 = vg[off + i1];
        if (a.rope_flags & 2) {
          const float2 cs = tab[(a.k_pos0 + c0 + c) * (D / 2) + i];
          const float t0 = k0 * cs.x - k1 * cs.y, t1 = k0 * cs.y + k1 * cs.x;
          k0 = t0; k1 = t1;
        }
      }
      ks[c][i0] = k0; ks[c][i1] = k1;
      vs[c][i0] = v0; vs[c][i1] = v1;
    }
    __syncthreads();
    for (int c = 0; c < 32; ++c) {
      const bool vis = row_ok && c0 + c < kend && visible(a, qpos, a.k_pos0 + c0 + c);
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) { s = fmaf(q[d], ks[c][d], s); dp = fmaf(dov[d], vs[c][d], dp); }
      const float p = vis ? exp2f(s * c2 - lse2) : 0.f;
      const float ds = p * (dp - dl);
#pragma unroll
      for (int d = 0; d < D; ++d) dq[d] = fmaf(ds, ks[c][d], dq[d]);
    }
  }
  if (!row_ok) return;
#pragma unroll
  for (int d = 0; d < D; ++d) dq[d] *= a.sm_scale;
  if (a.rope_flags & 1) {
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      const int i0 = half ? i : 2 * i, i1 = half ? i + D / 2 : 2 * i + 1;
      rotate_back(dq[i0], dq[i1], tab[qpos * (D / 2) + i]);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) a.dq[qrow * D + d] = dq[d];
}

template <int D>
__global__ void __launch_bounds__(64) bwd_dkdv_f32_kernel(BwdArgs a) {
  __shared__ float qs[32][D + 1];
  __shared__ float dos[32][D + 1];
  __shared__ float l2s[32], dls[32];
  const int lane = threadIdx.x, ktile = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int c = ktile * 64 + lane;
  const bool key_ok = c < a.Nk;
  const long long kpos = a.k_pos0 + c;
  const bool half = (a.rope_flags & 4) != 0;
  const long long krow = ((long long)b * a.Hkv + hk) * a.Nk + c;
  const float2* tab = reinterpret_cast<const float2*>(a.table);

  float kk[D], vv[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kk[d] = key_ok ? reinterpret_cast<const float*>(a.k)[krow * D + d] : 0.f;
    vv[d] = key_ok ? reinterpret_cast<const float*>(a.v)[krow * D + d] : 0.f;
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  if ((a.rope_flags & 2) && key_ok) {
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      const int i0 = half ? i : 2 * i, i1 = half ? i + D / 2 : 2 * i + 1;
      const float2 cs = tab[kpos * (D / 2) + i];
      const float x0 = kk[i0], x1 = kk[i1];
      kk[i0] = x0 * cs.x - x1 * cs.y;
      kk[i1] = x0 * cs.y + x1 * cs.x;
    }
  }
  const float c2 = a.sm_scale * kLog2e;
  // query rows that can see some key of this block
  const long long kp_first = a.k_pos0 + (long long)ktile * 64;
  const long long kp_last = a.k_pos0 + min(a.Nk, (ktile + 1) * 64) - 1;
  long long r_lo = 0, r_hi = a.Nq;
  if (a.causal) r_lo = max(0LL, min((long long)a.Nq, kp_first - a.q_pos0));
  if (a.causal && a.window > 0 && kp_first >= a.sink) r_hi = max(0LL, min((long long)a.Nq, kp_last + a.window - a.q_pos0));
  for (int g = 0; g < G; ++g) {
    const int h = hk * G + g;
    const long long hbase = ((long long)b * a.Hq + h) * a.Nq;
    for (long long rt = r_lo / 32 * 32; rt < r_hi; rt += 32) {
      __syncthreads();
      for (int e = lane; e < 32 * (D / 2); e += 64) {
        const int rr = e / (D / 2), i = e % (D / 2);
        const int i0 = half ? i : 2 * i, i1 = half ? i + D / 2 : 2 * i + 1;
        const long long r = rt + rr;
        float q0 = 0.f, q1 = 0.f, o0 = 0.f, o1 = 0.f;
        if (r < a.Nq) {
          const long long off = (hbase + r) * D;
          q0 = reinterpret_cast<const float*>(a.q)[off + i0];
          q1 = reinterpret_cast<const float*>(a.q)[off + i1];
          o0 = reinterpret_cast<const float*>(a.dout)[off + i0];
          o1 = reinterpret_cast<const float*>(a.dout)[off + i1];
          if (a.rope_flags & 1) {
            const float2 cs = tab[(a.q_pos0 + r) * (D / 2) + i];
            const float t0 = q0 * cs.x - q1 * cs.y, t1 = q0 * cs.y + q1 * cs.x;
            q0 = t0; q1 = t1;
          }
        }
        qs[rr][i0] = q0; qs[rr][i1] = q1;
        dos[rr][i0] = o0; dos[rr][i1] = o1;
      }
      if (lane < 32) {
        const long long r = rt + lane;
        l2s[lane] = r < a.Nq ? a.lse[hbase + r] * kLog2e : 0.f;
        dls[lane] = r < a.Nq ? a.delta[hbase + r] : 0.f;
      }
      __syncthreads();
      for (int rr = 0; rr < 32; ++rr) {
        const long long r = rt + rr;
        const bool vis = key_ok && r < a.Nq && visible(a, a.q_pos0 + r, kpos);
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) { s = fmaf(kk[d], qs[rr][d], s); dp = fmaf(vv[d], dos[rr][d], dp); }
        const float p = vis ? exp2f(s * c2 - l2s[rr]) : 0.f;
        const float ds = p * (dp - dls[rr]);
#pragma unroll
        for (int d = 0; d < D; ++d) {
          dv[d] = fmaf(p, dos[rr][d], dv[d]);
          dk[d] = fmaf(ds, qs[rr][d], dk[d]);
        }
      }
    }
  }
  if (!key_ok) return;
#pragma unroll
  for (int d = 0; d < D; ++d) dk[d] *= a.sm_scale;
  if (a.rope_flags & 2) {
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      const int i0 = half ? i : 2 * i, i1 = half ? i + D / 2 : 2 * i + 1;
      rotate_back(dk[i0], dk[i1], tab[kpos * (D / 2) + i]);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    a.dk[krow * D + d] = dk[d];
    a.dv[krow * D + d] = dv[d];
  }
}

// ------------------------------------------------------------------ bf16 (D = 128), matrix cores
//
// Tile layouts follow v_mfma_f32_32x32x16_bf16 (wave64): A operand lane l =
// row l % 32, k = (l / 32) * 8 + 0..7; B operand lane l = column l % 32, same
// k; accumulator lane l = column l % 32, rows (j / 4) * 8 + (l / 32) * 4 + j % 4.
// A product whose B operand comes straight from an accumulator (P, dS) takes
// its k elements in the accumulator's row order; the A operand is then read
// with the transposing LDS read in that same order, as the forward kernel does
// for O^T = V^T P^T.

constexpr int kD = 128;
// Row strides of LDS tiles.  272 B makes the 16-byte row reads conflict-free
// and 320 B the transposing reads; no stride does both.  Tiles read both ways
// use 304 B (row reads conflict-free, transposing reads two-way in part):
// storing such a tile twice, once per stride, measured slower.
// Tiles read both as 16-byte row chunks and with the transposing read: 272-byte
// rows, the 32 rows of a tile permuted, row r in slot prow(r) = (r & 16) +
// 4 (r & 3) + ((r >> 2) & 3).  The 16 rows of one row read then fall on 16
// distinct 16-byte bank groups and the 4 rows of one transposing read on the 4
// disjoint 64-byte quarters of the banks.
constexpr int kTStr = kD + 8;
__device__ constexpr int prow(int r) { return (r & 16) + 4 * (r & 3) + ((r >> 2) & 3); }
constexpr int kRStr = kD + 8;     // 272 B: tiles read only as 16-byte row chunks

// Load 8 d-chunks of one row (d = ks * 16 + hl * 8 + 0..7) and rotate them
// (interleaved pairs in-chunk; half-split pairs chunk ks with ks + 4).
// With scale != 1 the values are multiplied by it before the one rounding to
// bf16 (through the table when rotating).
template <bool HALF>
__device__ inline void load_row_rotated(const __hip_bfloat16* row, bool ok, bool rotate, const float4* tab4,
                                        long long pos, int hl, bf16x8 (&out)[8], float scale = 1.f) {
  uint4 w[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    w[ks] = ok ? *reinterpret_cast<const uint4*>(row + ks * 16 + hl * 8) : make_uint4(0, 0, 0, 0);
  auto sc4 = [&](float4 t) { return make_float4(t.x * scale, t.y * scale, t.z * scale, t.w * scale); };
  if (ok && rotate) {
    if (HALF) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int d0 = ks * 16 + hl * 8;
        const float4* t = tab4 + (pos * (kD / 2) + d0) / 2;
        const float4 tt[4] = {sc4(t[0]), sc4(t[1]), sc4(t[2]), sc4(t[3])};
        rotate_chunk_pair(w[ks], w[ks + 4], tt);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const float4* t = tab4 + (pos * (kD / 2) + (ks * 16 + hl * 8) / 2) / 2;
        w[ks] = rotate_chunk(w[ks], sc4(t[0]), sc4(t[1]));
      }
    }
  } else if (scale != 1.f) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint32_t in[4] = {w[ks].x, w[ks].y, w[ks].z, w[ks].w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack2(bf_lo(in[i]) * scale, bf_hi(in[i]) * scale);
      w[ks] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) out[ks] = as_bf16x8(w[ks]);
}

// acc[db] += X^T[d][rows] B[rows][cols] over a 32-row tile X held row-major in
// LDS (stride kTStr), B given as two 16-row k-steps in accumulator row order.
__device__ inline void mma_tr(f32x16 (&acc)[4], uint32_t x_lane, const bf16x8 (&bk)[2]) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const i16x4 lo = lds_read_tr(x_lane + ((half * 16) * kTStr + db * 32) * 2);
      const i16x4 hi = lds_read_tr(x_lane + ((half * 16 + 2) * kTStr + db * 32) * 2);   // rows + 8: slots + 2
      const bf16x8 xa = __builtin_bit_cast(
          bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){lo[0], lo[1], lo[2], lo[3], hi[0],
                                                                             hi[1], hi[2], hi[3]});
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, bk[half], acc[db], 0, 0, 0);
    }
  }
}


// acc1 = c1 + X1[rows][d] R1[d][cols] and acc2 = c2 + X2 R2, X1 and X2 32-row
// tiles in LDS (16-byte row reads), R1 and R2 in registers; the two
// independent chains are interleaved and each d-step's LDS operands are read
// one step ahead, so a pair of MFMAs waits on reads issued a pair earlier
// instead of each MFMA on its own read.
__device__ inline void mma_rows2c(uint32_t x1, const bf16x8 (&r1)[8], f32x16& acc1, const f32x16& c1, uint32_t x2,
                                  const bf16x8 (&r2)[8], f32x16& acc2, const f32x16& c2) {
  bf16x8 a1 = lds_read16(x1), a2 = lds_read16(x2);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    bf16x8 n1 = a1, n2 = a2;
    if (ks < 7) {
      n1 = lds_read16(x1 + (ks + 1) * 32);
      n2 = lds_read16(x2 + (ks + 1) * 32);
    }
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, r1[ks], ks == 0 ? c1 : acc1, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, r2[ks], ks == 0 ? c2 : acc2, 0, 0, 0);
    a1 = n1;
    a2 = n2;
  }
}

// acc = c + X[rows][d] R[d][cols], one chain, each d-step's LDS operand read one step ahead.
__device__ inline void mma_rows1c(uint32_t x, const bf16x8 (&r)[8], f32x16& acc, const f32x16& c) {
  bf16x8 a = lds_read16(x);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    bf16x8 n = a;
    if (ks < 7) n = lds_read16(x + (ks + 1) * 32);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, r[ks], ks == 0 ? c : acc, 0, 0, 0);
    a = n;
  }
}

__device__ inline void pack16(const float (&x)[16], bf16x8 (&out)[2]) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack2(x[half * 8 + 2 * i], x[half * 8 + 2 * i + 1]);
    out[half] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
  }
}

// Write a transposed accumulator (lane = one row of the result, d across
// (j / 4) * 8 + hl * 4 + j % 4 of each 32-wide d block) as fp32, scaled and,
// when asked, rotated back at position pos.
template <bool HALF>
__device__ inline void store_grad(float* dst, f32x16 (&acc)[4], float scale, bool rotate, const float2* tab,
                                  long long pos, int hl) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] *= scale;
  if (rotate) {
    if (HALF) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int d = db * 32 + (j >> 2) * 8 + hl * 4 + (j & 3);      // pairs (d, d + 64)
          float g0 = acc[db][j], g1 = acc[db + 2][j];
          rotate_back(g0, g1, tab[pos * (kD / 2) + d]);
          acc[db][j] = g0;
          acc[db + 2][j] = g1;
        }
    } else {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          const int d = db * 32 + (j >> 2) * 8 + hl * 4 + (j & 3);      // pairs (d, d + 1), d even
          float g0 = acc[db][j], g1 = acc[db][j + 1];
          rotate_back(g0, g1, tab[pos * (kD / 2) + d / 2]);
          acc[db][j] = g0;
          acc[db][j + 1] = g1;
        }
    }
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<float4*>(dst + db * 32 + g4 * 8 + hl * 4) =
          make_float4(acc[db][g4 * 4], acc[db][g4 * 4 + 1], acc[db][g4 * 4 + 2], acc[db][g4 * 4 + 3]);
}

constexpr int kKVKeys = 128;    // keys per dk/dv workgroup

// ---- dk / dv with two roles: a workgroup of 8 waves owns 128 keys of one KV
// head, four groups of 32.  Waves 0-3 ("P waves") hold k~ of their group and
// accumulate dV; waves 4-7 ("dS waves") hold v of the same group and
// accumulate dK.  The q~ tiles come from the entry point's copy of q, rotated
// and multiplied by sm_scale log2(e) with the one rounding the forward kernel
// applies, so S is the forward's score in log2 units and P = exp2(S - lse
// log2(e)) is the very softmax the forward normalised; dK~ = sm_scale dS^T q~
// then takes the factor ln 2.  Query tile i (32 rows of one head, staged in
// LDS, four buffers) goes through
//   P wave,  step i:   S(i+1) = q~ k~^T - lse next to P(i) = exp2(S(i)) (masked),
//                      P(i) to LDS, dV^T += dO(i)^T P(i)
//   dS wave, step i:   dP(i) = dO V^T - delta next to dS(i-1) = P(i-1) dP(i-1)
//                      (P read back from LDS), dK~^T += q~(i-1)^T dS(i-1)
// so every wave issues 16 MFMAs a step and two waves share each SIMD.
constexpr int kKV2Waves = 8;
constexpr int kKV2Threads = 64 * kKV2Waves;

struct Dkdv2Smem {
  alignas(16) __hip_bfloat16 q[4][32 * kTStr];
  alignas(16) __hip_bfloat16 o[4][32 * kTStr];
  alignas(16) float4 p[2][4][4][64];      // [step parity][key group][chunk of 4 floats][lane]
  alignas(16) float ld[4][64];            // [buffer][-lse log2(e) of the 32 rows, then -delta]
};


// EXACT_Q: q enters unrotated and unscaled (no SRT_ROTATE_Q), exactly as the
// forward kernel then uses it; the S accumulator starts at -lse / sm_scale
// and its product times sm_scale log2(e) is the forward's S - lse in log2
// units (one multiply per score instead of a rounding of q * sm_scale log2(e)).
template <bool HALF, bool WIN, bool EXACT_Q>
__global__ void __launch_bounds__(kKV2Threads) bwd_dkdv2_bf16_kernel(BwdArgs a) {
  __shared__ Dkdv2Smem sm;
  __shared__ int s_item;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave & 3, role = wave >> 2;
  const int l32 = lane & 31, hl = lane >> 5;
  // item (key block y, batch b, KV head x), x fastest, key blocks from the first (heavy first)
  int item = a.item0 + (int)blockIdx.x;
  if (a.sched) {
    if (tid == 0) s_item = sched_take(a.sched, a.Hkv, a.B, (a.Nk + kKVKeys - 1) / kKVKeys);
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(s_item);
  }
  const int hk = item % a.Hkv;
  const int kblk = item / a.Hkv / a.B;
  const int b = item / a.Hkv - kblk * a.B;
  const int G = a.Hq / a.Hkv;
  const int wk0 = kblk * kKVKeys + grp * 32;
  const int key = wk0 + l32;
  const bool key_ok = key < a.Nk;
  const long long kpos = a.k_pos0 + key;
  const float4* tab4 = reinterpret_cast<const float4*>(a.table);
  const float2* tab2 = reinterpret_cast<const float2*>(a.table);
  const float cq = a.sm_scale * kLog2e;   // (EXACT_Q)

  // query rows [r_lo, r_hi) that can see some key of this workgroup
  const int wg_k0 = kblk * kKVKeys;
  const long long kp_first = a.k_pos0 + wg_k0;
  const long long kp_last = a.k_pos0 + min(a.Nk, wg_k0 + kKVKeys) - 1;
  long long r_lo = 0, r_hi = a.Nq;
  if (a.causal) r_lo = max(0LL, min((long long)a.Nq, kp_first - a.q_pos0));
  if (WIN && kp_first >= a.sink) r_hi = max(0LL, min((long long)a.Nq, kp_last + a.window - a.q_pos0));
  const int t0 = (int)(r_lo / 32);
  const int ntq = r_hi > r_lo ? (int)((r_hi + 31) / 32) - t0 : 0;
  const int nit = G * ntq;

  // staging: thread t moves 16-byte chunk t & 15 of row t >> 4 of a q~ and a
  // dO tile through buffer descriptors whose range ends at Nq; threads 0..31
  // move lse and delta (negated, so they can start the accumulators)
  const __hip_bfloat16* qsrc = reinterpret_cast<const __hip_bfloat16*>(a.q_rot);
  const __hip_bfloat16* dog = reinterpret_cast<const __hip_bfloat16*>(a.dout);
  const int sc = tid & 15, sr = tid >> 4;
  const uint32_t soff = sr * (kD * 2) + sc * 16;
  uint4 qb, ob;
  // wave 0: lse (lanes r < 32) and delta (lanes 32 + r) of row r, raw; store()
  // writes -lse log2(e) and -delta a step later, when the loads have landed
  float lse_raw = 0.f, delta_raw = 0.f;
  // next tile to load: head ig of the group, row tile itq, first row hrow (all wave-uniform)
  int ig = 0, itq = t0;
  long long hrow = ((long long)b * a.Hq + hk * G) * a.Nq + (long long)t0 * 32;
  auto issue = [&]() {
    const int rows = ig < G ? min(32, max(0, a.Nq - itq * 32)) : 0;
    qb = buffer_ld16(raw_buffer(qsrc + hrow * kD, rows * (kD * 2)), soff);
    ob = buffer_ld16(raw_buffer(dog + hrow * kD, rows * (kD * 2)), soff);
    if (wave == 0) {
      // one descriptor per array (a per-lane choice of base would make the
      // descriptor divergent: a waterfall loop and a wait for the data here)
      lse_raw = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(raw_buffer(a.lse + hrow, rows * 4), l32 * 4, 0, 0));
      delta_raw = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(raw_buffer(a.delta + hrow, rows * 4), l32 * 4, 0, 0));
    }
    hrow += 32;
    if (++itq == t0 + ntq) {
      itq = t0;
      ++ig;
      hrow += a.Nq - ntq * 32;
    }
  };
  auto store = [&](int buf) {
    *reinterpret_cast<uint4*>(&sm.q[buf][prow(sr) * kTStr + sc * 8]) = qb;
    *reinterpret_cast<uint4*>(&sm.o[buf][prow(sr) * kTStr + sc * 8]) = ob;
    if (wave == 0) sm.ld[buf][lane] = lane < 32 ? lse_raw * (EXACT_Q ? -1.0f / a.sm_scale : -kLog2e) : -delta_raw;
  };
  auto init_rows = [&](const float* src) {     // the 16 accumulator rows (queries) of this lane
    f32x16 c;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 x = *reinterpret_cast<const float4*>(&src[g4 * 8 + hl * 4]);
      c[g4 * 4 + 0] = x.x; c[g4 * 4 + 1] = x.y; c[g4 * 4 + 2] = x.z; c[g4 * 4 + 3] = x.w;
    }
    return c;
  };

  const int gj = lane & 15;
  const int gd = ((lane >> 4) & 1) * 16 + 4 * (gj & 3);
  const int tr_off = prow(hl * 4 + (gj >> 2)) * kTStr + gd;
  bf16x8 breg[8];            // P waves: k~ (scaled); dS waves: v
  f32x16 acc[4];             // P waves: dV^T; dS waves: dK~^T
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;
  if (role == 0) {
    const __hip_bfloat16* kg = reinterpret_cast<const __hip_bfloat16*>(a.k) + ((long long)b * a.Hkv + hk) * a.Nk * kD;
    load_row_rotated<HALF>(kg + (long long)key * kD, key_ok, (a.rope_flags & 2) != 0, tab4, kpos, hl, breg);
  } else {
    const __hip_bfloat16* vg = reinterpret_cast<const __hip_bfloat16*>(a.v) + ((long long)b * a.Hkv + hk) * a.Nk * kD;
    load_row_rotated<HALF>(vg + (long long)key * kD, key_ok, false, tab4, 0, hl, breg);
  }

  if (nit > 0) {
    issue();
    store(0);
    issue();
    store(1);
    issue();
    __syncthreads();
    // Step i uses LDS buffers (i + 2) % 4 (staging), (i + 1) % 4, i % 4 and
    // (i - 1) % 4 and P slot i % 2: four steps per trip keep them compile-time
    // constants and let S / dP alternate between two register sets.
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    if (role == 0) {
      // the wave's keys are all visible to every row of row tile t iff tm_lo <= t <= tm_hi
      const long long kw_first = a.k_pos0 + wk0, kw_last = kw_first + 31;
      const bool is_sink = kpos < a.sink;
      auto cdiv = [](long long x, long long y) { return x >= 0 ? (x + y - 1) / y : -((-x) / y); };
      long long tlo = a.causal ? cdiv(kw_last - a.q_pos0, 32) : 0, thi = a.Nq / 32 - 1;
      if (WIN && kw_last >= a.sink) thi = min(thi, cdiv(a.window - 31 + kw_first - a.q_pos0, 32) - 1);
      const int tm_lo = (int)max((long long)INT_MIN, min((long long)INT_MAX, tlo));
      const int tm_hi = (int)max((long long)INT_MIN, min((long long)INT_MAX, thi));
      f32x16 s_a, s_b;
      mma_rows1c(lds_off(&sm.q[0][prow(l32) * kTStr + hl * 8]), breg, s_a, init_rows(&sm.ld[0][0]));
      int ct = t0;
      // step i = R (mod 4) on tile i: S(i+1) into s_out next to P(i) from s_in
      auto pstep = [&](auto rc, const f32x16& s_in, f32x16& s_out) {
        constexpr int R = decltype(rc)::value;
        constexpr int nb = (R + 1) & 3;
        store((R + 2) & 3);
        issue();
        mma_rows1c(lds_off(&sm.q[nb][prow(l32) * kTStr + hl * 8]), breg, s_out, init_rows(&sm.ld[nb][0]));   // stale past the end
        float p[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) p[j] = __builtin_amdgcn_exp2f(EXACT_Q ? s_in[j] * cq : s_in[j]);
        if (ct < tm_lo || ct > tm_hi) {
          const int qt0 = ct * 32;
          const long long relb = a.q_pos0 + qt0 - kpos;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int row = (j >> 2) * 8 + hl * 4 + (j & 3);
            const long long rel = relb + row;
            const bool vis = (qt0 + row < a.Nq) && (!a.causal || (rel >= 0 && (!WIN || rel < a.window || is_sink)));
            p[j] = vis ? p[j] : 0.f;
          }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
          sm.p[R & 1][grp][c][lane] = make_float4(p[4 * c], p[4 * c + 1], p[4 * c + 2], p[4 * c + 3]);
        bf16x8 pb[2];
        pack16(p, pb);
        // dV^T += dO^T P (transposing reads of the row-major dO tile)
        mma_tr(acc, lds_off(&sm.o[R][tr_off]), pb);
        if (++ct == t0 + ntq) ct = t0;
        __syncthreads();
      };
      int i = 0;
      for (; i + 4 <= nit; i += 4) {
        pstep(C0{}, s_a, s_b);
        pstep(C1{}, s_b, s_a);
        pstep(C2{}, s_a, s_b);
        pstep(C3{}, s_b, s_a);
      }
      if (i < nit) pstep(C0{}, s_a, s_b), ++i;
      if (i < nit) pstep(C1{}, s_b, s_a), ++i;
      if (i < nit) pstep(C2{}, s_a, s_b), ++i;
      // step nit: the dS waves' last step; only the staging and the barrier
      store((nit + 2) & 3);
      issue();
      __syncthreads();
    } else {
      f32x16 dp_a, dp_b;
      // step i = R (mod 4): dP(i) into dp_out (when i < nit) next to dS(i-1) from dp_in
      auto dstep = [&](auto rc, const f32x16& dp_in, f32x16& dp_out, bool dp_active) {
        constexpr int R = decltype(rc)::value;
        store((R + 2) & 3);
        issue();
        // (the loads stay here, a step ahead of the store that consumes them:
        // left alone the scheduler sinks them to the end of the step)
        __builtin_amdgcn_sched_barrier(0);
        if (dp_active) mma_rows1c(lds_off(&sm.o[R][prow(l32) * kTStr + hl * 8]), breg, dp_out, init_rows(&sm.ld[R][32]));
        float ds[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float4 pv = sm.p[(R + 1) & 1][grp][c][lane];
          ds[4 * c] = pv.x * dp_in[4 * c];
          ds[4 * c + 1] = pv.y * dp_in[4 * c + 1];
          ds[4 * c + 2] = pv.z * dp_in[4 * c + 2];
          ds[4 * c + 3] = pv.w * dp_in[4 * c + 3];
        }
        bf16x8 dsb[2];
        pack16(ds, dsb);
        // dK~^T += q~^T dS (transposing reads of the row-major q~ tile)
        mma_tr(acc, lds_off(&sm.q[(R + 3) & 3][tr_off]), dsb);
        __syncthreads();
      };
      // step 0: dP(0) only
      store(2);
      issue();
      mma_rows1c(lds_off(&sm.o[0][prow(l32) * kTStr + hl * 8]), breg, dp_a, init_rows(&sm.ld[0][32]));
      __syncthreads();
      int i = 1;
      for (; i + 3 < nit; i += 4) {
        dstep(C1{}, dp_a, dp_b, true);
        dstep(C2{}, dp_b, dp_a, true);
        dstep(C3{}, dp_a, dp_b, true);
        dstep(C0{}, dp_b, dp_a, true);
      }
      // steps i .. nit (at most four; the last one has no new dP)
      if (i <= nit) dstep(C1{}, dp_a, dp_b, i < nit), ++i;
      if (i <= nit) dstep(C2{}, dp_b, dp_a, i < nit), ++i;
      if (i <= nit) dstep(C3{}, dp_a, dp_b, i < nit), ++i;
      if (i <= nit) dstep(C0{}, dp_b, dp_a, i < nit), ++i;
    }
  }
  if (a.sched && tid == 0) sched_release(a.sched, gridDim.x);
  if (!key_ok) return;
  const long long krow = ((long long)b * a.Hkv + hk) * a.Nk + key;
  // dK~ = sm_scale dS^T q: with q~ carrying sm_scale log2(e) the factor is ln 2
  if (role == 0) store_grad<HALF>(a.dv + krow * kD, acc, 1.f, false, tab2, kpos, hl);
  else store_grad<HALF>(a.dk + krow * kD, acc, EXACT_Q ? a.sm_scale : kLn2, (a.rope_flags & 2) != 0, tab2, kpos, hl);
}

// ---- dq: a workgroup of 8 waves owns one KV head and 32 * (8 / HPW) query
// rows of HPW = min(G, 4) query heads (as the forward kernel); wave w holds
// rotated q (pre-multiplied by sm_scale log2(e), as in the forward) and dO of
// its 32 rows in registers and walks 32-key tiles of rotated k and v staged in
// LDS.  The S^T accumulator starts at -lse log2(e) and the dP^T accumulator at
// -delta, so P = exp2(S^T) and dS = P (dP - delta) = P dP^T.
constexpr int kQWaves = 8;
constexpr int kQThreads = 64 * kQWaves;

struct DqSmem {
  alignas(16) __hip_bfloat16 k[2][32 * kTStr];
  alignas(16) __hip_bfloat16 v[2][32 * kRStr];
};

template <bool HALF, bool WIN, bool EXACT_Q>
__global__ void __launch_bounds__(kQThreads, 1) bwd_dq_bf16_kernel(BwdArgs a) {
  __shared__ DqSmem sm;
  __shared__ int s_item;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int G = a.Hq / a.Hkv;
  const int HPW = G < 4 ? G : 4;
  const int RB = kQWaves / HPW;
  const int quads = G > 4 ? G / 4 : 1;
  const int HX = a.Hkv * quads;
  const int ntq = (a.Nq + 32 * RB - 1) / (32 * RB);
  // item (query-tile rank y, batch b, workgroup head x), x fastest, y = 0 the last query tile
  int item = a.item0 + (int)blockIdx.x;
  if (a.sched) {
    if (tid == 0) s_item = sched_take(a.sched, HX, a.B, ntq);
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(s_item);
  }
  const int xh = item % HX, yq = item / HX / a.B;
  const int b = item / HX - yq * a.B;
  const int hk = xh / quads, quad = xh - hk * quads;
  const int qt = a.causal ? (ntq - 1 - yq) : yq;
  const int hq = hk * G + quad * 4 + (wave % HPW);
  const int wrow0 = qt * (32 * RB) + (wave / HPW) * 32;
  const int wg_row_last = min(a.Nq, (qt + 1) * 32 * RB) - 1;
  const int row = wrow0 + l32;
  const bool row_ok = row < a.Nq;
  const long long qpos = a.q_pos0 + row;
  const float4* tab4 = reinterpret_cast<const float4*>(a.table);
  const float2* tab2 = reinterpret_cast<const float2*>(a.table);
  const long long qrow = ((long long)b * a.Hq + hq) * a.Nq + row;
  const __hip_bfloat16* kg = reinterpret_cast<const __hip_bfloat16*>(a.k) + ((long long)b * a.Hkv + hk) * a.Nk * kD;
  const __hip_bfloat16* vg = reinterpret_cast<const __hip_bfloat16*>(a.v) + ((long long)b * a.Hkv + hk) * a.Nk * kD;

  const float c2 = a.sm_scale * kLog2e;
  bf16x8 qreg[8], doreg[8];
  load_row_rotated<HALF>(reinterpret_cast<const __hip_bfloat16*>(a.q) + qrow * kD, row_ok, (a.rope_flags & 1) != 0,
                         tab4, qpos, hl, qreg, EXACT_Q ? 1.f : c2);
  load_row_rotated<HALF>(reinterpret_cast<const __hip_bfloat16*>(a.dout) + qrow * kD, row_ok, false, tab4, 0, hl,
                         doreg);
  // Rows past Nq have q = dO = 0, so S^T = dP^T = 0 and dS = 0.  A row with no
  // visible key (lse = -inf) only meets masked halves, where P is forced to 0.
  const float lse2 = row_ok ? a.lse[qrow] * kLog2e : 0.f;
  const float dl = row_ok ? a.delta[qrow] : 0.f;
  f32x16 negl, negd, dqacc[4];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    negl[j] = EXACT_Q ? -lse2 / c2 : -lse2;   // (EXACT_Q: the scores are multiplied by c2 after the product)
    negd[j] = -dl;
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) dqacc[db][j] = 0.f;

  // key tiles of 32: [0, sink tiles) then from the first row's window start to the causal end
  int kend = a.Nk;
  if (a.causal) kend = (int)max(0LL, min((long long)a.Nk, a.q_pos0 + wg_row_last - a.k_pos0 + 1));
  int nsk = 0, shift = 0, ntiles = (kend + 31) / 32, csink = 0;
  long long wave_lo_lim = -(1LL << 40);
  if (WIN) {
    const long long lo = a.q_pos0 + (long long)qt * (32 * RB) - a.window + 1 - a.k_pos0;
    csink = (int)min((long long)kend, max(0LL, (long long)a.sink - a.k_pos0));
    nsk = (csink + 31) / 32;
    const int tstart = lo >= kend ? ntiles : max(nsk, (int)(max(0LL, lo) / 32));
    shift = tstart - nsk;
    ntiles = nsk + max(0, ntiles - tstart);
    wave_lo_lim = a.q_pos0 + wrow0 + 31 - a.window + 1 - a.k_pos0;
  }
  auto tile_key0 = [&](int t) { return WIN ? (t < nsk ? t : t + shift) * 32 : t * 32; };
  // a 32-key tile at key0 needs the per-score mask iff key0 > mask_hi (past the
  // diagonal of the wave's first row, or past Nk) or, with a window, it starts
  // before some row's window while reaching past the sinks
  const long long wave_free_lim = a.causal ? (a.q_pos0 + wrow0 - a.k_pos0 + 1) : (long long)a.Nk;
  const int mask_hi = (int)max((long long)INT_MIN, min(wave_free_lim, (long long)a.Nk) - 32);
  const int mask_lo = (int)max((long long)INT_MIN, min((long long)INT_MAX, wave_lo_lim));
  int klim, klo;
  {
    long long lim = a.causal ? (qpos - a.k_pos0) : (long long)a.Nk - 1;
    lim = lim < (long long)a.Nk - 1 ? lim : (long long)a.Nk - 1;
    klim = (int)(lim < -1 ? -1 : lim);
    long long lo = WIN ? qpos - a.window + 1 - a.k_pos0 : -(1LL << 30);
    lo = lo < -(1LL << 30) ? -(1LL << 30) : lo;
    klo = (int)(lo > (1LL << 30) ? (1LL << 30) : lo);
  }

  // staging: thread t moves 16-byte chunk t & 15 of row t >> 4 of a k and a v
  // tile (16 threads per 256-byte row; with fewer than 512 threads also rows
  // (t >> 4) + kQThreads / 16, ...), through buffer descriptors whose range
  // ends at Nk (rows past it read as zero)
  const __hip_bfloat16* ksrc =
      a.k_rot ? reinterpret_cast<const __hip_bfloat16*>(a.k_rot) + ((long long)b * a.Hkv + hk) * a.Nk * kD : kg;
  const int sc = tid & 15, sr = tid >> 4;
  const uint32_t soff = sr * (kD * 2) + sc * 16;
  constexpr int kStg = 32 / (kQThreads / 16);     // rows per thread of a 32-row tile
  uint4 kb[kStg], vb[kStg];
  auto issue = [&](int key0) {
    const int bytes = min(32, max(0, a.Nk - key0)) * (kD * 2);
    const __amdgpu_buffer_rsrc_t rk = raw_buffer(ksrc + (long long)key0 * kD, bytes);
    const __amdgpu_buffer_rsrc_t rv = raw_buffer(vg + (long long)key0 * kD, bytes);
#pragma unroll
    for (int i = 0; i < kStg; ++i) {
      kb[i] = buffer_ld16(rk, soff + i * (kQThreads / 16) * (kD * 2));
      vb[i] = buffer_ld16(rv, soff + i * (kQThreads / 16) * (kD * 2));
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kStg; ++i) {
      *reinterpret_cast<uint4*>(&sm.k[buf][prow(sr + (kQThreads / 16) * i) * kTStr + sc * 8]) = kb[i];
      *reinterpret_cast<uint4*>(&sm.v[buf][(sr + (kQThreads / 16) * i) * kRStr + sc * 8]) = vb[i];
    }
  };
  const int gj = lane & 15;
  const int gd = ((lane >> 4) & 1) * 16 + 4 * (gj & 3);
  const uint32_t k_row = lds_off(&sm.k[0][prow(l32) * kTStr + hl * 8]);
  const uint32_t v_row = lds_off(&sm.v[0][l32 * kRStr + hl * 8]);
  const uint32_t k_tr = lds_off(&sm.k[0][prow(hl * 4 + (gj >> 2)) * kTStr + gd]);
  constexpr uint32_t kKBuf = 32 * kTStr * 2, kVBuf = 32 * kRStr * 2;

  // One 32-key tile in LDS buffer BUF (a compile-time constant: the loop takes
  // two tiles per trip).  The loads of the next tile were issued a tile
  // earlier; they go to the other buffer, which every wave left at the barrier
  // closing the previous tile.  Past the last tile the loads and stores only
  // touch the unused buffer.
  auto tile = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    const int key0 = tile_key0(t);
    issue(tile_key0(t + 1));
    // S^T = k~ q~^T - lse and dP^T = V dO^T - delta: lane = query, rows = 16 of the tile's keys
    f32x16 s, dp;
    mma_rows2c(k_row + BUF * kKBuf, qreg, s, negl, v_row + BUF * kVBuf, doreg, dp, negd);
    if constexpr (EXACT_Q) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] *= c2;
    }
    if (key0 > mask_hi || (WIN && key0 < mask_lo && key0 + 32 > csink)) {
      const int base = key0 + hl * 4;
      const int rel = klim - base, rlo = klo - base, rsk = csink - base;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int cj = (j >> 2) * 8 + (j & 3);
        const bool vis = WIN ? (cj <= rel && (cj >= rlo || cj < rsk)) : cj <= rel;
        s[j] = vis ? s[j] : -INFINITY;
      }
    }
    float ds[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) ds[j] = __builtin_amdgcn_exp2f(s[j]) * dp[j];
    bf16x8 dsb[2];
    pack16(ds, dsb);
    // dq~^T += k~^T dS^T (transposing reads of the row-major k~ tile)
    mma_tr(dqacc, k_tr + BUF * kKBuf, dsb);
    store(BUF ^ 1);
    __syncthreads();
  };
  if (ntiles > 0) {
    issue(tile_key0(0));
    store(0);
    __syncthreads();
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
      tile(B0{}, t);
      tile(B1{}, t + 1);
    }
    if (t < ntiles) tile(B0{}, t);
  }
  if (a.sched && tid == 0) sched_release(a.sched, gridDim.x);
  if (!row_ok) return;
  store_grad<HALF>(a.dq + qrow * kD, dqacc, a.sm_scale, (a.rope_flags & 1) != 0, tab2, qpos, hl);
}

__global__ void __launch_bounds__(256) fill_zero_kernel(float* p, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// grid of a grid-stride loop: enough waves to fill the chip, capped
inline unsigned grid_for(long long work, int block) {
  long long g = (work + block - 1) / block;
  const long long cap = 256LL * 64;
  return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

// grid with one thread per work item (no stride loop)
inline unsigned grid_exact(long long work, int block) {
  long long g = (work + block - 1) / block;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Hq * a.Nq;
  const long long work = rows * (a.D / 8);
  if (rows == 0) {                     // no query: dk = dv = 0 (a fill kernel, safe under graph capture)
    const long long n = (long long)a.B * a.Hkv * a.Nk * a.D;
    if (n > 0) {
      hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream, a.dk, n);
      hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream, a.dv, n);
    }
    return hipGetLastError();
  }
  if (a.bf16)
    hipLaunchKernelGGL(bwd_delta_kernel<true>, dim3(grid_exact(work, 256)), dim3(256), 0, stream, a.out, a.dout,
                       a.delta, rows, a.D);
  else
    hipLaunchKernelGGL(bwd_delta_kernel<false>, dim3(grid_exact(work, 256)), dim3(256), 0, stream, a.out, a.dout,
                       a.delta, rows, a.D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool half = (a.rope_flags & 4) != 0;
  if (a.bf16) {
    if (a.D != kD) return hipErrorInvalidValue;
    const int G = a.Hq / a.Hkv;
    if (!(G == 1 || G == 2 || G % 4 == 0)) return hipErrorInvalidValue;
    // run-time assignment (two scheduling blocks: dk/dv, then dq) when a
    // kernel runs more than two rounds of workgroups
    BwdArgs akv = a, aq = a;
    akv.sched = aq.sched = nullptr;
    akv.item0 = aq.item0 = 0;
    const long long nkv = (long long)a.Hkv * ((a.Nk + kKVKeys - 1) / kKVKeys) * a.B;
    const int HPW = G < 4 ? G : 4;
    const int rows_per_wg = 32 * (kQWaves / HPW);
    const int quads = G > 4 ? G / 4 : 1;
    const long long nq = (long long)a.Hkv * quads * ((a.Nq + rows_per_wg - 1) / rows_per_wg) * a.B;
    if (nkv > 0x7fffffffLL || nq > 0x7fffffffLL) return hipErrorInvalidValue;
    const bool win = a.causal && a.window > 0;
    if (a.sched) {
      e = launch_zero_words(a.sched, 2 * kSchedBlockWords, stream);
      if (e != hipSuccess) return e;
      if (nkv > 2LL * compute_units() && nkv <= kMaxLaunchItems) akv.sched = a.sched;
    }
    // a grid too large for one launch goes in launches of kMaxLaunchItems items (fixed assignment)
    auto launch_items = [&](auto kernel, BwdArgs& args, long long n_items, int threads) {
      for (long long base = 0; base < n_items; base += kMaxLaunchItems) {
        args.item0 = (int)base;
        const long long n = n_items - base < kMaxLaunchItems ? n_items - base : kMaxLaunchItems;
        hipLaunchKernelGGL(kernel, dim3((unsigned)n), dim3(threads), 0, stream, args);
      }
    };
    // q used exactly as given (no rotation of q, a non-zero scale): see EXACT_Q
    const bool exact = !(a.rope_flags & 1) && a.sm_scale != 0.f;
    auto kv_kernel = [&](auto h, auto w, auto x) {
      launch_items(bwd_dkdv2_bf16_kernel<decltype(h)::value, decltype(w)::value, decltype(x)::value>, akv, nkv,
                   kKV2Threads);
    };
    auto q_kernel = [&](auto h, auto w, auto x) {
      launch_items(bwd_dq_bf16_kernel<decltype(h)::value, decltype(w)::value, decltype(x)::value>, aq, nq,
                   kQThreads);
    };
    using T = std::true_type;
    using F = std::false_type;
    auto pick = [&](auto launch) {
      if (win) {
        if (half) { if (exact) launch(T{}, T{}, T{}); else launch(T{}, T{}, F{}); }
        else { if (exact) launch(F{}, T{}, T{}); else launch(F{}, T{}, F{}); }
      } else {
        if (half) { if (exact) launch(T{}, F{}, T{}); else launch(T{}, F{}, F{}); }
        else { if (exact) launch(F{}, F{}, T{}); else launch(F{}, F{}, F{}); }
      }
    };
    if (a.Nk > 0) {
      pick(kv_kernel);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (a.sched && nq > 2LL * compute_units() && nq <= kMaxLaunchItems)
      aq.sched = a.sched + kSchedBlockWords;
    pick(q_kernel);
    return hipGetLastError();
  }
  if (a.D != 64) return hipErrorInvalidValue;
  if (a.Nk > 0) {
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<64>, dim3((a.Nk + 63) / 64, a.Hkv, a.B), dim3(64), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, dim3((a.Nq + 63) / 64, a.Hq, a.B), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace srt
