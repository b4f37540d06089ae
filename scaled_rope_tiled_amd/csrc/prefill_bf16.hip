// bf16 tiled online-softmax attention, D = 128, on the gfx950 matrix cores.
//
// What it computes is FlashAttention's exact tiled softmax ("8.3 长上下文技术"
// §8.3.4: tiles of Q, K, V in on-chip memory, per-block max and exp-sum, the
// earlier accumulator rescaled; the N x N matrix never exists), with RoPE
// applied to q and k as they are loaded ("Long Context: RoPE / YaRN / NTK /
// MLA" §2.4 rope_attention; the YaRN temperature travels in the table, §6.4).
//
// Work decomposition (one workgroup = 8 waves = 512 threads, two per SIMD)
//   * A workgroup owns one KV head and 32 * (8 / HPW) query rows of HPW query
//     heads of its GQA group (HPW = min(Hq/Hkv, 4)): every K/V tile staged in
//     LDS serves all eight waves, i.e. up to four query heads.
//   * Wave w owns 32 query rows of one head and keeps them in registers:
//     rotated q as the B operand of S^T = K Q^T, the output as O^T (fp32).
//   * Items (workgroup head, batch, query tile) are numbered with the head
//     fastest and the query tiles from the last (most keys under the causal
//     mask) to the first, so the long tiles start first; consecutive
//     workgroups, which the dispatcher spreads round-robin over the 8 XCDs,
//     keep one head per XCD L2.  With a scheduling block the items are handed
//     out at run time instead (see sched_take), which evens out XCDs that run
//     at different speeds.
//   * Key tiles wholly above the causal diagonal, or wholly before the sliding
//     window of the workgroup's rows (sinks aside: "Long Context..." §10.1-10.2),
//     are never visited; only the 32-key halves that cross the diagonal, the
//     window's edge or the ragged end of K evaluate the mask (integer
//     compares per score).
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, wave64)
//   S^T[keys][queries] = K[keys][d] Q^T[d][queries]: A = 32x16 block of K read
//   from LDS (16 bytes per lane), B = Q^T from registers; the accumulator puts
//   one query per lane (lane & 31) with 16 of its keys, so the row max and row
//   sum of the softmax are in-lane, plus one v_permlane32_swap with lane ^ 32.
//   O^T[d][queries] = V^T[d][keys] P^T[keys][queries]: B = P^T comes straight
//   from the S^T accumulator (converted to bf16) because the contraction over
//   keys may use any key order as long as A uses the same one; A = V^T is read
//   from the row-major V tile with the gfx950 transposing LDS read
//   ds_read_b64_tr_b16, four consecutive keys of one d column per read.
//   The O^T accumulator again holds one query per lane, so the online-softmax
//   rescale is a per-lane multiply.  The reference m of the exponentials is
//   folded into the QK product: rotated q~ is stored pre-scaled by sm_scale
//   log2(e) and the accumulator starts at -m, so the scores arrive as
//   s sm_scale log2(e) - m and each probability is one exp2 (q that is not
//   rotated stays exact: its accumulator starts at -m / (sm_scale log2(e))
//   and one fp32 multiply per score gives the same value).  A half's
//   exponentials are taken against the current m at once (no row maximum on
//   the common path); m moves, in a rare branch, to the half's maximum only
//   when a lane's sum over the half exceeds a bound or the lane has no
//   reference yet.  The result is exact for any reference; the bound keeps
//   every term below it, far from bf16/fp32 overflow.
//
// Pipeline: the key range is walked in 32-key halves.  Step h issues PV of
// half h-1 and then QK of half h+1 (matrix work) next to the softmax of half
// h (VALU work that depends on neither), as one basic block, so a wave's
// exponentials overlap its own MFMAs as well as the other wave's on the SIMD.
//
// Staging: each thread moves two 16-byte chunks of K and of V per 64-key tile
// (16 threads per 256-byte row: fully coalesced) with buffer loads whose
// descriptor range ends at Nk, rotating K in fp32 on the way when asked.
// Tiles rotate through three LDS buffers with one barrier per tile (the loop
// takes three tiles per trip so that buffer indices are constants); a tile's
// global loads are in flight during two steps and its LDS stores sit at the
// start of the step before the barrier that publishes it.  Row strides are
// padded (K: 272 B, V: 320 B) so the 16-byte K reads and the transposing V
// reads of a wave hit distinct LDS banks.
#include "mfma_common.h"
#include "item_queue.h"

#include <type_traits>

namespace srt {
namespace {

using namespace mc;

constexpr int kD = 128;
constexpr int kWaves = 8;         // waves per workgroup (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32;           // query rows per wave
constexpr int kBN = 64;           // keys per tile
constexpr int kKStr = kD + 8;     // K tile row stride (bf16 elements) = 272 B
constexpr int kVStr = kD + 32;    // V tile row stride (bf16 elements) = 320 B
constexpr int kOStr = kD + 8;     // epilogue staging row stride (bf16 elements) = 272 B
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSumBound = 4096.0f;   // a lane's exponential sum over a half that moves the reference
constexpr int kStageRows = kBN * 16 / kThreads;   // 16-byte chunks per thread per tile and tensor
constexpr int kBufferWord3 = 0x00020000;          // buffer descriptor word 3 for raw 32-bit loads (gfx9 family)

struct Smem {
  __hip_bfloat16 k[3][kBN * kKStr];
  __hip_bfloat16 v[3][kBN * kVStr];
};
static_assert(kWaves * kBM * kOStr * 2 <= sizeof(Smem), "the epilogue staging fits in the tile buffers");

// ROT_K: rotate K on its way into LDS; HALF: half-split pairs; WIN: sliding
// window and sinks (without it, the window tests fold away); SCALE_S: q is
// not rotated, so it is kept exact (no rounding of q * sm_scale log2(e)) and
// the scores are multiplied by sm_scale log2(e) in fp32 instead.
template <bool ROT_K, bool HALF, bool WIN, bool SCALE_S>
__global__ void __launch_bounds__(kThreads, 1) prefill_bf16_kernel(PrefillArgs a) {
  __shared__ Smem sm;
  __shared__ int s_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.Hq / a.Hkv;
  const int HPW = G < 4 ? G : 4;                 // query heads per workgroup
  const int RB = kWaves / HPW;                   // 32-row blocks per workgroup
  const int quads = G > 4 ? G / 4 : 1;
  const int HX = a.Hkv * quads;                  // workgroup heads
  const int ntiles_q = (a.Nq + kBM * RB - 1) / (kBM * RB);
  int item = a.item0 + (int)blockIdx.x;
  if (a.sched) {
    if (tid == 0) s_item = sched_take(a.sched, HX, a.B, ntiles_q);
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(s_item);
  }
  const int xh = item % HX;
  const int yb = item / HX;
  const int yq = yb / a.B;                       // query-tile rank, 0 = most keys
  const int b = yb - yq * a.B;
  const int hk = xh / quads;
  const int quad = xh - hk * quads;
  const int qt = a.causal ? (ntiles_q - 1 - yq) : yq;
  const int hq = hk * G + quad * 4 + (wave % HPW);
  const int wrow0 = qt * (kBM * RB) + (wave / HPW) * kBM;     // first query row of this wave
  const int wg_row_last = min(a.Nq, (qt + 1) * kBM * RB) - 1;  // last valid row of the workgroup

  const __hip_bfloat16* qg = reinterpret_cast<const __hip_bfloat16*>(a.q) + ((long long)b * a.Hq + hq) * a.q_hstride;
  const __hip_bfloat16* kg = reinterpret_cast<const __hip_bfloat16*>(a.k) + ((long long)b * a.Hkv + hk) * a.kv_hstride;
  const __hip_bfloat16* vg = reinterpret_cast<const __hip_bfloat16*>(a.v) + ((long long)b * a.Hkv + hk) * a.kv_hstride;
  const float4* tab4 = reinterpret_cast<const float4*>(a.table);

  const int l32 = lane & 31;
  const int hl = lane >> 5;                      // lane half: 0 or 1

  // ---- Q^T operand: query wrow0 + l32, d = ks*16 + hl*8 + 0..7, rotated on load
  // With half-split pairs, dims d and d + 64 pair up; chunks ks and ks + 4
  // of the same lane hold exactly those, so the rotation stays in-lane.
  // Rotated q~ is stored pre-multiplied by cscale = sm_scale * log2(e), folded
  // into the rotation's one rounding, so S^T comes out in log2 units and the
  // softmax needs no multiply.  Unrotated q (SCALE_S) stays exact: a separate
  // rounding of q * cscale would shift a score by up to 2^-9 of its size,
  // which at |s| ~ 40 already exceeds the bf16 output bar; the scores are
  // scaled in fp32 instead.
  const float cscale = a.sm_scale * kLog2e;
  const float inv_cscale = cscale != 0.f ? 1.0f / cscale : 0.f;
  auto scale4 = [&](float4 t) { return make_float4(t.x * cscale, t.y * cscale, t.z * cscale, t.w * cscale); };
  // (loaded once the first K/V tile's loads are in flight, so the two
  // round trips to HBM overlap)
  //
  // The wave's 32 q rows and their table rows are read coalesced: load i of
  // lane j takes 16-byte chunk j % 16 of row 4i + j / 16, so each load
  // instruction covers four whole rows (the operand layout would spread one
  // instruction over 32 rows, and those scattered reads of q and the table
  // took about 4 us of a workgroup's start).  A chunk holds 8 dims = 4
  // interleaved pairs, whose 4 table entries are 32 contiguous bytes; with
  // half-split pairs chunk c < 8 pairs with chunk c + 8 of the same row, one
  // lane over (a lane exchange), and both take the 8 entries of pairs 8(c % 8)...
  // The rotated chunks then go through LDS (tile buffers 1 and 2, untouched
  // until the first barrier) into the MFMA operand layout.  Rows past the
  // last one read the last row (in bounds) and are zeroed.
  bf16x8 qreg[8];
  auto load_q = [&]() {
    const int cr = lane >> 4, cc = lane & 15;
    uint4 w[8];
    bool ok[8];
    long long qp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = wrow0 + 4 * i + cr;
      ok[i] = row < a.Nq;
      const int rowc = ok[i] ? row : a.Nq - 1;
      qp[i] = a.q_rope0 + (long long)rowc * a.rope_step;   // RoPE position
      w[i] = *reinterpret_cast<const uint4*>(qg + (long long)rowc * kD + cc * 8);
    }
    if constexpr (!SCALE_S) {
      if constexpr (HALF) {
        // (rows in two groups of four: eight rows of 64-byte table entries
        // at once would hold 128 registers)
        const bool first = cc < 8;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
        float4 t[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4* tp = tab4 + (qp[g * 4 + i] * (kD / 2) + (cc & 7) * 8) / 2;
#pragma unroll
          for (int e = 0; e < 4; ++e) t[i * 4 + e] = tp[e];
        }
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int i = g * 4 + i4;
          // partner chunk (the other half of the same pairs) from lane j ^ 8
          const uint4 o = make_uint4(__shfl_xor(w[i].x, 8), __shfl_xor(w[i].y, 8), __shfl_xor(w[i].z, 8),
                                     __shfl_xor(w[i].w, 8));
          const uint32_t m4[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
          const uint32_t p4[4] = {o.x, o.y, o.z, o.w};
          uint32_t r4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 tt = scale4(t[i4 * 4 + q]);   // pairs 2q, 2q + 1 of the chunk: (c, s, c, s)
            const float m0 = bf_lo(m4[q]), m1 = bf_hi(m4[q]), p0 = bf_lo(p4[q]), p1 = bf_hi(p4[q]);
            // first half: x c - y s; second half: x s + y c (x from the first half, y from the second)
            r4[q] = first ? pack2(m0 * tt.x - p0 * tt.y, m1 * tt.z - p1 * tt.w)
                          : pack2(p0 * tt.y + m0 * tt.x, p1 * tt.w + m1 * tt.z);
          }
          w[i] = make_uint4(r4[0], r4[1], r4[2], r4[3]);
        }
        }
      } else {
        float4 t[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4* tp = tab4 + (qp[i] * (kD / 2) + cc * 4) / 2;
          t[i * 2] = tp[0];
          t[i * 2 + 1] = tp[1];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = rotate_chunk(w[i], scale4(t[i * 2]), scale4(t[i * 2 + 1]));
      }
    }
    typedef __attribute__((address_space(3))) u32x4_t lds_u4q;
    const uint32_t stg = (wave < 4 ? lds_off(&sm.k[1][0]) : lds_off(&sm.v[1][0])) + (wave & 3) * (kBM * kKStr * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 x = ok[i] ? w[i] : make_uint4(0, 0, 0, 0);
      *(lds_u4q*)(uintptr_t)(stg + ((4 * i + cr) * kKStr + cc * 8) * 2) = (u32x4_t){x.x, x.y, x.z, x.w};
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = lds_read16(stg + (l32 * kKStr + ks * 16 + hl * 8) * 2);
  };
  static_assert(4 * kBM * kKStr * 2 <= 2 * kBN * kKStr * 2 && 4 * kBM * kKStr * 2 <= 2 * kBN * kVStr * 2,
                "the q staging of four waves fits in tile buffers 1 and 2 of K, and of V");

  // ---- key range of the workgroup (causal: up to its last query position)
  int kend = a.Nk;
  if (a.causal) {
    const long long lim = a.q_pos0 + wg_row_last - a.k_pos0 + 1;
    kend = (int)max(0LL, min((long long)a.Nk, lim));
  }
  // Sliding window: keys before the window of the workgroup's first row are
  // invisible to all its rows except the sinks (positions < sink).  Tiles run
  // over [0, nsk) and then from the window's first tile; tile t of the walk is
  // key tile t (t < nsk) or t + shift.  Each tile is visited once and the
  // per-key mask is exact, so the two ranges may touch.
  int nsk = 0, shift = 0, ntiles = (kend + kBN - 1) / kBN;
  int csink = 0;                                  // keys c < csink are sinks
  long long wave_lo_lim = -(1LL << 40);           // keys >= this are in every row's window
  if (WIN) {
    const long long lo = a.q_pos0 + (long long)qt * (kBM * RB) - a.window + 1 - a.k_pos0;
    csink = (int)min((long long)kend, max(0LL, (long long)a.sink - a.k_pos0));
    nsk = (csink + kBN - 1) / kBN;
    const int tstart = lo >= kend ? ntiles : max(nsk, (int)(max(0LL, lo) / kBN));
    shift = tstart - nsk;
    ntiles = nsk + max(0, ntiles - tstart);
    wave_lo_lim = a.q_pos0 + wrow0 + (kBM - 1) - a.window + 1 - a.k_pos0;
  }
  auto tile_key0 = [&](int t) { return WIN ? (t < nsk ? t : t + shift) * kBN : t * kBN; };
  // keys of a tile starting at key0 are all visible to every row of this wave iff
  // key0 + kBN <= Nk and k_pos0 + key0 + kBN - 1 <= q_pos0 + wrow0 (and, with a
  // window, the tile lies in every row's window or among the sinks)
  const long long wave_free_lim = a.causal ? (a.q_pos0 + wrow0 - a.k_pos0 + 1) : (long long)a.Nk;
  // The same tests in 32-bit scalar form: a 32-key half starting at key0h
  // evaluates the per-score mask iff key0h > mask_hi (it reaches past the
  // diagonal of the wave's first row or past Nk) or key0h < mask_lo while
  // reaching past the sinks (it starts before some row's window).  The
  // clamps to the int range keep both tests exact for 0 <= key0h < Nk.
  const int mask_hi = (int)max((long long)INT_MIN, min(wave_free_lim, (long long)a.Nk) - 32);
  const int mask_lo = (int)max((long long)INT_MIN, min((long long)INT_MAX, wave_lo_lim));

  // ---- staging assignment: chunk sc (16 bytes = dims 8sc..8sc+7) of rows sr and sr + 32
  const int sc = tid & 15;
  const int sr = tid >> 4;
  uint4 kbuf[kStageRows], vbuf[kStageRows];
  float4 tbuf[kStageRows][2];

  // K/V rows of a tile are read through buffer descriptors whose range ends
  // at the tile's last key below Nk: rows at or past Nk read as zero in
  // hardware, with no clamping, predication or per-tile vector arithmetic
  // (the descriptor is scalar; each thread's byte offset is fixed).
  // K rotated on load with half-split pairs needs chunks c and c + 8 of one
  // row in one thread: then thread t takes chunks (t & 7) and (t & 7) + 8 of
  // row t >> 3 (8 threads per 256-byte row, still coalesced).
  static_assert(kStageRows == 2 && kThreads / 8 == kBN, "half-split K staging covers one row per thread");
  const int hr = tid >> 3, hc = tid & 7;
  const uint32_t voff = sr * (kD * 2) + sc * 16;       // bytes of chunk sc of row sr within a tile
  constexpr uint32_t kRowStep = (kThreads / 16) * kD * 2;
  auto tile_rsrc = [&](const __hip_bfloat16* base, int key0) {
    // (readfirstlane keeps the wave-uniform row count scalar: a vector clamp
    // would make the descriptor divergent)
    const int rows = __builtin_amdgcn_readfirstlane(min(kBN, max(0, a.Nk - key0)));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (long long)key0 * kD), (short)0, rows * kD * 2,
                                             kBufferWord3);
  };
  auto ld16 = [](__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(w.x, w.y, w.z, w.w);
  };
  auto issue_loads = [&](int key0) {
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kg, key0), rv = tile_rsrc(vg, key0);
#pragma unroll
    for (int i = 0; i < kStageRows; ++i) {
      vbuf[i] = ld16(rv, voff + i * kRowStep);
      if (!(ROT_K && HALF)) {
        kbuf[i] = ld16(rk, voff + i * kRowStep);
        if (ROT_K) {
          const int key = key0 + sr + (kThreads / 16) * i;
          const int kc = key < a.Nk ? key : a.Nk - 1;    // rows past Nk are zero: any valid angle
          const float4* t = tab4 + ((a.k_rope0 + kc * a.rope_step) * (kD / 2) + sc * 4) / 2;
          tbuf[i][0] = t[0];
          tbuf[i][1] = t[1];
        }
      }
    }
    if (ROT_K && HALF) {
      const int key = key0 + hr;
      const int kc = key < a.Nk ? key : a.Nk - 1;
#pragma unroll
      for (int i = 0; i < 2; ++i) kbuf[i] = ld16(rk, hr * (kD * 2) + (hc + 8 * i) * 16);
      const float4* t = tab4 + ((a.k_rope0 + kc * a.rope_step) * (kD / 2) + hc * 8) / 2;   // pairs 8hc .. 8hc+7
#pragma unroll
      for (int q = 0; q < 4; ++q) tbuf[q >> 1][q & 1] = t[q];
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kStageRows; ++i) {
      const int r = sr + (kThreads / 16) * i;
      if (!(ROT_K && HALF)) {
        uint4 kw = kbuf[i];
        if (ROT_K) kw = rotate_chunk(kw, tbuf[i][0], tbuf[i][1]);
        *reinterpret_cast<uint4*>(&sm.k[buf][r * kKStr + sc * 8]) = kw;
      }
      *reinterpret_cast<uint4*>(&sm.v[buf][r * kVStr + sc * 8]) = vbuf[i];
    }
    if (ROT_K && HALF) {
      uint4 w1 = kbuf[0], w2 = kbuf[1];
      const float4 tt[4] = {tbuf[0][0], tbuf[0][1], tbuf[1][0], tbuf[1][1]};
      rotate_chunk_pair(w1, w2, tt);
      *reinterpret_cast<uint4*>(&sm.k[buf][hr * kKStr + hc * 8]) = w1;
      *reinterpret_cast<uint4*>(&sm.k[buf][hr * kKStr + (hc + 8) * 8]) = w2;
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
  // Mask as integer compares per score: key index c is visible to this lane's
  // query iff c <= klim (causal: k_pos0 + c <= q_pos0 + wrow0 + l32; and
  // c < Nk) and, with a window, c >= klo (inside the window) or c < csink.
  int klim, klo;
  {
    long long lim = a.causal ? (a.q_pos0 + wrow0 + l32 - a.k_pos0) : (long long)a.Nk - 1;
    lim = lim < (long long)a.Nk - 1 ? lim : (long long)a.Nk - 1;
    klim = (int)(lim < -1 ? -1 : lim);
    long long lo = WIN ? a.q_pos0 + wrow0 + l32 - a.window + 1 - a.k_pos0 : -(1LL << 30);
    lo = lo < -(1LL << 30) ? -(1LL << 30) : lo;
    klo = (int)(lo > (1LL << 30) ? (1LL << 30) : lo);
  }
  // Reference point of this lane's exponentials, in log2 units: scores enter
  // the softmax as s * cscale - m_run because the QK accumulator starts at
  // negm = -m_run.  It starts at 0.  After a half's exponentials are taken,
  // a lane whose sum over the half exceeds kSumBound (some term may be large)
  // or that has no reference yet sends the wave into a rare branch that sets
  // m_run to the half's maximum (when above it, or for the first visible half)
  // and takes the half's exponentials again.  The reference is then the value
  // of a visible score, so the row's sum stays >= 1; every term stays <=
  // kSumBound.  The two lanes of a query see the same pair maximum and take
  // the same decisions.  Rows that see no key at all need no reference.
  float m_run = 0.f;
  bool mset = !(klim >= 0 && (klim >= klo || csink > 0));
  bool all_set = __builtin_amdgcn_ballot_w64(!mset) == 0;    // wave-uniform: every lane has its reference
  float l_run = 0.f;             // this lane's partial sum (its 16 keys of every 32)
  f32x16 negm;
#pragma unroll
  for (int j = 0; j < 16; ++j) negm[j] = 0.f;
  const int gj = lane & 15;
  const int gd = ((lane >> 4) & 1) * 16 + 4 * (gj & 3);    // d offset inside a 32-wide block

  // ---- building blocks on one 32-key half of a K/V tile in LDS.  Buffer
  // index and half are compile-time constants, so every LDS address is a
  // per-lane base plus an immediate offset.
  const uint32_t k_lane = lds_off(&sm.k[0][l32 * kKStr + hl * 8]);
  const uint32_t v_lane = lds_off(&sm.v[0][(hl * 4 + (gj >> 2)) * kVStr + gd]);
  // S^T = K Q^T: 8 d-steps of one 32x32x16 MFMA
  auto qk = [&](auto bufc, auto kb, f32x16& acc) {
    constexpr int KB = decltype(kb)::value;
    uint32_t kl;
    if constexpr (std::is_same_v<decltype(bufc), int>)
      kl = opaque(k_lane + bufc * (kBN * kKStr * 2)) + KB * 32 * kKStr * 2;
    else
      kl = k_lane + decltype(bufc)::value * (kBN * kKStr * 2) + KB * 32 * kKStr * 2;
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read16(kl), qreg[0], negm, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < 8; ++ks) {
      const bf16x8 ka = lds_read16(kl + ks * 32);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], acc, 0, 0, 0);
    }
  };
  // O^T += V^T P^T: 4 d blocks x 2 key steps of 16
  auto pv = [&](const bf16x8 (&pb)[2], int buf, auto kb) {
    constexpr int KB = decltype(kb)::value;
    const uint32_t vl = opaque(v_lane + buf * (kBN * kVStr * 2)) + KB * 32 * kVStr * 2;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const i16x4 lo = lds_read_tr(vl + ((half * 16) * kVStr + db * 32) * 2);
        const i16x4 hi = lds_read_tr(vl + ((half * 16 + 8) * kVStr + db * 32) * 2);
        const bf16x8 va = __builtin_bit_cast(
            bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){lo[0], lo[1], lo[2], lo[3], hi[0],
                                                                               hi[1], hi[2], hi[3]});
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[half], oacc[db], 0, 0, 0);
      }
    }
  };

  f32x16 s_a, s_b;
  bf16x8 p_a[2], p_b[2];
  float alpha_prev = 1.f, d_prev = 0.f;
  bool need_prev = false;

  // exponentials of one half into packed bf16 P^T; returns this lane's fp32
  // sum of the probabilities, in two independent chains of adds (a v_dot2
  // over the packed pairs is one instruction per two terms, but it competes
  // with the matrix cores, adds do not)
  auto exps = [&](const f32x16& sv, bf16x8 (&pout)[2]) {
    float part[2] = {-0.f, -0.f};   // (-0 + x folds to x)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(sv[half * 8 + 2 * i]);
        const float p1 = __builtin_amdgcn_exp2f(sv[half * 8 + 2 * i + 1]);
        w[i] = pack2(p0, p1);
        part[half] += p0 + p1;
      }
      // (an empty asm that reads the packed words keeps the conversions in
      // the step's main block, among its MFMAs: otherwise they sink below the
      // reference-move branch and run after the last MFMA of the step)
      asm volatile("" :: "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]));
      pout[half] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
    }
    return part[0] + part[1];
  };

  // One pipeline step on half h = 2t + kb: scores of half h arrive in s_in,
  // the step computes QK(h+1) into s_out and PV(h-1) from p_in while the
  // softmax of half h writes p_out.  The matrix work does not depend on the
  // softmax, so with no branch in between the scheduler interleaves the wave's
  // MFMAs with its VALU softmax.  A reference moved at the end of step h-1
  // is applied at the start of step h: to O (after PV(h-2), before PV(h-1))
  // and to the scores of half h, whose QK was issued before the move.
  auto step = [&](auto has_pv, auto qbuf, auto qkb, int pbuf, auto pkb, int key0h, f32x16& s_in, f32x16& s_out,
                  const bf16x8 (&p_in)[2], bf16x8 (&p_out)[2]) {
    constexpr bool HAS_PV = decltype(has_pv)::value;
    if constexpr (SCALE_S) {
      // the accumulator held q.k - m_run / cscale: one multiply gives s cscale - m_run
#pragma unroll
      for (int j = 0; j < 16; ++j) s_in[j] *= cscale;
    }
    if (need_prev) {
      if (HAS_PV) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha_prev;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) s_in[j] -= d_prev;
    }
    if (key0h > mask_hi || (WIN && key0h < mask_lo && key0h + 32 > csink)) {
      const int base = key0h + hl * 4;
      const int rel = klim - base, rlo = klo - base, rsk = csink - base;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int cj = (j >> 2) * 8 + (j & 3);
        const bool vis = WIN ? (cj <= rel && (cj >= rlo || cj < rsk)) : cj <= rel;
        s_in[j] = vis ? s_in[j] : -INFINITY;
      }
    }

    // matrix work of this step (the QK of the half after the last one reads a
    // buffer holding stale data; its result is never used).  PV goes first: its
    // operands are ready, so its V reads and MFMAs cover the K reads of QK,
    // whose dependent chain then overlaps this half's softmax.
    if (HAS_PV) pv(p_in, pbuf, pkb);
    qk(qbuf, qkb, s_out);

    // online softmax of half h against the current reference
    float lsum = exps(s_in, p_out);
    need_prev = (__builtin_amdgcn_ballot_w64(lsum > kSumBound) != 0) | !all_set;
    if (need_prev) {
      float mx = fmaxf(fmaxf(s_in[0], s_in[1]), s_in[2]);
#pragma unroll
      for (int j = 3; j < 15; j += 2) mx = fmaxf(fmaxf(mx, s_in[j]), s_in[j + 1]);
      mx = pair_max(fmaxf(mx, s_in[15]));
      const bool first = !mset && mx > -INFINITY;
      mset = mset || first;
      all_set = __builtin_amdgcn_ballot_w64(!mset) == 0;
      const float d = (first || mx > 0.f) ? mx : 0.f;
      m_run += d;
      d_prev = d;
      // before its first visible key a row has l = 0 and O = 0; a first
      // reference far below 0 would overflow exp2(-d), so that move scales by 1
      alpha_prev = first ? 1.f : __builtin_amdgcn_exp2f(-d);
      l_run *= alpha_prev;
      const float nm = SCALE_S ? -m_run * inv_cscale : -m_run;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s_in[j] -= d;
        negm[j] = nm;
      }
      lsum = exps(s_in, p_out);
    }
    l_run += lsum;
  };
  // Tile t+1 goes into LDS buffer (t+1) % 3 at the start of step 2t, from
  // registers loaded two steps earlier; the loads of tile t+2 are issued into
  // the freed registers right after.  That buffer last served tile t-2,
  // whose last reader (PV of step 2t-2) every wave has passed at the barrier
  // closing step 2t-2; the barrier closing step 2t publishes tile t+1, first
  // read in step 2t+1.  Spreading the stores into the step's instruction
  // stream keeps them from bunching up in front of the barrier.  Past the
  // last tile the stores write stale registers into an unused buffer and the
  // loads, whose range is empty, return zeros without touching memory.
  auto tile_store = [&](int next_buf, int t) {
    store_lds(next_buf);
    issue_loads(tile_key0(t + 2));
  };
  using T = std::true_type;
  using F = std::false_type;
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;

  if (ntiles > 0) {
    issue_loads(tile_key0(0));
    load_q();
    store_lds(0);
    __syncthreads();
    issue_loads(tile_key0(1));
    qk(B0{}, K0{}, s_a);
    const int key00 = tile_key0(0);
    tile_store(1, 0);
    step(F{}, B0{}, K1{}, 0, K0{}, key00, s_a, s_b, p_b, p_a);
    __syncthreads();
    step(T{}, B1{}, K0{}, 0, K0{}, key00 + 32, s_b, s_a, p_a, p_b);
    // Tile t lives in LDS buffer t % 3.  Three tiles per trip keep every
    // buffer index a compile-time constant, so K operand addresses are one
    // base register plus immediate offsets and no buffer arithmetic is left
    // in the loop.
    auto tile = [&](auto curc, int t) {
      constexpr int C = decltype(curc)::value;
      using CUR = std::integral_constant<int, C>;
      using PRV = std::integral_constant<int, C == 0 ? 2 : C - 1>;
      using NXT = std::integral_constant<int, C == 2 ? 0 : C + 1>;
      const int key0 = tile_key0(t);
      tile_store(NXT::value, t);
      step(T{}, CUR{}, K1{}, PRV::value, K1{}, key0, s_a, s_b, p_b, p_a);
      __syncthreads();
      step(T{}, NXT{}, K0{}, C, K0{}, key0 + 32, s_b, s_a, p_a, p_b);
    };
    int t = 1;
    if constexpr (ROT_K) {
      // (rotating K on the way in needs the registers the unrolled walk
      // would take: one tile per trip, buffer indices at run time)
      int cur = 1;
      for (; t < ntiles; ++t) {
        const int prev = cur == 0 ? 2 : cur - 1, next = cur == 2 ? 0 : cur + 1;
        const int key0 = tile_key0(t);
        tile_store(next, t);
        step(T{}, cur, K1{}, prev, K1{}, key0, s_a, s_b, p_b, p_a);
        __syncthreads();
        step(T{}, next, K0{}, cur, K0{}, key0 + 32, s_b, s_a, p_a, p_b);
        cur = next;
      }
    } else {
      for (; t + 2 < ntiles; t += 3) {
        tile(B1{}, t);
        tile(B2{}, t + 1);
        tile(B0{}, t + 2);
      }
      if (t < ntiles) tile(B1{}, t);
      if (t + 1 < ntiles) tile(B2{}, t + 1);
    }
    if (need_prev) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha_prev;
    }
    // the last step, 2(ntiles-1)+1, left P of the last half in p_b
    pv(p_b, (ntiles - 1) % 3, K1{});
  }

  // ---- epilogue: combine the two lane halves' sums, normalise, write O and lse
  const float lt = pair_sum(l_run);
  const int row = wrow0 + l32;
  if (a.out_bf16 && !a.acc_o) {
    // A lane holds four d values of one row per 32-wide d block, so storing
    // straight from registers writes 32 scattered 16-byte pieces per
    // instruction.  Instead the wave's 32 x 128 block goes through its own
    // 8.5 KB of the (now idle) tile buffers and every 16 lanes then write one
    // whole 256-byte row: each store instruction covers four full rows.
    __syncthreads();                                 // every wave is done reading the last tiles
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const uint32_t stg = lds_off(&sm) + wave * (kBM * kOStr * 2);
    typedef __attribute__((address_space(3))) uint32_t lds_u32;
    typedef __attribute__((address_space(3))) u32x4_t lds_u4w;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint32_t at = stg + (l32 * kOStr + db * 32 + g4 * 8 + hl * 4) * 2;
        *(lds_u32*)(uintptr_t)at = pack2(oacc[db][g4 * 4 + 0] * inv, oacc[db][g4 * 4 + 1] * inv);
        *(lds_u32*)(uintptr_t)(at + 4) = pack2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv);
      }
    asm volatile("" ::: "memory");                    // the reads below follow the writes (one wave: in order)
    __hip_bfloat16* og = reinterpret_cast<__hip_bfloat16*>(a.out) + ((long long)b * a.Hq + hq) * a.o_hstride +
                         (long long)wrow0 * kD;
#pragma unroll
    for (int i = 0; i < kBM / 4; ++i) {
      const int r = i * 4 + (lane >> 4);
      const u32x4_t w = *(const lds_u4*)(uintptr_t)(stg + (r * kOStr + (lane & 15) * 8) * 2);
      if (wrow0 + r < a.Nq) *reinterpret_cast<uint4*>(og + (long long)r * kD + (lane & 15) * 8) = make_uint4(w.x, w.y, w.z, w.w);
    }
    if (a.lse && hl == 0 && row < a.Nq)
      a.lse[((long long)b * a.Hq + hq) * a.lse_hstride + row] = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
  } else if (row < a.Nq) {
    float inv = lt > 0.f ? 1.0f / lt : 0.f;
    float lse_row = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
    const long long obase = ((long long)b * a.Hq + hq) * a.o_hstride + (long long)row * kD;
    float wa = 0.f;                 // weight of the running state (ring step)
    f32x16 accv[4];                 // the running state's O, in the oacc layout
    if (a.acc_o) {
      // every load of the running state is issued before any is used, so the
      // epilogue waits for one round trip to memory instead of one per load
      const float* accp = a.acc_o + ((long long)b * a.Hq + hq) * a.acc_hstride + (long long)row * kD;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 x = *reinterpret_cast<const float4*>(accp + db * 32 + g4 * 8 + hl * 4);
          accv[db][g4 * 4 + 0] = x.x; accv[db][g4 * 4 + 1] = x.y; accv[db][g4 * 4 + 2] = x.z; accv[db][g4 * 4 + 3] = x.w;
        }
      // fold this launch's (O, lse) into the running state by the log-sum-exp
      // rule: lse = log(e^la + e^lb), O = e^(la-lse) O_a + e^(lb-lse) O_b
      // ("8.3 长上下文技术" §8.3.5: a ring step rescales the running result)
      const float la = a.acc_lse[((long long)b * a.Hq + hq) * a.acc_lse_hstride + row];
      const float mx = fmaxf(la, lse_row);
      if (mx == -INFINITY) {
        inv = 0.f;
      } else {
        const float ea = __expf(la - mx), eb = __expf(lse_row - mx);   // exp(-inf) = 0
        const float rs = 1.0f / (ea + eb);
        wa = ea * rs;
        inv *= eb * rs;
        lse_row = mx + __logf(ea + eb);
      }
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hl * 4;
        float o0 = oacc[db][g4 * 4 + 0] * inv, o1 = oacc[db][g4 * 4 + 1] * inv;
        float o2 = oacc[db][g4 * 4 + 2] * inv, o3 = oacc[db][g4 * 4 + 3] * inv;
        if (a.acc_o) {
          o0 = fmaf(wa, accv[db][g4 * 4 + 0], o0); o1 = fmaf(wa, accv[db][g4 * 4 + 1], o1);
          o2 = fmaf(wa, accv[db][g4 * 4 + 2], o2); o3 = fmaf(wa, accv[db][g4 * 4 + 3], o3);
        }
        if (a.out_bf16) {
          *reinterpret_cast<uint2*>(reinterpret_cast<__hip_bfloat16*>(a.out) + obase + d) =
              make_uint2(pack2(o0, o1), pack2(o2, o3));
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + obase + d) = make_float4(o0, o1, o2, o3);
        }
      }
    }
    if (a.lse && hl == 0) a.lse[((long long)b * a.Hq + hq) * a.lse_hstride + row] = lse_row;
  }
  if (a.sched && tid == 0) sched_release(a.sched, gridDim.x);
}

}  // namespace

// Compute units of the current device (cached per device).
int compute_units() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int n = 0;
    cache[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cache[dev];
}

__global__ void __launch_bounds__(64) zero_words_kernel(unsigned long long* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0ull;
}

hipError_t launch_zero_words(unsigned long long* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (n > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16_d128(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (a.D != kD || !(G == 1 || G == 2 || G % 4 == 0)) return hipErrorInvalidValue;
  const int HPW = G < 4 ? G : 4;
  const int rows_per_wg = kBM * (kWaves / HPW);
  const int quads = G > 4 ? G / 4 : 1;
  const long long items = (long long)a.Hkv * quads * ((a.Nq + rows_per_wg - 1) / rows_per_wg) * a.B;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  // the run-time assignment pays one atomic round trip per workgroup and
  // helps only when the XCDs run several workgroups each; a grid too large
  // for one launch goes in launches of kMaxLaunchItems with the fixed one
  PrefillArgs la = a;
  la.item0 = 0;
  if (la.sched && (items <= 2LL * compute_units() || items > kMaxLaunchItems)) la.sched = nullptr;
  const bool rot_k = (a.rope_flags & 2) != 0, half = (a.rope_flags & 4) != 0;
  const bool win = a.window > 0, scale_s = (a.rope_flags & 1) == 0;
  const dim3 block(kThreads);
  auto go = [&](auto kernel) {
    for (long long base = 0; base < items; base += kMaxLaunchItems) {
      la.item0 = (int)base;
      const long long n = items - base < kMaxLaunchItems ? items - base : kMaxLaunchItems;
      hipLaunchKernelGGL(kernel, dim3((unsigned)n), block, 0, stream, la);
    }
  };
  // half-split pairing changes only what is rotated: without a rotation it is
  // the same kernel
  auto pick = [&](auto wc, auto sc) {
    constexpr bool W = decltype(wc)::value, S = decltype(sc)::value;
    if (rot_k && half) go(prefill_bf16_kernel<true, true, W, S>);
    else if (rot_k) go(prefill_bf16_kernel<true, false, W, S>);
    else if constexpr (!S) {
      if (half) go(prefill_bf16_kernel<false, true, W, S>);
      else go(prefill_bf16_kernel<false, false, W, S>);
    } else {
      go(prefill_bf16_kernel<false, false, W, S>);
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  if (win) {
    if (scale_s) pick(T{}, T{});
    else pick(T{}, F{});
  } else {
    if (scale_s) pick(F{}, T{});
    else pick(F{}, F{});
  }
  return hipGetLastError();
}

}  // namespace srt
