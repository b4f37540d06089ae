// Internal declarations shared by the C-ABI layer (abi.cpp), the ring schedule
// (ring.cpp) and the kernel translation units.  Nothing here is part of the
// public ABI.  Only the runtime API is included, so the host sources also
// build with a plain C++ compiler (the kernel sources include the device
// headers themselves).
#pragma once

#include <hip/hip_runtime_api.h>
#include <cstdint>

namespace srt {

constexpr int kMaxHalf = 128;  // D <= 256

// Scaled frequencies passed by value as a kernel argument (1 KiB).
struct Theta {
  double v[kMaxHalf];
};

// ---------------------------------------------------------------- rope
hipError_t launch_rope_table(const Theta& th, int half, double mscale, long long npos, float* table,
                             hipStream_t stream);

// Position of row n (0 <= n < N) of a group: pos0 + n (kContiguous), or the
// shard-major layouts of a ring over P devices with C = N / P rows per shard:
// striped (shard n / C, row t = n % C sits at n / C + P t) and zigzag (rows
// t < C/2 of shard j at j C/2 + t, the rest at (2P - 1 - j) C/2 + t - C/2).
enum PosMode { kContiguous = 0, kStriped = 1, kZigzag = 2 };
struct PosMap {
  long long pos0;
  int mode, P, C;
};

// rows = B*H rows-groups of N rows each; row n of a group sits at position map(n).
// A null table means no rotation; outputs are multiplied by scale (one rounding).
hipError_t launch_rope_apply(const void* x, void* y, bool bf16, bool half_pairs, long long groups, int N, int D,
                             const PosMap& map, const float* table, hipStream_t stream, float scale = 1.f);

// ---------------------------------------------------------------- prefill
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const float* table;   // [npos][D/2] float2 or nullptr
  long long q_hstride, kv_hstride, o_hstride, lse_hstride;  // elements
  long long q_pos0, k_pos0;   // mask positions of row 0 of q and of k
  // RoPE positions: q row r turns by the table row q_rope0 + r * rope_step, k
  // row c by k_rope0 + c * rope_step (equal to the mask positions with step 1
  // except for strided ring shards, whose mask is stated in index space)
  long long q_rope0, k_rope0, rope_step;
  int B, Hq, Hkv, Nq, Nk, D;
  int causal;
  int rope_flags;       // bit0: rotate q, bit1: rotate k, bit2: half-split pairs
  int out_bf16;         // 1: out is bf16, 0: fp32
  int window;           // > 0: key j visible to query i only if i - j < window or j < sink
  int sink;             // first positions kept visible (used only with a window)
  float sm_scale;
  // One Ring Attention step: with acc_o set, the launch's own (O, lse) is
  // folded into the running state (acc_o fp32 [B][Hq][Nq][D], acc_lse fp32
  // [B][Hq][Nq], head strides acc_hstride / acc_lse_hstride) by the
  // log-sum-exp rule and the merged state is what goes to out / lse, which
  // may be acc_o / acc_lse themselves (in place: each lane reads the elements
  // it then writes).  acc_lse must be set with acc_o; lse may be NULL (then
  // only O is written).
  const float* acc_o;
  const float* acc_lse;
  long long acc_hstride, acc_lse_hstride;
  // Run-time assignment of the bf16 kernel's (head, query tile) items to
  // workgroups: kSchedWords zero-filled 64-bit counters, left zeroed by the
  // launch's last workgroup; nullptr keeps the fixed assignment by grid index.
  unsigned long long* sched;
  int item0;            // first item of this launch (launches of more than kMaxLaunchItems items are split)
};
constexpr int kMaxLaunchItems = 1 << 22;   // workgroups per launch: x-dimension work-items stay below 2^32
constexpr int kSchedWords = 10;   // 8 per-XCD queues, the shared pool, the count of finished workgroups
constexpr int kSchedBlockWords = 16;   // one block: SRT_PREFILL_SCHED_BYTES = 128 bytes

// Zero-fill n <= 64 64-bit words on the stream (a kernel, so that it may be captured).
hipError_t launch_zero_words(unsigned long long* p, int n, hipStream_t stream);
// Compute units of the current device.
int compute_units();

hipError_t launch_prefill_bf16_d128(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- merge
struct MergeArgs {
  const void* oa;
  const float* la;
  const void* ob;
  const float* lb;
  void* oo;
  float* lo;
  long long in_hstride, out_hstride, lse_out_hstride;
  int BH, N, D;
  int in_bf16, out_bf16;
};

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- decode
struct DecodeArgs {
  const void* q;          // [B][Hq][D] bf16
  const void* k;          // [B][Hkv][Nk][D] bf16, rotated
  const void* v;          // [B][Hkv][Nk][D] bf16
  const int* seq_lens;    // [B] or nullptr
  const float* table;     // or nullptr
  float* ws_o;            // [B][Hq][splits][D] fp32
  float* ws_lse;          // [B][Hq][splits] fp32
  void* out;              // [B][Hq][D] bf16
  float* lse;             // [B][Hq] or nullptr
  int B, Hq, Hkv, Nk, D, splits, split_len;
  int half_pairs;         // q rotated with pairs (x_i, x_{i+D/2})
  int window, sink;       // window > 0: keys [seq - window, seq) plus [0, sink) only
  float sm_scale;
};

size_t decode_workspace_bytes(int B, int Hq, int D, int splits);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Static device scratch of the allocation-free decode entry point (one copy
// per GPU, in decode.hip): its size, and its address on the current device
// (looked up once per device, then cached).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

// ---------------------------------------------------------------- backward
struct BwdArgs {
  const void* q;          // [B][Hq][Nq][D] dtype, raw (rotated on load with ROTATE_Q)
  const void* k;          // [B][Hkv][Nk][D]
  const void* v;
  const void* out;        // forward output [B][Hq][Nq][D] dtype
  const void* dout;       // upstream gradient [B][Hq][Nq][D] dtype
  const float* lse;       // forward lse [B][Hq][Nq]
  float* delta;           // workspace [B][Hq][Nq]: sum_d dO * O
  const void* q_rot;      // bf16: q rotated (ROTATE_Q) and multiplied by sm_scale log2(e), rounded once as the
                          // forward's q~ is, so the backward's S equals the forward's; always set for bf16
  const void* k_rot;      // the same for k (ROTATE_K)
  const float* table;
  float* dq;              // [B][Hq][Nq][D] fp32
  float* dk;              // [B][Hkv][Nk][D] fp32
  float* dv;              // [B][Hkv][Nk][D] fp32
  long long q_pos0, k_pos0;
  int B, Hq, Hkv, Nq, Nk, D;
  int causal, window, sink;
  int rope_flags;         // bit0: q rotated on load, bit1: k, bit2: half-split pairs
  int bf16;
  float sm_scale;
  // bf16: two scheduling blocks of kSchedBlockWords words in the workspace
  // (dk/dv, then dq), zero-filled by the launcher; see PrefillArgs::sched
  unsigned long long* sched;
  int item0;            // first item of this launch (see PrefillArgs::item0)
};

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- ring
struct RingArgs {
  const void* q;          // [B][Hq][N][D], shard-major rows
  const void* k;          // [B][Hkv][N][D], shard-major rows
  const void* v;
  const float* table;     // or nullptr
  void* workspace;        // ring_workspace_bytes(*this) bytes, 256-byte aligned
  void* out;              // [B][Hq][N][D] in the input dtype, shard-major
  float* lse;             // [B][Hq][N] or nullptr
  int B, Hq, Hkv, N, D;
  int P, mode;            // devices, PosMode of the shards
  int device;             // -1: every device, else that device's share only
  int window, sink;
  int rope_flags;         // as PrefillArgs; K is rotated once into the workspace
  bool bf16;
  float sm_scale;
};

size_t ring_workspace_bytes(const RingArgs& a);
hipError_t ring_prefill(const RingArgs& a, hipStream_t stream);

}  // namespace srt
