// Ring Attention over P devices, run on one GPU: the launch schedule.
//
// "8.3 长上下文技术" §8.3.5: device r holds one query shard and one K/V
// shard; it attends its own K/V shard first, then at step s the shard of
// device (r - s) mod P, which has travelled s hops around the ring, and folds
// each partial result into its running state with the online-softmax
// rescaling (here the log-sum-exp merge kernel).  The same page's causal load
// balancing picks which positions a shard holds: contiguous blocks, Striped
// (every P-th position) or Zig-Zag (chunk r with its mirror chunk 2P - 1 - r).
//
// On one GPU the devices' work runs one after another on one stream, device
// by device, in ring order; `device` >= 0 runs one device's share only (what
// that GPU of a real ring would compute).  Each (query run, key run) pair is
// one launch of the tiled prefill kernel at the runs' true positions, so the
// causal mask, the window and the sinks come out exactly; pairs with no
// visible key are not launched.  The first launch of a query run writes its
// (O, lse) as the run's fp32 running state; every later launch folds its own
// result into that state in its epilogue (log-sum-exp rule, in place), and
// the last one writes the merged state to the output rows, so no partial is
// written out and read back by a separate merge.  Striped shards have positions r + P t: the
// mask of a pair is then the causal mask in row-index space, shifted by one
// row when the key shard's device comes after the query shard's, and RoPE uses
// the strided positions.  K is rotated once, into the workspace, at its
// shard-major positions when asked to, and the prefill launches rotate q only.
#include "srt_internal.h"

#include <vector>

namespace srt {

namespace {

struct Run {
  long long row0;   // first row in the shard-major tensor
  int len;          // rows
  long long pos0;   // position of the first row
  int step;         // position stride between rows
};

// The runs of shard j: one for contiguous and striped, two for zigzag.
int shard_runs(const RingArgs& a, int j, Run (&out)[2]) {
  const int C = a.N / a.P;
  if (a.mode == kZigzag) {
    const int h = C / 2;
    out[0] = Run{(long long)j * C, h, (long long)j * h, 1};
    out[1] = Run{(long long)j * C + h, h, (long long)(2 * a.P - 1 - j) * h, 1};
    return 2;
  }
  if (a.mode == kStriped) {
    out[0] = Run{(long long)j * C, C, (long long)j, a.P};
    return 1;
  }
  out[0] = Run{(long long)j * C, C, (long long)j * C, 1};
  return 1;
}

// Does any key of run k stay visible to some query of run q (causal, window, sinks)?
bool any_visible(const RingArgs& a, const Run& q, const Run& k) {
  const long long qmin = q.pos0, qmax = q.pos0 + (long long)q.step * (q.len - 1);
  const long long kmin = k.pos0, kmax = k.pos0 + (long long)k.step * (k.len - 1);
  if (kmin > qmax) return false;
  if (a.window > 0) return kmax > qmin - a.window || kmin < a.sink;   // window only with step 1
  return true;
}

}  // namespace

size_t ring_workspace_bytes(const RingArgs& a) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t elt = a.bf16 ? 2 : 4;
  const int C = a.N / a.P;
  const size_t R = a.mode == kZigzag ? C / 2 : C;
  size_t n = 0;
  if (a.rope_flags & 2) n += up((size_t)a.B * a.Hkv * a.N * a.D * elt);
  n += up((size_t)a.B * a.Hq * R * a.D * 4) + up((size_t)a.B * a.Hq * R * 4);
  n += up(kSchedWords * 8);            // the prefill launches' scheduling block
  return n;
}

hipError_t ring_prefill(const RingArgs& a, hipStream_t stream) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t elt = a.bf16 ? 2 : 4;
  const int C = a.N / a.P;
  const size_t R = a.mode == kZigzag ? C / 2 : C;
  char* ws = static_cast<char*>(a.workspace);
  const void* kk = a.k;
  if (a.rope_flags & 2) {              // rotate every key once at its shard-major position
    void* krot = ws;
    ws += up((size_t)a.B * a.Hkv * a.N * a.D * elt);
    const PosMap map{0, a.mode, a.P, C};
    hipError_t e = launch_rope_apply(a.k, krot, a.bf16, (a.rope_flags & 4) != 0, (long long)a.B * a.Hkv, a.N, a.D,
                                     map, a.table, stream);
    if (e != hipSuccess) return e;
    kk = krot;
  }
  // running state of the current query run: fp32 O and lse
  float* acc_o = reinterpret_cast<float*>(ws);
  ws += up((size_t)a.B * a.Hq * R * a.D * 4);
  float* acc_l = reinterpret_cast<float*>(ws);
  ws += up((size_t)a.B * a.Hq * R * 4);
  // one scheduling block serves every launch of the call (they run one after
  // another on the stream, and each leaves it zero-filled)
  unsigned long long* sched = reinterpret_cast<unsigned long long*>(ws);
  if (hipError_t e = launch_zero_words(sched, kSchedWords, stream); e != hipSuccess) return e;

  const char* qb = static_cast<const char*>(a.q);
  const char* kb = static_cast<const char*>(kk);
  const char* vb = static_cast<const char*>(a.v);
  char* ob = static_cast<char*>(a.out);
  const long long hs = (long long)a.N * a.D;    // head stride of q, k, v, out

  // merge: fold the launch's result into the running state (acc_o, acc_l)
  auto prefill = [&](const Run& q, const Run& k, int r, int j, void* out, bool out_bf16, long long o_hstride,
                     float* lse, long long lse_hstride, bool merge) {
    PrefillArgs p{};
    p.q = qb + q.row0 * a.D * elt;
    p.k = kb + k.row0 * a.D * elt;
    p.v = vb + k.row0 * a.D * elt;
    p.out = out;
    p.lse = lse;
    p.table = a.table;
    p.sched = sched;
    p.q_hstride = hs; p.kv_hstride = hs; p.o_hstride = o_hstride; p.lse_hstride = lse_hstride;
    if (a.mode == kStriped) {
      // key u at j + P u is visible to query t at r + P t iff u <= t (j <= r) or u <= t - 1 (j > r)
      p.q_pos0 = 0;
      p.k_pos0 = j > r ? 1 : 0;
    } else {
      p.q_pos0 = q.pos0;
      p.k_pos0 = k.pos0;
    }
    p.q_rope0 = q.pos0; p.k_rope0 = k.pos0; p.rope_step = q.step;
    p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = q.len; p.Nk = k.len; p.D = a.D;
    p.causal = 1;
    p.rope_flags = a.rope_flags & ~2;
    p.out_bf16 = out_bf16 ? 1 : 0;
    p.window = a.window; p.sink = a.window > 0 ? a.sink : 0;
    p.sm_scale = a.sm_scale;
    if (merge) {
      p.acc_o = acc_o; p.acc_lse = acc_l;
      p.acc_hstride = (long long)R * a.D; p.acc_lse_hstride = (long long)R;
    }
    return a.bf16 ? launch_prefill_bf16_d128(p, stream) : launch_prefill_f32(p, stream);
  };

  const int r_lo = a.device >= 0 ? a.device : 0, r_hi = a.device >= 0 ? a.device + 1 : a.P;
  for (int r = r_lo; r < r_hi; ++r) {
    Run qruns[2];
    const int nq = shard_runs(a, r, qruns);
    for (int qi = 0; qi < nq; ++qi) {
      const Run& q = qruns[qi];
      // visible key runs in ring order: step s holds the shard of device (r - s) mod P
      std::vector<std::pair<Run, int>> todo;
      for (int s = 0; s < a.P; ++s) {
        const int j = ((r - s) % a.P + a.P) % a.P;
        Run kr[2];
        const int nk = shard_runs(a, j, kr);
        for (int ki = 0; ki < nk; ++ki)
          if (any_visible(a, q, kr[ki])) todo.push_back({kr[ki], j});
      }
      void* out = ob + q.row0 * a.D * elt;
      float* lse = a.lse ? a.lse + q.row0 : nullptr;
      hipError_t e = hipSuccess;
      if (todo.empty()) {              // no visible key (not reachable under a causal mask): O = 0, lse = -inf
        e = prefill(q, Run{0, 0, 0, q.step}, r, r, out, a.bf16, hs, lse, a.N, false);
        if (e != hipSuccess) return e;
        continue;
      }
      for (size_t i = 0; i < todo.size() && e == hipSuccess; ++i) {
        const bool last = i + 1 == todo.size();
        // the last launch writes the merged result to the output rows, the
        // others keep the running state in the workspace
        e = last ? prefill(q, todo[i].first, r, todo[i].second, out, a.bf16, hs, lse, a.N, i > 0)
                 : prefill(q, todo[i].first, r, todo[i].second, acc_o, false, (long long)R * a.D, acc_l,
                           (long long)R, i > 0);
      }
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace srt
