// Host-only harness for the ring launch schedule (csrc/ring.cpp): the kernel
// launchers are replaced by stubs that print each launch's arguments, so a
// CPU test can check which (query rows, key rows) pairs the schedule launches
// and where every partial state goes.  Buffers are fake addresses that are
// never dereferenced.
#include "srt_internal.h"

#include <cstdio>
#include <cstdlib>

namespace srt {

static const char* g_base[8];
static const char* g_name[8];
static int g_nbuf = 0;

static void name_ptr(const void* p, const char** name, long long* off) {
  const char* c = static_cast<const char*>(p);
  *name = p ? "?" : "none";
  *off = -1;
  for (int i = 0; i < g_nbuf; ++i)
    if (c >= g_base[i] && c < g_base[i] + (1LL << 36)) { *name = g_name[i]; *off = c - g_base[i]; }
}

hipError_t launch_rope_apply(const void* x, void* y, bool bf16, bool half_pairs, long long groups, int N, int D,
                             const PosMap& m, const float*, hipStream_t, float) {
  const char *nx, *ny;
  long long ox, oy;
  name_ptr(x, &nx, &ox);
  name_ptr(y, &ny, &oy);
  printf("rope %s %lld %s %lld bf16=%d half=%d groups=%lld N=%d D=%d mode=%d P=%d C=%d\n", nx, ox, ny, oy, (int)bf16,
         (int)half_pairs, groups, N, D, m.mode, m.P, m.C);
  return hipSuccess;
}

hipError_t launch_zero_words(unsigned long long* p, int n, hipStream_t) {
  const char* np;
  long long op;
  name_ptr(p, &np, &op);
  printf("zero at=%s:%lld n=%d\n", np, op, n);
  return hipSuccess;
}

static hipError_t log_prefill(const PrefillArgs& a, const char* kind) {
  const char *nq, *nk, *nv, *no, *nl, *na, *nal, *ns;
  long long oq, ok, ov, oo, ol, oa, oal, os;
  name_ptr(a.sched, &ns, &os);
  name_ptr(a.q, &nq, &oq);
  name_ptr(a.k, &nk, &ok);
  name_ptr(a.v, &nv, &ov);
  name_ptr(a.out, &no, &oo);
  name_ptr(a.lse, &nl, &ol);
  name_ptr(a.acc_o, &na, &oa);
  name_ptr(a.acc_lse, &nal, &oal);
  printf("prefill %s q=%s:%lld k=%s:%lld v=%s:%lld out=%s:%lld lse=%s:%lld acc=%s:%lld acclse=%s:%lld Nq=%d Nk=%d "
         "qp=%lld kp=%lld qr=%lld kr=%lld step=%lld qhs=%lld kvhs=%lld ohs=%lld lhs=%lld ahs=%lld alhs=%lld "
         "flags=%d obf16=%d window=%d sink=%d causal=%d sched=%s:%lld\n",
         kind, nq, oq, nk, ok, nv, ov, no, oo, nl, ol, na, oa, nal, oal, a.Nq, a.Nk, a.q_pos0, a.k_pos0, a.q_rope0,
         a.k_rope0, a.rope_step, a.q_hstride, a.kv_hstride, a.o_hstride, a.lse_hstride, a.acc_hstride,
         a.acc_lse_hstride, a.rope_flags, a.out_bf16, a.window, a.sink, a.causal, ns, os);
  return hipSuccess;
}

hipError_t launch_prefill_bf16_d128(const PrefillArgs& a, hipStream_t) { return log_prefill(a, "bf16"); }
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t) { return log_prefill(a, "f32"); }

hipError_t launch_merge(const MergeArgs& a, hipStream_t) {
  const char *na, *nb, *no, *nl;
  long long oa, ob, oo, ol;
  name_ptr(a.oa, &na, &oa);
  name_ptr(a.ob, &nb, &ob);
  name_ptr(a.oo, &no, &oo);
  name_ptr(a.lo, &nl, &ol);
  printf("merge a=%s:%lld b=%s:%lld out=%s:%lld lse=%s:%lld N=%d BH=%d inhs=%lld ohs=%lld lhs=%lld obf16=%d\n", na,
         oa, nb, ob, no, oo, nl, ol, a.N, a.BH, a.in_hstride, a.out_hstride, a.lse_out_hstride, a.out_bf16);
  return hipSuccess;
}

}  // namespace srt

int main(int argc, char** argv) {
  if (argc != 13) {
    fprintf(stderr, "usage: B Hq Hkv N D P mode device window sink rope_flags bf16\n");
    return 2;
  }
  srt::RingArgs a{};
  a.B = atoi(argv[1]); a.Hq = atoi(argv[2]); a.Hkv = atoi(argv[3]); a.N = atoi(argv[4]); a.D = atoi(argv[5]);
  a.P = atoi(argv[6]); a.mode = atoi(argv[7]); a.device = atoi(argv[8]); a.window = atoi(argv[9]);
  a.sink = atoi(argv[10]); a.rope_flags = atoi(argv[11]); a.bf16 = atoi(argv[12]) != 0;
  a.sm_scale = 0.1f;
  // fake, disjoint address ranges, 2^36 bytes apart (never dereferenced)
  const char* names[] = {"q", "k", "v", "out", "lse", "ws", "table"};
  for (int i = 0; i < 7; ++i) {
    srt::g_base[i] = reinterpret_cast<const char*>((unsigned long long)(i + 1) << 40);
    srt::g_name[i] = names[i];
  }
  srt::g_nbuf = 7;
  a.q = srt::g_base[0]; a.k = srt::g_base[1]; a.v = srt::g_base[2];
  a.out = const_cast<char*>(srt::g_base[3]);
  a.lse = reinterpret_cast<float*>(const_cast<char*>(srt::g_base[4]));
  a.workspace = const_cast<char*>(srt::g_base[5]);
  a.table = reinterpret_cast<const float*>(srt::g_base[6]);
  printf("workspace %zu\n", srt::ring_workspace_bytes(a));
  return srt::ring_prefill(a, nullptr) == hipSuccess ? 0 : 1;
}
