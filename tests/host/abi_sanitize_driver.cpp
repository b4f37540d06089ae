// Host-only driver of the C ABI (abi.cpp) and the ring schedule (ring.cpp),
// built with a plain C++ compiler under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Kernel launchers are stubs that check the
// arguments they receive and count launches; device pointers are fake,
// aligned addresses that nothing dereferences.  Every entry point is driven
// through valid and invalid arguments (host arrays of exactly the documented
// sizes, so a write past them is caught); the process exits 0 only if every
// expected status was returned and the sanitizers reported nothing.
#include "srt.h"
#include "srt_internal.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

static int g_fail = 0;
static long long g_launches = 0;
#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      fprintf(stderr, "FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond,       \
              srt_last_error());                                                  \
      ++g_fail;                                                                   \
    }                                                                             \
  } while (0)

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace srt {

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

hipError_t launch_rope_table(const Theta& th, int half, double mscale, long long npos, float* table, hipStream_t) {
  EXPECT(half >= 1 && half <= kMaxHalf && npos >= 1 && table && std::isfinite(mscale));
  for (int i = 0; i < half; ++i) EXPECT(std::isfinite(th.v[i]));
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_rope_apply(const void* x, void* y, bool, bool, long long groups, int N, int D, const PosMap& m,
                             const float*, hipStream_t, float) {
  EXPECT(x && y && groups >= 1 && N >= 1 && D % 8 == 0 && aligned16(x) && aligned16(y));
  EXPECT(m.P >= 1 && m.C >= 1);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_zero_words(unsigned long long* p, int n, hipStream_t) {
  EXPECT(p && n >= 1 && n <= 64 && (reinterpret_cast<uintptr_t>(p) & 7) == 0);
  ++g_launches;
  return hipSuccess;
}
static hipError_t check_prefill(const PrefillArgs& a) {
  EXPECT(!a.sched || (reinterpret_cast<uintptr_t>(a.sched) & 7) == 0);
  EXPECT(a.B >= 1 && a.Nq >= 1 && a.Nk >= 0 && a.Hq % a.Hkv == 0);
  EXPECT(a.q && a.out && aligned16(a.q) && aligned16(a.out));
  EXPECT(a.q_hstride >= (long long)a.Nq * a.D && a.o_hstride >= (long long)a.Nq * a.D);
  EXPECT(!a.acc_o || a.acc_lse);
  EXPECT(!(a.rope_flags & 3) || a.table);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_prefill_bf16_d128(const PrefillArgs& a, hipStream_t) {
  EXPECT(a.D == 128);
  return check_prefill(a);
}
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t) { return check_prefill(a); }
hipError_t launch_merge(const MergeArgs& a, hipStream_t) {
  EXPECT(a.BH >= 1 && a.N >= 1 && a.D % 8 == 0 && a.oa && a.ob && a.oo);
  ++g_launches;
  return hipSuccess;
}
size_t decode_workspace_bytes(int B, int Hq, int D, int splits) {
  return (size_t)B * Hq * splits * (size_t)(D + 1) * sizeof(float);
}
hipError_t launch_decode(const DecodeArgs& a, hipStream_t) {
  EXPECT(a.B >= 1 && a.splits >= 1 && a.split_len >= 0 && a.ws_o && a.ws_lse && aligned16(a.ws_o));
  EXPECT((char*)a.ws_lse - (char*)a.ws_o == (long long)a.B * a.Hq * a.splits * a.D * 4);
  ++g_launches;
  return hipSuccess;
}
hipError_t decode_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>((uintptr_t)1 << 41);
  return hipSuccess;
}
hipError_t launch_backward(const BwdArgs& a, hipStream_t) {
  EXPECT(a.B >= 1 && (a.Nq >= 1 || a.Nk >= 1) && a.delta);
  ++g_launches;
  return hipSuccess;
}

}  // namespace srt

static void* fake(int i) { return reinterpret_cast<void*>(((uintptr_t)(i + 1)) << 36); }

int main() {
  // ---- frequency step: outputs are host arrays of exactly D/2 entries
  for (int D : {2, 4, 64, 128, 256}) {
    for (int method = SRT_ROPE_NONE; method <= SRT_ROPE_YARN; ++method) {
      std::vector<double> th(D / 2);
      std::vector<signed char> band(D / 2);
      double ms = 0;
      const int st = srt_rope_inv_freq(method, 1e4, 16.0, 2048.0, 1.0, 32.0, D, th.data(), &ms, band.data());
      EXPECT(st == ((method == SRT_ROPE_NTK && D <= 2) ? SRT_ERR_INVALID : SRT_OK));
    }
    std::vector<double> th(D / 2), lam(D / 2, 2.0);
    double s = 0;
    EXPECT(srt_rope_inv_freq_dynamic_ntk(1e4, 65536, 2048.0, D, th.data(), &s) == (D < 4 ? SRT_ERR_INVALID : SRT_OK));
    EXPECT(srt_rope_inv_freq_factors(1e4, lam.data(), D, th.data()) == SRT_OK);
    EXPECT(srt_rope_cos_sin(th.data(), D, 1.0, 1024, (float*)fake(0), nullptr) == SRT_OK);
  }
  {
    double th[64];
    EXPECT(srt_rope_inv_freq(SRT_ROPE_YARN, 1e4, 16.0, 2048.0, 32.0, 1.0, 128, th, nullptr, nullptr) == SRT_ERR_INVALID);
    EXPECT(srt_rope_inv_freq(7, 1e4, 16.0, 0, 1, 32, 128, th, nullptr, nullptr) == SRT_ERR_INVALID);
    EXPECT(srt_rope_inv_freq(SRT_ROPE_NONE, 1e4, 1.0, 0, 1, 32, 258, th, nullptr, nullptr) == SRT_ERR_INVALID);
    EXPECT(srt_rope_inv_freq(SRT_ROPE_NONE, -1.0, 1.0, 0, 1, 32, 128, th, nullptr, nullptr) == SRT_ERR_INVALID);
    th[3] = NAN;
    EXPECT(srt_rope_cos_sin(th, 128, 1.0, 16, (float*)fake(0), nullptr) == SRT_ERR_INVALID);
    EXPECT(srt_rope_cos_sin(th, 128, 1.0, 0, (float*)fake(0), nullptr) == SRT_ERR_INVALID);
    EXPECT(srt_status_string(99) != nullptr && std::strlen(srt_last_error()) < 512);
  }
  // ---- rope_apply
  EXPECT(srt_rope_apply(fake(1), fake(1), SRT_BF16, 2, 8, 100, 128, 5, (float*)fake(0), 105, 0, nullptr) == SRT_OK);
  EXPECT(srt_rope_apply(fake(1), fake(2), SRT_F32, 1, 1, 100, 64, 6, (float*)fake(0), 105, 1, nullptr) ==
         SRT_ERR_INVALID);
  EXPECT(srt_rope_apply(fake(1), (char*)fake(2) + 8, SRT_BF16, 1, 1, 10, 128, 0, (float*)fake(0), 16, 0, nullptr) ==
         SRT_ERR_INVALID);
  EXPECT(srt_rope_apply(fake(1), fake(2), SRT_BF16, 1, 1, 10, 40, 0, (float*)fake(0), 16, 1, nullptr) ==
         SRT_ERR_UNSUPPORTED);
  // ---- prefill: every flag combination, fp32 and bf16, merge state off
  for (int dtype : {SRT_F32, SRT_BF16}) {
    const int D = dtype == SRT_BF16 ? 128 : 64;
    for (int flags = 0; flags < 8; ++flags) {
      const bool tab = (flags & 3) != 0;
      const int st = srt_attn_prefill(fake(1), fake(2), fake(3), dtype, 2, 8, 2, 300, 500, D, 300LL * D, 500LL * D,
                                      200, 0, 1, flags == 5 ? 64 : 0, 4, 0.1f, tab ? (float*)fake(0) : nullptr,
                                      tab ? 1000 : 0, flags, fake(4), SRT_F32, 300LL * D, (float*)fake(5), 300,
                                      flags == 3 ? fake(6) : nullptr, nullptr);
      EXPECT(st == SRT_OK);
    }
  }
  EXPECT(srt_attn_prefill(fake(1), fake(2), fake(3), SRT_BF16, 1, 8, 2, 64, 64, 128, 64 * 128 + 4, 64 * 128, 0, 0, 1,
                          0, 0, 0.1f, nullptr, 0, 0, fake(4), SRT_BF16, 64 * 128, nullptr, 0, nullptr, nullptr) ==
         SRT_ERR_INVALID);
  EXPECT(srt_attn_prefill(fake(1), fake(2), fake(3), SRT_BF16, 1, 8, 2, 64, 64, 128, 64 * 128, 64 * 128, 0, 0, 1, 0,
                          0, 0.1f, (float*)fake(0), 32, SRT_ROTATE_Q, fake(4), SRT_BF16, 64 * 128, nullptr, 0,
                          nullptr, nullptr) == SRT_ERR_INVALID);
  // a scheduling block off an 8-byte boundary
  EXPECT(srt_attn_prefill(fake(1), fake(2), fake(3), SRT_BF16, 1, 8, 2, 64, 64, 128, 64 * 128, 64 * 128, 0, 0, 1, 0,
                          0, 0.1f, nullptr, 0, 0, fake(4), SRT_BF16, 64 * 128, nullptr, 0,
                          static_cast<char*>(fake(6)) + 4, nullptr) == SRT_ERR_INVALID);
  EXPECT(srt_attn_prefill(fake(1), fake(2), fake(3), SRT_BF16, 1, 6, 4, 64, 64, 128, 64 * 128, 64 * 128, 0, 0, 1, 0,
                          0, 0.1f, nullptr, 0, 0, fake(4), SRT_BF16, 64 * 128, nullptr, 0, nullptr, nullptr) ==
         SRT_ERR_INVALID);
  EXPECT(srt_attn_prefill(fake(1), fake(2), fake(3), SRT_BF16, 1, 24, 8, 64, 64, 128, 64 * 128, 64 * 128, 0, 0, 1, 0,
                          0, 0.1f, nullptr, 0, 0, fake(4), SRT_BF16, 64 * 128, nullptr, 0, nullptr, nullptr) ==
         SRT_ERR_UNSUPPORTED);
  // ---- merge
  EXPECT(srt_attn_merge_states(fake(1), (float*)fake(2), fake(3), (float*)fake(4), SRT_F32, 1024, fake(1), SRT_F32,
                               1024, (float*)fake(2), 8, 2, 4, 8, 128, nullptr) == SRT_OK);
  EXPECT(srt_attn_merge_states(fake(1), (float*)fake(2), fake(3), (float*)fake(4), SRT_F32, 1024, fake(1), SRT_BF16,
                               1024, (float*)fake(2), 8, 2, 4, 8, 128, nullptr) == SRT_ERR_INVALID);
  // ---- decode, with a workspace and without
  {
    size_t n = 0;
    EXPECT(srt_attn_decode_workspace_size(16, 32, 128, 64, &n) == SRT_OK && n == 16ull * 32 * 64 * 129 * 4);
    EXPECT(srt_attn_decode_splitk(fake(1), fake(2), fake(3), SRT_BF16, 16, 32, 8, 131072, 128, nullptr, 64, 0.1f,
                                  (float*)fake(0), 131072, 0, 0, 0, fake(4), n, fake(5), (float*)fake(6), nullptr) ==
           SRT_OK);
    EXPECT(srt_attn_decode_splitk(fake(1), fake(2), fake(3), SRT_BF16, 16, 32, 8, 131072, 128, nullptr, 64, 0.1f,
                                  (float*)fake(0), 131072, 0, 4096, 4, fake(4), n - 1, fake(5), nullptr, nullptr) ==
           SRT_ERR_WORKSPACE);
    EXPECT(srt_attn_decode_splitk_noalloc(fake(1), fake(2), fake(3), SRT_BF16, 16, 32, 8, 131072, 128, nullptr, 64,
                                          0.1f, (float*)fake(0), 131072, 1, 4096, 4, fake(5), nullptr, nullptr) ==
           SRT_OK);
    EXPECT(srt_attn_decode_splitk_noalloc(fake(1), fake(2), fake(3), SRT_BF16, 64, 32, 8, 1024, 128, nullptr, 64,
                                          0.1f, nullptr, 0, 0, 0, 0, fake(5), nullptr, nullptr) == SRT_ERR_WORKSPACE);
    EXPECT(srt_attn_decode_noalloc_max_workspace() == srt::kDecodeScratchBytes);
  }
  // ---- backward
  for (int flags = 0; flags < 8; ++flags) {
    size_t n = 0;
    EXPECT(srt_attn_backward_workspace_size(SRT_BF16, 1, 8, 2, 300, 300, 128, flags, &n) == SRT_OK);
    std::vector<char> dummy(1);
    EXPECT(srt_attn_backward(fake(1), fake(2), fake(3), fake(4), fake(5), (float*)fake(6), SRT_BF16, 1, 8, 2, 300,
                             300, 128, 0, 0, 1, 0, 0, 0.1f, (flags & 3) ? (float*)fake(0) : nullptr, 300, flags,
                             fake(7), n, (float*)fake(8), (float*)fake(9), (float*)fake(10), nullptr) == SRT_OK);
  }
  // ---- ring: every partition, device count, window, one device or all
  for (int part : {SRT_PART_CONTIGUOUS, SRT_PART_STRIPED, SRT_PART_ZIGZAG}) {
    for (int P : {1, 2, 4, 8}) {
      for (int window : {0, 5, 40}) {
        if (window && part == SRT_PART_STRIPED) continue;
        for (int dev = -1; dev < P; ++dev) {
          const int N = 48 * P;
          size_t n = 0;
          EXPECT(srt_attn_ring_workspace_size(1, 4, 2, N, 128, SRT_BF16, P, part, 3, &n) == SRT_OK);
          EXPECT(srt_attn_ring_prefill(fake(1), fake(2), fake(3), SRT_BF16, 1, 4, 2, N, 128, P, part, dev, window, 3,
                                       0.1f, (float*)fake(0), N, 3, fake(4), n, fake(5), (float*)fake(6), nullptr) ==
                 SRT_OK);
          EXPECT(srt_attn_ring_prefill(fake(1), fake(2), fake(3), SRT_BF16, 1, 4, 2, N, 128, P, part, dev, window, 3,
                                       0.1f, (float*)fake(0), N, 3, fake(4), n - 1, fake(5), nullptr, nullptr) ==
                 SRT_ERR_WORKSPACE);
        }
      }
    }
  }
  EXPECT(srt_attn_ring_prefill(fake(1), fake(2), fake(3), SRT_BF16, 1, 4, 2, 100, 128, 8, SRT_PART_ZIGZAG, -1, 0, 0,
                               0.1f, nullptr, 0, 0, fake(4), 1 << 30, fake(5), nullptr, nullptr) == SRT_ERR_INVALID);
  printf("launches %lld failures %d\n", g_launches, g_fail);
  return g_fail == 0 && g_launches > 0 ? 0 : 1;
}
