// Host-side checks of the C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// against a host-only build of the library (no device code, no GPU needed): workspace
// sizing, argument validation and the refusal paths of every entry point, each of which
// must return before any device call.  Device pointers are aligned stand-in addresses
// that the host code must never dereference (a dereference faults here).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "spec_verify.h"

static int g_failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                    \
    }                                                                  \
  } while (0)

template <typename T>
static T *fake(uintptr_t addr) {
  return reinterpret_cast<T *>(addr);
}

static sv_weights weights(int d = 4096, int d_ff = 12288, int V = 151936, bool mlp = true) {
  sv_weights w;
  std::memset(&w, 0, sizeof(w));
  const uintptr_t z = 1u << 20;
  w.w_gate = mlp ? fake<void>(z) : nullptr;
  w.w_up = mlp ? fake<void>(2 * z) : nullptr;
  w.w_down = mlp ? fake<void>(3 * z) : nullptr;
  w.w_lm = fake<void>(4 * z);
  w.d = d;
  w.d_ff = mlp ? d_ff : 0;
  w.V = V;
  w.wtype = SV_WEIGHTS_BF16;
  return w;
}

static sv_weights weights_fp8(bool mlp = true) {
  sv_weights w = weights(4096, 12288, 151936, mlp);
  const uintptr_t z = 1u << 22;
  w.wtype = SV_WEIGHTS_FP8_E4M3;
  w.s_lm = fake<float>(5 * z);
  if (mlp) {
    w.s_gate = fake<float>(6 * z);
    w.s_up = fake<float>(7 * z);
    w.s_down = fake<float>(8 * z);
  }
  return w;
}

static sv_outputs outputs() {
  sv_outputs o;
  std::memset(&o, 0, sizeof(o));
  const uintptr_t z = 1u << 24;
  o.accepted_len = fake<int32_t>(z);
  o.emitted = fake<int32_t>(z + 4096);
  o.tau = fake<float>(z + 8192);
  return o;
}

static sv_cache cache() {
  sv_cache c;
  std::memset(&c, 0, sizeof(c));
  const uintptr_t z = 1u << 20;
  c.kv = fake<void>(z);
  c.layer_stride = 1 << 24;
  c.half_stride = 1 << 23;
  c.n_layers = 4;
  c.block_size = 16;
  c.entry_bytes = 2048;
  c.max_blocks = 64;
  c.n_blocks = 1024;
  c.block_table = fake<const int32_t>(2 * z);
  c.seq_len = fake<int32_t>(3 * z);
  c.rec_state = fake<void>(4 * z);
  c.rec_snap = fake<const void>(5 * z);
  c.rec_bytes = 1 << 16;
  return c;
}

static void workspace_sizes() {
  const sv_weights w = weights();
  const size_t g = sv_workspace_bytes(SV_MODE_GREEDY, 1, 15, &w);
  const size_t s = sv_workspace_bytes(SV_MODE_SAMPLE, 1, 15, &w);
  const size_t sch = sv_workspace_bytes(SV_MODE_SCHEDULED, 64, 15, &w);
  const size_t p = sv_workspace_bytes(SV_MODE_PROPOSE, 15, 0, &w);
  EXPECT(g > 0 && g < s);
  EXPECT(s >= 31ull * 151936 * 4);
  EXPECT(sch >= 64ull * 15 * 151936 * 4);
  EXPECT(p >= 15ull * 151936 * 4);
  EXPECT(g % 256 == 0 && s % 256 == 0 && sch % 256 == 0 && p % 256 == 0);
  EXPECT(sv_workspace_bytes(SV_MODE_GREEDY, 128, 7, &w) > g);
  // every batch size of the scheduled plan, including the ones with small-row plans
  for (int B = 1; B <= 128; B += 9)
    for (int K = 0; K <= 15; K += 5) EXPECT(sv_workspace_bytes(SV_MODE_SCHEDULED, B, K, &w) > 0);
  // bad shapes
  const sv_weights bad[] = {weights(100), weights(0), weights(4096, 100), weights(4096, 12288, 0),
                            weights(4096, 12288, (1 << 19) + 1)};
  for (const sv_weights &b : bad) EXPECT(sv_workspace_bytes(SV_MODE_SAMPLE, 1, 4, &b) == 0);
  sv_weights nomlp_ff = weights(4096, 12288, 151936, false);
  nomlp_ff.d_ff = 12288;
  EXPECT(sv_workspace_bytes(SV_MODE_SAMPLE, 1, 4, &nomlp_ff) == 0);
  EXPECT(sv_workspace_bytes(7, 1, 4, &w) == 0);
  EXPECT(sv_workspace_bytes(SV_MODE_SAMPLE, 0, 4, &w) == 0);
  EXPECT(sv_workspace_bytes(SV_MODE_SAMPLE, 1, 4, nullptr) == 0);
  // FP8 rules
  const sv_weights w8 = weights_fp8();
  EXPECT(sv_workspace_bytes(SV_MODE_SAMPLE, 1, 15, &w8) > 0);
  EXPECT(sv_workspace_bytes(SV_MODE_GREEDY, 8, 7, &w8) == 0);
  sv_weights w8b = w8;
  w8b.s_down = nullptr;
  EXPECT(sv_workspace_bytes(SV_MODE_SAMPLE, 1, 15, &w8b) == 0);
  const sv_weights w8n = weights_fp8(false);
  EXPECT(sv_workspace_bytes(SV_MODE_SAMPLE, 1, 15, &w8n) > 0);
}

static void invalid_arguments() {
  const sv_weights w = weights();
  sv_outputs o = outputs();
  const uint16_t *P16 = fake<const uint16_t>(1u << 28);
  const int32_t *P32 = fake<const int32_t>(1u << 28);
  const float *PF = fake<const float>(1u << 28);
  void *ws = fake<void>(1u << 30);
  const size_t wsn = 1ull << 40;
  EXPECT(spec_verify_greedy(&w, nullptr, P32, 1, 4, ws, wsn, &o, nullptr) == SV_EINVAL);
  EXPECT(spec_verify_greedy(nullptr, P16, P32, 1, 4, ws, wsn, &o, nullptr) == SV_EINVAL);
  EXPECT(spec_verify_greedy(&w, P16, P32, 1, 4, ws, wsn, nullptr, nullptr) == SV_EINVAL);
  EXPECT(spec_verify_greedy(&w, P16, nullptr, 1, 4, ws, wsn, &o, nullptr) == SV_EINVAL);
  EXPECT(spec_verify_greedy(&w, fake<const uint16_t>((1u << 28) + 2), P32, 1, 4, ws, wsn, &o, nullptr) == SV_EINVAL);
  EXPECT(spec_verify_greedy(&w, P16, P32, 0, 4, ws, wsn, &o, nullptr) == SV_EINVAL);
  EXPECT(spec_verify_greedy(&w, P16, P32, 1, -1, ws, wsn, &o, nullptr) == SV_EINVAL);
  const float Ts[] = {0.f, -1.f, INFINITY, NAN};
  for (float T : Ts) {
    EXPECT(spec_verify_sample(&w, P16, P16, P32, PF, T, 1, 4, ws, wsn, &o, nullptr) == SV_EINVAL);
    EXPECT(spec_verify_sample_noalloc(&w, P16, P16, P32, PF, T, 1, 15, &o, nullptr) == SV_EINVAL);
    if (T != 0.f)  // T = 0 is the tree's greedy rule
      EXPECT(spec_verify_tree(&w, P16, P16, P32, P32, PF, T, 1, 4, ws, wsn, &o, nullptr, -1, nullptr) == SV_EINVAL);
  }
  EXPECT(spec_verify_sample(&w, P16, P16, P32, nullptr, 1.f, 1, 4, ws, wsn, &o, nullptr) == SV_EINVAL);
  EXPECT(spec_verify_sample(&w, P16, nullptr, P32, PF, 1.f, 1, 4, ws, wsn, &o, nullptr) == SV_EINVAL);
  EXPECT(spec_verify_scheduled(&w, P16, P16, P32, PF, 1.f, 0.3f, 3, 4, 15, ws, wsn, &o, nullptr) == SV_EINVAL);
  const float thrs[] = {0.f, 1.5f, NAN};
  for (float thr : thrs)
    EXPECT(spec_verify_scheduled(&w, P16, P16, P32, PF, 1.f, thr, 64, 4, 15, ws, wsn, &o, nullptr) == SV_EINVAL);
  EXPECT(spec_verify_scheduled(&w, P16, P16, P32, PF, 1.f, 0.3f, 16384, 8193, 1, ws, wsn, &o, nullptr) == SV_EINVAL);
  EXPECT(spec_verify_scheduled(&w, P16, P16, P32, PF, 1.f, 0.3f, 16384, 8193, 0, ws, wsn, &o, nullptr) == SV_EINVAL);
  sv_outputs o2 = outputs();
  o2.accepted_len = nullptr;
  EXPECT(spec_verify_greedy(&w, P16, P32, 1, 4, ws, wsn, &o2, nullptr) == SV_EINVAL);
  int32_t *D = fake<int32_t>(1u << 28);
  EXPECT(spec_draft_propose(&w, P16, nullptr, 1.f, 4, ws, wsn, D, nullptr, nullptr) == SV_EINVAL);
  EXPECT(spec_draft_propose(&w, P16, PF, -1.f, 4, ws, wsn, D, nullptr, nullptr) == SV_EINVAL);
  EXPECT(spec_draft_propose(&w, P16, PF, 1.f, 0, ws, wsn, D, nullptr, nullptr) == SV_EINVAL);
}

static void small_workspace() {
  const sv_weights w = weights();
  sv_outputs o = outputs();
  const uint16_t *P16 = fake<const uint16_t>(1u << 28);
  const int32_t *P32 = fake<const int32_t>(1u << 28);
  const float *PF = fake<const float>(1u << 28);
  void *ws = fake<void>(1u << 30);
  size_t need = sv_workspace_bytes(SV_MODE_SAMPLE, 1, 15, &w);
  EXPECT(spec_verify_sample(&w, P16, P16, P32, PF, 1.f, 1, 15, ws, need - 256, &o, nullptr) == SV_EWORKSPACE);
  need = sv_workspace_bytes(SV_MODE_GREEDY, 2, 7, &w);
  EXPECT(spec_verify_greedy(&w, P16, P32, 2, 7, ws, need - 1, &o, nullptr) == SV_EWORKSPACE);
  need = sv_workspace_bytes(SV_MODE_SCHEDULED, 64, 15, &w);
  // the workspace size covers any budget; at the largest (B * (Kmax + 1)) it is exact
  EXPECT(spec_verify_scheduled(&w, P16, P16, P32, PF, 1.f, 0.3f, 64 * 16, 64, 15, ws, need - 256, &o, nullptr) ==
         SV_EWORKSPACE);
  need = sv_workspace_bytes(SV_MODE_PROPOSE, 15, 0, &w);
  EXPECT(spec_draft_propose(&w, P16, PF, 1.f, 15, ws, need - 1, fake<int32_t>(1u << 28), nullptr, nullptr) ==
         SV_EWORKSPACE);
  EXPECT(spec_verify_greedy(&w, P16, P32, 2, 7, fake<void>((1u << 30) + 16), 1ull << 40, &o, nullptr) == SV_EINVAL);
  // the allocation-free call: sizes beyond its static scratch
  EXPECT(spec_verify_sample_noalloc(&w, P16, P16, P32, PF, 1.f, 8, 7, &o, nullptr) == SV_ESCRATCH);
  EXPECT(spec_verify_sample_noalloc(&w, nullptr, P16, P32, PF, 1.f, 1, 15, &o, nullptr) == SV_EINVAL);
}

static void commit_rejections() {
  const int32_t *acc = fake<const int32_t>(6u << 20);
  sv_cache good = cache();
  EXPECT(spec_commit(nullptr, acc, nullptr, nullptr, 8, 15, nullptr, nullptr) == SV_EINVAL);
  EXPECT(spec_commit(&good, nullptr, nullptr, nullptr, 8, 15, nullptr, nullptr) == SV_EINVAL);
  EXPECT(spec_commit(&good, acc, nullptr, nullptr, 0, 15, nullptr, nullptr) == SV_EINVAL);
  EXPECT(spec_commit(&good, acc, nullptr, nullptr, 8, -1, nullptr, nullptr) == SV_EINVAL);
  EXPECT(spec_commit(&good, acc, nullptr, nullptr, 8, 64, nullptr, nullptr) == SV_EINVAL);
  for (int k = 0; k < 12; ++k) {
    sv_cache c = cache();
    switch (k) {
      case 0: c.seq_len = nullptr; break;
      case 1: c.entry_bytes = 24; break;
      case 2: c.entry_bytes = 0; break;
      case 3: c.block_size = 0; break;
      case 4: c.kv = fake<void>((1u << 20) + 8); break;
      case 5: c.block_table = nullptr; break;
      case 6: c.n_blocks = 0; break;
      case 7: c.layer_stride = (1 << 24) + 4; break;
      case 8: c.rec_bytes = 100; break;
      case 9: c.rec_snap = nullptr; break;
      case 10: c.rec_state = fake<void>((1u << 22) + 4); break;
      default: c.n_layers = -1; break;
    }
    EXPECT(spec_commit(&c, acc, nullptr, nullptr, 8, 15, nullptr, nullptr) == SV_EINVAL);
  }
}

static void strings() {
  EXPECT(std::strstr(sv_version(), "gfx950") != nullptr);
  EXPECT(std::strcmp(sv_strerror(SV_EINVAL), "invalid argument") == 0);
  EXPECT(std::strcmp(sv_strerror(SV_EWORKSPACE), "workspace too small") == 0);
  for (int c = -10; c <= 10; ++c) EXPECT(sv_strerror(c) != nullptr);
  EXPECT(sv_last_hip_error() != nullptr);
}

int main() {
  workspace_sizes();
  invalid_arguments();
  small_workspace();
  commit_rejections();
  strings();
  if (g_failures) {
    std::fprintf(stderr, "%d host ABI check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("host ABI checks passed\n");
  return 0;
}
