// Sweep of the library's host entry points under AddressSanitizer and
// UndefinedBehaviorSanitizer, with the kernel launchers replaced by checking
// stand-ins (stub_launch.cpp): every size query, plan and call over the
// weight formats, activation formats, shapes at and beyond the documented
// limits, and explicit tunings (valid and invalid, drawn from a fixed
// generator).  Consistency checked on the way:
//   * a call succeeds exactly when its plan and workspace query succeed, and
//     gives the same status as the plan otherwise;
//   * a call with one byte less workspace than its query fails with
//     HM_ERR_WORKSPACE (when the query is not 0);
//   * plan texts are NUL-terminated within any buffer length.
// Device pointers are fake aligned addresses: the stand-ins never touch them.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hm.h"

namespace hm { extern long g_launches; }

static void* dev(uintptr_t slot) { return reinterpret_cast<void*>((uintptr_t)0x7f0000000000ull + slot * 0x100000000ull); }
static long g_checks = 0;

#define EXPECT(cond, ...)                                    \
  do {                                                       \
    ++g_checks;                                              \
    if (!(cond)) {                                           \
      fprintf(stderr, "%s:%d: ", __FILE__, __LINE__);        \
      fprintf(stderr, __VA_ARGS__);                          \
      fprintf(stderr, "\n");                                 \
      exit(1);                                               \
    }                                                        \
  } while (0)

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static int32_t draw(int32_t lo, int32_t hi) {  // inclusive, splitmix64
  g_rng += 0x9E3779B97F4A7C15ull;
  uint64_t z = g_rng;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return lo + (int32_t)(z % (uint64_t)(hi - lo + 1));
}

static hm_tuning random_tuning() {
  hm_tuning t;
  memset(&t, 0, sizeof t);
  t.abi = draw(0, 20) == 0 ? HM_ABI_VERSION + 1 : HM_ABI_VERSION;
  t.path = draw(-1, 5);
  static const int32_t ks[] = {0, 1, 2, 3, 4, 8, 16};
  t.stream_ks = ks[draw(0, 6)];
  t.stream_nbw = draw(0, 3);
  t.stream_splits = draw(0, 9) == 0 ? draw(-2, 1 << 20) : draw(0, 8);
  static const int32_t waves[] = {0, 4, 8, 5};
  t.stream_waves = waves[draw(0, 3)];
  static const int32_t rows[] = {0, 16, 32, 8};
  t.moe_stream_rows = rows[draw(0, 3)];
  t.moe_stream_max = draw(-1, 5000);
  t.moe_stream_nbw = draw(0, 3);
  t.moe_stream_ks = ks[draw(0, 6)];
  t.moe_stream_lds_kb = draw(0, 3) == 0 ? draw(-5, 200) : 0;
  t.moe_big_min = draw(-2, 300);
  t.moe_tile = draw(-1, 3);
  return t;
}

static void check_plan_text(hm_status st, const char* buf, size_t len) {
  if (st == HM_OK && len > 0) EXPECT(memchr(buf, 0, len) != nullptr, "plan text not terminated");
}

static void dense_sweep(const hm_wdesc& d) {
  static const int64_t ms[] = {0, 1, 2, 15, 16, 17, 31, 32, 64, 127, 128, 129, 255, 256, 257, 1000, 1024,
                               4096, 4097, 65536, (int64_t)1 << 24, (int64_t)1 << 31, -1};
  for (int32_t afmt = -1; afmt <= 3; ++afmt) {
    for (int64_t m : ms) {
      for (int rep = 0; rep < 6; ++rep) {
        hm_tuning tt = random_tuning();
        const hm_tuning* t = rep == 0 ? nullptr : &tt;
        size_t ws = 0;
        const hm_status s_ws = hm_gemm_workspace_size(&d, afmt, m, t, &ws);
        char buf[512];
        const hm_status s_plan = hm_gemm_plan(&d, afmt, m, t, buf, sizeof buf);
        check_plan_text(s_plan, buf, sizeof buf);
        const size_t lens[] = {1, 7, 0};
        const size_t len = lens[rep % 3];
        char small[8];
        const hm_status s_small = hm_gemm_plan(&d, afmt, m, t, len ? small : nullptr, len);
        check_plan_text(s_small, small, len);
        const void* xs = dev(3);
        const hm_status s = hm_gemm(&d, dev(1), afmt, dev(2), xs, m, (uint16_t*)dev(4), ws ? dev(5) : nullptr,
                                    ws, t, nullptr);
        if (m == 0 && s_ws == HM_OK) {
          EXPECT(s == HM_OK, "m = 0 call: %d", (int)s);
          continue;
        }
        if (s_ws == HM_OK && s_plan == HM_OK) {
          EXPECT(s == HM_OK, "gemm wfmt %d afmt %d n %lld k %lld m %lld: plan ok, call %d", d.wfmt, afmt,
                 (long long)d.n, (long long)d.k, (long long)m, (int)s);
          if (ws > 0) {
            const hm_status s2 = hm_gemm(&d, dev(1), afmt, dev(2), xs, m, (uint16_t*)dev(4), dev(5), ws - 1, t,
                                         nullptr);
            EXPECT(s2 == HM_ERR_WORKSPACE, "short workspace: %d", (int)s2);
          }
        } else {
          EXPECT(s != HM_OK, "gemm wfmt %d afmt %d m %lld: plan/size failed (%d/%d) but the call ran",
                 d.wfmt, afmt, (long long)m, (int)s_plan, (int)s_ws);
          if (s_plan != HM_OK) EXPECT(s == s_plan || s_ws != HM_OK, "status %d vs plan %d", (int)s, (int)s_plan);
        }
      }
    }
  }
}

static void moe_sweep(const hm_wdesc& d) {
  static const int64_t ts[] = {0, 1, 3, 64, 1024, 8192, 16384, (int64_t)1 << 20, (int64_t)1 << 28, -1};
  static const int32_t topks[] = {1, 2, 8, 0};
  for (int32_t afmt = 0; afmt <= 2; ++afmt) {
    for (int64_t t : ts) {
      for (int32_t topk : topks) {
        for (int32_t rp = 0; rp <= 2; ++rp) {
          for (int rep = 0; rep < 3; ++rep) {
            hm_tuning tt = random_tuning();
            const hm_tuning* tn = rep == 0 ? nullptr : &tt;
            size_t ws = 0;
            const hm_status s_ws = hm_moe_gemm_workspace_size(&d, afmt, t, topk, tn, &ws);
            char buf[512];
            const hm_status s_plan = hm_moe_gemm_plan(&d, afmt, t, topk, rp, tn, buf, sizeof buf);
            check_plan_text(s_plan, buf, sizeof buf);
            const hm_status s = hm_moe_gemm(&d, dev(1), afmt, dev(2), dev(3), rp, t, topk, (const int32_t*)dev(6),
                                            (const int32_t*)dev(7), (uint16_t*)dev(4), dev(5), ws, tn, nullptr);
            if (t == 0 && s_ws == HM_OK && s_plan == HM_OK) {
              EXPECT(s == HM_OK, "moe t = 0: %d", (int)s);
              continue;
            }
            if (s_ws == HM_OK && s_plan == HM_OK) {
              EXPECT(s == HM_OK, "moe wfmt %d afmt %d t %lld topk %d rp %d: plan ok, call %d", d.wfmt, afmt,
                     (long long)t, topk, rp, (int)s);
              const hm_status s2 = hm_moe_gemm(&d, dev(1), afmt, dev(2), dev(3), rp, t, topk, (const int32_t*)dev(6),
                                               (const int32_t*)dev(7), (uint16_t*)dev(4), dev(5), ws - 1, tn,
                                               nullptr);
              EXPECT(s2 == HM_ERR_WORKSPACE, "moe short workspace: %d", (int)s2);
            } else {
              EXPECT(s != HM_OK || t == 0, "moe wfmt %d afmt %d t %lld topk %d rp %d: plan/size failed (%d/%d) but the call ran", d.wfmt, afmt, (long long)t, topk, rp, (int)s_plan, (int)s_ws);
            }
            // the gated variant: same schedule, its own plan
            {
              const hm_status g_plan = hm_moe_gemm_gated_plan(&d, afmt, t, topk, rp, tn, buf, sizeof buf);
              check_plan_text(g_plan, buf, sizeof buf);
              const hm_status g = hm_moe_gemm_gated(&d, dev(1), afmt, dev(2), dev(3), rp, t, topk,
                                                    (const int32_t*)dev(6), (const int32_t*)dev(7),
                                                    (uint16_t*)dev(4), dev(5), ws, tn, nullptr);
              if (s_ws == HM_OK && g_plan == HM_OK)
                EXPECT(g == HM_OK, "gated moe wfmt %d n %lld t %lld: plan ok, call %d", d.wfmt, (long long)d.n,
                       (long long)t, (int)g);
              else
                EXPECT(g != HM_OK || t == 0, "gated moe: plan/size failed (%d/%d) but the call ran", (int)g_plan,
                       (int)s_ws);
              if (g_plan == HM_OK) EXPECT(d.n % 32 == 0, "gated plan accepted n = %lld", (long long)d.n);
            }
            // the allocation-free variant: its device lookup may fail here (no GPU)
            (void)hm_moe_gemm_static(&d, dev(1), afmt, dev(2), dev(3), rp, t, topk, (const int32_t*)dev(6),
                                     (const int32_t*)dev(7), (uint16_t*)dev(4), tn, nullptr);
          }
        }
      }
    }
  }
}

int main() {
  static const int32_t wfmts[] = {-1, 0, 1, 2, 3, 4, 5, 6, 7};
  static const int64_t ns[] = {1, 16, 17, 1000, 4096, 7168, 14336, 0};
  static const int64_t ks[] = {128, 256, 2048, 4096, 7168, 1 << 20, (1 << 20) + 128, 100, 0};
  static const int32_t es[] = {1, 8, 256, 512, 513, 0};
  static const int32_t groups[] = {128, 32, 64};
  long descs = 0;
  for (int32_t wf : wfmts)
    for (int64_t n : ns)
      for (int64_t k : ks)
        for (int32_t e : es)
          for (int32_t g : groups) {
            hm_wdesc d;
            memset(&d, 0, sizeof d);
            d.abi = HM_ABI_VERSION;
            d.wfmt = wf;
            d.group = g;
            d.num_experts = e;
            d.n = n;
            d.k = k;
            size_t bytes = 0;
            const hm_status st = hm_transform_size(&d, &bytes);
            const hm_status tr = hm_transform(&d, (const uint8_t*)dev(1), dev(2), (const uint8_t*)dev(3), dev(4),
                                              bytes, nullptr);
            const hm_status trg = hm_transform_gated(&d, (const uint8_t*)dev(1), dev(2), (const uint8_t*)dev(3),
                                                     dev(4), bytes, nullptr);
            if (st != HM_OK) {
              EXPECT(tr != HM_OK && trg != HM_OK, "transform ran on a rejected descriptor");
              continue;
            }
            EXPECT((trg == HM_OK) == (tr == HM_OK && n % 32 == 0), "gated transform status %d", (int)trg);
            ++descs;
            EXPECT(bytes > 0 && bytes % 256 == 0, "transform size %zu", bytes);
            if (bytes > 1) EXPECT(hm_transform(&d, (const uint8_t*)dev(1), dev(2), (const uint8_t*)dev(3), dev(4),
                                               bytes - 1, nullptr) != HM_OK, "short weight buffer accepted");
            for (int32_t ex = -1; ex <= e; ++ex) {
              const hm_status dq = hm_dequant(&d, dev(1), bytes, ex, (float*)dev(2), nullptr);
              EXPECT((dq == HM_OK) == (ex >= 0 && ex < e), "dequant expert %d of %d: %d", ex, e, (int)dq);
            }
            if (k <= 7168 && n <= 14336) {
              if (e == 1) dense_sweep(d);
              if (e == 8 || e == 256) moe_sweep(d);
            }
          }
  // sort, row quantizers, block steps, read probe
  for (int64_t t : {(int64_t)0, (int64_t)1, (int64_t)512, (int64_t)4096, (int64_t)16384, (int64_t)1 << 28})
    for (int32_t topk : {1, 8, 9})
      for (int32_t e : {1, 8, 256, 512, 513}) {
        size_t ws = 0;
        const hm_status sw = hm_moe_sort_workspace_size(t, topk, e, &ws);
        const hm_status s = hm_moe_sort((const int32_t*)dev(1), t, topk, e, (int32_t*)dev(2), (int32_t*)dev(3),
                                        (int32_t*)dev(4), ws ? dev(5) : nullptr, ws, nullptr);
        EXPECT((sw == HM_OK) == (s == HM_OK) || (t == 0 && s == HM_OK), "sort t %lld topk %d e %d: %d/%d",
               (long long)t, topk, e, (int)sw, (int)s);
        if (sw == HM_OK && ws > 0)
          EXPECT(hm_moe_sort((const int32_t*)dev(1), t, topk, e, (int32_t*)dev(2), (int32_t*)dev(3),
                             (int32_t*)dev(4), dev(5), ws - 1, nullptr) == HM_ERR_WORKSPACE, "sort short ws");
      }
  for (int64_t m : {(int64_t)0, (int64_t)1, (int64_t)4097, (int64_t)-1})
    for (int64_t k : {(int64_t)1, (int64_t)32, (int64_t)33, (int64_t)7168, (int64_t)0}) {
      (void)hm_quant_fp8_rows((const uint16_t*)dev(1), m, k, (uint8_t*)dev(2), (float*)dev(3), nullptr);
      (void)hm_quant_mxfp4_rows((const uint16_t*)dev(1), m, k, (uint8_t*)dev(2), (uint8_t*)dev(3), nullptr);
      (void)hm_silu_mul((const uint16_t*)dev(1), m, k, (uint16_t*)dev(2), nullptr);
      (void)hm_silu_mul_fp8((const uint16_t*)dev(1), m, k, (uint8_t*)dev(2), (float*)dev(3), nullptr);
      for (int32_t topk : {0, 1, 8})
        (void)hm_moe_combine((const uint16_t*)dev(1), (const float*)dev(2), m, topk, k, (uint16_t*)dev(3), nullptr);
      (void)hm_read_probe(dev(1), m * 4096, (int32_t)k, 4, (uint32_t*)dev(2), nullptr);
    }
  for (int32_t s = -1; s <= 10; ++s) EXPECT(hm_status_string(s) != nullptr, "status string");
  EXPECT(hm_moe_gemm_static_max_workspace() > 0, "static workspace size");
  printf("host sweep ok: %ld descriptors, %ld checks, %ld stub launches\n", descs, g_checks, hm::g_launches);
  return 0;
}
