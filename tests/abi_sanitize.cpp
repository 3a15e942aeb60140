// Host-side checks of the C-ABI front end (argument validation, split planning, launch
// arguments) built with the address and undefined-behaviour sanitizers. The kernel launchers
// are stubs here: they record the arguments the front end hands to them and succeed, so no call
// touches a device. Each case names the status it must return; the sanitizers report any
// overflow, out-of-bounds access or other undefined behaviour on the way.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "fa.h"
#include "fa_bwd_internal.h"
#include "fa_internal.h"

namespace {
int g_launches = 0;
fa::FwdArgs g_last;
int g_last_ncol = 0;
}  // namespace

// ---- stubs of the kernel side (same row and tile geometry as the kernels) -------------------
namespace fa {
int bf16_rows_per_block(int d, int64_t BH, int N) {
  if (d == 64 && BH * (((int64_t)N + 255) / 256) >= 256) return 256;   // tuned kernel
  if (d <= 64) return BH * (((int64_t)N + 127) / 128) >= 256 ? 128 : 64;
  return d == 128 ? 256 : (d <= 128 ? 256 : 128);
}
int f32_rows_per_block(int d) { return d <= 64 ? 32 : (d <= 128 ? 64 : 128); }
int bf16_split_rows_per_block(int d_pad) { return d_pad <= 64 ? 64 : (d_pad <= 128 ? 256 : 128); }
int bf16_split_key_tile(int d_pad) { return d_pad <= 128 ? 64 : 32; }
int f32_split_key_tile(int) { return 32; }
int bwd_rows_per_block() { return 128; }
static hipError_t record(const FwdArgs& a, int ncol) {
  ++g_launches;
  g_last = a;
  g_last_ncol = ncol;
  return hipSuccess;
}
hipError_t launch_bf16(const FwdArgs& a, int, bool, hipStream_t) { return record(a, 1); }
hipError_t launch_f32(const FwdArgs& a, int, bool, hipStream_t) { return record(a, 1); }
hipError_t launch_bf16_partial(const FwdArgs& a, int, bool, int ns, hipStream_t) { return record(a, ns); }
hipError_t launch_f32_partial(const FwdArgs& a, int, bool, int ns, hipStream_t) { return record(a, ns); }
hipError_t launch_merge(const FwdArgs& a, int, bool, int ns, bool, bool, hipStream_t) { return record(a, ns); }
hipError_t launch_bwd_bf16(const BwdArgs&, bool, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace fa

static int g_fail = 0;
static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    ++g_fail;
  }
}

int main() {
  const uintptr_t G = (uintptr_t)1 << 40;   // well-separated fake device addresses (never touched)
  void *q = (void*)G, *k = (void*)(2 * G), *v = (void*)(3 * G), *o = (void*)(4 * G);
  float* lse = (float*)(5 * G);
  const float nan = NAN, inf = INFINITY;
  struct Case { const char* what; int B, H, N, d; float scale; int causal; int want; };
  const Case cases[] = {
      {"ok small", 1, 1, 16, 64, 0.125f, 0, FA_OK},
      {"ok causal d=128", 2, 3, 1000, 128, 0.088f, 1, FA_OK},
      {"ok d=1", 1, 1, 3, 1, 1.0f, 0, FA_OK},
      {"ok d=256", 1, 2, 77, 256, -0.3f, 1, FA_OK},
      {"B=0", 0, 1, 16, 64, 0.125f, 0, FA_ERR_INVALID_ARG},
      {"H<0", 1, -5, 16, 64, 0.125f, 0, FA_ERR_INVALID_ARG},
      {"N=INT_MIN", 1, 1, INT_MIN, 64, 0.125f, 0, FA_ERR_INVALID_ARG},
      {"d=0", 1, 1, 16, 0, 0.125f, 0, FA_ERR_INVALID_ARG},
      {"causal=2", 1, 1, 16, 64, 0.125f, 2, FA_ERR_INVALID_ARG},
      {"scale nan", 1, 1, 16, 64, nan, 0, FA_ERR_INVALID_ARG},
      {"scale inf", 1, 1, 16, 64, inf, 0, FA_ERR_INVALID_ARG},
      {"d=257", 1, 1, 16, 257, 0.125f, 0, FA_ERR_UNSUPPORTED},
      {"d=INT_MAX", 1, 1, 16, INT_MAX, 0.125f, 0, FA_ERR_UNSUPPORTED},
      {"count > 2^62", INT_MAX, INT_MAX, INT_MAX, 128, 0.125f, 0, FA_ERR_INVALID_ARG},
      {"N*d >= 2^31", 1, 1, 1 << 24, 256, 0.125f, 0, FA_ERR_UNSUPPORTED},
      {"B*H overflows int", 65536, 65536, 1, 1, 1.0f, 0, FA_ERR_UNSUPPORTED},
      {"grid above INT_MAX", 1 << 16, 1 << 15, 1, 1, 1.0f, 0, FA_ERR_UNSUPPORTED},
  };
  for (const Case& c : cases) {
    char buf[160];
    snprintf(buf, sizeof buf, "fa_fwd %s", c.what);
    expect(buf, fa_fwd(q, k, v, o, lse, c.B, c.H, c.N, c.d, c.scale, c.causal, nullptr), c.want);
    snprintf(buf, sizeof buf, "fa_fwd_f32 %s", c.what);
    expect(buf, fa_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)o, lse, c.B, c.H, c.N, c.d,
                           c.scale, c.causal, nullptr), c.want);
    for (int ns : {0, 1, 7, 64}) {
      for (int dt : {FA_BF16, FA_F32}) {
        int nsplit = -1;
        size_t wb = 0;
        const int st = fa_fwd_splitkv_plan(c.B, c.H, c.N, c.d, dt, c.causal, ns, &nsplit, &wb);
        snprintf(buf, sizeof buf, "fa_fwd_splitkv %s ns=%d dt=%d", c.what, ns, dt);
        // the plan checks sizes only; the call checks pointers, scale and the plan
        const int want_call = (st != FA_OK) ? st : c.want;
        expect(buf, fa_fwd_splitkv(q, k, v, o, lse, c.B, c.H, c.N, c.d, c.scale, c.causal, dt, ns,
                                   (void*)(8 * G), wb, nullptr), want_call);
      }
    }
  }
  // pointers and overlaps
  expect("null q", fa_fwd(nullptr, k, v, o, lse, 1, 1, 16, 64, 0.125f, 0, nullptr), FA_ERR_INVALID_ARG);
  expect("o overlaps q", fa_fwd(q, k, v, (char*)q + 64, lse, 1, 1, 16, 64, 0.125f, 0, nullptr), FA_ERR_INVALID_ARG);
  expect("lse overlaps o", fa_fwd(q, k, v, o, (float*)((char*)o + 8), 1, 1, 16, 64, 0.125f, 0, nullptr),
         FA_ERR_INVALID_ARG);
  expect("q misaligned", fa_fwd((char*)q + 8, k, v, o, lse, 1, 1, 16, 64, 0.125f, 0, nullptr), FA_ERR_INVALID_ARG);
  expect("lse misaligned", fa_fwd(q, k, v, o, (float*)((char*)lse + 2), 1, 1, 16, 64, 0.125f, 0, nullptr),
         FA_ERR_INVALID_ARG);
  expect("splitkv small workspace",
         fa_fwd_splitkv(q, k, v, o, lse, 1, 1, 256, 64, 0.125f, 0, FA_F32, 8, (void*)(8 * G), 16, nullptr),
         FA_ERR_WORKSPACE);
  expect("splitkv misaligned workspace",
         fa_fwd_splitkv(q, k, v, o, lse, 1, 1, 256, 64, 0.125f, 0, FA_F32, 8, (void*)(8 * G + 4), 1 << 30, nullptr),
         FA_ERR_INVALID_ARG);
  // launch arguments the front end computes
  expect("headline shape", fa_fwd(q, k, v, o, lse, 1, 16, 8192, 128, 0.088f, 0, nullptr), FA_OK);
  if (g_last.BH != 16 || g_last.n_qtiles != 32 || g_last.N != 8192 || g_last.part_u != nullptr ||
      g_last.wg_shift != 0) {
    fprintf(stderr, "FAIL headline launch arguments: BH=%d n_qtiles=%d wg_shift=%d\n", g_last.BH, g_last.n_qtiles,
            g_last.wg_shift);
    ++g_fail;
  }
  // one head, 8 query tiles: packed onto one XCD (8 launched workgroups per work item)
  expect("single head fp32", fa_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)o, lse, 1, 1,
                                        256, 64, 0.125f, 0, nullptr), FA_OK);
  if (g_last.n_qtiles != 8 || g_last.wg_shift != 3) {
    fprintf(stderr, "FAIL single-head launch arguments: n_qtiles=%d wg_shift=%d\n", g_last.n_qtiles, g_last.wg_shift);
    ++g_fail;
  }
  // 8 heads or more, or more than 32 workgroups: not packed
  expect("eight heads", fa_fwd(q, k, v, o, lse, 2, 4, 256, 64, 0.125f, 0, nullptr), FA_OK);
  if (g_last.wg_shift != 0) {
    fprintf(stderr, "FAIL eight-head launch arguments: wg_shift=%d\n", g_last.wg_shift);
    ++g_fail;
  }
  expect("one long head", fa_fwd(q, k, v, o, lse, 1, 1, 2048, 128, 0.088f, 0, nullptr), FA_OK);
  if (g_last.n_qtiles != 8 || g_last.wg_shift != 0) {
    fprintf(stderr, "FAIL long-head launch arguments: n_qtiles=%d wg_shift=%d\n", g_last.n_qtiles, g_last.wg_shift);
    ++g_fail;
  }
  expect("one head, 64 tiles", fa_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)o, lse, 1, 1,
                                          2048, 64, 0.125f, 0, nullptr), FA_OK);
  if (g_last.wg_shift != 0) {
    fprintf(stderr, "FAIL 64-tile launch arguments: wg_shift=%d\n", g_last.wg_shift);
    ++g_fail;
  }
  expect("split fp32 256", fa_fwd_splitkv(q, k, v, o, lse, 1, 1, 256, 64, 0.125f, 0, FA_F32, 8, (void*)(8 * G),
                                          1 << 30, nullptr), FA_OK);
  if (g_last_ncol != 8 || g_last.kv_chunk != 32 || (uintptr_t)g_last.part_u != 8 * G || g_last.wg_shift != 0) {
    fprintf(stderr, "FAIL split launch arguments: ncol=%d kv_chunk=%d\n", g_last_ncol, g_last.kv_chunk);
    ++g_fail;
  }
  // backward
  void *dout = (void*)(6 * G), *dq = (void*)(7 * G), *dk = (void*)(9 * G), *dv = (void*)(10 * G);
  float* delta = (float*)(11 * G);
  expect("bwd ok", fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, 1, 2, 100, 128, 0.088f, 1, nullptr), FA_OK);
  expect("bwd d=96", fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, 1, 2, 100, 96, 0.1f, 0, nullptr),
         FA_ERR_UNSUPPORTED);
  expect("bwd huge", fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, INT_MAX, INT_MAX, INT_MAX, 64, 0.1f, 0, nullptr),
         FA_ERR_INVALID_ARG);
  expect("bwd dq overlaps dk", fa_bwd(q, k, v, o, dout, lse, dq, (char*)dq + 16, dv, delta, 1, 1, 16, 64, 0.1f, 0,
                                      nullptr), FA_ERR_INVALID_ARG);
  for (int s = -3; s <= 6; ++s)
    if (fa_status_string(s) == nullptr) {
      fprintf(stderr, "FAIL status string %d\n", s);
      ++g_fail;
    }
  printf("cases failed: %d, launches recorded: %d\n", g_fail, g_launches);
  return g_fail ? 1 : 0;
}
