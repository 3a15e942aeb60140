// C-ABI front end: argument validation, kernel selection and launch (declared in fa.h).
#include <hip/hip_runtime.h>
#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_internal.h"
#include "fa_bwd_internal.h"

namespace {

// Checks shared by both entry points. Runs before any HIP call; a rejected call writes
// nothing. On success fills `args` and the padded head width.
int validate(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, float scale, int causal, size_t elem,
             int (*rows_per_block)(int), fa::FwdArgs* args, int* d_pad) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  // element count B*H*N*d must stay below 2^62 (byte offsets then fit in 64 bits)
  const unsigned __int128 count = (unsigned __int128)B * H * N * d;
  if (count > ((unsigned __int128)1 << 62)) return FA_ERR_INVALID_ARG;
  if (d > 256) return FA_ERR_UNSUPPORTED;
  // per-head offsets are computed in 64 bits, but row indices and N*d in 32 bits
  if ((int64_t)N * d > INT_MAX) return FA_ERR_UNSUPPORTED;

  // outputs must not overlap inputs
  const uint64_t bytes = (uint64_t)count * elem;
  const uint64_t lse_bytes = (uint64_t)B * H * N * sizeof(float);
  auto overlap = [](const void* x, uint64_t nx, const void* y, uint64_t ny) {
    const uintptr_t a0 = (uintptr_t)x, b0 = (uintptr_t)y;
    return a0 < b0 + ny && b0 < a0 + nx;
  };
  const void* ins[3] = {q, k, v};
  for (const void* in : ins) {
    if (overlap(o, bytes, in, bytes)) return FA_ERR_INVALID_ARG;
    if (lse != nullptr && overlap(lse, lse_bytes, in, bytes)) return FA_ERR_INVALID_ARG;
  }
  if (lse != nullptr && overlap(lse, lse_bytes, o, bytes)) return FA_ERR_INVALID_ARG;

  const int dp = d <= 64 ? 64 : (d <= 128 ? 128 : 256);
  const int br = rows_per_block(d);
  const int64_t n_qtiles = ((int64_t)N + br - 1) / br;
  if ((int64_t)B * H * n_qtiles > INT_MAX) return FA_ERR_UNSUPPORTED;

  args->q = q;
  args->k = k;
  args->v = v;
  args->o = o;
  args->lse = lse;
  args->N = N;
  args->d = d;
  args->BH = B * H;
  args->n_qtiles = (int)n_qtiles;
  // |scale| * log2(e), floored at the smallest normal float so that a zero scale still
  // keeps -inf (masked) scores at -inf after scaling; the floor changes no finite result.
  args->sl2 = fmaxf(fabsf(scale) * 1.4426950408889634f, FLT_MIN);
  args->neg = scale < 0.0f ? 1 : 0;
  *d_pad = dp;
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
  fa::FwdArgs args;
  int d_pad = 0;
  const int st = validate(q, k, v, o, lse, B, H, N, d, scale, causal, 2,
                          fa::bf16_rows_per_block, &args, &d_pad);
  if (st != FA_OK) return st;
  return fa::launch_bf16(args, d_pad, causal != 0, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
  fa::FwdArgs args;
  int d_pad = 0;
  const int st = validate(q, k, v, o, lse, B, H, N, d, scale, causal, 4,
                          fa::f32_rows_per_block, &args, &d_pad);
  if (st != FA_OK) return st;
  return fa::launch_f32(args, d_pad, causal != 0, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                      int d, float scale, int causal, hipStream_t stream) {
  const void* ins[6] = {q, k, v, o, dout, lse};
  void* outs[4] = {dq, dk, dv, delta};
  for (const void* p : ins) if (p == nullptr) return FA_ERR_INVALID_ARG;
  for (const void* p : outs) if (p == nullptr) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  const unsigned __int128 count = (unsigned __int128)B * H * N * d;
  if (count > ((unsigned __int128)1 << 62)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((int64_t)N * d > INT_MAX) return FA_ERR_UNSUPPORTED;
  const int64_t nblk = ((int64_t)N + fa::bwd_rows_per_block() - 1) / fa::bwd_rows_per_block();
  if ((int64_t)B * H * nblk > INT_MAX) return FA_ERR_UNSUPPORTED;

  // no output may overlap an input or another output
  const uint64_t tb = (uint64_t)count * 2, rb = (uint64_t)B * H * N * sizeof(float);
  const uint64_t in_bytes[6] = {tb, tb, tb, tb, tb, rb};
  const uint64_t out_bytes[4] = {tb, tb, tb, rb};
  auto overlap = [](const void* x, uint64_t nx, const void* y, uint64_t ny) {
    const uintptr_t a0 = (uintptr_t)x, b0 = (uintptr_t)y;
    return a0 < b0 + ny && b0 < a0 + nx;
  };
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], out_bytes[i], ins[j], in_bytes[j])) return FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], out_bytes[i], outs[j], out_bytes[j])) return FA_ERR_INVALID_ARG;
  }

  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.N = N;
  a.d = d;
  a.BH = B * H;
  a.sl2 = fmaxf(fabsf(scale) * 1.4426950408889634f, FLT_MIN);
  a.neg = scale < 0.0f ? 1 : 0;
  return fa::launch_bwd_bf16(a, causal != 0, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported problem (head dimension above 256 or problem too large)";
    case FA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}
