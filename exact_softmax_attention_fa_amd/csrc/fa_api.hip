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
// nothing. `br` is the query rows per workgroup of the kernel that will run. On success fills
// `args` and the padded head width.
int validate(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, float scale, int causal, size_t elem,
             int br, fa::FwdArgs* args, int* d_pad) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FA_ERR_INVALID_ARG;
  // rows move in 16-byte pieces: q, k, v, o 16-byte aligned, lse 4-byte aligned
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_INVALID_ARG;
  if ((uintptr_t)lse & 3) return FA_ERR_INVALID_ARG;
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
  args->kv_chunk = N;
  args->part_u = nullptr;
  args->part_ml = nullptr;
  // One-XCD packing for short sequences only: there it cuts the HBM traffic of the K/V
  // re-reads at no cost in time, while long ones (all workgroups streaming K/V at once through
  // one XCD) ran slower packed.
  args->wg_shift = ((int64_t)B * H < 8 && (int64_t)B * H * n_qtiles <= 32 && N <= 1024) ? 3 : 0;
  *d_pad = dp;
  return FA_OK;
}

constexpr int kMaxSplits = 64;
constexpr int kMinColumnKeys = 1024;   // shortest key column of the default split

using fa::SplitPlan;

int plan_split(int B, int H, int N, int d, int dtype, int causal, int num_splits, SplitPlan* p) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  // the size limits of the single-pass calls, before any product of the sizes below
  if ((unsigned __int128)B * H * N * d > ((unsigned __int128)1 << 62)) return FA_ERR_INVALID_ARG;
  if (d > 256) return FA_ERR_UNSUPPORTED;
  if ((int64_t)N * d > INT_MAX) return FA_ERR_UNSUPPORTED;
  const int dp = d <= 64 ? 64 : (d <= 128 ? 128 : 256);
  const int tile = dtype == FA_BF16 ? fa::bf16_split_key_tile(dp) : fa::f32_split_key_tile(dp);
  const int rows = dtype == FA_BF16 ? fa::bf16_split_rows_per_block(dp) : fa::f32_rows_per_block(dp);
  const int64_t tiles = ((int64_t)N + tile - 1) / tile;
  const int64_t base = (int64_t)B * H * (((int64_t)N + rows - 1) / rows);   // workgroups of one column
  int64_t want = num_splits;
  if (want == 0) {
    // Library choice, for grids of fewer than one workgroup per CU of the 256 (larger grids
    // keep one column): about 256 workgroups without the mask. Under the causal mask the key
    // ranges of the query tiles grow from one tile to all of them, so the last query tile
    // would finish long after the rest; columns of fewer keys (about 2048 workgroups, of which
    // the ones past the diagonal exit at once) even that out. Columns keep at least
    // kMinColumnKeys keys: below that, writing and merging the partial states costs more than
    // the spread gains.
    const int64_t target = causal ? 2048 : 256;
    const int64_t by_len = ((int64_t)N + kMinColumnKeys - 1) / kMinColumnKeys;
    want = base >= 256 ? 1 : (target + base - 1) / base;
    if (want > by_len) want = by_len;
  }
  want = want < 1 ? 1 : (want > kMaxSplits ? kMaxSplits : want);
  if (want > tiles) want = tiles;
  const int64_t per = (tiles + want - 1) / want;              // tiles per column
  const int64_t chunk = per * tile;
  const int64_t ns = ((int64_t)N + chunk - 1) / chunk;        // no column without keys
  p->nsplit = (int)ns;
  p->kv_chunk = (int)(ns == 1 ? N : chunk);
  p->d_pad = dp;
  if (ns == 1) {
    p->u_bytes = 0;
    p->ws_bytes = 0;
    return FA_OK;
  }
  const unsigned __int128 rows_all = (unsigned __int128)ns * B * H * N;
  const unsigned __int128 ub = rows_all * dp * sizeof(float);
  const unsigned __int128 total = ((ub + 255) / 256) * 256 + rows_all * 2 * sizeof(float);
  if (total > ((unsigned __int128)1 << 62)) return FA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * (((int64_t)N + rows - 1) / rows) > INT_MAX) return FA_ERR_UNSUPPORTED;
  p->u_bytes = (size_t)ub;
  p->ws_bytes = (size_t)total;
  return FA_OK;
}

bool ranges_overlap(const void* x, uint64_t nx, const void* y, uint64_t ny) {
  const uintptr_t a0 = (uintptr_t)x, b0 = (uintptr_t)y;
  return a0 < b0 + ny && b0 < a0 + nx;
}

}  // namespace

namespace fa {

int splitkv_check(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                  float scale, int causal, int dtype, int num_splits, SplitPlan* plan, fa::FwdArgs* args) {
  const int st = plan_split(B, H, N, d, dtype, causal, num_splits, plan);
  if (st != FA_OK) return st;
  int d_pad = 0;
  const bool bf = dtype == FA_BF16;
  return validate(q, k, v, o, lse, B, H, N, d, scale, causal, bf ? 2 : 4,
                  bf ? fa::bf16_split_rows_per_block(plan->d_pad) : fa::f32_rows_per_block(d), args, &d_pad);
}

int splitkv_run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                float scale, int causal, int dtype, const SplitPlan& plan, fa::FwdArgs args, void* ws,
                hipStream_t stream) {
  const bool bf = dtype == FA_BF16;
  if (plan.nsplit == 1) {
    return bf ? fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream)
              : fa_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)o, lse, B, H, N, d, scale,
                           causal, stream);
  }
  const int d_pad = plan.d_pad;
  args.kv_chunk = plan.kv_chunk;
  args.wg_shift = 0;   // the split pass spreads its columns over the whole chip
  args.part_u = (float*)ws;
  args.part_ml = (float*)((uint8_t*)ws + ((plan.u_bytes + 255) / 256) * 256);
  const hipError_t e1 = bf ? fa::launch_bf16_partial(args, d_pad, causal != 0, plan.nsplit, stream)
                           : fa::launch_f32_partial(args, d_pad, causal != 0, plan.nsplit, stream);
  if (e1 != hipSuccess) return FA_ERR_HIP;
  const hipError_t e2 = fa::launch_merge(args, d_pad, causal != 0, plan.nsplit, /*m_unscaled=*/!bf,
                                         /*out_f32=*/!bf, stream);
  return e2 == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
  fa::FwdArgs args;
  int d_pad = 0;
  const int st = validate(q, k, v, o, lse, B, H, N, d, scale, causal, 2,
                          fa::bf16_rows_per_block(d, (int64_t)B * H, N), &args, &d_pad);
  if (st != FA_OK) return st;
  return fa::launch_bf16(args, d_pad, causal != 0, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
  fa::FwdArgs args;
  int d_pad = 0;
  const int st = validate(q, k, v, o, lse, B, H, N, d, scale, causal, 4,
                          fa::f32_rows_per_block(d), &args, &d_pad);
  if (st != FA_OK) return st;
  return fa::launch_f32(args, d_pad, causal != 0, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_splitkv_plan(int B, int H, int N, int d, int dtype, int causal, int num_splits,
                                   int* nsplit_out, size_t* workspace_bytes_out) {
  SplitPlan plan;
  const int st = plan_split(B, H, N, d, dtype, causal, num_splits, &plan);
  if (st != FA_OK) return st;
  if (nsplit_out != nullptr) *nsplit_out = plan.nsplit;
  if (workspace_bytes_out != nullptr) *workspace_bytes_out = plan.ws_bytes;
  return FA_OK;
}

extern "C" int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int N, int d, float scale, int causal, int dtype, int num_splits,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  SplitPlan plan;
  fa::FwdArgs args;
  const int st = fa::splitkv_check(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, num_splits, &plan, &args);
  if (st != FA_OK) return st;
  if (plan.nsplit > 1) {
    if (workspace == nullptr || workspace_bytes < plan.ws_bytes) return FA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return FA_ERR_INVALID_ARG;
    // the workspace may not overlap any input or output
    const size_t elem = dtype == FA_BF16 ? 2 : 4;
    const uint64_t tb = (uint64_t)B * H * N * d * elem, lb = (uint64_t)B * H * N * sizeof(float);
    const void* bufs[4] = {q, k, v, o};
    for (const void* b : bufs)
      if (b != nullptr && ranges_overlap(workspace, plan.ws_bytes, b, tb)) return FA_ERR_INVALID_ARG;
    if (lse != nullptr && ranges_overlap(workspace, plan.ws_bytes, lse, lb)) return FA_ERR_INVALID_ARG;
  }
  return fa::splitkv_run(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, plan, args, workspace, stream);
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                      int d, float scale, int causal, hipStream_t stream) {
  const void* ins[6] = {q, k, v, o, dout, lse};
  void* outs[4] = {dq, dk, dv, delta};
  for (const void* p : ins) if (p == nullptr) return FA_ERR_INVALID_ARG;
  for (const void* p : outs) if (p == nullptr) return FA_ERR_INVALID_ARG;
  // 16-byte aligned row arrays, 4-byte aligned row statistics
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv) & 15)
    return FA_ERR_INVALID_ARG;
  if (((uintptr_t)lse | (uintptr_t)delta) & 3) return FA_ERR_INVALID_ARG;
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
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than fa_fwd_splitkv_plan reports";
    case FA_ERR_SCRATCH:
      return "problem needs more partial-state memory than the fixed 64 MiB buffer of fa_fwd_splitkv_noalloc";
    default: return "unknown status";
  }
}
