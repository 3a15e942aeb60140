// Internal launch interface between the C-ABI front end (fa_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Arguments shared by every forward kernel. Pointers are per-call device pointers;
// each (b, h) slice of q/k/v/o is N*d contiguous elements, lse holds N floats per slice.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;     // may be null
  int N;          // sequence length (queries = keys)
  int d;          // head dimension actually stored (<= the kernel's padded width)
  int BH;         // B * H
  int n_qtiles;   // ceil(N / rows per workgroup)
  float sl2;      // |scale| * log2(e): scores are kept in base-2 exponent units
  int neg;        // 1 when scale < 0: the kernel negates q (exact) and uses |scale|
  // Key-range split over workgroups (generic kernels only). Workgroup column y = blockIdx.y
  // takes keys [y * kv_chunk, (y + 1) * kv_chunk); kv_chunk is a multiple of the kernel's key
  // tile. With part_u == nullptr there is one column (kv_chunk >= N) and the kernel writes o
  // and lse; otherwise it writes its partial state (m, l, u) instead:
  //   part_u  [split][BH][N][d_pad] fp32: unnormalised numerator u
  //   part_ml [split][BH][N][2]     fp32: reference m (units: launch_merge's m_unscaled) and
  //                                 denominator l
  int kv_chunk;
  float* part_u;
  float* part_ml;
  // Single-pass grids of fewer than 8 short heads, small enough for one XCD (the dispatcher
  // places workgroup i on XCD i mod 8), launch 2^wg_shift workgroups per work item along x,
  // and only those with blockIdx.x a multiple of 2^wg_shift work: every workgroup then runs on
  // the same XCD and the heads' K/V come from HBM once into its L2, not once per XCD.
  int wg_shift;
};

// Rows of queries per workgroup of the kernel that will run for head width d (host needs it
// for the grid). The bf16 choice at head widths up to 64 also depends on the grid: BH heads
// (B * H) of N queries.
int bf16_rows_per_block(int d, int64_t BH, int N);
int f32_rows_per_block(int d);

// Enqueue one forward pass. d_pad (64, 128 or 256) is the padded head width of the generic
// kernels. Return hipSuccess or the launch error.
hipError_t launch_bf16(const FwdArgs& a, int d_pad, bool causal, hipStream_t stream);
hipError_t launch_f32(const FwdArgs& a, int d_pad, bool causal, hipStream_t stream);

// Tuned bf16 kernels for head width exactly 128 or 64 (a.d): rows per workgroup, whether a grid
// of BH heads of N queries at d = 64 takes the tuned kernel (enough work items for the chip),
// and the launch.
int bf16_tuned_rows_per_block();
bool bf16_tuned_d64(int64_t BH, int N);
hipError_t launch_bf16_tuned(const FwdArgs& a, bool causal, hipStream_t stream);

// ---- key-range split (split-KV) -------------------------------------------------------------
// Rows per workgroup and keys per tile of the generic kernel that runs the partial pass
// (split path: the generic kernels serve every width, d = 128 included).
int bf16_split_rows_per_block(int d_pad);
int bf16_split_key_tile(int d_pad);
int f32_split_key_tile(int d_pad);
// Partial pass: grid (BH * n_qtiles, nsplit); every workgroup writes part_u / part_ml for its
// rows and keys (workgroups whose key range lies past their last query under the causal mask
// write nothing; the merge never reads those entries).
hipError_t launch_bf16_partial(const FwdArgs& a, int d_pad, bool causal, int nsplit, hipStream_t stream);
hipError_t launch_f32_partial(const FwdArgs& a, int d_pad, bool causal, int nsplit, hipStream_t stream);
// Merge pass: o and lse from the nsplit partial states of every row. m_unscaled = 1 when the
// partial kernels keep m on unscaled scores (fp32 kernel: weights 2^((m_s - m*) * sl2)),
// 0 when m is already in base-2 units (bf16 kernel: weights 2^(m_s - m*)). out_f32 selects
// the output type (fp32 or bf16).
hipError_t launch_merge(const FwdArgs& a, int d_pad, bool causal, int nsplit, bool m_unscaled, bool out_f32,
                        hipStream_t stream);

// ---- split-KV front end (shared by the entry points with and without a caller workspace) ----
// Plan of a split-KV call: the number of split columns actually used, the keys per column and
// the workspace bytes they need (0 when one column remains, i.e. the single-pass kernels run).
struct SplitPlan {
  int nsplit;
  int kv_chunk;
  int d_pad;
  size_t u_bytes;    // partial numerators: nsplit * B*H * N * d_pad fp32
  size_t ws_bytes;   // u_bytes rounded up to 256, plus the (m, l) pairs
};
// Host checks of a split-KV call (before any HIP call): the plan and the arguments of the
// single-pass call of that dtype. Fills `plan` and `args`; returns an fa_status code.
int splitkv_check(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                  float scale, int causal, int dtype, int num_splits, SplitPlan* plan, FwdArgs* args);
// The split-KV call once the checks have passed: partial pass over (query tile, key column)
// into `ws` (plan.ws_bytes, 256-byte aligned), then the merge; with one column, the
// single-pass call. Returns an fa_status code.
int splitkv_run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                float scale, int causal, int dtype, const SplitPlan& plan, FwdArgs args, void* ws,
                hipStream_t stream);

}  // namespace fa
