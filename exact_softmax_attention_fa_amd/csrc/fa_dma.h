// Address arithmetic of the loads that move K/V (forward) and Q/dO/K/V (backward) tiles from
// global memory straight into LDS with global_load_lds_dwordx4: each lane of one instruction
// moves 16 bytes, read at (scalar base + the lane's unsigned 32-bit offset) and written to LDS
// bytes [m0 + 16 lane, m0 + 16 lane + 16). Rows are stored unpadded with their 16-byte chunks
// permuted (swizzled), so a lane fetches the logical chunk that belongs at its physical place.
//
// Plain integer functions, shared by the kernels and by a host-side checker that walks every
// load of every wave for a sweep of sequence lengths and checks that each one reads inside its
// head's rows, reads the row and chunk it should, and writes inside its LDS slot.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

namespace fa {
namespace dma {

FA_HD int imin(int a, int b) { return a < b ? a : b; }

// Rows at or past the last one (N-1) of a sequence read row N-1 instead (their scores are
// masked later): the bytes to pull the offset of row r of a tile starting at row0 back by.
// With row0 <= N-1 the result never exceeds r * row_bytes, so the unsigned per-lane offset
// (at least r * row_bytes) stays non-negative.
FA_HD uint32_t past_end_back(int row0, int r, int N, int row_bytes) {
  const int over = row0 + r - (N - 1);
  return over > 0 ? (uint32_t)over * (uint32_t)row_bytes : 0u;
}

// ---- tuned forward kernels, head width D = 64 or 128: 64-key tiles of K and V, 8 waves ------
// A tile is 64 rows of 2D bytes, D/8 chunks of 16 bytes per row. Wave w's load instruction i
// (0 <= i < D/64) fills LDS bytes [((D/64) w + i) KiB, +1 KiB) of the tile: lane l takes row
// ((D/64) w + i) (512/D) + l/(D/8) and physical chunk l%(D/8), i.e. the logical K chunk
// (l%(D/8)) ^ fwd_k_swz(row) or V chunk (l%(D/8)) ^ fwd_v_swz(row) of that row.
// The K permutation makes the 16-byte operand reads of 16 consecutive rows hit distinct banks
// (D = 128: 256-byte rows, chunk ^ (r & 15); D = 64: 128-byte rows, pairs of rows share a bank
// row, chunk ^ ((r >> 1) & 7)); the V permutation does the same for the transpose reads of 4
// consecutive rows and two 16-feature halves (4(r & 3), or 4((r >> 1) & 1) for D = 64). Both are
// periodic in 16 rows, so row offsets of 16 and 32 keep them.
template <int D> constexpr int fwd_row_bytes() { return 2 * D; }
template <int D>
FA_HD int fwd_k_swz(int r) {
  static_assert(D == 64 || D == 128, "head width");
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
FA_HD int fwd_v_swz(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
template <int D>
FA_HD int fwd_row(int wave, int lane, int i) { return ((D / 64) * wave + i) * (512 / D) + lane / (D / 8); }
template <int D>
FA_HD uint32_t fwd_k_off(int wave, int lane, int i) {
  const int r = fwd_row<D>(wave, lane, i);
  return (uint32_t)(r * fwd_row_bytes<D>() + ((lane % (D / 8)) ^ fwd_k_swz<D>(r)) * 16);
}
template <int D>
FA_HD uint32_t fwd_v_off(int wave, int lane, int i) {
  const int r = fwd_row<D>(wave, lane, i);
  return (uint32_t)(r * fwd_row_bytes<D>() + ((lane % (D / 8)) ^ fwd_v_swz<D>(r)) * 16);
}

// ---- backward kernels: [32][D] tiles, 16-byte chunk L of row r stored at L ^ swz(r) --------
// With this permutation the 16 rows that one 16-lane quarter of a 16-byte row read touches land
// in 16 different bank groups, and so do the 4 rows x 4 chunks each half of a transposed read
// touches.
template <int D>
FA_HD int swz(int r) {
  static_assert(D == 64 || D == 128, "head width");
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
// Load instruction i into a [32][D] tile fills its i-th KiB: lane l writes physical chunk
// l % (D/8) of row i (512/D) + l / (D/8), i.e. fetches that row's chunk (l % (D/8)) ^ swz(row).
template <int D>
FA_HD int tile_row(int i, int lane) { return i * (512 / D) + lane / (D / 8); }
template <int D>
FA_HD uint32_t tile_off(int i, int lane) {
  const int r = tile_row<D>(i, lane);
  return (uint32_t)(r * 2 * D + 16 * ((lane % (D / 8)) ^ swz<D>(r)));
}
// dQ kernel: first key of sub-tile (wave & 1) of 64-key step t, clamped to N-1 (a sub-tile that
// starts past the sequence then reads row N-1 throughout, and past_end_back stays below the
// per-lane offsets).
FA_HD int dq_row0(int t, int wave, int N) { return imin(2 * t * 32 + (wave & 1) * 32, N - 1); }

}  // namespace dma
}  // namespace fa
