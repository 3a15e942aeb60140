// Host-side walk of every global -> LDS tile load the kernels issue, for a list of sequence
// lengths, with the address arithmetic the kernels use (fa_dma.h). For each 16-byte load it
// checks that the global offset is non-negative and inside the head's N rows, that it reads the
// row it should (rows past N-1 read row N-1) and the logical chunk the swizzle places at its LDS
// position, that it writes inside its LDS slot, and that every 16-byte place of a tile is
// written exactly once. The loop structure (which tiles each kernel issues for a given N and
// mask) restates the kernels' own.
//
// It also walks the forward ring schedule (which interval requests, reads and reuses each
// slot) for every tile count the lengths give.
//
// usage: dma_bounds [--old-dq-base | --no-back | --deep-lead] N1 N2 ...
//   --old-dq-base  plants the dQ kernel's earlier base row (not clamped to N-1)
//   --no-back      plants loads that never pull rows past N-1 back
//   --deep-lead    plants a forward ring lead one tile deeper than the ring allows
// Prints the counts and the first violations; exit status 1 if any load violates a check.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "fa_dma.h"

using namespace fa::dma;

static bool g_old_dq = false, g_no_back = false, g_deep_lead = false;
static long g_loads = 0, g_bad = 0;

static void bad(const char* what, const char* kernel, int N, int D, int a, int b, int c, long long v) {
  if (g_bad < 20)
    fprintf(stderr, "VIOLATION %s: %s N=%d D=%d (%d,%d,%d) value=%lld\n", what, kernel, N, D, a, b, c, v);
  ++g_bad;
}

static uint32_t back_of(int row0, int r, int N, int row_bytes) {
  return g_no_back ? 0u : past_end_back(row0, r, N, row_bytes);
}

// one 16-byte load: global byte offset (as the kernel forms it: unsigned 32-bit lane offset minus
// the pull-back, added to a row base) and its expected value
static void check_load(const char* k, int N, int D, int row_bytes, int64_t base, uint32_t off, uint32_t back,
                       int want_row, int want_chunk, int a, int b, int c) {
  ++g_loads;
  const uint32_t lane_off = off - back;                  // unsigned, as in the kernel
  const int64_t src = base + (int64_t)lane_off;
  if ((int64_t)off - (int64_t)back < 0) bad("lane offset wraps below 0", k, N, D, a, b, c, (long long)off - back);
  if (src < 0 || src + 16 > (int64_t)N * row_bytes) bad("read outside the head", k, N, D, a, b, c, src);
  const int64_t want = (int64_t)want_row * row_bytes + 16 * (int64_t)want_chunk;
  if (src != want) bad("reads the wrong row or chunk", k, N, D, a, b, c, src - want);
}

// ---- forward, tuned kernels (head width D = 128 or 64) ---------------------------------------
// The expected chunks restate the permutations: D = 128 K c ^ (r & 15), V c ^ 4(r & 3);
// D = 64 K c ^ ((r >> 1) & 7), V c ^ 4((r >> 1) & 1).
template <int D>
static void fwd(int N, bool causal) {
  const int BR = 256, BC = 64, SLOTS = 4, ROWB = fwd_row_bytes<D>(), TILEB = BC * ROWB;
  const int VREGION = SLOTS * TILEB, LDS = 2 * SLOTS * TILEB, CPR = D / 8, NLD = D / 64;
  if (LDS > 160 * 1024) bad("rings exceed the CU's LDS", "fwd", N, D, 0, 0, 0, LDS);
  const char* kn = D == 128 ? "fwd128" : "fwd64";
  const int nqt = (N + BR - 1) / BR;
  for (int qt = 0; qt < nqt; ++qt) {
    const int kv_end = causal ? (N < (qt + 1) * BR ? N : (qt + 1) * BR) : N;
    const int nkv = (kv_end + BC - 1) / BC;
    for (int t = 0; t < nkv; ++t) {
      const int key0 = t * BC, slot = t % SLOTS;
      const bool full = key0 + BC <= N;
      std::vector<int> hits(TILEB / 16, 0);
      for (int wave = 0; wave < 8; ++wave)
        for (int i = 0; i < NLD; ++i)
          for (int lane = 0; lane < 64; ++lane) {
            const int r = fwd_row<D>(wave, lane, i);
            const uint32_t back = full ? 0u : back_of(key0, r, N, ROWB);
            const int row = key0 + r < N - 1 ? key0 + r : N - 1;
            const int64_t base = (int64_t)key0 * ROWB;
            const int c = lane % CPR;
            const int kc = D == 128 ? c ^ (r & 15) : c ^ ((r >> 1) & 7);
            const int vc = D == 128 ? c ^ ((r & 3) << 2) : c ^ (((r >> 1) & 1) << 2);
            check_load(D == 128 ? "fwd128 K" : "fwd64 K", N, D, ROWB, base, fwd_k_off<D>(wave, lane, i), back, row, kc,
                       t, wave, lane);
            check_load(D == 128 ? "fwd128 V" : "fwd64 V", N, D, ROWB, base, fwd_v_off<D>(wave, lane, i), back, row, vc,
                       t, wave, lane);
            const int dk = slot * TILEB + (NLD * wave + i) * 1024 + 16 * lane;   // K ring; V at +VREGION
            if (dk < slot * TILEB || dk + 16 > (slot + 1) * TILEB || dk + VREGION + 16 > LDS)
              bad("LDS write outside the slot", kn, N, D, t, wave, lane, dk);
            if ((dk - slot * TILEB) / ROWB != r || ((dk - slot * TILEB) % ROWB) / 16 != c)
              bad("LDS place is not the loaded row's physical chunk", kn, N, D, t, wave, lane, dk);
            ++hits[(dk - slot * TILEB) / 16];
          }
      for (int p = 0; p < TILEB / 16; ++p)
        if (hits[p] != 1) bad("tile place not written exactly once", kn, N, D, t, p, 0, hits[p]);
    }
  }
}

// ---- forward, tuned kernels: the ring schedule ------------------------------------------------
// Restated from the phase definitions: group g runs M_j in interval 2j+g and V_j in 2j+1+g
// (j < nkv), and the final M_nkv in 2nkv+g. M_j reads K_j (j < nkv) and V_{j-1}; the end of V_j
// requests V_j operands for M_{j+1}. Group g requests tiles 0 .. lead_g-1 before interval 0 and
// tile j+lead_g at the start of V_j (lead = S-2, S-1), into slot t mod S. The barrier closing
// interval k waits until at most `ahead` of the wave's newest tiles are in flight, with
// ahead = (last tile requested) - (k+1)/2 and at most 4 supported. Checks: every slot is
// rewritten only after every read of its previous tile; every tile is requested by both groups
// before the barrier that closes the interval before its first read, and that barrier waits for
// it; the in-flight count never exceeds 4.
static void fwd_schedule(int nkv, int S) {
  const char* kn = "fwd ring";
  std::vector<int> last_read(nkv, -1), first_read(nkv, 1 << 30);
  auto read = [&](int t, int k) {
    if (t < 0 || t >= nkv) return;
    last_read[t] = k > last_read[t] ? k : last_read[t];
    first_read[t] = k < first_read[t] ? k : first_read[t];
  };
  for (int g = 0; g < 2; ++g)
    for (int j = 0; j <= nkv; ++j) {
      const int km = 2 * j + g;
      if (j < nkv) read(j, km);    // K_j in M_j
      read(j - 1, km);             // V_{j-1} in M_j
      if (j < nkv) read(j, km + 1);   // V_j operand requests at the end of V_j
    }
  for (int g = 0; g < 2; ++g) {
    const int lead = (g == 0 ? S - 2 : S - 1) + (g_deep_lead ? 1 : 0);
    std::vector<int> issue(nkv, 0);   // interval at whose start the group requests tile t (-1: prologue)
    for (int t = 0; t < nkv; ++t) issue[t] = t < lead ? -1 : 2 * (t - lead) + 1 + g;
    for (int t = 0; t < nkv; ++t) {
      if (t >= S && issue[t] <= last_read[t - S])
        bad("slot rewritten before its last read", kn, nkv, S, t, g, issue[t], last_read[t - S]);
      // the barrier closing interval first_read-1 waits for tiles up to first_read/2
      if (first_read[t] < 2 * t) bad("tile read before a barrier waits for it", kn, nkv, S, t, g, first_read[t], 0);
      if (issue[t] > first_read[t] - 1)
        bad("tile requested after the barrier before its first read", kn, nkv, S, t, g, issue[t], first_read[t]);
    }
    // both groups close intervals 0 .. 2nkv with a barrier (group 1: an extra one first, none
    // after its final M phase); requests at the start of interval k count at its barrier
    for (int k = 0; k <= 2 * nkv; ++k) {
      int last = -1;
      for (int t = 0; t < nkv; ++t)
        if (issue[t] <= k) last = t;
      const int ahead = last - ((k + 1) >> 1);
      if (ahead > 4) bad("more tiles in flight than the barrier waits for", kn, nkv, S, k, g, ahead, 0);
    }
  }
}

// ---- backward, dQ kernel (4 waves, 128 queries; 64-key steps of two 32-row sub-tiles) --------
template <int D>
static void dq(int N, bool causal) {
  const int KT = 32 * D, SLOTB = 4 * KT * 2, KB_SUB = 2 * KT / 1024, RB = 2 * D;
  const int nqt = (N + 127) / 128;
  for (int qt = 0; qt < nqt; ++qt) {
    const int kv_end = causal ? (N < (qt + 1) * 128 ? N : (qt + 1) * 128) : N;
    const int nst = (kv_end + 63) / 64;
    for (int t = 0; t < nst; ++t) {
      const int slot = t & 1;
      for (int wave = 0; wave < 4; ++wave) {
        const int u0 = 2 * t * 32 + (wave & 1) * 32;       // sub-tile's first key (unclamped)
        const int row0 = g_old_dq ? u0 : dq_row0(t, wave, N);
        std::vector<int> hits(2 * KT / 16, 0);
        for (int i = 0; i < KB_SUB; ++i)
          for (int lane = 0; lane < 64; ++lane) {
            const int r = tile_row<D>(i, lane);
            const int row = u0 + r < N - 1 ? u0 + r : N - 1;
            check_load("dq", N, D, RB, (int64_t)row0 * RB, tile_off<D>(i, lane), back_of(row0, r, N, RB), row,
                       (lane % (D / 8)) ^ swz<D>(r), t, wave, lane);
            const int lo = slot * SLOTB + wave * KT * 2, d = lo + i * 1024 + 16 * lane;
            if (d + 16 > lo + KT * 2 || d + 16 > 2 * SLOTB) bad("LDS write outside the sub-tile", "dq", N, D, t, wave, d, 0);
            ++hits[(d - lo) / 16];
          }
        for (int p = 0; p < 2 * KT / 16; ++p)
          if (hits[p] != 1) bad("sub-tile place not written exactly once", "dq", N, D, t, wave, p, hits[p]);
      }
    }
  }
}

// ---- backward, dK/dV kernel (128 keys; query blocks of 32 rows into 5 slots) ---------------
template <int D>
static void dkdv(int N, bool causal) {
  const int NW = 4, RPW = 2 * (D / 64), KB_TILE = 2 * 32 * D / 1024, TILEB = 2 * 32 * D;
  const int SLOTB = 2 * TILEB + 512, SLOTS = 5, RB = 2 * D;
  const int nkb = (N + 127) / 128, nqb = (N + 31) / 32;
  for (int kblk = 0; kblk < nkb; ++kblk) {
    const int qb0 = causal ? kblk * 128 / 32 : 0;
    for (int qb = qb0; qb < nqb; ++qb) {
      const int row0 = qb * 32;
      {
        const int slot = (qb - qb0) % SLOTS;   // block qb0 + j goes to slot j mod 5
        std::vector<int> hits(SLOTB / 16, 0);
        for (int lw = 0; lw < NW; ++lw) {
          const int tile = (lw * RPW) / KB_TILE;   // 0: Q, 1: dO
          for (int i = 0; i < RPW; ++i) {
            const int kb = (lw * RPW + i) % KB_TILE;
            for (int lane = 0; lane < 64; ++lane) {
              const int r = tile_row<D>(kb, lane);
              const int row = row0 + r < N - 1 ? row0 + r : N - 1;
              check_load("dkdv", N, D, RB, (int64_t)row0 * RB, tile_off<D>(kb, lane), back_of(row0, r, N, RB), row,
                         (lane % (D / 8)) ^ swz<D>(r), qb, lw, lane);
              const int lo = slot * SLOTB + tile * TILEB, d = lo + kb * 1024 + 16 * lane;
              if (d + 16 > lo + TILEB) bad("LDS write outside the tile", "dkdv", N, D, qb, lw, d, 0);
              ++hits[(d - slot * SLOTB) / 16];
            }
          }
          if (lw < 2) {   // 32 log-normalisers (wave 0) or deltas (wave 1), lanes 32..63 repeat
            for (int lane = 0; lane < 64; ++lane) {
              ++g_loads;
              const int lr = lane & 31;
              const int idx = row0 + (lr < N - 1 - row0 ? lr : N - 1 - row0);
              if (N - 1 - row0 < 0 || idx < 0 || idx >= N) bad("row statistic outside the head", "dkdv", N, D, qb, lw, lane, idx);
              const int d = slot * SLOTB + 2 * TILEB + lw * 256 + 4 * lane;
              if (d + 4 > (slot + 1) * SLOTB) bad("LDS write outside the slot", "dkdv stats", N, D, qb, lw, lane, d);
            }
          }
        }
        for (int p = 0; p < 2 * TILEB / 16; ++p)
          if (hits[p] != 1) bad("slot place not written exactly once", "dkdv", N, D, qb, slot, p, hits[p]);
      }
    }
  }
}

int main(int argc, char** argv) {
  std::vector<int> Ns;
  for (int a = 1; a < argc; ++a) {
    if (!strcmp(argv[a], "--old-dq-base")) g_old_dq = true;
    else if (!strcmp(argv[a], "--no-back")) g_no_back = true;
    else if (!strcmp(argv[a], "--deep-lead")) g_deep_lead = true;
    else Ns.push_back(atoi(argv[a]));
  }
  for (int N : Ns) {
    if (N < 1) continue;
    for (int causal = 0; causal < 2; ++causal) {
      fwd<128>(N, causal);
      fwd<64>(N, causal);
      const int nkv = (N + 63) / 64;   // key tiles of the longest item (whole N)
      for (int S = 4; S <= 6; ++S) fwd_schedule(nkv, S);
      dq<64>(N, causal);
      dq<128>(N, causal);
      if (N <= 8192) {   // (the dK/dV walk is quadratic in N; it is covered up to 8192)
        dkdv<64>(N, causal);
        dkdv<128>(N, causal);
      }
    }
  }
  printf("loads checked: %ld, violations: %ld\n", g_loads, g_bad);
  return g_bad ? 1 : 0;
}
