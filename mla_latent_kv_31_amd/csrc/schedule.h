// Work-balanced split of a decode batch, shared by the decode and combine kernels.
//
// Every sequence costs tiles + MLA_BALANCED_SEG_COST (0 when empty), with tiles = ceil(len / 32);
// the costs are laid end to end in batch order, and unit w of n owns the cost range
// [w*q, (w+1)*q) with q = ceil(total / n).  The first MLA_BALANCED_SEG_COST cost positions of a
// sequence stand for the fixed price of one segment (query load, pipeline fill, partial write);
// its tiles follow.  The segment of sequence b in unit w is the set of b's tiles inside w's
// range; its partial goes to slot w + b, which no other non-empty segment shares.  Both sides
// derive everything from seq_lens, so no schedule is stored anywhere.
//
// Row groups.  With a group size G > 1 the batch is read as batch / G groups of G consecutive
// rows that read the same keys up to their own lengths (the draft rows of one sequence in a
// multi-token verify step).  A group costs like its longest row and the split above runs over
// groups with n / G group-units; unit u = G*w + i runs row i of every group segment of
// group-unit w, clamped to that row's own tiles, and writes its partial to slot G*(w + g) + i for
// group g.  The G units of a group-unit read the same pages at the same time, and consecutive
// units share an L2 (see the decode kernel's unit placement), so the cache is fetched from HBM
// about once per group instead of once per row.  G = 1 is the plain split.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

constexpr int kSchedTile = MLA_BALANCED_TILE;
constexpr int kSchedSegCost = MLA_BALANCED_SEG_COST;

__host__ __device__ inline int sched_len(int len, int cap) { return len < 0 ? 0 : (len > cap ? cap : len); }
__host__ __device__ inline int sched_tiles(int len) { return (len + kSchedTile - 1) / kSchedTile; }
__host__ __device__ inline int sched_cost(int len) {
  const int t = sched_tiles(len);
  return t > 0 ? t + kSchedSegCost : 0;
}
__host__ __device__ inline int sched_quota(int total, int n_units) { return (total + n_units - 1) / n_units; }

// Tiles [k0, k1) of a sequence (cost prefix cb, `tiles` tiles) inside unit w; empty when k1 <= k0.
__host__ __device__ inline void sched_segment(int cb, int tiles, int w, int q, int& k0, int& k1) {
  const int s = cb + kSchedSegCost;
  const int lo = w * q, hi = lo + q;
  k0 = (lo > s ? lo : s) - s;
  k1 = (hi < s + tiles ? hi : s + tiles) - s;
}

// Row segment: tiles [k0, k1) of one row of a group inside group-unit w, the group's segment
// clamped to the row's own tiles (empty when k1 <= k0).
__host__ __device__ inline void sched_row_segment(int cb, int group_tiles, int row_tiles, int w, int q, int& k0,
                                                  int& k1) {
  sched_segment(cb, group_tiles, w, q, k0, k1);
  k1 = k1 < row_tiles ? k1 : row_tiles;
}

// Partial slot of row i of group g in group-unit w.
__host__ __device__ inline int sched_slot(int w, int g, int group, int i) { return (w + g) * group + i; }

// Units whose segments of a non-empty sequence are non-empty: [w0, w1].
__host__ __device__ inline void sched_units(int cb, int tiles, int q, int& w0, int& w1) {
  const int s = cb + kSchedSegCost;
  w0 = s / q;
  w1 = (s + tiles - 1) / q;
}

// ---- wave-cooperative helpers (wave64); every lane receives the results

__device__ inline int sched_wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Length that sets the cost of group g: its longest row.
__host__ __device__ inline int sched_group_len(const int32_t* __restrict__ seq_lens, int g, int group, int cap) {
  int m = 0;
  for (int i = 0; i < group; ++i) {
    const int l = sched_len(seq_lens[g * group + i], cap);
    m = l > m ? l : m;
  }
  return m;
}

// Cost prefix of group b and the total cost of the n_groups groups.
__device__ inline void sched_prefix(const int32_t* __restrict__ seq_lens, int n_groups, int group, int cap, int b,
                                    int& cb, int& total) {
  const int lane = threadIdx.x & 63;
  int before = 0, all = 0;
  for (int i = lane; i < n_groups; i += 64) {
    const int c = sched_cost(sched_group_len(seq_lens, i, group, cap));
    all += c;
    if (i < b) before += c;
  }
  cb = sched_wave_sum(before);
  total = sched_wave_sum(all);
}

// First group whose cost range ends past `pos`, with its cost prefix (n_groups and the total
// cost when there is none).
__device__ inline void sched_find(const int32_t* __restrict__ seq_lens, int n_groups, int group, int cap, int pos,
                                  int& b, int& cb) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  const int batch = n_groups;
  for (int c0 = 0; c0 < batch; c0 += 64) {
    const int i = c0 + lane;
    const int c = i < batch ? sched_cost(sched_group_len(seq_lens, i, group, cap)) : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const uint64_t m = __ballot(i < batch && base + incl > pos);
    if (m) {
      const int f = __builtin_ctzll(m);
      b = c0 + f;
      cb = base + __shfl(incl - c, f, 64);
      return;
    }
    base += __shfl(incl, 63, 64);
  }
  b = batch;
  cb = base;
}

}  // namespace mla
