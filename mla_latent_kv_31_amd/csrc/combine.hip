// Log-sum-exp merge of split-K partials for latent widths up to 512 (a multiple of 8):
//   LSE = ln sum_i exp(lse_i),  z = sum_i exp(lse_i - LSE) o_i
// over any split equal to the single-pass softmax of the scores ([ase] Fig. 2).  One wave per
// (sequence, head): lanes first reduce the chunk maxima and weights (kept in LDS), then each lane
// accumulates eight latent columns over the chunks with 16-byte loads, eight chunks' loads in
// flight at a time; chunks of weight zero (empty or negligible) never contribute.  The balanced split (schedule.h) merges the slots of each
// sequence's segments.

#include <math.h>

#include "common.h"
#include "launch.h"
#include "schedule.h"

namespace mla {
namespace {

constexpr int kCombineMaxSplits = 2048;

// grid (H / 4, batch); wave w handles head 4*blockIdx.x + w.  The partials of sequence b are the
// `count` slots base, base + step, ...: the S chunks b*S .. b*S+S-1 of the fixed split, or the
// slots of b's segments in the balanced split with row groups of `group` rows (recomputed from
// seq_lens, see schedule.h; consecutive for group 1, every group-th slot otherwise).
template <bool kBalanced>
__global__ __launch_bounds__(256) void combine_kernel(int H, int dc, int S, int group,
                                                      const int32_t* __restrict__ seq_lens,
                                                      int batch, int cap, const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part, float* __restrict__ z,
                                                      float* __restrict__ lse_out) {
  __shared__ float wts[4][kCombineMaxSplits];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = 4 * blockIdx.x + wave, b = blockIdx.y;
  if (h >= H) return;  // whole wave leaves; no block-wide barrier follows
  int base = b * S, count = S, step = 1;
  if constexpr (kBalanced) {
    const int grp = b / group, gi = b - grp * group;
    int cb, total;
    sched_prefix(seq_lens, batch / group, group, cap, grp, cb, total);
    const int tiles = sched_tiles(sched_len(seq_lens[b], cap));  // this row's own tiles
    count = 0;
    if (tiles > 0) {
      int w0, w1;
      sched_units(cb, tiles, sched_quota(total, S / group), w0, w1);
      base = sched_slot(w0, grp, group, gi);
      count = w1 - w0 + 1;
      step = group;
    }
  }
  const float* lp = lse_part + size_t(base) * H + h;
  const size_t lstride = size_t(step) * H;
  float mx = -INFINITY;
  for (int s = lane; s < count; s += 64) mx = fmaxf(mx, lp[s * lstride]);
  mx = wave_max(mx);
  float* zo = z + (size_t(b) * H + h) * dc;
  if (mx == -INFINITY) {
    for (int c = lane * 4; c < dc; c += 256) *reinterpret_cast<float4*>(zo + c) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane == 0 && lse_out) lse_out[size_t(b) * H + h] = -INFINITY;
    return;
  }
  float tot = 0.f;
  for (int s = lane; s < count; s += 64) {
    const float w = expf(lp[s * lstride] - mx);
    wts[wave][s] = w;
    tot += w;
  }
  tot = wave_sum(tot);
  const float inv = 1.f / tot;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
  const int c0 = 8 * lane;
  if (c0 < dc) {
    const float* op = o_part + (size_t(base) * H + h) * dc + c0;
    const size_t stride = size_t(step) * H * dc;
    // eight slots per round: all sixteen loads are issued before the first FMA.  Rows of zero
    // weight (empty chunks, possibly never written) are loaded but dropped by a select.
    constexpr int kG = 8;
    for (int s0 = 0; s0 < count; s0 += kG) {
      float4 x0[kG], x1[kG];
      float w[kG];
#pragma unroll
      for (int k = 0; k < kG; ++k) {
        const int s = min(s0 + k, count - 1);
        w[k] = s0 + k < count ? wts[wave][s] * inv : 0.f;
        x0[k] = *reinterpret_cast<const float4*>(op + s * stride);
        x1[k] = *reinterpret_cast<const float4*>(op + s * stride + 4);
      }
#pragma unroll
      for (int k = 0; k < kG; ++k) {
        const bool use = w[k] != 0.f;
        a0.x = use ? fmaf(w[k], x0[k].x, a0.x) : a0.x;
        a0.y = use ? fmaf(w[k], x0[k].y, a0.y) : a0.y;
        a0.z = use ? fmaf(w[k], x0[k].z, a0.z) : a0.z;
        a0.w = use ? fmaf(w[k], x0[k].w, a0.w) : a0.w;
        a1.x = use ? fmaf(w[k], x1[k].x, a1.x) : a1.x;
        a1.y = use ? fmaf(w[k], x1[k].y, a1.y) : a1.y;
        a1.z = use ? fmaf(w[k], x1[k].z, a1.z) : a1.z;
        a1.w = use ? fmaf(w[k], x1[k].w, a1.w) : a1.w;
      }
    }
    *reinterpret_cast<float4*>(zo + c0) = a0;
    *reinterpret_cast<float4*>(zo + c0 + 4) = a1;
  }
  if (lane == 0 && lse_out) lse_out[size_t(b) * H + h] = mx + logf(tot);
}

}  // namespace

bool combine_fast_supported(const Dims& d, int n_splits) {
  return d.dc % 8 == 0 && d.dc <= 512 && n_splits <= kCombineMaxSplits;
}

hipError_t launch_combine_fast(const Dims& d, int batch, int n_splits, const float* o_part, const float* lse_part,
                               float* z, float* lse, hipStream_t s) {
  combine_kernel<false><<<dim3((d.H + 3) / 4, batch), 256, 0, s>>>(d.H, d.dc, n_splits, 1, nullptr, batch, 0, o_part,
                                                                   lse_part, z, lse);
  return hipGetLastError();
}

hipError_t launch_combine_fast_balanced(const Dims& d, const Cache& c, int n_units, int group, const float* o_part,
                                        const float* lse_part, float* z, float* lse, hipStream_t s) {
  combine_kernel<true><<<dim3((d.H + 3) / 4, c.batch), 256, 0, s>>>(
      d.H, d.dc, n_units, group, c.seq_lens, c.batch, c.max_pages * c.page_size, o_part, lse_part, z, lse);
  return hipGetLastError();
}

}  // namespace mla
