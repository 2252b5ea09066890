// Dimension-generic kernels: any head count and widths within the limits in launch.h, float32 or
// bfloat16 storage, float32 arithmetic.  They serve small and odd shapes (the toy workload), the
// upstream projections, and the split-K combine.  The V3-shaped hot path uses the MFMA kernels.
//
// Score convention: q_hat already carries sm_scale * log2(e) (see mla_absorb_query), so a dot
// product with a cached row is a base-2 logit; partial lse values are converted back to natural
// log on output.

#include <math.h>

#include "common.h"
#include "launch.h"
#include "schedule.h"

namespace mla {

namespace {

constexpr int kThreads = 256;

// -------------------------------------------------------------------------------- absorb
// One block per (query row, head).  q_hat = [q_c . W_UK[h]^T | RoPE_pos(q_r)] * qscale.
template <typename T, typename Q = typename QHatOf<T>::type>
__global__ __launch_bounds__(kThreads) void absorb_generic_kernel(Dims d, const T* __restrict__ q_c,
                                                                  const T* __restrict__ q_r,
                                                                  const T* __restrict__ w_uk,
                                                                  const int32_t* __restrict__ pos,
                                                                  Q* __restrict__ q_hat, float qscale) {
  extern __shared__ float qs[];  // [d_k]
  const int r = blockIdx.x, h = blockIdx.y;
  const size_t qi = size_t(r) * d.H + h;
  for (int k = threadIdx.x; k < d.dk; k += blockDim.x) qs[k] = Elem<T>::load(q_c, qi * d.dk + k);
  __syncthreads();
  const T* w = w_uk + size_t(h) * d.dc * d.dk;
  Q* out = q_hat + qi * d.W();
  for (int j = threadIdx.x; j < d.dc; j += blockDim.x) {
    float acc = 0.f;
    for (int k = 0; k < d.dk; ++k) acc = fmaf(qs[k], Elem<T>::load(w, size_t(j) * d.dk + k), acc);
    Elem<Q>::store(out, j, acc * qscale);
  }
  const double p = double(pos[r]);
  for (int i = threadIdx.x; i < d.dr / 2; i += blockDim.x) {
    const double ang = p * pow(double(d.rope_base), -2.0 * i / d.dr);
    const double cs = cos(ang), sn = sin(ang);
    const double x1 = Elem<T>::load(q_r, qi * d.dr + 2 * i), x2 = Elem<T>::load(q_r, qi * d.dr + 2 * i + 1);
    Elem<Q>::store(out, d.dc + 2 * i, float(x1 * cs - x2 * sn) * qscale);
    Elem<Q>::store(out, d.dc + 2 * i + 1, float(x1 * sn + x2 * cs) * qscale);
  }
}

// -------------------------------------------------------------------------------- attend
// One block per (chunk or query row or unit, sequence, head).  Online softmax over the key range in
// tiles of 256 tokens: every thread scores one token, then every thread accumulates its latent
// columns over the tile.  MODE kPrefill: blockIdx.x is the query row, keys t <= q_start + row.
// MODE kBalanced: blockIdx.x is a unit of the balanced split (schedule.h); a block whose segment
// is empty writes nothing.
enum { kFixed = 0, kPrefill = 1, kBalanced = 2 };
template <typename T, int MODE, typename Q = typename QHatOf<T>::type>
__global__ __launch_bounds__(kThreads) void attend_generic_kernel(Dims d, Cache c, const Q* __restrict__ q_hat,
                                                                  int split_tokens, int n_splits, int q_len,
                                                                  const int32_t* __restrict__ q_start,
                                                                  float* __restrict__ o_out,
                                                                  float* __restrict__ lse_out) {
  extern __shared__ float sm[];
  const int W = d.W();
  float* qs = sm;               // [W]
  float* ps = sm + W;           // [kThreads]
  float* red = ps + kThreads;   // [16]
  const int x = blockIdx.x, b = blockIdx.y, h = blockIdx.z;
  const int len = sched_len(c.seq_lens[b], c.max_pages * c.page_size);
  int t0, t1;
  size_t qrow, orow;
  if (MODE == kPrefill) {
    t0 = 0;
    t1 = min(len, q_start[b] + x + 1);
    qrow = (size_t(b) * q_len + x) * d.H + h;
    orow = qrow;
  } else if (MODE == kBalanced) {
    // split_tokens carries the row-group size G: unit x runs row x % G of its group-unit x / G
    const int group = split_tokens, cap = c.max_pages * c.page_size;
    const int gu = x / group, gi = x - gu * group, grp = b / group;
    if (b - grp * group != gi) return;  // another unit's row (uniform over the block)
    int cb, total;
    sched_prefix(c.seq_lens, c.batch / group, group, cap, grp, cb, total);
    int k0, k1;
    sched_row_segment(cb, sched_tiles(sched_group_len(c.seq_lens, grp, group, cap)), sched_tiles(len), gu,
                      sched_quota(total, n_splits / group), k0, k1);
    if (k1 <= k0) return;  // uniform over the block
    t0 = k0 * kSchedTile;
    t1 = min(k1 * kSchedTile, len);
    qrow = size_t(b) * d.H + h;
    orow = size_t(sched_slot(gu, grp, group, gi)) * d.H + h;
  } else {
    t0 = x * split_tokens;
    t1 = min(t0 + split_tokens, len);
    qrow = size_t(b) * d.H + h;
    orow = (size_t(b) * n_splits + x) * d.H + h;
  }
  for (int k = threadIdx.x; k < W; k += blockDim.x) qs[k] = Elem<Q>::load(q_hat, qrow * W + k);
  __syncthreads();
  const T* pool = static_cast<const T*>(c.pool);
  float acc[kGenericMaxDc / kThreads];
#pragma unroll
  for (int i = 0; i < kGenericMaxDc / kThreads; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int base = t0; base < t1; base += kThreads) {
    const int t = base + threadIdx.x;
    const bool valid = t < t1;
    float sc = -INFINITY;
    if (valid) {
      const T* row = pool + row_index(c.page_table, c.max_pages, c.page_size, b, t) * W;
      float a = 0.f;
      for (int k = 0; k < W; ++k) a = fmaf(qs[k], Elem<T>::load(row, k), a);
      sc = a;
    }
    const float mn = fmaxf(m, block_max(sc, red));
    const float alpha = fast_exp2(m - mn);
    const float p = valid ? fast_exp2(sc - mn) : 0.f;
    ps[threadIdx.x] = p;
    l = l * alpha + block_sum(p, red);
#pragma unroll
    for (int i = 0; i < kGenericMaxDc / kThreads; ++i) acc[i] *= alpha;
    const int n = min(kThreads, t1 - base);
    for (int tt = 0; tt < n; ++tt) {
      const float pt = ps[tt];
      const T* row = pool + row_index(c.page_table, c.max_pages, c.page_size, b, base + tt) * W;
#pragma unroll
      for (int i = 0; i < kGenericMaxDc / kThreads; ++i) {
        const int j = threadIdx.x + i * kThreads;
        if (j < d.dc) acc[i] = fmaf(pt, Elem<T>::load(row, j), acc[i]);
      }
    }
    m = mn;
    __syncthreads();
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < kGenericMaxDc / kThreads; ++i) {
    const int j = threadIdx.x + i * kThreads;
    if (j < d.dc) o_out[orow * d.dc + j] = acc[i] * inv;
  }
  if (threadIdx.x == 0 && lse_out) lse_out[orow] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

// -------------------------------------------------------------------------------- combine
// One block per (head, sequence): LSE-weighted merge of the sequence's partials, the S chunks of
// the fixed split or the segment slots of the balanced split (schedule.h).
template <bool BAL>
__global__ __launch_bounds__(kThreads) void combine_generic_kernel(Dims d, Cache c, int S, int group,
                                                                   const float* __restrict__ o_part,
                                                                   const float* __restrict__ lse_part,
                                                                   float* __restrict__ z,
                                                                   float* __restrict__ lse_out) {
  __shared__ float red[16];
  __shared__ float wts[1024];
  const int h = blockIdx.x, b = blockIdx.y;
  size_t base = size_t(b) * S;
  int count = S, step = 1;
  if (BAL) {
    const int cap = c.max_pages * c.page_size;
    const int grp = b / group, gi = b - grp * group;
    int cb, total;
    sched_prefix(c.seq_lens, c.batch / group, group, cap, grp, cb, total);
    const int tiles = sched_tiles(sched_len(c.seq_lens[b], cap));  // this row's own tiles
    count = 0;
    if (tiles > 0) {
      int w0, w1;
      sched_units(cb, tiles, sched_quota(total, S / group), w0, w1);
      base = size_t(sched_slot(w0, grp, group, gi));
      count = w1 - w0 + 1;
      step = group;
    }
  }
  const float* lp = lse_part + base * d.H + h;  // stride step * H over partials
  const size_t lstride = size_t(step) * d.H;
  float mx = -INFINITY;
  for (int s = threadIdx.x; s < count; s += blockDim.x) mx = fmaxf(mx, lp[s * lstride]);
  mx = block_max(mx, red);
  float* zo = z + (size_t(b) * d.H + h) * d.dc;
  if (mx == -INFINITY) {
    for (int j = threadIdx.x; j < d.dc; j += blockDim.x) zo[j] = 0.f;
    if (threadIdx.x == 0 && lse_out) lse_out[size_t(b) * d.H + h] = -INFINITY;
    return;
  }
  float tot = 0.f;
  for (int s = threadIdx.x; s < count; s += blockDim.x) tot += expf(lp[s * lstride] - mx);
  tot = block_sum(tot, red);
  const float inv = 1.f / tot;
  float acc[kGenericMaxDc / kThreads];
#pragma unroll
  for (int i = 0; i < kGenericMaxDc / kThreads; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < count; s0 += 1024) {
    const int ns = min(1024, count - s0);
    __syncthreads();
    for (int s = threadIdx.x; s < ns; s += blockDim.x) wts[s] = expf(lp[(s0 + s) * lstride] - mx) * inv;
    __syncthreads();
    for (int s = 0; s < ns; ++s) {
      const float w = wts[s];
      if (w == 0.f) continue;  // empty chunk: its partial is never read
      const float* op = o_part + ((base + size_t(s0 + s) * step) * d.H + h) * d.dc;
#pragma unroll
      for (int i = 0; i < kGenericMaxDc / kThreads; ++i) {
        const int j = threadIdx.x + i * kThreads;
        if (j < d.dc) acc[i] = fmaf(w, op[j], acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kGenericMaxDc / kThreads; ++i) {
    const int j = threadIdx.x + i * kThreads;
    if (j < d.dc) zo[j] = acc[i];
  }
  if (threadIdx.x == 0 && lse_out) lse_out[size_t(b) * d.H + h] = mx + logf(tot);
}

// -------------------------------------------------------------------------------- out_proj
template <typename T>
__global__ __launch_bounds__(128) void out_proj_generic_kernel(Dims d, const float* __restrict__ z,
                                                               const T* __restrict__ w_uv, float* __restrict__ out) {
  extern __shared__ float zs[];  // [d_c]
  const int h = blockIdx.x, r = blockIdx.y;
  const size_t zi = size_t(r) * d.H + h;
  for (int j = threadIdx.x; j < d.dc; j += blockDim.x) zs[j] = z[zi * d.dc + j];
  __syncthreads();
  const T* w = w_uv + size_t(h) * d.dc * d.dv;
  for (int v = threadIdx.x; v < d.dv; v += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < d.dc; ++j) acc = fmaf(zs[j], Elem<T>::load(w, size_t(j) * d.dv + v), acc);
    out[zi * d.dv + v] = acc;
  }
}

// -------------------------------------------------------------------------------- projections
template <typename T>
__global__ __launch_bounds__(kThreads) void project_query_kernel(Dims d, int dm, int dcq, const T* __restrict__ hh,
                                                                 const T* __restrict__ w_dq, const T* __restrict__ w_uq,
                                                                 const T* __restrict__ w_qr, T* __restrict__ q_c,
                                                                 T* __restrict__ q_r) {
  extern __shared__ float sm[];
  float* hs = sm;       // [dm]
  float* cq = sm + dm;  // [dcq]
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < dm; i += blockDim.x) hs[i] = Elem<T>::load(hh, size_t(r) * dm + i);
  __syncthreads();
  for (int c = threadIdx.x; c < dcq; c += blockDim.x) {
    float acc = 0.f;
    for (int i = 0; i < dm; ++i) acc = fmaf(hs[i], Elem<T>::load(w_dq, size_t(i) * dcq + c), acc);
    cq[c] = acc;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < d.H * d.dk; idx += blockDim.x) {
    const int hd = idx / d.dk, k = idx % d.dk;
    float acc = 0.f;
    for (int c = 0; c < dcq; ++c) acc = fmaf(cq[c], Elem<T>::load(w_uq, (size_t(hd) * dcq + c) * d.dk + k), acc);
    Elem<T>::store(q_c, size_t(r) * d.H * d.dk + idx, acc);
  }
  for (int idx = threadIdx.x; idx < d.H * d.dr; idx += blockDim.x) {
    const int hd = idx / d.dr, k = idx % d.dr;
    float acc = 0.f;
    for (int c = 0; c < dcq; ++c) acc = fmaf(cq[c], Elem<T>::load(w_qr, (size_t(hd) * dcq + c) * d.dr + k), acc);
    Elem<T>::store(q_r, size_t(r) * d.H * d.dr + idx, acc);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(Dims d, Cache c, int dm, const T* __restrict__ hh,
                                                             const T* __restrict__ w_dkv, const T* __restrict__ w_kr,
                                                             const int32_t* __restrict__ seq_ids,
                                                             const int32_t* __restrict__ positions, float rms_eps) {
  extern __shared__ float sm[];
  float* hs = sm;           // [dm]
  float* cs = hs + dm;      // [dc]
  float* ks = cs + d.dc;    // [dr]
  float* red = ks + d.dr;   // [16]
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < dm; i += blockDim.x) hs[i] = Elem<T>::load(hh, size_t(r) * dm + i);
  __syncthreads();
  float ss = 0.f;
  for (int j = threadIdx.x; j < d.dc; j += blockDim.x) {
    float acc = 0.f;
    for (int i = 0; i < dm; ++i) acc = fmaf(hs[i], Elem<T>::load(w_dkv, size_t(i) * d.dc + j), acc);
    cs[j] = acc;
    ss = fmaf(acc, acc, ss);
  }
  for (int p = threadIdx.x; p < d.dr; p += blockDim.x) {
    float acc = 0.f;
    for (int i = 0; i < dm; ++i) acc = fmaf(hs[i], Elem<T>::load(w_kr, size_t(i) * d.dr + p), acc);
    ks[p] = acc;
  }
  ss = block_sum(ss, red);  // also orders the cs/ks writes before the reads below
  const float scale = rms_eps > 0.f ? 1.f / sqrtf(ss / float(d.dc) + rms_eps) : 1.f;
  const int b = seq_ids[r], t = positions[r];
  T* row = const_cast<T*>(static_cast<const T*>(c.pool)) + row_index(c.page_table, c.max_pages, c.page_size, b, t) * d.W();
  for (int j = threadIdx.x; j < d.dc; j += blockDim.x) Elem<T>::store(row, j, cs[j] * scale);
  const double pd = double(t);
  for (int i = threadIdx.x; i < d.dr / 2; i += blockDim.x) {
    const double ang = pd * pow(double(d.rope_base), -2.0 * i / d.dr);
    const double cn = cos(ang), sn = sin(ang);
    const double x1 = ks[2 * i], x2 = ks[2 * i + 1];
    Elem<T>::store(row, d.dc + 2 * i, float(x1 * cn - x2 * sn));
    Elem<T>::store(row, d.dc + 2 * i + 1, float(x1 * sn + x2 * cn));
  }
}

float q_scale(const Dims& d) { return d.sm_scale * kLog2e; }

}  // namespace

// -------------------------------------------------------------------------------- launchers
hipError_t launch_absorb_generic(const Dims& d, const void* q_c, const void* q_r, const void* w_uk,
                                 const int32_t* pos, int rows, void* q_hat, hipStream_t s) {
  const dim3 grid(rows, d.H);
  const size_t shm = sizeof(float) * d.dk;
  if (d.dtype == MLA_BF16)
    absorb_generic_kernel<uint16_t><<<grid, kThreads, shm, s>>>(
        d, (const uint16_t*)q_c, (const uint16_t*)q_r, (const uint16_t*)w_uk, pos, (f16_t*)q_hat, q_scale(d));
  else
    absorb_generic_kernel<float><<<grid, kThreads, shm, s>>>(d, (const float*)q_c, (const float*)q_r,
                                                             (const float*)w_uk, pos, (float*)q_hat, q_scale(d));
  return hipGetLastError();
}

hipError_t launch_decode_generic(const Dims& d, const Cache& c, const void* q_hat, int n_splits, int split_tokens,
                                 float* o_part, float* lse_part, hipStream_t s) {
  const dim3 grid(n_splits, c.batch, d.H);
  const size_t shm = sizeof(float) * (d.W() + kThreads + 16);
  if (d.dtype == MLA_BF16)
    attend_generic_kernel<uint16_t, kFixed><<<grid, kThreads, shm, s>>>(d, c, (const f16_t*)q_hat, split_tokens,
                                                                       n_splits, 1, nullptr, o_part, lse_part);
  else
    attend_generic_kernel<float, kFixed><<<grid, kThreads, shm, s>>>(d, c, (const float*)q_hat, split_tokens, n_splits,
                                                                    1, nullptr, o_part, lse_part);
  return hipGetLastError();
}

hipError_t launch_prefill_generic(const Dims& d, const Cache& c, const void* q_hat, int q_len,
                                  const int32_t* q_start, float* z, float* lse, hipStream_t s) {
  const dim3 grid(q_len, c.batch, d.H);
  const size_t shm = sizeof(float) * (d.W() + kThreads + 16);
  if (d.dtype == MLA_BF16)
    attend_generic_kernel<uint16_t, kPrefill><<<grid, kThreads, shm, s>>>(d, c, (const f16_t*)q_hat, 0, 1, q_len,
                                                                      q_start, z, lse);
  else
    attend_generic_kernel<float, kPrefill><<<grid, kThreads, shm, s>>>(d, c, (const float*)q_hat, 0, 1, q_len, q_start,
                                                                   z, lse);
  return hipGetLastError();
}

hipError_t launch_combine_generic(const Dims& d, int batch, int n_splits, const float* o_part, const float* lse_part,
                                  float* z, float* lse, hipStream_t s) {
  Cache none{};
  combine_generic_kernel<false><<<dim3(d.H, batch), kThreads, 0, s>>>(d, none, n_splits, 1, o_part, lse_part, z, lse);
  return hipGetLastError();
}

hipError_t launch_decode_generic_balanced(const Dims& d, const Cache& c, const void* q_hat, int n_units, int group,
                                          float* o_part, float* lse_part, hipStream_t s) {
  const dim3 grid(n_units, c.batch, d.H);
  const size_t shm = sizeof(float) * (d.W() + kThreads + 16);
  if (d.dtype == MLA_BF16)
    attend_generic_kernel<uint16_t, kBalanced><<<grid, kThreads, shm, s>>>(d, c, (const f16_t*)q_hat, group, n_units,
                                                                          1, nullptr, o_part, lse_part);
  else
    attend_generic_kernel<float, kBalanced><<<grid, kThreads, shm, s>>>(d, c, (const float*)q_hat, group, n_units,
                                                                       1, nullptr, o_part, lse_part);
  return hipGetLastError();
}

hipError_t launch_combine_generic_balanced(const Dims& d, const Cache& c, int n_units, int group,
                                           const float* o_part, const float* lse_part, float* z, float* lse,
                                           hipStream_t s) {
  combine_generic_kernel<true><<<dim3(d.H, c.batch), kThreads, 0, s>>>(d, c, n_units, group, o_part, lse_part, z,
                                                                       lse);
  return hipGetLastError();
}

hipError_t launch_out_proj_generic(const Dims& d, const float* z, const void* w_uv, int rows, float* out,
                                   hipStream_t s) {
  const dim3 grid(d.H, rows);
  const size_t shm = sizeof(float) * d.dc;
  if (d.dtype == MLA_BF16)
    out_proj_generic_kernel<uint16_t><<<grid, 128, shm, s>>>(d, z, (const uint16_t*)w_uv, out);
  else
    out_proj_generic_kernel<float><<<grid, 128, shm, s>>>(d, z, (const float*)w_uv, out);
  return hipGetLastError();
}

hipError_t launch_project_query(const Dims& d, int d_model, int d_cq, const void* h, const void* w_dq,
                                const void* w_uq, const void* w_qr, int rows, void* q_c, void* q_r, hipStream_t s) {
  const size_t shm = sizeof(float) * (d_model + d_cq);
  if (d.dtype == MLA_BF16)
    project_query_kernel<uint16_t><<<rows, kThreads, shm, s>>>(d, d_model, d_cq, (const uint16_t*)h,
                                                               (const uint16_t*)w_dq, (const uint16_t*)w_uq,
                                                               (const uint16_t*)w_qr, (uint16_t*)q_c, (uint16_t*)q_r);
  else
    project_query_kernel<float><<<rows, kThreads, shm, s>>>(d, d_model, d_cq, (const float*)h, (const float*)w_dq,
                                                            (const float*)w_uq, (const float*)w_qr, (float*)q_c,
                                                            (float*)q_r);
  return hipGetLastError();
}

hipError_t launch_kv_append(const Dims& d, const Cache& c, int d_model, const void* h, const void* w_dkv,
                            const void* w_kr, const int32_t* seq_ids, const int32_t* positions, int rows,
                            float rms_eps, hipStream_t s) {
  const size_t shm = sizeof(float) * (d_model + d.dc + d.dr + 16);
  if (d.dtype == MLA_BF16)
    kv_append_kernel<uint16_t><<<rows, kThreads, shm, s>>>(d, c, d_model, (const uint16_t*)h, (const uint16_t*)w_dkv,
                                                           (const uint16_t*)w_kr, seq_ids, positions, rms_eps);
  else
    kv_append_kernel<float><<<rows, kThreads, shm, s>>>(d, c, d_model, (const float*)h, (const float*)w_dkv,
                                                        (const float*)w_kr, seq_ids, positions, rms_eps);
  return hipGetLastError();
}

}  // namespace mla
