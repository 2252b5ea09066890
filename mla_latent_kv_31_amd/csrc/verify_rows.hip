// Rows of a multi-token verify step for the split-K decode path.
//
// A verify step (speculative decoding) scores q_len new tokens per sequence at once, each with
// the causal rule of a chunk ([ase] causal-mask remark after Fig. 2): query i of sequence b sits
// at position q_start[b] + i and reads keys t <= q_start[b] + i, t < seq_lens[b].  Each such query
// is an ordinary decode query over its own prefix, so the step can run as decode over
// batch * q_len rows: row r = b * q_len + i reads sequence b's pages with length
// clamp(q_start[b] + i + 1, 0, seq_lens[b]).  This kernel writes those rows' page table (a copy
// of sequence b's row), lengths and positions; the work-balanced decode then spreads all rows over
// every compute unit, where a one-workgroup-per-query-row prefill would wait on its longest row.

#include "launch.h"

namespace mla {
namespace {

__global__ void verify_rows_kernel(const int32_t* __restrict__ table, const int32_t* __restrict__ lens,
                                   const int32_t* __restrict__ q_start, int q_len, int max_pages,
                                   int32_t* __restrict__ row_table, int32_t* __restrict__ row_lens,
                                   int32_t* __restrict__ row_pos) {
  const int r = blockIdx.y;
  const int b = r / q_len, i = r - b * q_len;
  const int32_t* src = table + size_t(b) * max_pages;
  int32_t* dst = row_table + size_t(r) * max_pages;
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < max_pages; p += gridDim.x * blockDim.x) dst[p] = src[p];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const int pos = q_start[b] + i;
    row_lens[r] = min(max(pos + 1, 0), lens[b]);
    if (row_pos) row_pos[r] = pos;
  }
}

}  // namespace

hipError_t launch_verify_rows(const Cache& c, const int32_t* q_start, int q_len, int32_t* row_table,
                              int32_t* row_lens, int32_t* row_pos, hipStream_t stream) {
  const int rows = c.batch * q_len;
  const dim3 grid(min((c.max_pages + 255) / 256, 64), rows);
  hipLaunchKernelGGL(verify_rows_kernel, grid, dim3(256), 0, stream, c.page_table, c.seq_lens, q_start, q_len,
                     c.max_pages, row_table, row_lens, row_pos);
  return hipGetLastError();
}

}  // namespace mla
