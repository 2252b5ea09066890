// Cache write for new tokens on bf16 MFMA (gfx950), DeepSeek-V3 latent shape (d_c 512, d_r 64).
//
// For each new token r ([molayo] formal definition, KV compression; [huny] section 2, decoupled
// RoPE; [ase] Fig. 1 note on the norm that follows the latent):
//   y = h_r . [W_DKV | W_KR]                      (576 wide, fp32 accumulate)
//   c = y[0:512], RMS-normalised with unit gain when rms_eps > 0
//   k^R = RoPE_{pos_r}(y[512:576]), interleaved pairs, inverse frequencies base^(-2i/64)
//   pool row of (seq_ids[r], positions[r]) = bf16([c | k^R])
//
// Two launches.  The product is a skinny GEMM (rows x d_model) . (d_model x 576) that is bound by
// reading the weights at decode batch sizes, so its K range is split over enough workgroups to
// keep every CU streaming: kv_gemm_kernel writes fp32 partial products [split][row][576] to the
// caller's workspace.  kv_finish_kernel (one workgroup per row, its four waves sharing the splits)
// sums the splits, normalises, rotates, rounds to bf16 and stores the 1,152-byte row through the
// page table.
//
// kv_gemm_kernel: a workgroup of two waves computes a 64-row x 32-column tile over its K range,
// wave w rows 32w..32w+31, with v_mfma_f32_32x32x16_bf16.  A operand (h) comes straight from
// global memory, 16 bytes per lane (row l%32, k 8*(l/32)..+7 of the k-step).  The weight slice
// [256 k x 32 columns] is staged in LDS per chunk (row-major, 64-byte rows) and read with
// ds_read_b64_tr_b16: lane i of each 16-lane group receives column i of the 4 x 16 block the
// group addresses, which is the B-operand layout (column l%32, k 8*(l/32)..+7) in two reads.

#include <math.h>

#include <mutex>

#include "common.h"
#include "fp8.h"
#include "launch.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kDc = 512, kDr = 64, kW = kDc + kDr;
constexpr int kXcds = 8;  // accelerator complex dies, one L2 each
constexpr int kCols = 32;             // output columns per workgroup
constexpr int kColTiles = kW / kCols; // 18
constexpr int kRowsWg = 64;           // output rows per workgroup (two waves)
constexpr int kChunk = 256;           // k rows of the weight slice staged per LDS chunk
constexpr int kThreads = 128;
constexpr int kChunkB = kChunk * kCols * 2;          // 16 KiB
constexpr int kLoadsPerThread = kChunkB / 16 / kThreads;  // 8 x 16 B

__global__ __launch_bounds__(kThreads) void kv_gemm_kernel(const uint16_t* __restrict__ h, int d_model, int rows,
                                                          const uint16_t* __restrict__ w_dkv,
                                                          const uint16_t* __restrict__ w_kr, int k_per_split,
                                                          float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kChunkB];
  lds_u8* const lbase = (lds_u8*)smem;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ct = blockIdx.x, rt = blockIdx.y, ks = blockIdx.z;
  const int col0 = ct * kCols;
  // the weight slice: columns col0..col0+31 of W_DKV, or of W_KR for the last two tiles
  const uint16_t* wsrc = col0 < kDc ? w_dkv + col0 : w_kr + (col0 - kDc);
  const int wstride = col0 < kDc ? kDc : kDr;
  const int k_begin = ks * k_per_split;
  const int nchunks = k_per_split / kChunk;

  // A operand rows (clamped: rows past the end compute garbage that is never stored)
  const int row = min(rt * kRowsWg + wave * 32 + (lane & 31), rows - 1);
  const uint16_t* hrow = h + size_t(row) * d_model + 8 * (lane >> 5);

  // cooperative staging of one chunk: thread t moves 16-byte pieces t + 128 x of the slice,
  // piece p = (k row p / 4, quarter p % 4 of its 64 bytes)
  u32x4 stage[kLoadsPerThread];
  auto load_chunk = [&](int c) {
    const int k0 = k_begin + c * kChunk;
#pragma unroll
    for (int x = 0; x < kLoadsPerThread; ++x) {
      const int p = threadIdx.x + kThreads * x;
      stage[x] = *reinterpret_cast<const u32x4*>(wsrc + size_t(k0 + (p >> 2)) * wstride + 8 * (p & 3));
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int x = 0; x < kLoadsPerThread; ++x) {
      const int p = threadIdx.x + kThreads * x;
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(lbase + buf * kChunkB + 16 * p) = stage[x];
    }
  };
  // transposing reads: group g = lane/16 addresses k rows 8*(g/2) + 4*half + (lane%16)/4 and
  // columns 16*(g%2) + 4*(lane%4) .. +3 of a 16-row k-step
  const int g = lane >> 4, i16 = lane & 15;
  const int tr_off = (8 * (g >> 1) + (i16 >> 2)) * (kCols * 2) + 2 * (16 * (g & 1) + 4 * (i16 & 3));

  f32x16 acc;
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = 0.f;

  // A operands of one chunk: 16 k-steps, 16 bytes per lane each
  bf16x8 a[kChunk / 16], a_next[kChunk / 16];
  auto load_a = [&](bf16x8* dst, int c) {
    const int k0 = k_begin + c * kChunk;
#pragma unroll
    for (int s = 0; s < kChunk / 16; ++s) dst[s] = *reinterpret_cast<const bf16x8*>(hrow + k0 + 16 * s);
  };
  load_a(a, 0);
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    // the next chunk's operands are in flight while this one is multiplied (issued after this
    // chunk's A loads, so the in-order wait counts only wait for what the MFMAs use)
    if (c + 1 < nchunks) {
      load_a(a_next, c + 1);
      load_chunk(c + 1);
    }
    const lds_u8* wb = lbase + buf * kChunkB + tr_off;
#pragma unroll
    for (int s = 0; s < kChunk / 16; ++s) {
      const lds_u8* p = wb + s * 16 * (kCols * 2);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(p + 4 * (kCols * 2)));
      const bf16x8 b = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b, acc, 0, 0, 0);
    }
    if (c + 1 < nchunks) {
      store_chunk(buf ^ 1);  // that buffer was last read before the previous barrier
      __syncthreads();
#pragma unroll
      for (int s = 0; s < kChunk / 16; ++s) a[s] = a_next[s];
    }
  }

  // D layout: column l%32, rows 8*(x/4) + 4*(l/32) + x%4
  float* const out = part + (size_t(ks) * rows) * kW + col0 + (lane & 31);
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int r = rt * kRowsWg + wave * 32 + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
    if (r < rows) out[size_t(r) * kW] = acc[x];
  }
}

// kv_gemm_tiled_kernel, for 512 rows and more (prefill-sized writes), where reusing h and the weight
// slice from LDS matters more than streaming the weights: a workgroup of four waves computes a
// 64-row x 64-column tile over its K range, wave w rows 32(w&1).., columns 32(w>>1)...  Both
// operands are staged per 64-k chunk with global_load_lds transfers, three chunks ahead of the one
// multiplied (16 KiB per chunk: h rows and weight k-rows of 128 bytes each).  Workgroups are dealt to
// the eight XCDs in turn; the tiles of one row tile (all column tiles and K splits, which share its
// h rows) go to one XCD, so that they share its L2.  16-byte chunks of an h row are XOR-swizzled
// by (row>>1)&7, so 16 consecutive rows at one logical chunk (an A-operand read) hit 16 distinct
// bank groups; those of a weight k-row by 4((k>>1)&1), so the 4 k-rows x 64 bytes of a transposing
// read do.  Each lane's transfer fetches the global piece the swizzle places at its position.
constexpr int kTM = 64, kTN = 64, kKC = 64;                // tile rows, columns, k per chunk
constexpr int kTThreads = 256, kTStages = 4;
constexpr int kTRowB = kKC * 2;                            // 128 bytes per staged row
constexpr int kTAB = kTM * kTRowB, kTBB = kKC * kTRowB;    // 8 KiB each
constexpr int kTStageB = kTAB + kTBB;
constexpr int kTColTiles = kW / kTN;                       // 9: eight of W_DKV, one of W_KR
static_assert(kW % kTN == 0 && kDc % kTN == 0, "column tiles");

__device__ __forceinline__ void dma16(uint32_t lds_dst, uint32_t voff, const void* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_dst), "v"(voff), "s"(gbase)
               : "memory");
}

__global__ __launch_bounds__(kTThreads) void kv_gemm_tiled_kernel(const uint16_t* __restrict__ h, int d_model,
                                                                 int rows, const uint16_t* __restrict__ w_dkv,
                                                                 const uint16_t* __restrict__ w_kr, int k_per_split,
                                                                 float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kTStages * kTStageB];
  lds_u8* const lbase = (lds_u8*)smem;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(lbase));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // workgroup id -> (column tile, row tile, split): XCD x = id % 8 takes row tiles x, x + 8, ...
  const int n_rt = (rows + kTM - 1) / kTM, n_split = gridDim.x / (kTColTiles * n_rt);
  int ct, rt, ks;
  {
    const int id = blockIdx.x;
    if (n_rt % kXcds == 0) {
      const int per = kTColTiles * n_split, slot = id / kXcds;
      rt = id % kXcds + kXcds * (slot / per);
      ct = (slot % per) % kTColTiles;
      ks = (slot % per) / kTColTiles;
    } else {
      ct = id % kTColTiles;
      rt = (id / kTColTiles) % n_rt;
      ks = id / (kTColTiles * n_rt);
    }
  }
  const int col0 = ct * kTN, row0 = rt * kTM;
  const uint16_t* const wsrc = col0 < kDc ? w_dkv + col0 : w_kr + (col0 - kDc);
  const int wstride = col0 < kDc ? kDc : kDr;
  const int k_begin = ks * k_per_split, nchunks = k_per_split / kKC;

  // transfers: wave w moves staged rows 8(2w+x) .. +7 (x = 0, 1) of h and of the weight slice; lane
  // L writes 16 bytes at position L of that 1 KiB, i.e. row +L/8, physical chunk L%8
  uint32_t a_voff[2], b_voff[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int r = 8 * (2 * wave + x) + (lane >> 3), p = lane & 7;
    const int grow = min(row0 + r, rows - 1);  // rows past the end: a valid row, never stored
    a_voff[x] = uint32_t((size_t(grow) * d_model + 8 * (p ^ ((r >> 1) & 7))) * 2);
    b_voff[x] = uint32_t((r * wstride + 8 * (p ^ (4 * ((r >> 1) & 1)))) * 2);
  }
  auto issue = [&](int c) {  // chunk c into stage c % 3
    const int k0 = k_begin + c * kKC;
    const uint32_t st = lds0 + uint32_t((c % kTStages) * kTStageB);
    const uint16_t* ga = h + k0;
    const uint16_t* gb = wsrc + size_t(k0) * wstride;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      dma16(st + uint32_t(1024 * (2 * wave + x)), a_voff[x], ga);
      dma16(st + uint32_t(kTAB + 1024 * (2 * wave + x)), b_voff[x], gb);
    }
  };

  // operand reads.  A (32 rows x 16 k of k-step s): lane l reads row 32(w&1) + l%32, logical chunk
  // 2s + l/32.  B (16 k x 32 columns): two transposing reads of 4 k-rows x 16 columns per 16-lane
  // group; group g, lane i: k-rows 8(g/2) + i/4 (and +4) of the k-step, columns 32(w>>1) +
  // 16(g%2) + 4(i%4) .. +3.
  const int wm = wave & 1, wn = wave >> 1;
  const int ar = 32 * wm + (lane & 31);
  const uint32_t a_off = uint32_t(ar * kTRowB + 16 * ((lane >> 5) ^ ((ar >> 1) & 7)));
  const int g = lane >> 4, i16 = lane & 15;
  const int q = 4 * wn + 2 * (g & 1) + ((i16 & 3) >> 1);  // logical 16-byte chunk of the columns
  const int kr0 = 8 * (g >> 1) + (i16 >> 2);
  const uint32_t b_lo = uint32_t(kTAB + kr0 * kTRowB + 16 * (q ^ (4 * ((kr0 >> 1) & 1))) + 8 * (i16 & 1));
  const uint32_t b_hi = uint32_t(kTAB + (kr0 + 4) * kTRowB + 16 * (q ^ (4 * (((kr0 + 4) >> 1) & 1))) + 8 * (i16 & 1));

  f32x16 acc[2];  // even and odd k-steps: two independent accumulation chains
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[0][x] = acc[1][x] = 0.f;

#pragma unroll
  for (int c = 0; c < kTStages - 1; ++c)
    if (c < nchunks) issue(c);
  for (int c = 0; c < nchunks; ++c) {
    // chunk c landed (the four transfers of each later chunk issued may still fly), for every wave
    // after the barrier; the stage of chunk c-1 is then free for chunk c+3
    if (c + 2 < nchunks)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (c + 1 < nchunks)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (c + kTStages - 1 < nchunks) issue(c + kTStages - 1);
    const uint32_t st = lds0 + uint32_t((c % kTStages) * kTStageB);
    bf16x8 a[kKC / 16], b[kKC / 16];
#pragma unroll
    for (int s = 0; s < kKC / 16; ++s) {
      // the k-steps of A's 32 rows sit 32 bytes apart in the logical row: XOR of the chunk bit 1
      a[s] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
          reinterpret_cast<lds_u8*>(uintptr_t(st + (a_off ^ uint32_t(32 * s)))));
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<__attribute__((address_space(3))) i16x4*>(uintptr_t(st + b_lo + 16 * kTRowB * s)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<__attribute__((address_space(3))) i16x4*>(uintptr_t(st + b_hi + 16 * kTRowB * s)));
      b[s] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int s = 0; s < kKC / 16; ++s)
      acc[s & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], acc[s & 1], 0, 0, 0);
  }

  // D layout: column l%32, rows 8*(x/4) + 4*(l/32) + x%4
  float* const out = part + (size_t(ks) * rows) * kW + col0 + 32 * wn + (lane & 31);
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int r = row0 + 32 * wm + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
    if (r < rows) out[size_t(r) * kW] = acc[0][x] + acc[1][x];
  }
}

// RoPE inverse frequencies base^(-2i/d_r), computed on the host in double.
struct InvFreq {
  double v[kDr / 2];
};

constexpr int kFinishWaves = 4;  // waves per row in the finish: they share out the K splits

template <bool F8>
__global__ __launch_bounds__(64 * kFinishWaves) void kv_finish_kernel(const float* __restrict__ part, int rows,
                                                                     int splits, Cache c,
                                                                     const int32_t* __restrict__ seq_ids,
                                                                     const int32_t* __restrict__ positions,
                                                                     float rms_eps, InvFreq inv_freq) {
  __shared__ float red[kFinishWaves - 1][10][64];
  const int r = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // lane: latent columns 8*lane .. +7 and, for lane < 32, rotary pair lane; wave q sums the splits
  // q, q+4, ... (unrolled, so the loads of several splits are in flight together), then wave 0
  // adds the other waves' sums
  float v[10] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = wave; s < splits; s += kFinishWaves) {
    const float* p = part + (size_t(s) * rows + r) * kW;
    const float4 x0 = *reinterpret_cast<const float4*>(p + 8 * lane);
    const float4 x1 = *reinterpret_cast<const float4*>(p + 8 * lane + 4);
    const float2 y = *reinterpret_cast<const float2*>(p + kDc + 2 * (lane & 31));
    v[0] += x0.x; v[1] += x0.y; v[2] += x0.z; v[3] += x0.w;
    v[4] += x1.x; v[5] += x1.y; v[6] += x1.z; v[7] += x1.w;
    v[8] += y.x; v[9] += y.y;
  }
  if (wave > 0) {
#pragma unroll
    for (int x = 0; x < 10; ++x) red[wave - 1][x][lane] = v[x];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int q = 0; q < kFinishWaves - 1; ++q)
#pragma unroll
    for (int x = 0; x < 10; ++x) v[x] += red[q][x][lane];
  const float k1 = v[8], k2 = v[9];
  float ss = 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x) ss = fmaf(v[x], v[x], ss);
  ss = wave_sum(ss);
  const float scale = rms_eps > 0.f ? 1.f / sqrtf(ss / float(kDc) + rms_eps) : 1.f;

  const int b = seq_ids[r], t = positions[r];
  uint16_t* row;
  if constexpr (F8) {
    // E4M3 codes of the normalised fp32 latent under the token's power-of-two scale (fp8.h)
    unsigned char* row8 = const_cast<unsigned char*>(static_cast<const unsigned char*>(c.pool)) +
                          row_index(c.page_table, c.max_pages, c.page_size, b, t) * kFp8RowB;
    float amax = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      v[x] *= scale;
      amax = fmaxf(amax, fabsf(v[x]));
    }
    const int e = fp8_scale_exp(wave_max(amax));
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      w0 |= e4m3_code(ldexpf(v[x], -e)) << (8 * x);
      w1 |= e4m3_code(ldexpf(v[4 + x], -e)) << (8 * x);
    }
    *reinterpret_cast<uint2*>(row8 + 8 * lane) = make_uint2(w0, w1);
    if (lane == 0) *reinterpret_cast<u32x4*>(row8 + kFp8ScaleOff) = u32x4{__float_as_uint(ldexpf(1.f, e)), 0u, 0u, 0u};
    row = reinterpret_cast<uint16_t*>(row8);  // the rotary values follow the 512 code bytes
  } else {
    row = const_cast<uint16_t*>(static_cast<const uint16_t*>(c.pool)) +
          row_index(c.page_table, c.max_pages, c.page_size, b, t) * kW;
    u32x4 o;
#pragma unroll
    for (int x = 0; x < 4; ++x)
      o[x] = uint32_t(f32_to_bf16(v[2 * x] * scale)) | (uint32_t(f32_to_bf16(v[2 * x + 1] * scale)) << 16);
    *reinterpret_cast<u32x4*>(row + 8 * lane) = o;
  }
  if (lane < kDr / 2) {
    // angle pos * base^(-2i/d_r), i = lane, in double, reduced to [-pi, pi] before the float32
    // sine and cosine
    const double ang = double(t) * inv_freq.v[lane];
    const double rd = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
    float sn, cn;
    sincosf(float(rd), &sn, &cn);
    const float r1 = k1 * cn - k2 * sn, r2 = k1 * sn + k2 * cn;
    // (bf16 rotary values start at element 512 of a bf16 row, byte 512 of an FP8 row)
    uint16_t* kr = F8 ? row + kDc / 2 : row + kDc;
    *reinterpret_cast<uint32_t*>(kr + 2 * lane) = uint32_t(f32_to_bf16(r1)) | (uint32_t(f32_to_bf16(r2)) << 16);
  }
}

// K splits for `rows` new tokens: enough workgroups (about two per CU) to keep every CU
// streaming weights, each split a whole number of 256-row chunks.
constexpr int kTiledMinRows = 512;  // from here on kv_gemm_tiled_kernel (same splits, same partials)

int kv_splits(int d_model, int rows) {
  const int nchunk = d_model / kChunk;
  const int tiles = kColTiles * ((rows + kRowsWg - 1) / kRowsWg);
  const int want = max(1, (512 + tiles - 1) / tiles);
  int best = 1;
  for (int s = 1; s <= nchunk; ++s)
    if (nchunk % s == 0 && s <= want) best = s;
  return best;
}

// Scratch of the allocation-free cache write (mla_kv_append_noalloc): the split-K partial products
// go to this file-scope device array instead of a caller workspace.  Every GPU the library runs on
// holds its own copy until the process ends.  In host code the array's name is only a stand-in:
// kernels get the device address hipGetSymbolAddress returns for the current device, looked up on
// the first call on each device and kept per device.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

}  // namespace

hipError_t kv_append_noalloc_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = p;
  }
  *ptr = static_cast<float*>(g_scratch_addr[dev]);
  return hipSuccess;
}

bool kv_append_mfma_supported(const Dims& d, int d_model) {
  return d.dtype == MLA_BF16 && d.dc == kDc && d.dr == kDr && d_model >= kChunk && d_model % kChunk == 0;
}

size_t kv_append_mfma_workspace(int d_model, int rows) {
  return size_t(kv_splits(d_model, rows)) * size_t(rows) * kW * sizeof(float);
}

hipError_t launch_kv_append_mfma(const Dims& d, const Cache& c, int d_model, const void* h, const void* w_dkv,
                                 const void* w_kr, const int32_t* seq_ids, const int32_t* positions, int rows,
                                 float rms_eps, float* workspace, hipStream_t s, bool fp8) {
  const int splits = kv_splits(d_model, rows);
  if (rows >= kTiledMinRows)
    kv_gemm_tiled_kernel<<<kTColTiles * ((rows + kTM - 1) / kTM) * splits, kTThreads, 0, s>>>(
        static_cast<const uint16_t*>(h), d_model, rows, static_cast<const uint16_t*>(w_dkv),
        static_cast<const uint16_t*>(w_kr), d_model / splits, workspace);
  else
    kv_gemm_kernel<<<dim3(kColTiles, (rows + kRowsWg - 1) / kRowsWg, splits), kThreads, 0, s>>>(
        static_cast<const uint16_t*>(h), d_model, rows, static_cast<const uint16_t*>(w_dkv),
        static_cast<const uint16_t*>(w_kr), d_model / splits, workspace);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  InvFreq inv;
  for (int i = 0; i < kDr / 2; ++i) inv.v[i] = pow(double(d.rope_base), -2.0 * i / kDr);
  auto fin = fp8 ? kv_finish_kernel<true> : kv_finish_kernel<false>;
  fin<<<rows, 64 * kFinishWaves, 0, s>>>(workspace, rows, splits, c, seq_ids, positions, rms_eps, inv);
  return hipGetLastError();
}

}  // namespace mla
