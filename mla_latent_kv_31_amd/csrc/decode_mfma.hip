// Split-K flash-decode over the latent cache on bf16 MFMA (gfx950), DeepSeek-V3 shape:
// 128 heads, rows of 576 values = [c^KV (512) | k^R (64)], bf16 cache and q_hat, fp32 accumulate.
// The same kernel runs chunked prefill: a prefill query row is a decode query with its own causal
// key range.
//
// A workgroup runs a list of segments (query row, sequence, token range, output row): one chunk
// of the fixed split, all segments of one unit of the work-balanced split (schedule.h), or one
// prefill row.  Four waves.  All 128 heads read the same cached rows, so each 32-token tile
// (36,864 B) is fetched from HBM once per workgroup, straight into LDS with 16-byte
// global_load_lds transfers.  Four LDS buffers rotate: tile j is being scored, tile j-1 is being
// summed, tiles j+1 and j+2 are streaming in.
//
// Wave w scores heads 32w..32w+31 and runs their softmax.  The weighted sum is split the other
// way: waves 2p and 2p+1 (a pair) both accumulate heads 64p..64p+63, wave 2p latent columns
// 0..255 and wave 2p+1 columns 256..511.  Each wave hands its bf16 probabilities of a tile to
// its partner through LDS, so every transposing operand read feeds two MFMAs (one per head
// block of the pair) and the weighted sum needs half the LDS reads of a one-wave-per-head-block
// split, with the same 256-register accumulator.
//
// Scores ([ase] Fig. 2: content dot plus position dot over the concatenated row) are computed
// transposed, S^T = tile . q_hat^T, with v_mfma_f32_32x32x16_bf16: tokens on M, heads on N, so
// every lane holds the 16 scores of one head and the softmax max/sum stay inside the lane plus
// one v_permlane32_swap between the two lane halves.  The weighted latent sum ([ase] Fig. 4,
// z = a.C, rotary columns never summed) is accumulated transposed as well, O^T += C^T . P^T,
// with the 512 latent columns on M (16 blocks of 32) and heads on N.  C^T operands come from
// ds_read_b64_tr_b16, the gfx950 transposing LDS read, so the row-major tile needs no reshuffle.
// The token order inside each 16-wide MFMA k-step follows the score layout; both operands use
// the same order.
//
// Per tile and wave, phase A runs the 36 dependent score MFMAs of tile j (operands read three
// steps ahead) with the nine transfers of tile j+2 issued in its first steps, and picks up the
// partner's probabilities of tile j-1; phase B runs the 32 independent weighted-sum MFMAs of tile
// j-1 with the softmax of tile j woven between them, so that the VALU work hides behind the
// matrix cores, and publishes this wave's probabilities of tile j for the partner.
//
// LDS tile layout: a latent region (32 rows x 1,024 B) followed by a rotary region (32 rows x
// 128 B).  gfx950 LDS has 64 banks (256 B per cycle).  Latent 16-byte chunks are XOR-swizzled
// inside each 256-byte block by f(row) = ((row & 3) << 2) | ((row >> 2) & 3): any 16
// consecutive rows at one logical chunk (score reads, 16 lanes per cycle) and any 4 rows x 4
// chunks (transposing reads, 32 lanes per cycle) hit 16 distinct bank groups.  Rotary chunks are
// swizzled by g(row) = (row >> 1) & 7, two 128-byte rows sharing one 256-byte bank line.
// One 1 KiB latent row is exactly one wave-wide 16-byte transfer.
//
// The tile transfers are issued with inline global_load_lds_dwordx4 and waited for explicitly
// (s_waitcnt vmcnt + barrier at the top of each tile): the compiler cannot see that the
// transfers in flight target other buffers and would otherwise wait for them before every LDS
// read.  M0 carries the LDS destination; this kernel has no other M0 user.
//
// Softmax uses base-2 logits (q_hat carries sm_scale*log2 e) against a fixed reference per
// segment: the maximum of its first tile.  Probabilities of later tiles may then exceed one, by
// at most 2^64 (fp32 and bf16 keep their relative precision there), so the 256-register
// accumulator is never rescaled inside the loop.  If some head's scores climb more than 64
// above its reference, the workgroup runs the segment a second time with the segment maximum
// (now known) as reference; with realistic scores that pass never happens.

#include <math.h>

#include "common.h"
#include "launch.h"
#include "schedule.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kH = 128, kDc = 512, kW = 576;
constexpr int kRowB = kW * 2;                    // 1,152 bytes per cached row
constexpr int kLatB = kDc * 2;                   // 1,024 latent bytes per row
constexpr int kRopeB = kRowB - kLatB;            // 128 rotary bytes per row
constexpr int kTile = 32;                        // tokens per tile (one MFMA block)
constexpr int kNBuf = 4;                         // LDS tile buffers
constexpr int kTileB = kTile * kRowB;            // 36,864 bytes
constexpr int kRopeOff = kTile * kLatB;          // rotary region offset inside a tile buffer
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLatPerWave = kTile / kWaves;      // 8 latent-row transfers per wave per tile
constexpr int kDmaPerWave = kLatPerWave + 1;     // + 1 rotary transfer (8 rotary rows)
constexpr int kKSteps = kW / 16;                 // 36 score k-steps
constexpr int kKLat = kDc / 16;                  // 32 of them over the latent columns
constexpr int kXWaveB = 2 * 64 * 16;             // one wave's bf16 probabilities of a tile (2 k-steps)
constexpr int kXBufB = kWaves * kXWaveB;         // probability exchange of one tile: 8 KiB
constexpr int kXOff = kNBuf * kTileB;            // two exchange buffers (tiles of even / odd index)
constexpr int kLdsB = kXOff + 2 * kXBufB;        // 160 KiB: the whole CU
constexpr int kMBlk = kDc / 2 / 32;              // 8 latent blocks of 32 columns per wave
constexpr int kAcc = 2 * kMBlk;                  // x 2 head blocks = 16 accumulator blocks
constexpr int kPvOps = 2 * kMBlk;                // 16 transposed operands per tile (2 k-steps)
constexpr int kPvSteps = 2 * kPvOps;             // 32 weighted-sum MFMAs per tile
constexpr float kRerunMargin = 64.0f;  // reference may lag the running max by this much

// FP8 cache rows (E4M3 latent codes with one power-of-two scale per token): 512 codes | 64 bf16
// rotary values | fp32 scale | 12 zero bytes.  The FP8 variant of the kernel stages each tile's
// codes (and scales) in LDS, converts them once per tile into the bf16 tile layout above, and runs
// the unchanged MFMA phases on that.  Three bf16 tile buffers (tile j scored, tile j-1 summed,
// tile j+1 being converted) and two code staging slots fit next to the exchange buffers.
constexpr int kRowB8 = 656;
constexpr int kNBuf8 = 3;
constexpr int kStgCodesB = kTile * kDc;           // 16 KiB of codes per staged tile
constexpr int kStgB = kStgCodesB + 1024;          // + one transfer of the 32 rows' scale chunks
constexpr int kStgOff = kNBuf8 * kTileB;
constexpr int kXOff8 = kStgOff + 2 * kStgB;
constexpr int kLdsB8 = kXOff8 + 2 * kXBufB;       // 158 KiB
static_assert(kLdsB8 <= 160 * 1024, "FP8 layout fits the CU's LDS");

__host__ __device__ constexpr int lat_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__host__ __device__ constexpr int rope_swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ float lane_swap_max(float v) {
  // v_permlane32_swap(v, v): lanes < 32 receive the upper half in .y, lanes >= 32 the lower
  // half in .x; the max of both is the max over the lane pair (l, l^32).
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_swap_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One step of the score chain, accumulated in VGPRs (the 256 accumulator registers hold the
// weighted sums).  The first step starts from zero; consecutive steps accumulate into exactly the
// same registers, which the matrix core forwards; after the last one the wave waits out the
// result latency before any VALU instruction reads the scores.
__device__ __forceinline__ void score_step(bool first, bool last, f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if (first) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  } else if (last) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(acc) : "v"(a), "v"(b));
  } else {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  }
}

__device__ __forceinline__ bf16x8 lds16(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

__device__ __forceinline__ void dma16(uint32_t lds_dst, uint32_t voff, const unsigned char* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_dst), "v"(voff), "s"(gbase)
               : "memory");
}

// Page ids of 64 consecutive pages of a sequence's table, one per lane, loaded and waited for in
// one asm block.  Tile addresses are then taken with v_readlane: a compiler-visible load here
// would leave a pending-load state at the loop joins and make the compiler drain every tile
// transfer in flight before the next use.  Lanes past the last page read the final table entry.
__device__ __forceinline__ int load_page_window(const int32_t* row, int first, int count, int max_pages, int lane) {
  const uint32_t off = 4u * uint32_t(min(first + lane, max_pages - 1));
  int v;
  asm volatile("global_load_dword %0, %1, %2\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(off), "s"(row) : "memory");
  return lane < count ? v : 0;
}

// What a workgroup runs: a list of segments (query row, sequence, token range, output row).
enum Mode {
  kFixed = 0,     // one chunk of the fixed split; grid = chunks x sequences
  kBalanced = 1,  // every segment of one unit of the balanced split; grid = units (schedule.h)
  kPrefill = 2,   // one query row of a prefill chunk over its whole causal key range, written
                  // straight to z / lse; grid = rows, longest rows first
};

template <int MODE, bool F8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(const uint16_t* __restrict__ pool, const int32_t* __restrict__ page_table,
                        const int32_t* __restrict__ seq_lens, int batch, int max_pages, int page_size,
                        int tiles_per_page_log2, const uint16_t* __restrict__ q_hat, int n_splits,
                        int split_tokens, const int32_t* __restrict__ q_start, float* __restrict__ o_part,
                        float* __restrict__ lse_part) {
  constexpr bool kBal = MODE == kBalanced;
  constexpr int kNB = F8 ? kNBuf8 : kNBuf;          // bf16 tile buffers
  constexpr int kXO = F8 ? kXOff8 : kXOff;          // exchange buffers
  __shared__ __attribute__((aligned(16))) unsigned char smem[F8 ? kLdsB8 : kLdsB];
  lds_u8* const lbase = (lds_u8*)smem;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hi = lane >> 5;
  const int head = wave * 32 + (lane & 31);  // scored by this lane (lanes l and l^32 share it)
  const int lh = wave & 1;                   // latent half summed by this wave
  const int cap = max_pages * page_size;  // never index past the page table

  // ---- per-lane constants of the tile transfers.  Latent row n = 4x + wave (x < 8) is one 1 KiB
  // transfer; rotary rows 8*wave .. 8*wave+7 are this wave's ninth.  Lane L writes LDS chunk L of
  // the transfer; the global chunk it reads is the one that the XOR swizzle places there.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // (lane & ~15) | ((lane ^ c) & 15) = lane ^ c for a 4-bit c: one XOR with a scalar per transfer
  // from a single per-lane base (kept opaque in the tile loop, so no per-transfer copies are held)
  uint32_t lane16 = 16u * uint32_t(lane);
  auto lat_off = [&](int x) {  // the swizzle of row n = 4x + wave depends on n & 15
    return lane16 ^ uint32_t(16 * lat_swz(4 * (x & 3) + wave_u));
  };
  auto rope_off = [&]() {
    constexpr int rb = F8 ? kRowB8 : kRowB, ro = F8 ? kDc : kLatB;  // row stride, rotary offset
    return uint32_t((lane >> 3) * rb + ro + 16 * ((lane & 7) ^ ((4 * wave_u + (lane >> 4)) & 7)));
  };
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(lbase));

  // ---- per-lane LDS offsets
  // score reads: row (lane&31), logical chunk 2k + hi (latent) or 2(k-32) + hi (rotary).  The
  // swizzle XORs the chunk index, so the place of step k is the place of step 0 XOR 32*k bytes
  // (k < 8 within a 256-byte block; rotary k < 4).
  int qk_x, qr_x;
  {
    const int fl = lat_swz(lane & 15), gr = rope_swz(lane & 31);
    qk_x = (lane & 31) * kLatB + 16 * (hi ^ fl);
    qr_x = kRopeOff + (lane & 31) * kRopeB + 16 * (hi ^ gr);
  }
  // transposing reads: lane group g = lane/16 reads rows r0 = 4*(g/2) + (lane%16)/4 (+16a, +8 for
  // the second half of the k-step), columns 32*mb + 16*(g%2) + 4*(lane%4) .. +3 of this wave's
  // latent half.  Column block 4*m4 + y lands at the place of m4 = 0 XOR 64*m4; the row +8 flips
  // bit 1 of the swizzle, so the second read sits a fixed per-lane distance from the first.
  int pv_x, pv_d8;
  {
    const int g = lane >> 4, ii = lane & 15, qq = ii & 3;
    const int r0 = 4 * (g >> 1) + (ii >> 2);
    const int y = 2 * (g & 1) + (qq >> 1);
    pv_x = r0 * kLatB + 512 * lh + 16 * (y ^ lat_swz(r0)) + 8 * (qq & 1);
    pv_d8 = 8 * kLatB + 16 * (((4 + y) ^ lat_swz(8 + r0)) - ((4 + y) ^ lat_swz(r0)));
  }
  // probability exchange: this lane's 16 bytes of k-step s in the buffer of tile parity t
  const uint32_t x_mine = uint32_t(kXO + wave * kXWaveB + 16 * lane);
  const uint32_t x_peer = uint32_t(kXO + (wave ^ 1) * kXWaveB + 16 * lane);
  auto x_at = [&](uint32_t base, int t, int s) { return lbase + base + t * kXBufB + s * 1024; };
  auto a_src = [&](const lds_u8* tb, int kk) -> const lds_u8* {
    return kk < kDc / 16 ? tb + 256 * (kk >> 3) + (qk_x ^ (32 * (kk & 7))) : tb + (qr_x ^ (32 * (kk & 3)));
  };
  // weighted-sum operand o = 8 * kstep + mb (mb: block of this wave's latent half): two
  // transposing reads, tokens +0..3 / +8..11
  auto tr8 = [&](const lds_u8* tb, int o) {
    const lds_u8* base = tb + 16 * (o >> 3) * kLatB + 256 * ((o & 7) >> 2);
    const lds_u8* p0 = base + (pv_x ^ (64 * (o & 3)));
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
    const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0 + pv_d8));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // ---- the segment list
  const int unit = blockIdx.x;
  int next_b, next_cb = 0, unit_end = 0, quota = 0;
  if constexpr (kBal) {
    int total;
    sched_prefix(seq_lens, batch, cap, 0, next_cb, total);
    total = __builtin_amdgcn_readfirstlane(total);  // wave-uniform: keep the segment loop scalar
    quota = sched_quota(total, n_splits);
    if (quota == 0 || unit * quota >= total) return;  // idle unit (uniform)
    unit_end = min(unit * quota + quota, total);
    sched_find(seq_lens, batch, cap, unit * quota, next_b, next_cb);
    next_b = __builtin_amdgcn_readfirstlane(next_b);
    next_cb = __builtin_amdgcn_readfirstlane(next_cb);
  } else {
    next_b = blockIdx.y;
  }

  for (bool first_seg = true;; first_seg = false) {
    int b, t0, t1;
    size_t slot, qrow;  // output row group and q_hat row group (128 heads each)
    if constexpr (kBal) {
      if (next_b >= batch || next_cb >= unit_end) break;
      b = next_b;
      const int len = sched_len(seq_lens[b], cap);
      int k0, k1;
      sched_segment(next_cb, sched_tiles(len), unit, quota, k0, k1);
      next_cb += sched_cost(len);
      ++next_b;
      if (k1 <= k0) continue;  // this unit holds only the segment price of sequence b
      t0 = k0 * kTile;
      t1 = min(k1 * kTile, len);
      slot = size_t(unit) + b;
      qrow = b;
    } else if constexpr (MODE == kPrefill) {
      // n_splits carries the chunk length; row i of sequence b reads keys t <= q_start[b] + i
      const int i = n_splits - 1 - unit / batch;
      b = unit % batch;
      qrow = slot = size_t(b) * n_splits + i;
      t0 = 0;
      t1 = min(sched_len(seq_lens[b], cap), max(q_start[b] + i + 1, 0));
      if (t1 <= 0) {  // no visible key: z = 0, lse = -inf
        float* zr = o_part + (slot * kH + head) * kDc + 4 * hi;
        for (int c = 0; c < kDc; c += 8) *reinterpret_cast<float4*>(zr + c) = make_float4(0.f, 0.f, 0.f, 0.f);
        if (hi == 0 && lse_part) lse_part[slot * kH + head] = -INFINITY;
        return;
      }
    } else {
      b = next_b;
      qrow = b;
      t0 = unit * split_tokens;
      t1 = min(t0 + split_tokens, sched_len(seq_lens[b], cap));
      slot = size_t(b) * n_splits + unit;
      if (t0 >= t1) {  // empty chunk: lse = -inf; its o_part is never read by the combine
        if (hi == 0) lse_part[slot * kH + head] = -INFINITY;
        return;
      }
    }
    if (!first_seg) __syncthreads();  // the previous segment is done with every LDS buffer
    const size_t orow = slot * kH + head;
    const int ntiles = (t1 - t0 + kTile - 1) / kTile;

    // Page ids of the segment, 64 per window, one per lane.  t0 is a multiple of the tile.
    const int kt0 = t0 / kTile;  // first tile, counted from the sequence start
    const int p0 = kt0 >> tiles_per_page_log2;
    const int npg = ((kt0 + ntiles - 1) >> tiles_per_page_log2) - p0 + 1;
    const int32_t* pt_row = page_table + size_t(b) * max_pages;
    int wbase = 0;  // first page of the window held in my_page
    int my_page = load_page_window(pt_row, p0, npg, max_pages, lane);
    auto tile_src = [&](int k) {
      const int kt = kt0 + k;
      const int pg = __builtin_amdgcn_readlane(my_page, ((kt >> tiles_per_page_log2) - p0 - wbase) & 63);
      const int in_page = (kt & ((1 << tiles_per_page_log2) - 1)) * kTile;
      if constexpr (F8)
        return reinterpret_cast<const unsigned char*>(pool) + (size_t(pg) * page_size + in_page) * kRowB8;
      else
        return reinterpret_cast<const unsigned char*>(pool + (size_t(pg) * page_size + in_page) * kW);
    };
    auto dma_one = [&](const unsigned char* g, uint32_t dst, int x) {  // x-th transfer of a tile
      if (x < kLatPerWave) {
        const int n = 4 * x + wave_u;
        dma16(dst + uint32_t(n * kLatB), lat_off(x), g + size_t(n) * kRowB);
      } else {
        dma16(dst + uint32_t(kRopeOff + wave_u * 1024), rope_off(), g + size_t(8 * wave_u) * kRowB);
      }
    };
    auto dma_tile = [&](int k) {
      const unsigned char* g = tile_src(k);
      const uint32_t dst = lds0 + uint32_t((k % kNB) * kTileB);
#pragma unroll
      for (int x = 0; x < kDmaPerWave; ++x) dma_one(g, dst, x);
    };
    // ---- FP8: transfer x of a tile's codes and scales into staging slot `slot`.  Transfer
    // T = 4*wave + x (x < 4) moves rows 2T, 2T+1 (512 code bytes each; lane L: row 2T + L/32, chunk
    // L%32); x = 4 (wave 0 only) moves the 16-byte scale chunk of row L%32 (lanes 32..63 repeat
    // rows 0..31).  The rotary rows go straight into the bf16 tile buffer (dma_rope8).
    const uint32_t c8_off = uint32_t((lane >> 5) * kRowB8 + 16 * (lane & 31));
    const uint32_t s8_off = uint32_t((lane & 31) * kRowB8 + kDc + 2 * (kW - kDc));
    auto dma_codes8 = [&](const unsigned char* g, int slot, int x) {
      const uint32_t dst = lds0 + uint32_t(kStgOff + slot * kStgB);
      if (x < 4) {
        const int T = 4 * wave_u + x;
        dma16(dst + uint32_t(T * 1024), c8_off, g + size_t(2 * T) * kRowB8);
      } else if (wave_u == 0) {
        dma16(dst + uint32_t(kStgCodesB), s8_off, g);
      }
    };
    auto dma_rope8 = [&](const unsigned char* g, int k) {
      dma16(lds0 + uint32_t((k % kNB) * kTileB + kRopeOff + wave_u * 1024), rope_off(), g + size_t(8 * wave_u) * kRowB8);
    };
    auto dma_tile8 = [&](int k) {  // codes and scales of tile k into slot k&1, its rotary rows into buffer k%3
      const unsigned char* g = tile_src(k);
#pragma unroll
      for (int x = 0; x < 5; ++x) dma_codes8(g, k & 1, x);
      dma_rope8(g, k);
    };
    // ---- FP8: convert the staged codes of tile k (slot k&1) into the bf16 latent rows of buffer
    // k%3, code x scale (exact: a power-of-two scale), rows >= nval as zeros.  Wave w converts rows
    // 8w..8w+7; lane l takes row 8w + l/8 and code chunks q = l%8 + 8u (16 codes, two bf16 chunks).
    const int cv_row = 8 * wave + (lane >> 3);
    auto cv_read = [&](int k, int u) {  // 16 codes of chunk u
      const lds_u8* stg = lbase + kStgOff + (k & 1) * kStgB;
      return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(stg + cv_row * kDc +
                                                                                16 * ((lane & 7) + 8 * u));
    };
    auto cv_scale = [&](int k) {
      const lds_u8* stg = lbase + kStgOff + (k & 1) * kStgB + kStgCodesB;
      return *reinterpret_cast<const __attribute__((address_space(3))) float*>(stg + 16 * cv_row);
    };
    // the two bf16 output chunks (8 values each) of code chunk u, half h (dwords 2h, 2h+1)
    auto cv_write = [&](int k, int u, int h, const u32x4& codes, float scale, bool valid) {
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint32_t w = codes[2 * h + d];
        o[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, false));
        o[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, true));
      }
      if (!valid) o = u32x4{0u, 0u, 0u, 0u};
      const int c = 2 * ((lane & 7) + 8 * u) + h;  // bf16 chunk of the 1,024-byte latent row
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
          lbase + (k % kNB) * kTileB + cv_row * kLatB + 256 * (c >> 4) + 16 * ((c & 15) ^ lat_swz(cv_row))) = o;
    };
    auto cv_valid = [&](int k) { return cv_row < t1 - (t0 + k * kTile); };
    auto convert_tile8 = [&](int k) {  // all at once (the prologue's tile 0)
      const float sc = cv_scale(k);
      const bool v = cv_valid(k);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 cd = cv_read(k, u);
        cv_write(k, u, 0, cd, sc, v);
        cv_write(k, u, 1, cd, sc, v);
      }
    };

    if constexpr (F8) {
      dma_tile8(0);
    } else {
      dma_tile(0);
    }

    // ---- this wave's 32 heads of q_hat, as the B operand of S^T = tile . q_hat^T, held in
    // registers for the whole segment: 32 latent and 4 rotary k-steps.
    bf16x8 qf[kKLat], rq[kKSteps - kKLat];
    {
      const uint16_t* qp = q_hat + (qrow * kH + head) * kW + 8 * hi;
#pragma unroll
      for (int k = 0; k < kKLat; ++k) qf[k] = *reinterpret_cast<const bf16x8*>(qp + 16 * k);
#pragma unroll
      for (int k = 0; k < kKSteps - kKLat; ++k) rq[k] = *reinterpret_cast<const bf16x8*>(qp + kDc + 16 * k);
    }
    // Consume these loads here: an empty asm that reads every fragment makes the compiler wait for
    // them before the tile loop (tile 0 and the previous segment's stores complete too).  Otherwise
    // its waits for them land inside the loop, where the vmcnt they use would also drain the tile
    // transfers in flight.
#pragma unroll
    for (int k = 0; k < kKLat; ++k) asm volatile("" : "+v"(qf[k]));
#pragma unroll
    for (int k = 0; k < kKSteps - kKLat; ++k) asm volatile("" : "+v"(rq[k]));
    if constexpr (F8) {
      // codes of tile 1 (past a one-tile segment: a copy of tile 0 into the free slot)
      const unsigned char* g1 = tile_src(min(1, ntiles - 1));
#pragma unroll
      for (int x = 0; x < 5; ++x) dma_codes8(g1, 1, x);
    } else {
      if (ntiles > 1) dma_tile(1);
    }

    f32x16 acc[kAcc];  // acc[2 * mb + 0]: own heads, acc[2 * mb + 1]: the partner's
    float m_ref = -INFINITY, m_max = -INFINITY, l_lane = 0.f;
    bf16x8 pb0, pb1;  // own probabilities of the previous tile, bf16, k-steps 0 and 1

    for (int pass = 0; pass < 2; ++pass) {
      if (pass > 0) {
        if (wbase != 0) {
          wbase = 0;
          my_page = load_page_window(pt_row, p0, npg, max_pages, lane);
        }
        if constexpr (F8) {
          dma_tile8(0);
          const unsigned char* g1 = tile_src(min(1, ntiles - 1));
#pragma unroll
          for (int x = 0; x < 5; ++x) dma_codes8(g1, 1, x);
        } else {
          dma_tile(0);
          if (ntiles > 1) dma_tile(1);
        }
      }
      // source of the transfers issued in the next tile step: tile j+2 of step j, or, past the
      // segment end, a harmless copy of its last tile into the buffer that is free anyway
      const unsigned char* g_dma = tile_src(min(2, ntiles - 1));
      // FP8: source of tile j+1, whose rotary rows go out at the top of step j (its address was
      // the code transfers' source one step earlier, taken before any page-window move)
      const unsigned char* g_rope = F8 ? tile_src(min(1, ntiles - 1)) : nullptr;
#pragma unroll
      for (int a = 0; a < kAcc; ++a)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[a][x] = 0.f;
      l_lane = 0.f;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        pb0[x] = (__bf16)0.f;
        pb1[x] = (__bf16)0.f;
      }
      // The weighted sum of the tile before tile 0 runs on a zeroed buffer with zero
      // probabilities (own and, in the exchange buffer of odd tiles, the partner's), which keeps
      // the pipelined loop uniform.
      {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (int x = threadIdx.x; x < kRopeOff / 16; x += kThreads)
          *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(lbase + (kNB - 1) * kTileB + 16 * x) = zero;
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(x_at(x_mine, 1, 0)) = zero;
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(x_at(x_mine, 1, 1)) = zero;
      }
      if constexpr (F8) {  // tile 0's codes landed: convert them before the loop
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        convert_tile8(0);
      }

      bool over = false;
      for (int j = 0; j < ntiles; ++j) {
        // A segment longer than 64 pages moves its page window once tile j+3, whose address this
        // step computes, leaves it (the wait inside the load also drains tile j+1, a bubble every
        // 64 pages).  Tiles whose addresses are already computed are not affected.
        if (j + 3 < ntiles && ((kt0 + j + 3) >> tiles_per_page_log2) - p0 - wbase >= 64) {
          wbase += 64;
          my_page = load_page_window(pt_row, p0 + wbase, npg - wbase, max_pages, lane);
        }
        if (F8 || j + 1 >= ntiles)
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // FP8: codes of j+1 and rotary rows of j landed
        else
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerWave) : "memory");  // tile j landed, j+1 may fly
        __syncthreads();  // every wave's part of tile j landed; tile j-2 fully consumed
        // Keep the per-step offsets derived inside the loop (one XOR each) instead of letting the
        // compiler hoist a dozen precomputed copies into registers next to the q_hat fragments.
        asm volatile("" : "+v"(qk_x), "+v"(qr_x), "+v"(pv_x), "+v"(pv_d8), "+v"(lane16));
        lds_u8* const tb = lbase + (j % kNB) * kTileB;
        lds_u8* const tp = lbase + ((j + kNB - 1) % kNB) * kTileB;
        const int nvalid = min(kTile, t1 - (t0 + j * kTile));
        // FP8: the rotary rows of tile j+1 go to the buffer tile j-2 left (past the segment end a
        // copy of the last tile's); its latent rows are converted in phase B below
        if constexpr (F8) dma_rope8(g_rope, j + 1);
        if (!F8 && nvalid < kTile) {  // tail tile: latent rows past the sequence end read as zeros
          // (FP8 tiles get their zero rows from the conversion)
          const u32x4 zero = {0u, 0u, 0u, 0u};
          for (int x = threadIdx.x; x < (kTile - nvalid) * (kLatB / 16); x += kThreads)
            *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(tb + nvalid * kLatB + 16 * x) = zero;
          __syncthreads();
        }
        // Tile j+2 goes to the buffer that tile j-2 left; past the segment end the transfers copy
        // the segment's last tile there instead, which keeps the wait counts uniform and the loop
        // free of branches.  Every transfer lands before the loop ends (drained below).
        const uint32_t dnext = lds0 + uint32_t(((j + 2) % kNB) * kTileB);
        const unsigned char* g_dma_next = g_dma;

        // ---- phase A: scores of tile j, one dependent MFMA chain, operands read kQA steps
        // ahead; the nine transfers of tile j+2 go out in its first steps, the partner's
        // probabilities of tile j-1 are read after them, and the first kPB operand reads of phase B
        // are issued during its last steps
        constexpr int kQA = 3, kPB = 3;
        f32x16 sacc;
        bf16x8 pa[kPB + 1], pq0, pq1;
        {
          bf16x8 qa[kQA + 1];
#pragma unroll
          for (int i = 0; i < kQA; ++i) qa[i] = lds16(a_src(tb, i));
          __builtin_amdgcn_sched_barrier(0);  // the first operand reads go out right after the barrier
#pragma unroll
          for (int i = 0; i < kKSteps; ++i) {
            if (i + kQA < kKSteps) {
              qa[(i + kQA) % (kQA + 1)] = lds16(a_src(tb, i + kQA));
            } else if (i + kQA - kKSteps < kPB) {
              const int k = i + kQA - kKSteps;
              pa[k] = tr8(tp, k);
            }
            if (i == kDmaPerWave + 2) pq0 = lds16(x_at(x_peer, (j + 1) & 1, 0));
            if (i == kDmaPerWave + 3) pq1 = lds16(x_at(x_peer, (j + 1) & 1, 1));
            score_step(i == 0, i == kKSteps - 1, sacc, qa[i % (kQA + 1)], i < kKLat ? qf[i] : rq[i - kKLat]);
            if constexpr (F8) {
              if (i % 4 == 1 && i / 4 < 5) dma_codes8(g_dma, j & 1, i / 4);  // codes of tile j+2
            } else {
              if (i % 4 == 1) dma_one(g_dma, dnext, i / 4);
            }
            if (i == 22) g_dma_next = tile_src(min(j + 3, ntiles - 1));  // for the next step
            __builtin_amdgcn_sched_barrier(0);
          }
        }

        // tail tile: scores of tokens past the segment end drop out of the softmax
        if (nvalid < kTile) {
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int tok = 8 * (x >> 2) + 4 * hi + (x & 3);
            if (tok >= nvalid) sacc[x] = -INFINITY;
          }
        }

        // ---- phase B: weighted sum of tile j-1 (16 operands x 2 head blocks = 32 independent
        // MFMAs) with the online softmax of tile j (base-2 logits; lane = one head, lanes l and l^32
        // share it) woven between them, so the VALU work runs in the shadow of the matrix cores.
        // Branch-free: the reference update is a select.
        {
          const bool first = pass == 0 && j == 0;  // the segment's first tile fixes the reference
          float mx0 = 0.f, mx = 0.f, pr[16], tsum = 0.f;
          bf16x8 pn0, pn1;
          u32x4 cv_cd[2];  // FP8: code chunks of tile j+1 in flight
          float cv_sc = 0.f;
          bool cv_ok = false;
#pragma unroll
          for (int i = 0; i < kPvSteps; ++i) {
            const int o = i >> 1, nb = i & 1;  // operand, head block (0: own, 1: partner)
            if (nb == 0 && o + kPB < kPvOps) pa[(o + kPB) % (kPB + 1)] = tr8(tp, o + kPB);
            const bf16x8 pp = o < kMBlk ? (nb ? pq0 : pb0) : (nb ? pq1 : pb1);
            acc[2 * (o & 7) + nb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[o % (kPB + 1)], pp, acc[2 * (o & 7) + nb], 0, 0, 0);
            if (i == 1 || i == 2) {  // row maximum, one half per step
              float m = -INFINITY;
#pragma unroll
              for (int x = 8 * (i - 1); x < 8 * i; ++x) m = fmaxf(m, sacc[x]);
              if (i == 1) {
                mx0 = m;
              } else {
                mx = lane_swap_max(fmaxf(mx0, m));
                m_ref = first ? mx : m_ref;
                m_max = fmaxf(m_max, mx);
                over |= mx > m_ref + kRerunMargin;
              }
            }
            // one probability per step (the exp2 is a quarter-rate instruction), summed and
            // packed to bf16 pairwise as they come, so that no step outgrows its MFMA
            if (i >= 3 && i < 19) pr[i - 3] = fast_exp2(sacc[i - 3] - m_ref);
            if (i == 4) tsum = pr[0];
            if (i >= 5 && i < 20) tsum += pr[i - 4];
            if (i >= 5 && i < 20 && (i & 1)) {  // pair (i-5)/2 is complete
              const int x = i - 5;
              if (x < 8) {
                pn0[x] = (__bf16)pr[x];
                pn0[x + 1] = (__bf16)pr[x + 1];
              } else {
                pn1[x - 8] = (__bf16)pr[x];
                pn1[x - 7] = (__bf16)pr[x + 1];
              }
            }
            if (i == 20) l_lane += tsum;
            // for the partner, read after the next tile's barrier
            if (i == 13) *reinterpret_cast<__attribute__((address_space(3))) bf16x8*>(x_at(x_mine, j & 1, 0)) = pn0;
            if (i == 21) *reinterpret_cast<__attribute__((address_space(3))) bf16x8*>(x_at(x_mine, j & 1, 1)) = pn1;
            if constexpr (F8) {
              // the codes of tile j+1 become its bf16 latent rows in the shadow of the last
              // weighted-sum MFMAs, once the scores and probabilities are dead: chunk u is read two
              // steps before its two halves are converted and written (steps 20 .. 27)
              if (i == 17) {
                cv_sc = cv_scale(j + 1);
                cv_ok = cv_valid(j + 1);
              }
              if (i >= 20 && i < 28) cv_write(j + 1, (i - 20) >> 1, i & 1, cv_cd[((i - 20) >> 1) & 1], cv_sc, cv_ok);
              if (i >= 18 && i < 26 && !(i & 1)) cv_cd[((i - 18) >> 1) & 1] = cv_read(j + 1, (i - 18) >> 1);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          pb0 = pn0;
          pb1 = pn1;
          if constexpr (F8) g_rope = g_dma;
          g_dma = g_dma_next;
        }
      }

      // ---- weighted sum of the last tile, once the partner's probabilities of it are published
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      {
        lds_u8* const tp = lbase + ((ntiles - 1) % kNB) * kTileB;
        const bf16x8 pq0 = lds16(x_at(x_peer, (ntiles - 1) & 1, 0));
        const bf16x8 pq1 = lds16(x_at(x_peer, (ntiles - 1) & 1, 1));
        bf16x8 pa[3];
        pa[0] = tr8(tp, 0);
        pa[1] = tr8(tp, 1);
#pragma unroll
        for (int i = 0; i < kPvSteps; ++i) {
          const int o = i >> 1, nb = i & 1;
          if (nb == 0 && o + 2 < kPvOps) pa[(o + 2) % 3] = tr8(tp, o + 2);
          const bf16x8 pp = o < kMBlk ? (nb ? pq0 : pb0) : (nb ? pq1 : pb1);
          acc[2 * (o & 7) + nb] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[o % 3], pp, acc[2 * (o & 7) + nb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- rerun the segment if some head outgrew its reference (uniform decision)
      // the flags go to the buffer after the last tile's, idle now
      __attribute__((address_space(3))) int* rerun_flag =
          reinterpret_cast<__attribute__((address_space(3))) int*>(lbase + (ntiles % kNB) * kTileB);
      const bool wave_over = __builtin_amdgcn_ballot_w64(over) != 0;
      if (lane == 0) rerun_flag[wave] = wave_over;
      __syncthreads();
      const bool rerun = rerun_flag[0] | rerun_flag[1] | rerun_flag[2] | rerun_flag[3];
      if (!rerun) break;
      m_ref = m_max;
      __syncthreads();
    }

    // ---- normalise and write the segment's partial.  The sums of the partner's heads come
    // through the exchange buffer that no tile uses any more.  The MFMA layout gives each lane
    // 16-byte pieces of 32 different rows; staged through LDS (the tile buffers are idle now),
    // every store instruction writes 1 KiB of one contiguous half row instead.
    const float l_tot = lane_swap_sum(l_lane);
    __attribute__((address_space(3))) float* const l_x =
        reinterpret_cast<__attribute__((address_space(3))) float*>(lbase + kXO + (ntiles & 1) * kXBufB);
    if (hi == 0) l_x[head] = l_tot;
    __syncthreads();  // every wave is done with the tile buffers and the rerun flags; sums published
    const float inv_own = 1.f / l_tot, inv_peer = 1.f / l_x[(wave ^ 1) * 32 + (lane & 31)];
    {
      constexpr int kStRow = 256 * 4 + 16;  // one staged half row, padded against bank conflicts
      static_assert(kWaves * 32 * kStRow <= kXOff && kWaves * 32 * kStRow <= kXOff8,
                    "staging stays clear of the exchange buffers");
      lds_u8* const stg = lbase + wave * 32 * kStRow;
#pragma unroll
      for (int half = 0; half < 2; ++half) {  // head block: own, then the partner's
        float* const orow0 = o_part + (slot * kH + (half ? wave ^ 1 : wave) * 32) * kDc + 256 * lh;
        const float inv = half ? inv_peer : inv_own;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const f32x16 v = acc[2 * m + half] * inv;
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const u32x4 f = {__float_as_uint(v[4 * j4]), __float_as_uint(v[4 * j4 + 1]), __float_as_uint(v[4 * j4 + 2]),
                             __float_as_uint(v[4 * j4 + 3])};
            *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
                stg + (lane & 31) * kStRow + 4 * (32 * m + 8 * j4 + 4 * hi)) = f;
          }
        }
        // the same wave reads back what it wrote: LDS operations of one wave complete in order
#pragma unroll 8
        for (int r = 0; r < 32; ++r) {
          const u32x4 x = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(stg + r * kStRow + 16 * lane);
          *reinterpret_cast<u32x4*>(orow0 + size_t(r) * kDc + 4 * lane) = x;
        }
      }
    }
    if (hi == 0 && lse_part) lse_part[orow] = (m_ref + log2f(l_tot)) * kLn2;
    if constexpr (!kBal) break;
  }
}

}  // namespace

bool decode_mfma_supported(const Dims& d, const Cache& c, int split_tokens) {
  const int tpp = c.page_size / kTile;  // tiles per page: a power of two
  return d.dtype == MLA_BF16 && d.H == kH && d.dc == kDc && d.dr == kW - kDc && c.page_size % kTile == 0 &&
         tpp > 0 && (tpp & (tpp - 1)) == 0 && (split_tokens == 0 || split_tokens % c.page_size == 0);
}

hipError_t launch_decode_mfma(const Dims& d, const Cache& c, const void* q_hat, int n_splits, int split_tokens,
                              float* o_part, float* lse_part, hipStream_t s, bool fp8) {
  (void)d;
  const int tpp_log2 = __builtin_ctz(unsigned(c.page_size / kTile));
  auto k = fp8 ? decode_mfma_kernel<kFixed, true> : decode_mfma_kernel<kFixed, false>;
  k<<<dim3(n_splits, c.batch), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(c.pool), c.page_table, c.seq_lens, c.batch, c.max_pages, c.page_size, tpp_log2,
      static_cast<const uint16_t*>(q_hat), n_splits, split_tokens, nullptr, o_part, lse_part);
  return hipGetLastError();
}

hipError_t launch_decode_mfma_balanced(const Dims& d, const Cache& c, const void* q_hat, int n_units, float* o_part,
                                       float* lse_part, hipStream_t s, bool fp8) {
  (void)d;
  const int tpp_log2 = __builtin_ctz(unsigned(c.page_size / kTile));
  auto k = fp8 ? decode_mfma_kernel<kBalanced, true> : decode_mfma_kernel<kBalanced, false>;
  k<<<dim3(n_units), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(c.pool), c.page_table, c.seq_lens, c.batch, c.max_pages, c.page_size, tpp_log2,
      static_cast<const uint16_t*>(q_hat), n_units, 0, nullptr, o_part, lse_part);
  return hipGetLastError();
}

bool prefill_mfma_supported(const Dims& d, const Cache& c) { return decode_mfma_supported(d, c, 0); }

hipError_t launch_prefill_mfma(const Dims& d, const Cache& c, const void* q_hat, int q_len, const int32_t* q_start,
                               float* z, float* lse, hipStream_t s, bool fp8) {
  (void)d;
  const int tpp_log2 = __builtin_ctz(unsigned(c.page_size / kTile));
  auto k = fp8 ? decode_mfma_kernel<kPrefill, true> : decode_mfma_kernel<kPrefill, false>;
  k<<<dim3(c.batch * q_len), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(c.pool), c.page_table, c.seq_lens, c.batch, c.max_pages, c.page_size, tpp_log2,
      static_cast<const uint16_t*>(q_hat), q_len, 0, q_start, z, lse);
  return hipGetLastError();
}

}  // namespace mla
