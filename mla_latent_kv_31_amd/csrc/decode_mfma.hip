// Split-K flash-decode over the latent cache on MFMA (gfx950), DeepSeek-V3 shape: 128 heads, rows of
// 576 values = [c^KV (512) | k^R (64)], a bf16 (or FP8) cache, an IEEE binary16 absorbed query, fp32
// accumulation.  The same kernel runs chunked prefill: a prefill query row is a decode query with
// its own causal key range.
//
// A workgroup runs a list of segments (query row, sequence, token range, output row): one chunk
// of the fixed split, all segments of one unit of the work-balanced split (schedule.h), or one
// prefill row.  Four waves.  All 128 heads read the same cached rows, so each 32-token tile
// (36,864 B) is fetched from HBM once per workgroup, straight into LDS with 16-byte
// global_load_lds transfers.  Four LDS buffers rotate: tile j is being scored, tile j-1 is being
// summed, tile j+1 is converted, tile j+2 is streaming in.
//
// Precision.  The matrix products run in binary16: every wave converts, in place, the bf16 values
// it transferred itself (exact for the latents' range; binary16 has three more significand bits
// than bf16), the absorbed query arrives in binary16, and the probabilities are rounded to
// binary16.  Rounding q_hat and P to bf16 instead would put single heads of short or peaked rows
// past the bf16 tolerance on the output; binary16 keeps them an order of magnitude inside it.
//
// Wave w scores heads 32w..32w+31 and runs their softmax.  Scores ([ase] Fig. 2: content dot plus
// position dot over the concatenated row) are computed transposed, S^T = tile . q_hat^T, with
// v_mfma_f32_16x16x32_f16 in four independent accumulation chains (two 16-token blocks x two
// 16-head blocks, 18 k-steps each), interleaved so that no MFMA waits on the one before it.  Lane
// l then holds, for heads 32w + l%16 and 32w + 16 + l%16, the scores of tokens 4g..4g+3 and
// 16+4g..16+4g+3 (g = l/16): the softmax max/sum stay inside the lane plus one permlane16_swap
// and one permlane32_swap.
//
// The weighted latent sum ([ase] Fig. 4, z = a.C, rotary columns never summed) is accumulated
// transposed, O^T += C^T . P^T, on v_mfma_f32_32x32x16_f16, latent columns on M, heads on N.
// Waves 2p and 2p+1 (a pair) both accumulate heads 64p..64p+63, wave 2p latent columns 0..255
// and wave 2p+1 columns 256..511; each wave hands its probabilities of a tile to its partner
// through LDS, so every transposing operand read (ds_read_b64_tr_b16) feeds two MFMAs.  One
// permlane16_swap turns the two head blocks of probabilities into the B operands of the two
// 16-token k-steps: k-step s, lane half h takes tokens {4(2h+s)..+3} u {16+4(2h+s)..+3}, and the
// transposing reads of C^T follow the same token order.
//
// Per tile and wave, phase A runs the 72 score MFMAs of tile j, issues the nine transfers of tile
// j+2 in its first steps and converts this wave's part of tile j+1 in its second half; phase B runs
// the 32 independent weighted-sum MFMAs of tile j-1 with the online softmax of tile j woven
// between them, and publishes this wave's probabilities of tile j for the partner.
//
// LDS tile layout: a latent region (32 rows x 1,024 B) followed by a rotary region (32 rows x
// 128 B).  gfx950 LDS has 64 banks (256 B per cycle), and its bank index is not just address bits
// 2..7: bank-conflict counters on single access patterns show 16 rows at 1 KiB pitch that are
// distinct modulo 256 B still colliding in pairs, so the row bits of the address take part.
// Latent 16-byte chunks are XOR-swizzled inside each 256-byte block by
// f(row) = ((row & 3) << 2) | 3 * ((row >> 3) & 1), one of the swizzles measured conflict-free for
// the score reads (16 consecutive rows at one logical chunk) and the transposing reads (4 aligned
// rows x 4 chunks) on all four tile buffers.  Rotary chunks are swizzled by g(row) = (row >> 1) & 7, two 128-byte rows
// sharing one 256-byte bank line.  One 1 KiB latent row is exactly one wave-wide 16-byte transfer.
//
// The tile transfers are issued with inline global_load_lds_dwordx4 and waited for explicitly: the
// compiler cannot see that the transfers in flight target other buffers and would otherwise wait
// for them before every LDS read.  M0 carries the LDS destination; this kernel has no other M0 user.
//
// Softmax uses base-2 logits (q_hat carries sm_scale*log2 e) against a fixed reference per segment
// and head: the maximum of its first tile.  Probabilities of later tiles may then exceed one, by at
// most 2^15 (binary16 holds them with full relative precision), so the 256-register accumulator is
// never rescaled inside the loop.  If some head's scores climb more than 15 above its reference,
// the workgroup runs the segment a second time with the segment maximum (now known) as reference;
// with scores of unit scale that pass does not happen.

#include <math.h>

#include "common.h"
#include "launch.h"
#include "schedule.h"

namespace mla {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kH = 128, kDc = 512, kW = 576;
constexpr int kRowB = kW * 2;                    // 1,152 bytes per cached row
constexpr int kLatB = kDc * 2;                   // 1,024 latent bytes per row
constexpr int kRopeB = kRowB - kLatB;            // 128 rotary bytes per row
constexpr int kTile = 32;                        // tokens per tile
constexpr int kNBuf = 4;                         // LDS tile buffers
constexpr int kTileB = kTile * kRowB;            // 36,864 bytes
constexpr int kRopeOff = kTile * kLatB;          // rotary region offset inside a tile buffer
constexpr int kWaves = 4;
constexpr int kXcds = 8;                         // accelerator complex dies, one L2 each
constexpr int kThreads = 64 * kWaves;
constexpr int kLatPerWave = kTile / kWaves;      // 8 latent-row transfers per wave per tile
constexpr int kDmaPerWave = kLatPerWave + 1;     // + 1 rotary transfer (8 rotary rows)
constexpr int kKs = kW / 32;                     // 18 score k-steps (K = 32 each)
constexpr int kKsLat = kDc / 32;                 // 16 of them over the latent columns
constexpr int kScoreSteps = 4 * kKs;             // 72 score MFMAs per tile and wave
constexpr int kXWaveB = 2 * 64 * 16;             // one wave's binary16 probabilities of a tile (2 k-steps)
constexpr int kXBufB = kWaves * kXWaveB;         // probability exchange of one tile: 8 KiB
constexpr int kXOff = kNBuf * kTileB;            // two exchange buffers (tiles of even / odd index)
constexpr int kLdsB = kXOff + 2 * kXBufB;        // 160 KiB: the whole CU
constexpr int kMBlk = kDc / 2 / 32;              // 8 latent blocks of 32 columns per wave
constexpr int kAcc = 2 * kMBlk;                  // x 2 head blocks = 16 accumulator blocks
constexpr int kPvOps = 2 * kMBlk;                // 16 transposed operands per tile (2 k-steps)
constexpr int kPvSteps = 2 * kPvOps;             // 32 weighted-sum MFMAs per tile
constexpr float kRerunMargin = 15.0f;  // reference may lag the running max by this much (2^15 < 65504)

// Phase A schedule of the binary16 conversion of this wave's part of tile j+1 (bf16 cache): chunk
// x (0..8) is read at step kCvStart + 4x, its four dwords are converted kCvLead steps later, one per
// step, and it is written back after the last one.  The transfers of tile j+2 go out every other
// step from step 0.
constexpr int kCvStart = 20, kCvLead = 8, kCvRing = kCvLead / 4 + 1;
static_assert(kCvStart + 4 * 8 + kCvLead + 3 < kScoreSteps, "conversion fits in phase A");

// FP8 cache rows (E4M3 latent codes with one power-of-two scale per token): 512 codes | 64 bf16
// rotary values | fp32 scale | 12 zero bytes.  The FP8 variant stages each tile's codes (and
// scales) in LDS and converts them once per tile into the binary16 tile layout above; its rotary
// rows go straight into the tile buffer and are converted in place by the wave that moved them.
// Three tile buffers (tile j scored, tile j-1 summed, tile j+1 being converted) and two code
// staging slots fit next to the exchange buffers.
constexpr int kRowB8 = 656;
constexpr int kNBuf8 = 3;
constexpr int kStgCodesB = kTile * kDc;           // 16 KiB of codes per staged tile
constexpr int kStgB = kStgCodesB + 1024;          // + one transfer of the 32 rows' scale chunks
constexpr int kStgOff = kNBuf8 * kTileB;
constexpr int kXOff8 = kStgOff + 2 * kStgB;
constexpr int kLdsB8 = kXOff8 + 2 * kXBufB;       // 158 KiB
static_assert(kLdsB8 <= 160 * 1024, "FP8 layout fits the CU's LDS");

__host__ __device__ constexpr int lat_swz(int row) { return ((row & 3) << 2) | (3 * ((row >> 3) & 1)); }
__host__ __device__ constexpr int rope_swz(int row) { return (row >> 1) & 7; }

// v_max_f32 / v_max3_f32 as such.  fmaxf would first quiet each operand with a v_max_f32 of the
// value with itself (for signalling NaNs); the scores here come out of MFMAs, which never produce
// one.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Max / sum over the four lanes l%16 + 16g (g = 0..3) that hold one head's scores.
__device__ __forceinline__ float head_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float head_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One score MFMA, accumulated in VGPRs (the 256 accumulator registers hold the weighted sums).
// The first k-step starts from zero.  Four chains interleave, so consecutive MFMAs never depend on
// each other; after the last one the wave waits out the result latency before any VALU
// instruction touches the scores (score_drain).
__device__ __forceinline__ void score_mfma(bool first, f32x4& acc, const f16x8& a, const f16x8& b) {
  if (first)
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4"); }

// LDS byte address of a pointer into the kernel's one shared array, and back.  Tile buffers start
// at multiples of 4 KiB, so a per-lane offset whose swizzle bits lie below 4 KiB can be XORed after
// the buffer address is added.
__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) { return uint32_t(reinterpret_cast<uintptr_t>(p)); }
__device__ __forceinline__ lds_u8* lds_ptr(uint32_t a) { return reinterpret_cast<lds_u8*>(uintptr_t(a)); }

__device__ __forceinline__ f16x8 lds16(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) f16x8*>(p);
}
__device__ __forceinline__ u32x4 lds_u4(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}
__device__ __forceinline__ void lds_put(lds_u8* p, const u32x4& v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(p) = v;
}

// Two bf16 values (one dword) as two binary16 values: exact for magnitudes in [2^-14, 65504],
// nearest-even below (the latents' scale keeps those out of the products' significant digits).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t d) {
  const float lo = __uint_as_float(d << 16), hi = __uint_as_float(d & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float __attribute__((ext_vector_type(2)))){lo, hi}, f16x2));
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float __attribute__((ext_vector_type(2)))){a, b}, f16x2));
}

// One 16-byte-per-lane transfer of cached rows into LDS.  Where a bf16 row (1,152 B, nine whole
// 128-byte lines) is read by one workgroup only, the transfer carries the non-temporal hint (kNT):
// the streamed cache then does not displace the lines that are read again (q_hat and page-table
// rows of other units, and what the launches after the decode read: the partials, W_UV, W_UK).
// FP8 rows (656 B) share lines between the code, rotary and scale transfers of a row and its
// neighbours, which the hint would evict between those reads, so they are loaded normally.
template <bool kNT>
__device__ __forceinline__ void dma16(uint32_t lds_dst, uint32_t voff, const unsigned char* gbase) {
  if constexpr (kNT)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds_dst), "v"(voff), "s"(gbase)
                 : "memory");
  else
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

// NT: the bf16 tile transfers carry the non-temporal hint; set where each cached row is read by one
// workgroup only (fixed split, plain balanced split), clear where other workgroups read the same
// rows shortly after and should find them in L2 (row groups, prefill rows of one sequence).
template <int MODE, bool F8, bool NT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(const uint16_t* __restrict__ pool, const int32_t* __restrict__ page_table,
                        const int32_t* __restrict__ seq_lens, int batch, int max_pages, int page_size,
                        int tiles_per_page_log2, const uint16_t* __restrict__ q_hat, int n_splits,
                        int split_tokens, const int32_t* __restrict__ q_start, float* __restrict__ o_part,
                        float* __restrict__ lse_part) {
  constexpr bool kBal = MODE == kBalanced;
  constexpr int kNB = F8 ? kNBuf8 : kNBuf;          // tile buffers
  constexpr int kXO = F8 ? kXOff8 : kXOff;          // exchange buffers
  __shared__ __attribute__((aligned(16))) unsigned char smem[F8 ? kLdsB8 : kLdsB];
  lds_u8* const lbase = (lds_u8*)smem;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, ii = lane & 15;   // score layout: lane group, row / head within it
  const int hi = lane >> 5;                  // 32 x 32 layout: lane half
  const int head32 = wave * 32 + (lane & 31);  // one head of this wave in the 32 x 32 layout
  const int lh = wave & 1;                   // latent half summed by this wave
  const int cap = max_pages * page_size;     // never index past the page table

  // ---- per-lane constants of the tile transfers.  Latent row n = 4x + wave (x < 8) is one 1 KiB
  // transfer; rotary rows 8*wave .. 8*wave+7 are this wave's ninth.  Lane L writes LDS chunk L of
  // the transfer; the global chunk it reads is the one that the XOR swizzle places there.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
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
  // score operand of token block t, k-step ks: row 16t + ii, logical 16-byte chunk 4ks + g
  // (latent) or 4(ks-16) + g (rotary).  The swizzle XORs the chunk index, so k-step ks sits at the
  // place of k-step 0 XOR 64*(ks & 3) bytes inside its 256-byte block.
  int qa_x = ii * kLatB + 16 * (g ^ lat_swz(ii));
  int qr_x = kRopeOff + ii * kRopeB + 16 * (g ^ rope_swz(ii));
  // transposing reads: lane group g reads rows 8(g>>1) + 4s + ii/4 (k-step s) and the same +16,
  // columns 32mb + 16(g&1) + 4(ii&3) .. +3 of this wave's latent half.  k-step s adds 4 rows, which
  // leaves the row swizzle as it is; column block 4*m4 + c sits at the place of m4 = 0 XOR 64*m4.
  int pv_x;
  {
    const int r0 = 8 * (g >> 1) + (ii >> 2);
    const int y = 2 * (g & 1) + ((ii >> 1) & 1);
    pv_x = r0 * kLatB + 512 * lh + 16 * (y ^ lat_swz(r0)) + 8 * (ii & 1);
  }
  // probability exchange: this lane's 16 bytes of k-step s in the buffer of tile parity t
  const uint32_t x_mine = uint32_t(kXO + wave * kXWaveB + 16 * lane);
  const uint32_t x_peer = uint32_t(kXO + (wave ^ 1) * kXWaveB + 16 * lane);
  auto x_at = [&](uint32_t base, int t, int s) { return lbase + base + t * kXBufB + s * 1024; };
  auto a_src = [&](const lds_u8* tb, int t, int ks) -> const lds_u8* {
    return ks < kKsLat ? tb + 16 * kLatB * t + 256 * (ks >> 2) + (qa_x ^ (64 * (ks & 3)))
                       : tb + 16 * kRopeB * t + (qr_x ^ (64 * (ks - kKsLat)));
  };
  // weighted-sum operand o = 8 * kstep + mb (mb: block of this wave's latent half): two
  // transposing reads, tokens 4(2h+s) + 0..3 and 16 + the same
  // pb: the tile buffer's address plus pv_x
  auto tr8 = [&](uint32_t pb, int o) {
    const int s = o >> 3, mb = o & 7;
    const lds_u8* p0 = lds_ptr((pb ^ uint32_t(64 * (mb & 3))) + 4 * kLatB * s + 256 * (mb >> 2));
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
    const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0 + 16 * kLatB));
    return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // LDS place of this wave's own transfer x of a tile (bf16 cache: the chunk it converts in place)
  auto own_chunk = [&](lds_u8* tbuf, int x) -> lds_u8* {
    return x < kLatPerWave ? tbuf + (4 * x + wave_u) * kLatB + lane16 : tbuf + kRopeOff + wave_u * 1024 + lane16;
  };

  // ---- the segment list.  Workgroups are dealt to the chip's eight XCDs (each with its own L2) in
  // turn, workgroup id modulo 8; consecutive units of the work-balanced split, which mostly share
  // a sequence (and so its q_hat rows and page-table row), or are the rows of one row group
  // reading the same pages side by side, are placed on one XCD.
  int unit = blockIdx.x;
  if constexpr (kBal) {
    if (gridDim.x % kXcds == 0) unit = (unit % kXcds) * (gridDim.x / kXcds) + unit / kXcds;
  }
  // kBalanced: split_tokens carries the row-group size G (schedule.h); this unit runs row g_row of
  // the groups in group-unit g_unit
  const int group = kBal ? split_tokens : 1;
  const int g_unit = unit / group, g_row = unit - g_unit * group;
  const int n_groups = batch / group;
  int next_b, next_cb = 0, unit_end = 0, quota = 0;
  if constexpr (kBal) {
    int total;
    sched_prefix(seq_lens, n_groups, group, cap, 0, next_cb, total);
    total = __builtin_amdgcn_readfirstlane(total);  // wave-uniform: keep the segment loop scalar
    quota = sched_quota(total, n_splits / group);
    if (quota == 0 || g_unit * quota >= total) return;  // idle unit (uniform)
    unit_end = min(g_unit * quota + quota, total);
    sched_find(seq_lens, n_groups, group, cap, g_unit * quota, next_b, next_cb);
    next_b = __builtin_amdgcn_readfirstlane(next_b);
    next_cb = __builtin_amdgcn_readfirstlane(next_cb);
  } else {
    next_b = blockIdx.y;
  }

  for (bool first_seg = true;; first_seg = false) {
    int b, t0, t1;
    size_t slot, qrow;  // output row group and q_hat row group (128 heads each)
    if constexpr (kBal) {
      if (next_b >= n_groups || next_cb >= unit_end) break;
      const int grp = next_b;
      b = grp * group + g_row;
      const int glen = group == 1 ? sched_len(seq_lens[b], cap) : sched_group_len(seq_lens, grp, group, cap);
      const int len = group == 1 ? glen : sched_len(seq_lens[b], cap);
      int k0, k1;
      sched_row_segment(next_cb, sched_tiles(glen), sched_tiles(len), g_unit, quota, k0, k1);
      next_cb += sched_cost(glen);
      ++next_b;
      if (k1 <= k0) continue;  // only the segment price of this group, or past this row's end
      t0 = k0 * kTile;
      t1 = min(k1 * kTile, len);
      slot = size_t(sched_slot(g_unit, grp, group, g_row));
      qrow = b;
    } else if constexpr (MODE == kPrefill) {
      // n_splits carries the chunk length; row i of sequence b reads keys t <= q_start[b] + i
      const int i = n_splits - 1 - unit / batch;
      b = unit % batch;
      qrow = slot = size_t(b) * n_splits + i;
      t0 = 0;
      t1 = min(sched_len(seq_lens[b], cap), max(q_start[b] + i + 1, 0));
      if (t1 <= 0) {  // no visible key: z = 0, lse = -inf
        float* zr = o_part + (slot * kH + head32) * kDc + 4 * hi;
        for (int c = 0; c < kDc; c += 8) *reinterpret_cast<float4*>(zr + c) = make_float4(0.f, 0.f, 0.f, 0.f);
        if (hi == 0 && lse_part) lse_part[slot * kH + head32] = -INFINITY;
        return;
      }
    } else {
      b = next_b;
      qrow = b;
      t0 = unit * split_tokens;
      t1 = min(t0 + split_tokens, sched_len(seq_lens[b], cap));
      slot = size_t(b) * n_splits + unit;
      if (t0 >= t1) {  // empty chunk: lse = -inf; its o_part is never read by the combine
        if (hi == 0) lse_part[slot * kH + head32] = -INFINITY;
        return;
      }
    }
    if (!first_seg) __syncthreads();  // the previous segment is done with every LDS buffer
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
    auto dma_one = [&](const unsigned char* gsrc, uint32_t dst, int x) {  // x-th transfer of a tile
      if (x < kLatPerWave) {
        const int n = 4 * x + wave_u;
        dma16<NT>(dst + uint32_t(n * kLatB), lat_off(x), gsrc + size_t(n) * kRowB);
      } else {
        dma16<NT>(dst + uint32_t(kRopeOff + wave_u * 1024), rope_off(), gsrc + size_t(8 * wave_u) * kRowB);
      }
    };
    auto dma_tile = [&](int k) {  // tile min(k, ntiles-1) into buffer k % kNB
      const unsigned char* gsrc = tile_src(min(k, ntiles - 1));
      const uint32_t dst = lds0 + uint32_t((k % kNB) * kTileB);
#pragma unroll
      for (int x = 0; x < kDmaPerWave; ++x) dma_one(gsrc, dst, x);
    };
    // ---- bf16 cache: this wave's nine chunks of a landed tile become binary16 in place; latent rows
    // at or past `nvalid` become zeros (their probabilities are zero, and 0 x NaN would not be)
    auto convert_own = [&](int k, int nvalid) {
      lds_u8* const tbuf = lbase + (k % kNB) * kTileB;
#pragma unroll
      for (int x = 0; x < kDmaPerWave; ++x) {
        const u32x4 v = lds_u4(own_chunk(tbuf, x));
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = bf16x2_to_f16x2(v[d]);
        if (x < kLatPerWave && 4 * x + wave_u >= nvalid) o = u32x4{0u, 0u, 0u, 0u};
        lds_put(own_chunk(tbuf, x), o);
      }
    };
    auto zero_tail_own = [&](int k, int nvalid) {  // after the piecewise conversion of a tail tile
      lds_u8* const tbuf = lbase + (k % kNB) * kTileB;
#pragma unroll
      for (int x = 0; x < kLatPerWave; ++x)
        if (4 * x + wave_u >= nvalid) lds_put(own_chunk(tbuf, x), u32x4{0u, 0u, 0u, 0u});
    };
    // ---- FP8: transfer x of a tile's codes and scales into staging slot `slot`.  Transfer
    // T = 4*wave + x (x < 4) moves rows 2T, 2T+1 (512 code bytes each; lane L: row 2T + L/32, chunk
    // L%32); x = 4 (wave 0 only) moves the 16-byte scale chunk of row L%32 (lanes 32..63 repeat
    // rows 0..31).  The rotary rows go straight into the tile buffer (dma_rope8).
    const uint32_t c8_off = uint32_t((lane >> 5) * kRowB8 + 16 * (lane & 31));
    const uint32_t s8_off = uint32_t((lane & 31) * kRowB8 + kDc + 2 * (kW - kDc));
    auto dma_codes8 = [&](const unsigned char* gsrc, int stg, int x) {
      const uint32_t dst = lds0 + uint32_t(kStgOff + stg * kStgB);
      if (x < 4) {
        const int T = 4 * wave_u + x;
        dma16<false>(dst + uint32_t(T * 1024), c8_off, gsrc + size_t(2 * T) * kRowB8);
      } else if (wave_u == 0) {
        dma16<false>(dst + uint32_t(kStgCodesB), s8_off, gsrc);
      }
    };
    auto dma_rope8 = [&](const unsigned char* gsrc, int k) {
      dma16<false>(lds0 + uint32_t((k % kNB) * kTileB + kRopeOff + wave_u * 1024), rope_off(), gsrc + size_t(8 * wave_u) * kRowB8);
    };
    auto dma_tile8 = [&](int k) {  // codes and scales of tile k into slot k&1, its rotary rows into buffer k%3
      const unsigned char* gsrc = tile_src(min(k, ntiles - 1));
#pragma unroll
      for (int x = 0; x < 5; ++x) dma_codes8(gsrc, k & 1, x);
      dma_rope8(gsrc, k);
    };
    // ---- FP8: convert the staged codes of tile k (slot k&1) into the binary16 latent rows of
    // buffer k%3, code x scale (exact: a power-of-two scale), rows >= nval as zeros.  Wave w
    // converts rows 8w..8w+7; lane l takes row 8w + l/8 and code chunks q = l%8 + 8u (16 codes,
    // two output chunks).  Those are also the rows of this wave's rotary transfer, converted in
    // place by rope8_convert.
    const int cv_row = 8 * wave + (lane >> 3);
    auto cv_read = [&](int k, int u) {  // 16 codes of chunk u
      const lds_u8* stg = lbase + kStgOff + (k & 1) * kStgB;
      return lds_u4(stg + cv_row * kDc + 16 * ((lane & 7) + 8 * u));
    };
    auto cv_scale = [&](int k) {
      const lds_u8* stg = lbase + kStgOff + (k & 1) * kStgB + kStgCodesB;
      return *reinterpret_cast<const __attribute__((address_space(3))) float*>(stg + 16 * cv_row);
    };
    // the two binary16 output chunks (8 values each) of code chunk u, half h (dwords 2h, 2h+1)
    auto cv_write = [&](int k, int u, int h, const u32x4& codes, float scale, bool valid) {
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint32_t w = codes[2 * h + d];
        o[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, scale, false));
        o[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, scale, true));
      }
      if (!valid) o = u32x4{0u, 0u, 0u, 0u};
      const int c = 2 * ((lane & 7) + 8 * u) + h;  // 16-byte chunk of the 1,024-byte latent row
      lds_put(lbase + (k % kNB) * kTileB + cv_row * kLatB + 256 * (c >> 4) + 16 * ((c & 15) ^ lat_swz(cv_row)), o);
    };
    auto cv_valid = [&](int k) { return cv_row < t1 - (t0 + k * kTile); };
    auto rope8_convert = [&](int k) {  // this wave's rotary transfer of tile k, in place
      lds_u8* const p = lbase + (k % kNB) * kTileB + kRopeOff + wave_u * 1024 + lane16;
      const u32x4 v = lds_u4(p);
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[d] = bf16x2_to_f16x2(v[d]);
      lds_put(p, o);
    };
    auto convert_tile8 = [&](int k) {  // all at once (the prologue's tile 0)
      const float sc = cv_scale(k);
      const bool v = cv_valid(k);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 cd = cv_read(k, u);
        cv_write(k, u, 0, cd, sc, v);
        cv_write(k, u, 1, cd, sc, v);
      }
      rope8_convert(k);
    };

    if constexpr (F8) {
      dma_tile8(0);
    } else {
      dma_tile(0);
    }

    // ---- this wave's 32 heads of q_hat, as the B operand of S^T = tile . q_hat^T, held in
    // registers for the whole segment: head block hb (16 heads), 18 k-steps of 32 columns.
    f16x8 qf[2][kKs];
    {
      const uint16_t* qp = q_hat + (qrow * kH + wave * 32 + ii) * kW + 8 * g;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks)
          qf[hb][ks] = *reinterpret_cast<const f16x8*>(qp + size_t(16 * hb) * kW + 32 * ks);
    }
    // Consume these loads here: an empty asm that reads every fragment makes the compiler wait for
    // them before the tile loop (tile 0 and the previous segment's stores complete too).  Otherwise
    // its waits for them land inside the loop, where the vmcnt they use would also drain the tile
    // transfers in flight.
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) asm volatile("" : "+v"(qf[hb][ks]));

    f32x16 acc[kAcc];  // acc[2 * mb + 0]: own heads, acc[2 * mb + 1]: the partner's
    float m_ref[2] = {-INFINITY, -INFINITY}, m_max[2] = {-INFINITY, -INFINITY}, l_lane[2] = {0.f, 0.f};
    f16x8 pb0, pb1;  // own probabilities of the previous tile, B operands of k-steps 0 and 1

    for (int pass = 0; pass < 2; ++pass) {
      if (pass > 0) {
        if (wbase != 0) {
          wbase = 0;
          my_page = load_page_window(pt_row, p0, npg, max_pages, lane);
        }
        if constexpr (F8)
          dma_tile8(0);
        else
          dma_tile(0);
      }
      // tile 0 landed (the q_hat loads behind it too): make it binary16, then start tile 1 (past
      // a one-tile segment: a copy of tile 0 into the buffer that is free anyway)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if constexpr (F8) {
        __syncthreads();  // every wave's codes of tile 0 are staged
        convert_tile8(0);
        const unsigned char* g1 = tile_src(min(1, ntiles - 1));
#pragma unroll
        for (int x = 0; x < 5; ++x) dma_codes8(g1, 1, x);
      } else {
        convert_own(0, min(kTile, t1 - t0));
        dma_tile(1);
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
      l_lane[0] = l_lane[1] = 0.f;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        pb0[x] = (_Float16)0.f;
        pb1[x] = (_Float16)0.f;
      }
      // The weighted sum of the tile before tile 0 runs on a zeroed buffer with zero
      // probabilities (own and, in the exchange buffer of odd tiles, the partner's), which keeps
      // the pipelined loop uniform.
      {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (int x = threadIdx.x; x < kRopeOff / 16; x += kThreads) lds_put(lbase + (kNB - 1) * kTileB + 16 * x, zero);
        lds_put(x_at(x_mine, 1, 0), zero);
        lds_put(x_at(x_mine, 1, 1), zero);
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
        if constexpr (F8) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // codes of j+1, rotary rows of j landed
        // bf16: every wave converted its part of tile j (previous step or the prologue); tile j-2
        // is fully consumed.  FP8: every wave's codes of tile j+1 are staged.
        __syncthreads();
        // Keep the per-step offsets derived inside the loop (one XOR each) instead of letting the
        // compiler hoist dozens of precomputed copies into registers next to the q_hat fragments.
        asm volatile("" : "+v"(qa_x), "+v"(qr_x), "+v"(pv_x), "+v"(lane16));
        lds_u8* const tb = lbase + (j % kNB) * kTileB;
        const uint32_t tp = lds_addr(lbase + ((j + kNB - 1) % kNB) * kTileB) + uint32_t(pv_x);
        lds_u8* const tn = lbase + ((j + 1) % kNB) * kTileB;
        const int nvalid = min(kTile, t1 - (t0 + j * kTile));
        const int nvalid_next = min(kTile, t1 - (t0 + (j + 1) * kTile));
        // FP8: the rotary rows of tile j+1 go to the buffer tile j-2 left (past the segment end a
        // copy of the last tile's); its latent rows are converted in phase B below
        if constexpr (F8) dma_rope8(g_rope, j + 1);
        // Tile j+2 goes to the buffer that tile j-2 left; past the segment end the transfers copy
        // the segment's last tile there instead, which keeps the wait counts uniform and the loop
        // free of branches.  Every transfer lands before the loop ends (drained below).
        const uint32_t dnext = lds0 + uint32_t(((j + 2) % kNB) * kTileB);
        const unsigned char* g_dma_next = g_dma;

        // ---- phase A: scores of tile j in four interleaved chains (step i: k-step i/4, token
        // block (i/2)&1, head block i&1), operands read kQD k-steps ahead; the transfers of tile
        // j+2 go out in its first steps; from step kCvStart on, this wave's part of tile j+1 (landed
        // by then) is converted to binary16 in place (bf16 cache); the partner's probabilities of
        // tile j-1 and the first kPB operands of phase B are read in its last steps
        constexpr int kQD = 2, kPB = 3;
        f32x4 sacc[2][2];
        f16x8 pa[kPB + 1], pq0, pq1;
        {
          f16x8 qa[2][kQD + 1];
          u32x4 cin[kCvRing];  // bf16 cache: this wave's chunks of tile j+1 in flight, converted in place
#pragma unroll
          for (int ks = 0; ks < kQD; ++ks) {
            qa[0][ks] = lds16(a_src(tb, 0, ks));
            qa[1][ks] = lds16(a_src(tb, 1, ks));
          }
          __builtin_amdgcn_sched_barrier(0);  // the first operand reads go out right after the barrier
#pragma unroll
          for (int i = 0; i < kScoreSteps; ++i) {
            const int ks = i >> 2, t = (i >> 1) & 1, hb = i & 1;
            if (hb == 0 && ks + kQD < kKs) qa[t][(ks + kQD) % (kQD + 1)] = lds16(a_src(tb, t, ks + kQD));
            if constexpr (F8) {
              if (i < 5) dma_codes8(g_dma, j & 1, i);  // codes of tile j+2
            } else {
              if (!(i & 1) && i / 2 < kDmaPerWave) dma_one(g_dma, dnext, i / 2);
              // conversion of this wave's part of tile j+1: chunk x read at kCvStart + 4x, dword d
              // converted at kCvStart + 4x + kCvLead + d, the chunk written back after the last dword
              if (i == kCvStart) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerWave) : "memory");
              if (i >= kCvStart && (i - kCvStart) % 4 == 0 && (i - kCvStart) / 4 < kDmaPerWave)
                cin[((i - kCvStart) / 4) % kCvRing] = lds_u4(own_chunk(tn, (i - kCvStart) / 4));
              if (i >= kCvStart + kCvLead) {
                const int x = (i - kCvStart - kCvLead) / 4, d = (i - kCvStart - kCvLead) % 4;
                if (x < kDmaPerWave) {
                  cin[x % kCvRing][d] = bf16x2_to_f16x2(cin[x % kCvRing][d]);
                  if (d == 3) lds_put(own_chunk(tn, x), cin[x % kCvRing]);
                }
              }
            }
            if (i == 20) g_dma_next = tile_src(min(j + 3, ntiles - 1));  // for the next step
            if (i == kScoreSteps - 8) pq0 = lds16(x_at(x_peer, (j + 1) & 1, 0));
            if (i == kScoreSteps - 6) pq1 = lds16(x_at(x_peer, (j + 1) & 1, 1));
            if (i >= kScoreSteps - 2 * kPB && (i & 1)) {
              const int k = (i - (kScoreSteps - 2 * kPB)) >> 1;
              pa[k] = tr8(tp, k);
            }
            score_mfma(ks == 0, sacc[t][hb], qa[t][ks % (kQD + 1)], qf[hb][ks]);
            __builtin_amdgcn_sched_barrier(0);
          }
          score_drain();
        }
        // bf16 tail tile next: its latent rows past the segment end read as zeros (FP8 tiles get
        // their zero rows from the conversion)
        if (!F8 && nvalid_next < kTile) zero_tail_own(j + 1, nvalid_next);

        // tail tile: scores of tokens past the segment end drop out of the softmax
        if (nvalid < kTile) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
              for (int x = 0; x < 4; ++x)
                if (16 * t + 4 * g + x >= nvalid) sacc[t][hb][x] = -INFINITY;
        }

        // ---- phase B: weighted sum of tile j-1 (16 operands x 2 head blocks = 32 independent
        // MFMAs) with the online softmax of tile j (base-2 logits; this lane's two heads) woven
        // between them, so that the VALU work runs in the shadow of the matrix cores.  Branch-free:
        // the reference update is a select.
        {
          const bool first = pass == 0 && j == 0;  // the segment's first tile fixes the reference
          float mx[2] = {0.f, 0.f}, pr0 = 0.f, tsum[2] = {0.f, 0.f};
          uint32_t pk[2][4];  // binary16 probability pairs: [head block][token block * 2 + pair]
          u32x4 cv_cd[2];  // FP8: code chunks of tile j+1 in flight
          float cv_sc = 0.f;
          bool cv_ok = false;
#pragma unroll
          for (int i = 0; i < kPvSteps; ++i) {
            const int o = i >> 1, nb = i & 1;  // operand, head block (0: own, 1: partner)
            if (nb == 0 && o + kPB < kPvOps) pa[(o + kPB) % (kPB + 1)] = tr8(tp, o + kPB);
            const f16x8 pp = o < kMBlk ? (nb ? pq0 : pb0) : (nb ? pq1 : pb1);
            acc[2 * (o & 7) + nb] =
                __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[o % (kPB + 1)], pp, acc[2 * (o & 7) + nb], 0, 0, 0);
            if (i == 1 || i == 2) {  // row maximum of head block i-1 over this lane's 8 tokens, then the head
              const int hb = i - 1;
              const f32x4 u = sacc[0][hb], v = sacc[1][hb];
              const float m = vmax(vmax3(u[0], u[1], u[2]), vmax3(u[3], v[0], vmax3(v[1], v[2], v[3])));
              mx[hb] = head_max(m);
              m_ref[hb] = first ? mx[hb] : m_ref[hb];
              m_max[hb] = vmax(m_max[hb], mx[hb]);
              over |= mx[hb] > m_ref[hb] + kRerunMargin;
            }
            // one probability per step (the exp2 is a quarter-rate instruction), summed and packed
            // to binary16 pairwise as they come, so that no step outgrows its MFMA.  Probability e
            // (0..15): head block e/8, token block (e/4)&1, row e&3.
            if (i >= 3 && i < 19) {
              const int e = i - 3, hb = e >> 3, t = (e >> 2) & 1, x = e & 3;
              const float p = fast_exp2(sacc[t][hb][x] - m_ref[hb]);
              tsum[hb] += p;
              if (e & 1)
                pk[hb][2 * t + (x >> 1)] = pack_f16(pr0, p);
              else
                pr0 = p;
            }
            if (i == 19) {  // head block 0 -> the tokens of k-step 0, head block 1 -> k-step 1
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                const auto sw = __builtin_amdgcn_permlane16_swap(pk[0][d], pk[1][d], false, false);
                pk[0][d] = sw[0];
                pk[1][d] = sw[1];
              }
            }
            if (i == 20) {
              l_lane[0] += tsum[0];
              l_lane[1] += tsum[1];
            }
            // for the partner, read after the next tile's barrier
            if (i == 21) lds_put(x_at(x_mine, j & 1, 0), u32x4{pk[0][0], pk[0][1], pk[0][2], pk[0][3]});
            if (i == 23) lds_put(x_at(x_mine, j & 1, 1), u32x4{pk[1][0], pk[1][1], pk[1][2], pk[1][3]});
            if constexpr (F8) {
              // the codes of tile j+1 become its binary16 latent rows in the shadow of the last
              // weighted-sum MFMAs, once the scores and probabilities are dead: chunk u is read two
              // steps before its two halves are converted and written (steps 22 .. 29); the rotary
              // rows of tile j+1 (this wave's transfer, issued at the top of the step) follow
              if (i == 19) {
                cv_sc = cv_scale(j + 1);
                cv_ok = cv_valid(j + 1);
              }
              if (i >= 22 && i < 30) cv_write(j + 1, (i - 22) >> 1, i & 1, cv_cd[((i - 22) >> 1) & 1], cv_sc, cv_ok);
              if (i >= 20 && i < 28 && !(i & 1)) cv_cd[((i - 20) >> 1) & 1] = cv_read(j + 1, (i - 20) >> 1);
              if (i == 30) {
                // four code transfers of tile j+2 (five on wave 0) were issued after the rotary rows
                asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
                rope8_convert(j + 1);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          pb0 = __builtin_bit_cast(f16x8, u32x4{pk[0][0], pk[0][1], pk[0][2], pk[0][3]});
          pb1 = __builtin_bit_cast(f16x8, u32x4{pk[1][0], pk[1][1], pk[1][2], pk[1][3]});
          if constexpr (F8) g_rope = g_dma;
          g_dma = g_dma_next;
        }
      }

      // ---- weighted sum of the last tile, once the partner's probabilities of it are published
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      {
        const uint32_t tp = lds_addr(lbase + ((ntiles - 1) % kNB) * kTileB) + uint32_t(pv_x);
        const f16x8 pq0 = lds16(x_at(x_peer, (ntiles - 1) & 1, 0));
        const f16x8 pq1 = lds16(x_at(x_peer, (ntiles - 1) & 1, 1));
        f16x8 pa[3];
        pa[0] = tr8(tp, 0);
        pa[1] = tr8(tp, 1);
#pragma unroll
        for (int i = 0; i < kPvSteps; ++i) {
          const int o = i >> 1, nb = i & 1;
          if (nb == 0 && o + 2 < kPvOps) pa[(o + 2) % 3] = tr8(tp, o + 2);
          const f16x8 pp = o < kMBlk ? (nb ? pq0 : pb0) : (nb ? pq1 : pb1);
          acc[2 * (o & 7) + nb] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[o % 3], pp, acc[2 * (o & 7) + nb], 0, 0, 0);
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
      m_ref[0] = m_max[0];
      m_ref[1] = m_max[1];
      __syncthreads();
    }

    // ---- normalise and write the segment's partial.  The row sums of all 128 heads go through
    // the exchange buffer that no tile uses any more.  The MFMA layout gives each lane 16-byte
    // pieces of 32 different rows; staged through LDS (the tile buffers are idle now), every store
    // instruction writes 1 KiB of one contiguous half row instead.
    const float l_tot[2] = {head_sum(l_lane[0]), head_sum(l_lane[1])};
    __attribute__((address_space(3))) float* const l_x =
        reinterpret_cast<__attribute__((address_space(3))) float*>(lbase + kXO + (ntiles & 1) * kXBufB);
    if (g == 0) {
      l_x[wave * 32 + ii] = l_tot[0];
      l_x[wave * 32 + 16 + ii] = l_tot[1];
      if (lse_part) {
        lse_part[slot * kH + wave * 32 + ii] = (m_ref[0] + log2f(l_tot[0])) * kLn2;
        lse_part[slot * kH + wave * 32 + 16 + ii] = (m_ref[1] + log2f(l_tot[1])) * kLn2;
      }
    }
    __syncthreads();  // every wave is done with the tile buffers and the rerun flags; sums published
    const float inv_own = 1.f / l_x[head32], inv_peer = 1.f / l_x[(wave ^ 1) * 32 + (lane & 31)];
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
            lds_put(stg + (lane & 31) * kStRow + 4 * (32 * m + 8 * j4 + 4 * hi), f);
          }
        }
        // the same wave reads back what it wrote: LDS operations of one wave complete in order
#pragma unroll 8
        for (int r = 0; r < 32; ++r) {
          const u32x4 x = lds_u4(stg + r * kStRow + 16 * lane);
          *reinterpret_cast<u32x4*>(orow0 + size_t(r) * kDc + 4 * lane) = x;
        }
      }
    }
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
  auto k = fp8 ? decode_mfma_kernel<kFixed, true> : decode_mfma_kernel<kFixed, false, true>;
  k<<<dim3(n_splits, c.batch), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(c.pool), c.page_table, c.seq_lens, c.batch, c.max_pages, c.page_size, tpp_log2,
      static_cast<const uint16_t*>(q_hat), n_splits, split_tokens, nullptr, o_part, lse_part);
  return hipGetLastError();
}

hipError_t launch_decode_mfma_balanced(const Dims& d, const Cache& c, const void* q_hat, int n_units, int group,
                                       float* o_part, float* lse_part, hipStream_t s, bool fp8) {
  (void)d;
  const int tpp_log2 = __builtin_ctz(unsigned(c.page_size / kTile));
  auto k = fp8        ? decode_mfma_kernel<kBalanced, true>
           : group == 1 ? decode_mfma_kernel<kBalanced, false, true>
                        : decode_mfma_kernel<kBalanced, false, false>;
  k<<<dim3(n_units), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(c.pool), c.page_table, c.seq_lens, c.batch, c.max_pages, c.page_size, tpp_log2,
      static_cast<const uint16_t*>(q_hat), n_units, group, nullptr, o_part, lse_part);
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
