// Precomposed weights (row N2): products of consecutive projections taken once, offline, and the
// two per-step products that use them.
//
// Query side ([molayo] formal definition, absorbed weight W_UQ[h] . W_UK[h]^T; [ase] section on
// multiplying consecutive projections ahead of time): the weight w_qcat [d_cq, H, d_c + d_r] holds,
// for every head, [W_UQ[h] . W_UK[h]^T | W_QR[h]], so that one product c^Q . w_qcat gives every
// head's latent-space query and unrotated rotary query at once; an epilogue rotates the rotary part
// at the query position, applies sm_scale * log2(e) and rounds q_hat to binary16.
//
// Value side ([ase] same section, value side; [huny] section 2, output-projection fusion): the
// weight w_uvo [H, d_c, d_model] holds W_UV[h] . W_O[h], so the layer output is
// out = z_concat . w_uvo with z the weighted latents of every head concatenated.
//
// gemm_kernel: part[s, m, n] = sum over the s-th K range of A[m, k] . B[k, n], B bf16 row-major,
// A bf16 or float32 (split into bf16 hi + lo parts, two MFMAs, about 16 significant bits).  A
// workgroup of four waves owns 64 rows x 128 columns (wave w: columns 32w..32w+31, both 32-row
// blocks) and walks its K range in chunks of 64: the chunk of A (64 x 64) and of B (64 x 128) is
// loaded into registers one chunk ahead (every load instruction covering whole rows), then stored
// to LDS (double-buffered); A operands are read row-wise, B operands with the transposing
// ds_read_b64_tr_b16.  Reads of A are shared by the 128 columns of a workgroup; B, the weight,
// is read from HBM exactly once over the grid.

#include <math.h>

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTM = 64, kTN = 128, kKC = 64;  // workgroup tile and K chunk
constexpr int kThreads = 256;
constexpr int kBChunkB = kKC * kTN * 2;       // 16 KiB
constexpr int kAChunkB = kTM * kKC * 2;       // 8 KiB per bf16 part
constexpr int kBufB = kBChunkB + 2 * kAChunkB;  // B | A hi | A lo

template <bool AF32>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const void* __restrict__ a_ptr, int64_t lda,
                                                        const uint16_t* __restrict__ b, int64_t ldb, int M,
                                                        int64_t n_total, int k_per_split, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kBufB];
  lds_u8* const lbase = (lds_u8*)smem;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, t = threadIdx.x;
  const int64_t n0 = int64_t(blockIdx.x) * kTN;
  const int m0 = blockIdx.y * kTM;
  const int64_t k_begin = int64_t(blockIdx.z) * k_per_split;
  const int nchunks = k_per_split / kKC;

  // global -> register staging of one chunk; every load instruction reads whole rows.  B: 64 k
  // rows x 256 bytes, thread t moves the 16-byte pieces t + 256x (k row p/16, piece p%16), x < 4.
  // A: 64 rows x 64 k; bf16: thread t moves rows 32x + t/8 (x < 2), bytes 16(t%8) .. +15 of the
  // row's 128; float32: rows 16x + t/16 (x < 4), floats 4(t%16) .. +3 of the row's 64.
  constexpr int kAPer = AF32 ? 4 : 2;
  constexpr int kARowStep = kTM / kAPer, kAThrPerRow = kThreads / kARowStep;
  u32x4 sb[4];
  u32x4 sa[kAPer];
  auto load = [&](int c) {
    const int64_t k0 = k_begin + int64_t(c) * kKC;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int p = t + kThreads * x;
      sb[x] = *reinterpret_cast<const u32x4*>(b + (k0 + (p >> 4)) * ldb + n0 + 8 * (p & 15));
    }
#pragma unroll
    for (int x = 0; x < kAPer; ++x) {
      const int64_t row = min(m0 + kARowStep * x + t / kAThrPerRow, M - 1);  // rows past M: computed, never stored
      if constexpr (AF32)
        sa[x] = *reinterpret_cast<const u32x4*>(static_cast<const float*>(a_ptr) + row * lda + k0 + 4 * (t % kAThrPerRow));
      else
        sa[x] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a_ptr) + row * lda + k0 + 8 * (t % kAThrPerRow));
    }
  };
  // LDS layout of a buffer: B [64 k][128 n] bf16 (256-byte rows, 16-byte chunk c of k row k at
  // c ^ 4(k & 3), so that the 4 k rows x 64 bytes of a transposing read fall in distinct bank
  // groups); A hi and A lo [64 m][64 k] bf16 (128-byte rows, chunk c of row r at c ^ ((r >> 1) & 7):
  // 16 consecutive rows at one logical chunk, two rows per 256-byte bank line, hit 16 bank groups)
  auto a_chunk_off = [](int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); };
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  auto store = [&](int buf) {
    lds_u8* const bb = lbase + buf * kBufB;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int p = t + kThreads * x, k = p >> 4;
      *reinterpret_cast<lds_u32x4*>(bb + 256 * k + 16 * ((p & 15) ^ (4 * (k & 3)))) = sb[x];
    }
#pragma unroll
    for (int x = 0; x < kAPer; ++x) {
      const int r = kARowStep * x + t / kAThrPerRow;
      if constexpr (AF32) {
        // four floats -> four bf16 hi (round to nearest even) and four bf16 lo (the rounded
        // remainder, exact in float32): half h = t%2 of logical chunk (t%16)/2 of row r
        const int q = t & 15, c = q >> 1, h = q & 1;
        u32x2 hi, lo;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float f0 = __uint_as_float(sa[x][2 * e]), f1 = __uint_as_float(sa[x][2 * e + 1]);
          const uint32_t hv = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){f0, f1}, bf16x2));
          const float r0 = f0 - __uint_as_float(hv << 16), r1 = f1 - __uint_as_float(hv & 0xffff0000u);
          hi[e] = hv;
          lo[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){r0, r1}, bf16x2));
        }
        *reinterpret_cast<lds_u32x2*>(bb + kBChunkB + a_chunk_off(r, c) + 8 * h) = hi;
        *reinterpret_cast<lds_u32x2*>(bb + kBChunkB + kAChunkB + a_chunk_off(r, c) + 8 * h) = lo;
      } else {
        *reinterpret_cast<lds_u32x4*>(bb + kBChunkB + a_chunk_off(r, t % kAThrPerRow)) = sa[x];
      }
    }
  };

  // operand reads.  A (row block rb): row 32rb + l%32, k 16s + 8(l/32) .. +7 = chunk 2s + l/32.
  // B: transposing reads, group g = l/16 addresses k rows 8(g/2) + (l%16)/4 (+4) of step s and
  // columns 32w + 16(g%2) + 4(l%4) .. +3 (the kv-append GEMM's B layout with 256-byte rows).
  const int g = lane >> 4, i16 = lane & 15;
  // k row 8(g/2) + i16/4 (k & 3 = i16/4 for every step and the +4 read), 16-byte chunk
  // 4w + 2(g%2) + (i16%4)/2, 8-byte half i16%2
  const int b_off = (8 * (g >> 1) + (i16 >> 2)) * (kTN * 2) +
                    16 * ((4 * wave + 2 * (g & 1) + ((i16 & 3) >> 1)) ^ (4 * (i16 >> 2))) + 8 * (i16 & 1);
  auto a_op = [&](const lds_u8* ab, int rb, int s) {
    const int r = 32 * rb + (lane & 31);
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(ab + a_chunk_off(r, 2 * s + (lane >> 5)));
  };
  auto b_op = [&](const lds_u8* bb, int s) {
    const lds_u8* p = bb + b_off + s * 16 * (kTN * 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 4 * (kTN * 2)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 acc[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[rb][x] = 0.f;

  load(0);
  store(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunks) load(c + 1);  // in flight while this chunk is multiplied
    const lds_u8* const bb = lbase + buf * kBufB;
#pragma unroll
    for (int s = 0; s < kKC / 16; ++s) {
      const bf16x8 bo = b_op(bb, s);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op(bb + kBChunkB, rb, s), bo, acc[rb], 0, 0, 0);
        if constexpr (AF32)
          acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op(bb + kBChunkB + kAChunkB, rb, s), bo, acc[rb], 0, 0, 0);
      }
    }
    if (c + 1 < nchunks) {
      store(buf ^ 1);  // that buffer was last read before the previous barrier
      __syncthreads();
    }
  }

  // D layout (A rows on M, B columns on N): lane holds column 32w + l%32 of rows
  // 8(x/4) + 4(l/32) + x%4 of each row block
  float* const out = part + int64_t(blockIdx.z) * M * n_total + n0 + 32 * wave + (lane & 31);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int m = m0 + 32 * rb + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
      if (m < M) out[int64_t(m) * n_total] = acc[rb][x];
    }
}

// Query epilogue: q_hat[r, h, :] = [sum_s part[s, r, h, 0:d_c] | RoPE_pos(sum_s part[s, r, h, d_c:])] *
// qscale, rounded to binary16 (the q_hat format of the bf16 path).  One wave per (row, head); lane l holds columns 8l..8l+7 of the 512
// latent columns and, for l < 32, rotary pair l.
struct RopeFreqP {
  double v[32];
};
__global__ __launch_bounds__(256) void query_epilogue_kernel(const float* __restrict__ part, int splits, int rows,
                                                             int H, const int32_t* __restrict__ pos, float qscale,
                                                             RopeFreqP freq, uint16_t* __restrict__ q_hat) {
  const int64_t rh = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (rh >= int64_t(rows) * H) return;
  const int lane = threadIdx.x & 63;
  const int r = int(rh / H);
  constexpr int W = 576;
  const int64_t stride = int64_t(rows) * H * W;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, x1 = 0.f, x2 = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float* p = part + s * stride + rh * W;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p + 8 * lane), c = *reinterpret_cast<const f32x4*>(p + 8 * lane + 4);
    v[0] += a[0]; v[1] += a[1]; v[2] += a[2]; v[3] += a[3];
    v[4] += c[0]; v[5] += c[1]; v[6] += c[2]; v[7] += c[3];
    if (lane < 32) {
      const float2 y = *reinterpret_cast<const float2*>(p + 512 + 2 * lane);
      x1 += y.x;
      x2 += y.y;
    }
  }
  uint16_t* o = q_hat + rh * W;
  u32x4 w;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = uint32_t(f32_to_f16(v[2 * q] * qscale)) | (uint32_t(f32_to_f16(v[2 * q + 1] * qscale)) << 16);
  *reinterpret_cast<u32x4*>(o + 8 * lane) = w;
  if (lane < 32) {
    // angle pos * base^(-2i/d_r) in double, reduced to [-pi, pi] before the float sine and cosine
    const double ang = double(pos[r]) * freq.v[lane];
    const double rd = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
    float sn, cs;
    sincosf(float(rd), &sn, &cs);
    const float r1 = (x1 * cs - x2 * sn) * qscale, r2 = (x1 * sn + x2 * cs) * qscale;
    *reinterpret_cast<uint32_t*>(o + 512 + 2 * lane) = uint32_t(f32_to_f16(r1)) | (uint32_t(f32_to_f16(r2)) << 16);
  }
}

// out[r, n] = sum_s part[s, r, n] (float32)
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part, int splits, int64_t count,
                                                         float* __restrict__ out) {
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
  for (int s = 1; s < splits; ++s) acc += *reinterpret_cast<const f32x4*>(part + s * count + i);
  *reinterpret_cast<f32x4*>(out + i) = acc;
}

// Offline precomposition: out[h, i, j] = bf16(sum_k X[h, i, k] Y[h, k, j]) for arbitrary strides,
// 16 x 16 outputs per workgroup, K in tiles of 16 through LDS, float32 accumulation.
struct Strides3 {
  int64_t h, i, k;
};
__global__ __launch_bounds__(256) void precompose_kernel(const uint16_t* __restrict__ x, Strides3 sx,
                                                         const uint16_t* __restrict__ y, Strides3 sy, int I, int J,
                                                         int K, uint16_t* __restrict__ out, Strides3 so) {
  __shared__ float xs[16][17], ys[16][17];
  const int h = blockIdx.z, ti = threadIdx.x >> 4, tj = threadIdx.x & 15;
  const int i = blockIdx.y * 16 + ti, j = blockIdx.x * 16 + tj;
  float acc = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    // X tile rows i0.., k k0..; Y tile k k0.., columns j0..  (sy.i is the k stride, sy.k the j stride)
    const int xi = blockIdx.y * 16 + ti, xk = k0 + tj;
    xs[ti][tj] = (xi < I && xk < K) ? bf16_to_f32(x[h * sx.h + xi * sx.i + xk * sx.k]) : 0.f;
    const int yk = k0 + ti, yj = blockIdx.x * 16 + tj;
    ys[ti][tj] = (yk < K && yj < J) ? bf16_to_f32(y[h * sy.h + yk * sy.i + yj * sy.k]) : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(xs[ti][kk], ys[kk][tj], acc);
    __syncthreads();
  }
  if (i < I && j < J) out[h * so.h + i * so.i + j * so.k] = f32_to_bf16(acc);
}

// copy W_QR[h] [d_cq, d_r] into the rotary columns of w_qcat [d_cq, H, d_c + d_r]
__global__ void copy_qr_kernel(const uint16_t* __restrict__ w_qr, int d_cq, int H, int d_c, int d_r,
                               uint16_t* __restrict__ w_qcat) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = int64_t(H) * d_cq * d_r;
  if (idx >= total) return;
  const int rr = int(idx % d_r), q = int((idx / d_r) % d_cq), h = int(idx / (int64_t(d_r) * d_cq));
  w_qcat[(int64_t(q) * H + h) * (d_c + d_r) + d_c + rr] = w_qr[idx];
}

// K splits of a product: the most that divide its chunks and keep the grid within 512 workgroups,
// i.e. one round at two workgroups per CU (64 KiB of LDS each); a second round of short
// workgroups left the matrix weight stream idle at every start.
int gemm_splits(int64_t n_total, int M, int64_t K) {
  const int64_t tiles = (n_total / kTN) * ((M + kTM - 1) / kTM);
  const int64_t chunks = K / kKC;
  int best = 1;
  for (int s = 1; s <= 64; ++s)
    if (chunks % s == 0 && tiles * s <= 512) best = s;
  return best;
}

template <bool AF32>
hipError_t launch_gemm(const void* a, int64_t lda, const uint16_t* b, int64_t ldb, int M, int64_t n_total, int64_t K,
                       int splits, float* part, hipStream_t s) {
  const dim3 grid(unsigned(n_total / kTN), unsigned((M + kTM - 1) / kTM), unsigned(splits));
  gemm_kernel<AF32><<<grid, kThreads, 0, s>>>(a, lda, b, ldb, M, n_total, int(K / splits), part);
  return hipGetLastError();
}

}  // namespace

bool precomposed_supported(const Dims& d) { return d.dtype == MLA_BF16 && d.dc == 512 && d.dr == 64; }

// Workspaces (float32 split partials) of the two per-step products.
size_t absorb_precomposed_workspace(const Dims& d, int d_cq, int rows) {
  const int64_t n = int64_t(d.H) * (d.dc + d.dr);
  return size_t(gemm_splits(n, rows, d_cq)) * size_t(rows) * size_t(n) * sizeof(float);
}
size_t out_fused_workspace(const Dims& d, int d_model, int rows) {
  return size_t(gemm_splits(d_model, rows, int64_t(d.H) * d.dc)) * size_t(rows) * size_t(d_model) * sizeof(float);
}

hipError_t launch_precompose_query(const Dims& d, int d_cq, const void* w_uq, const void* w_uk, const void* w_qr,
                                   void* w_qcat, hipStream_t s) {
  const int W = d.dc + d.dr;
  // out[h, q, c] = sum_k W_UQ[h, q, k] W_UK[h, c, k], stored at w_qcat[q, h, c]
  const Strides3 sx{int64_t(d_cq) * d.dk, d.dk, 1};
  const Strides3 sy{int64_t(d.dc) * d.dk, 1, d.dk};  // Y[h, k, c] = W_UK[h, c, k]
  const Strides3 so{W, int64_t(d.H) * W, 1};
  const dim3 grid((d.dc + 15) / 16, (d_cq + 15) / 16, d.H);
  precompose_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(w_uq), sx, static_cast<const uint16_t*>(w_uk), sy,
                                         d_cq, d.dc, d.dk, static_cast<uint16_t*>(w_qcat), so);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = int64_t(d.H) * d_cq * d.dr;
  copy_qr_kernel<<<unsigned((total + 255) / 256), 256, 0, s>>>(static_cast<const uint16_t*>(w_qr), d_cq, d.H, d.dc,
                                                               d.dr, static_cast<uint16_t*>(w_qcat));
  return hipGetLastError();
}

hipError_t launch_precompose_out(const Dims& d, int d_model, const void* w_uv, const void* w_o, void* w_uvo,
                                 hipStream_t s) {
  // out[h, c, m] = sum_v W_UV[h, c, v] W_O[h * d_v + v, m]
  const Strides3 sx{int64_t(d.dc) * d.dv, d.dv, 1};
  const Strides3 sy{int64_t(d.dv) * d_model, d_model, 1};
  const Strides3 so{int64_t(d.dc) * d_model, d_model, 1};
  const dim3 grid((d_model + 15) / 16, (d.dc + 15) / 16, d.H);
  precompose_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(w_uv), sx, static_cast<const uint16_t*>(w_o), sy,
                                         d.dc, d_model, d.dv, static_cast<uint16_t*>(w_uvo), so);
  return hipGetLastError();
}

hipError_t launch_absorb_precomposed(const Dims& d, int d_cq, const void* c_q, const void* w_qcat, const int32_t* pos,
                                     int rows, void* q_hat, float* workspace, hipStream_t s) {
  const int64_t n = int64_t(d.H) * (d.dc + d.dr);
  const int splits = gemm_splits(n, rows, d_cq);
  hipError_t e = launch_gemm<false>(c_q, d_cq, static_cast<const uint16_t*>(w_qcat), n, rows, n, d_cq, splits,
                                    workspace, s);
  if (e != hipSuccess) return e;
  RopeFreqP f;
  for (int i = 0; i < d.dr / 2; ++i) f.v[i] = pow(double(d.rope_base), -2.0 * i / d.dr);
  const float qscale = d.sm_scale * 1.4426950408889634f;
  const int64_t waves = int64_t(rows) * d.H;
  query_epilogue_kernel<<<unsigned((waves + 3) / 4), 256, 0, s>>>(workspace, splits, rows, d.H, pos, qscale, f,
                                                                   static_cast<uint16_t*>(q_hat));
  return hipGetLastError();
}

hipError_t launch_out_fused(const Dims& d, int d_model, const float* z, const void* w_uvo, int rows, float* out,
                            float* workspace, hipStream_t s) {
  const int64_t K = int64_t(d.H) * d.dc;
  const int splits = gemm_splits(d_model, rows, K);
  hipError_t e = launch_gemm<true>(z, K, static_cast<const uint16_t*>(w_uvo), d_model, rows, d_model, K, splits,
                                   workspace, s);
  if (e != hipSuccess) return e;
  const int64_t count = int64_t(rows) * d_model;
  sum_splits_kernel<<<unsigned((count / 4 + 255) / 256), 256, 0, s>>>(workspace, splits, count, out);
  return hipGetLastError();
}

// o_concat [rows, H*d_v] float32 . W_O [H*d_v, d_model] bf16 -> out [rows, d_model] float32
size_t output_projection_workspace(const Dims& d, int d_model, int rows) {
  return size_t(gemm_splits(d_model, rows, int64_t(d.H) * d.dv)) * size_t(rows) * size_t(d_model) * sizeof(float);
}
hipError_t launch_output_projection(const Dims& d, int d_model, const float* o, const void* w_o, int rows, float* out,
                                    float* workspace, hipStream_t s) {
  const int64_t K = int64_t(d.H) * d.dv;
  const int splits = gemm_splits(d_model, rows, K);
  hipError_t e = launch_gemm<true>(o, K, static_cast<const uint16_t*>(w_o), d_model, rows, d_model, K, splits,
                                   workspace, s);
  if (e != hipSuccess) return e;
  const int64_t count = int64_t(rows) * d_model;
  sum_splits_kernel<<<unsigned((count / 4 + 255) / 256), 256, 0, s>>>(workspace, splits, count, out);
  return hipGetLastError();
}

}  // namespace mla
