// Pre-pass kernels: K smoothing, per-block INT8 quantisation of Q and K, and
// V preparation (packed FP16 tiles, or per-channel e4m3) for the attention
// kernel.  All of them are HBM-bound streaming kernels: 16-byte coalesced
// loads, one workgroup per quantisation block, values kept in registers
// between the block reduction and the quantisation (one read of each input).
//
// Pages (by title): "⚡️SageAttention — brand new attention" (postsniper.ru),
// quantisation introduction: scale = max|A|/127, Â = round(A/scale); dtcms.com
// SageAttention summary, section "SageAttention（v1）": smooth K by its mean,
// per-block quantisation of q and k; section "SageAttention 2": V in FP8.
#include "sage_common.h"
#include "sage_internal.h"

namespace sage {

// ---------------------------------------------------------------------------
// Zero fill (used instead of hipMemsetAsync so the sequence stays capturable).
__global__ void zero_kernel(v4i* __restrict__ p, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = v4i{0, 0, 0, 0};
}

// ---------------------------------------------------------------------------
// K column sums in exact int64 fixed point (value * 2^24), per head-sequence.
// Grid (ceil(Nmax/256), H, B); each block sums up to 256 tokens and adds its
// partial sums with integer atomics (exact and order-independent).
constexpr int kColsumChunk = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void k_colsum_kernel(const uint16_t* __restrict__ k, SeqGeom g,
                                                            unsigned long long* __restrict__ colsum) {
  constexpr int CG = D / 8;            // 16-byte channel groups per row
  constexpr int RPP = kThreads / CG;   // rows per pass
  const int b = blockIdx.z, h = blockIdx.y;
  int64_t row0;
  int n;
  hs_rows(g, b, h, row0, n);
  const int t0 = blockIdx.x * kColsumChunk;
  if (t0 >= n) return;
  const int t1 = min(n, t0 + kColsumChunk);
  const int cg = threadIdx.x % CG, rr = threadIdx.x / CG;
  // fp64 partial sums are exact: every fp16 value is a multiple of 2^-24 below
  // 2^16 in magnitude, and a thread adds at most kColsumChunk / RPP of them
  constexpr int ITER = kColsumChunk / RPP;
  v4i raw[ITER];  // all loads in flight before the adds
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int t = t0 + rr + i * RPP;
    raw[i] = (t < t1) ? *reinterpret_cast<const v4i*>(k + (row0 + t) * D + cg * 8) : v4i{0, 0, 0, 0};
  }
  double acc[8] = {0., 0., 0., 0., 0., 0., 0., 0.};
#pragma unroll
  for (int i = 0; i < ITER; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = (uint32_t)raw[i][j];
      acc[2 * j] += (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
      acc[2 * j + 1] += (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
  static_assert(kColsumChunk / RPP <= 8192, "fp64 partial sums must stay exact");
  __shared__ int64_t red[RPP][D];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[rr][cg * 8 + j] = (int64_t)(acc[j] * 0x1p24);  // integral, < 2^53
  __syncthreads();
  if (threadIdx.x < D) {
    int64_t s = 0;
    for (int r = 0; r < RPP; ++r) s += red[r][threadIdx.x];
    const int64_t hs = (int64_t)b * g.H + h;
    atomicAdd(colsum + hs * D + threadIdx.x, (unsigned long long)s);
  }
}

// Block-wide max of a non-negative value over 256 threads.
__device__ __forceinline__ float block_max256(float v) {
  __shared__ float wmax[kThreads / 64];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = wmax[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, wmax[i]);
  return r;
}

// ---------------------------------------------------------------------------
// Per-block INT8 of one block of ROWS tokens x D channels of fp32 values
// x = fp16 input - shift.  MODE selects the shift:
//   kShiftNone  — Q without smoothing;
//   kShiftKMean — K: the head-sequence's token mean (from the column sums),
//                 written to mean[hs][D] by block 0;
//   kShiftBlock — smoothed Q: the block's own token mean, written to
//                 mean[hs][blk][D] (dtcms summary, section "SageAttention 2":
//                 Q is smoothed as well).
// Grid (ceil(Nmax/ROWS), H, B).
enum { kShiftNone = 0, kShiftKMean = 1, kShiftBlock = 2 };

template <int D, int ROWS, int MODE>
__global__ __launch_bounds__(kThreads) void quant_block_kernel(const uint16_t* __restrict__ x16, SeqGeom g,
                                                               const long long* __restrict__ colsum,
                                                               float out_scale_mul, int8_t* __restrict__ codes,
                                                               float* __restrict__ scales,
                                                               float* __restrict__ mean) {
  constexpr int CG = D / 8, RPP = kThreads / CG, PASSES = ROWS / RPP;
  static_assert(PASSES * RPP == ROWS, "block rows must be a multiple of rows per pass");
  const int b = blockIdx.z, h = blockIdx.y, blk = blockIdx.x;
  int64_t row0;
  int n;
  hs_rows(g, b, h, row0, n);
  const int t0 = blk * ROWS;
  if (t0 >= n) return;
  const int cg = threadIdx.x % CG, rr = threadIdx.x / CG;
  const int64_t hs = (int64_t)b * g.H + h;
  // all of the block's loads first (raw fp16, 16 bytes per pass and thread)
  v4i raw[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int t = t0 + rr + p * RPP;
    raw[p] = (t < n) ? *reinterpret_cast<const v4i*>(x16 + (row0 + t) * D + cg * 8) : v4i{0, 0, 0, 0};
  }
  float shift[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) shift[j] = 0.f;
  if (MODE == kShiftKMean) {
    // km = fp32(exact sum * 2^-24 / n): one fp64 divide per channel, one rounding
    __shared__ float km_s[D];
    if (threadIdx.x < D) {
      const float km = (float)((double)colsum[hs * D + threadIdx.x] * 0x1p-24 / (double)n);
      km_s[threadIdx.x] = km;
      if (blk == 0) mean[hs * D + threadIdx.x] = km;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) shift[j] = km_s[cg * 8 + j];
  } else if (MODE == kShiftBlock) {
    // the block's own mean, by the same exact rule: fp64 sums of fp16 values
    // are exact (multiples of 2^-24 below 2^16, at most ROWS of them), one
    // fp64 divide by the block's token count, one rounding to fp32
    double acc[8] = {0., 0., 0., 0., 0., 0., 0., 0.};
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = (uint32_t)raw[p][j];  // rows past n were loaded as zeros
        acc[2 * j] += (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
        acc[2 * j + 1] += (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
      }
    __shared__ double part[RPP][D];
    __shared__ float qm_s[D];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[rr][cg * 8 + j] = acc[j];
    __syncthreads();
    if (threadIdx.x < D) {
      double sum = 0.;  // exact in any order
      for (int r = 0; r < RPP; ++r) sum += part[r][threadIdx.x];
      const float qm = (float)(sum / (double)min(ROWS, n - t0));
      qm_s[threadIdx.x] = qm;
      mean[(hs * ceil_div(g.N, ROWS) + blk) * D + threadIdx.x] = qm;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) shift[j] = qm_s[cg * 8 + j];
  }
  // x = fp32(fp16) - shift; rows past n are zero (their codes are not stored)
  auto unpack = [&](int p, float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = (uint32_t)raw[p][j];
      x[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)) - shift[2 * j];
      x[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)) - shift[2 * j + 1];
    }
  };
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    if (t0 + rr + p * RPP < n) {
      float x[8];
      unpack(p, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
    }
  }
  amax = block_max256(amax);
  const float s = amax / kInt8Max;
  const float r = 1.0f / s;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int t = t0 + rr + p * RPP;
    if (t < n) {
      uint2 w = {0u, 0u};  // an all-zero block (s = 0) has all codes 0
      if (s > 0.f) {
        float x[8];
        unpack(p, x);
        w.x = pack4_i8(int8_code(x[0], s, r), int8_code(x[1], s, r), int8_code(x[2], s, r), int8_code(x[3], s, r));
        w.y = pack4_i8(int8_code(x[4], s, r), int8_code(x[5], s, r), int8_code(x[6], s, r), int8_code(x[7], s, r));
      }
      *reinterpret_cast<uint2*>(codes + (row0 + t) * D + cg * 8) = w;
    }
  }
  if (threadIdx.x == 0) {
    const int nblk = ceil_div(g.N, ROWS);
    scales[hs * nblk + blk] = s * out_scale_mul;
  }
}

// ---------------------------------------------------------------------------
// Per-token INT8 of Q (dtcms summary, "SageAttention（v1）": per-token
// quantisation of q; "SageAttention 2": finer granularity): the quantiser of
// quant_block_kernel on each row alone.  D/8 threads share a row (16 bytes
// each); a workgroup takes ROWS rows, all loads first.  scales[row0 + t] =
// fp32(max|x|/127) · out_scale_mul, i.e. indexed like the token itself.
// Grid (ceil(Nmax/ROWS), H, B).
template <int D, int ROWS>
__global__ __launch_bounds__(kThreads) void quant_row_kernel(const uint16_t* __restrict__ x16, SeqGeom g,
                                                             float out_scale_mul, int8_t* __restrict__ codes,
                                                             float* __restrict__ scales) {
  constexpr int CG = D / 8, RPP = kThreads / CG, PASSES = ROWS / RPP;
  static_assert(PASSES * RPP == ROWS, "rows must be a multiple of rows per pass");
  const int b = blockIdx.z, h = blockIdx.y;
  int64_t row0;
  int n;
  hs_rows(g, b, h, row0, n);
  const int t0 = blockIdx.x * ROWS;
  if (t0 >= n) return;
  const int cg = threadIdx.x % CG, rr = threadIdx.x / CG;
  v4i raw[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int t = t0 + rr + p * RPP;
    raw[p] = (t < n) ? *reinterpret_cast<const v4i*>(x16 + (row0 + t) * D + cg * 8) : v4i{0, 0, 0, 0};
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int t = t0 + rr + p * RPP;
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = (uint32_t)raw[p][j];
      x[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
      x[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
    for (int o = 1; o < CG; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));  // the row's CG lanes
    const float sc = amax / kInt8Max;
    const float r = 1.0f / sc;
    if (t < n) {
      uint2 w = {0u, 0u};  // an all-zero row (scale 0) has all codes 0
      if (sc > 0.f) {
        w.x = pack4_i8(int8_code(x[0], sc, r), int8_code(x[1], sc, r), int8_code(x[2], sc, r), int8_code(x[3], sc, r));
        w.y = pack4_i8(int8_code(x[4], sc, r), int8_code(x[5], sc, r), int8_code(x[6], sc, r), int8_code(x[7], sc, r));
      }
      *reinterpret_cast<uint2*>(codes + (row0 + t) * D + cg * 8) = w;
      if (cg == 0) scales[row0 + t] = sc * out_scale_mul;
    }
  }
}

// ---------------------------------------------------------------------------
// V per-channel absolute maximum (as fp32 bits; non-negative floats order like
// their bit patterns, so an integer atomic max is exact).
template <int D>
__global__ __launch_bounds__(kThreads) void v_absmax_kernel(const uint16_t* __restrict__ v, SeqGeom g,
                                                            unsigned* __restrict__ amax_bits) {
  constexpr int CG = D / 8, RPP = kThreads / CG;
  const int b = blockIdx.z, h = blockIdx.y;
  int64_t row0;
  int n;
  hs_rows(g, b, h, row0, n);
  const int t0 = blockIdx.x * kColsumChunk;
  if (t0 >= n) return;
  const int t1 = min(n, t0 + kColsumChunk);
  const int cg = threadIdx.x % CG, rr = threadIdx.x / CG;
  constexpr int ITER = kColsumChunk / RPP;
  v4i raw[ITER];  // all loads in flight before the reduction
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int t = t0 + rr + i * RPP;
    raw[i] = (t < t1) ? *reinterpret_cast<const v4i*>(v + (row0 + t) * D + cg * 8) : v4i{0, 0, 0, 0};
  }
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < ITER; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = (uint32_t)raw[i][j];
      m[2 * j] = fmaxf(m[2 * j], fabsf((float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu))));
      m[2 * j + 1] = fmaxf(m[2 * j + 1], fabsf((float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16))));
    }
  __shared__ float red[RPP][D];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[rr][cg * 8 + j] = m[j];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
    for (int r = 0; r < RPP; ++r) s = fmaxf(s, red[r][threadIdx.x]);
    const int64_t hs = (int64_t)b * g.H + h;
    atomicMax(amax_bits + hs * D + threadIdx.x, __float_as_uint(s));
  }
}

// scale = fp32(amax / 448), in place over the amax bits.
__global__ void v_scale_finalize_kernel(float* __restrict__ vs, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) vs[i] = vs[i] / kE4M3Max;
}

// OCP e4m3 byte of fp32(v / s): IEEE divide, saturate to ±448, then the
// hardware round-to-nearest-even conversion.  s == 0 -> code 0.
__device__ __forceinline__ float e4m3_operand(float v, float s) {
  if (!(s > 0.f)) return 0.f;
  return __builtin_amdgcn_fmed3f(v / s, -kE4M3Max, kE4M3Max);
}

__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// ---------------------------------------------------------------------------
// V preparation, one 64-key tile per workgroup.  Grid (ceil(Nmax/64), H, B).
//   FP8 = false: packed fp16 tile in MFMA-operand order (see attn.hip).
//   FP8 = true, ROWMAJOR = false: packed e4m3 tile in MFMA-operand order.
//   FP8 = true, ROWMAJOR = true: row-major e4m3 codes [.., n, D].
// Packed fp16 tile: 16-byte chunk (f, lane), f = kc*(D/32) + dt, holds the
//   8 values V[key][d] with d = 32dt + lane%32 and, for j = 0..7,
//   key = 16kc + 8(j/4) + 4(lane/32) + j%4.
// Packed e4m3 tile: 32-byte chunk (dt, lane) holds, for j = 0..31,
//   key = 32(j/16) + 8((j%16)/4) + 4(lane/32) + j%4, d = 32dt + lane%32.
// Keys past the sequence end are written as zeros.
template <int D, bool FP8, bool ROWMAJOR>
__global__ __launch_bounds__(kThreads) void v_prepare_kernel(const uint16_t* __restrict__ v, SeqGeom g,
                                                             const float* __restrict__ vscale,
                                                             uint8_t* __restrict__ out) {
  const int b = blockIdx.z, h = blockIdx.y, kb = blockIdx.x;
  int64_t row0;
  int n;
  hs_rows(g, b, h, row0, n);
  const int t0 = kb * kKBlock;
  if (t0 >= n) return;
  const int64_t hs = (int64_t)b * g.H + h;
  __shared__ uint16_t tile[kKBlock][D + 2];
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  for (int idx = threadIdx.x; idx < kKBlock * CPR; idx += kThreads) {
    const int r = idx / CPR, c = idx % CPR;
    v4i val = {0, 0, 0, 0};
    if (t0 + r < n) val = *reinterpret_cast<const v4i*>(v + (row0 + t0 + r) * D + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[r][c * 8 + 2 * j] = (uint16_t)((uint32_t)val[j] & 0xffffu);
      tile[r][c * 8 + 2 * j + 1] = (uint16_t)((uint32_t)val[j] >> 16);
    }
  }
  __syncthreads();
  if (!FP8) {
    constexpr int TILE_BYTES = kKBlock * D * 2;
    uint8_t* dst = out + vtile_index(g, b, h, kb) * TILE_BYTES;
    for (int idx = threadIdx.x; idx < TILE_BYTES / 16; idx += kThreads) {
      const int f = idx / 64, lane = idx % 64;
      const int kc = f / (D / 32), dt = f % (D / 32);
      const int d = 32 * dt + (lane & 31), g4 = 4 * (lane >> 5);
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const int k0 = 16 * kc + 8 * (j / 4) + g4 + (j & 3);
        w[j / 2] = (uint32_t)tile[k0][d] | ((uint32_t)tile[k0 + 1][d] << 16);
      }
      *reinterpret_cast<v4i*>(dst + (int64_t)idx * 16) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  } else if (!ROWMAJOR) {
    constexpr int TILE_BYTES = kKBlock * D;
    uint8_t* dst = out + vtile_index(g, b, h, kb) * TILE_BYTES;
    for (int idx = threadIdx.x; idx < TILE_BYTES / 32; idx += kThreads) {
      const int dt = idx / 64, lane = idx % 64;
      const int d = 32 * dt + (lane & 31), g4 = 4 * (lane >> 5);
      const float s = vscale[hs * D + d];
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float f[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * q + jj;
          const int key = 32 * (j / 16) + 8 * ((j % 16) / 4) + g4 + (j & 3);
          f[jj] = e4m3_operand((float)__builtin_bit_cast(_Float16, tile[key][d]), s);
        }
        w[q] = pack4_e4m3(f[0], f[1], f[2], f[3]);
      }
      v4i* o = reinterpret_cast<v4i*>(dst + (int64_t)idx * 32);
      o[0] = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      o[1] = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    }
  } else {
    // row-major codes: each thread converts 16 channels of one row
    constexpr int C16 = D / 16;
    for (int idx = threadIdx.x; idx < kKBlock * C16; idx += kThreads) {
      const int r = idx / C16, c = idx % C16;
      if (t0 + r >= n) continue;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float f[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d = 16 * c + 4 * q + jj;
          f[jj] = e4m3_operand((float)__builtin_bit_cast(_Float16, tile[r][d]), vscale[hs * D + d]);
        }
        w[q] = pack4_e4m3(f[0], f[1], f[2], f[3]);
      }
      *reinterpret_cast<v4i*>(out + (row0 + t0 + r) * D + 16 * c) =
          v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP4 (dtcms summary, section "SageAttention 3": microscaling FP4 attention,
// two-level quantisation, range adjusted against block outliers): OCP MX
// blocks of 32 e2m1 elements sharing one E8M0 (power-of-two) scale, the
// smallest one under which the block maximum fits e2m1's largest value 6.

// LDS row of key κ of a 64-key tile in the MXFP4 attention kernel: the K̂ rows
// are stored so that each MFMA lane half's 32 scores are 32 consecutive keys
// (LDS row 32s + 8q + 4g + t holds key 32g + 16s + 4q + t).
__device__ __forceinline__ int mx_krow_of_key(int kappa) {
  return 32 * ((kappa >> 4) & 1) + 8 * ((kappa >> 2) & 3) + 4 * (kappa >> 5) + (kappa & 3);
}

// Q, the smoothed K or the smoothed Q as MX FP4 along channels (per token,
// 32-channel blocks).  MODE (the shifts of quant_block_kernel):
//   kShiftNone  — Q;
//   kShiftKMean — K: x = fp32(k) - km, km from the exact column sums, written
//                 to mean[hs][D] by the first workgroup;
//   kShiftBlock — smoothed Q: x = fp32(q) - q̄ of the workgroup's own 128-token
//                 block (ROWS = 128), the exact block mean written to
//                 mean[hs][blk][D].
// Codes [row][D/2] bytes, channel c in nibble c%2 of byte c/2.  Scale bytes
// (X + 127) of block b = 2kk + g: Q into qscale[row][g] dword, byte kk; K
// into the K/V tile's aux region at (LDS row of the key)·8 + 4g + kk.  D/8
// threads per token.  Grid (ceil(Nmax/ROWS), H, B).
template <int D, int ROWS, int MODE>
__global__ __launch_bounds__(kThreads) void mx_rows_kernel(const uint16_t* __restrict__ x16, SeqGeom g,
                                                           const long long* __restrict__ colsum,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ qscale,
                                                           uint8_t* __restrict__ aux, float* __restrict__ mean) {
  constexpr bool SMOOTH = MODE == kShiftKMean;
  constexpr int CG = D / 8, RPP = kThreads / CG, PASSES = ROWS / RPP;
  static_assert(PASSES * RPP == ROWS, "rows must be a multiple of rows per pass");
  const int b = blockIdx.z, h = blockIdx.y;
  int64_t row0;
  int n;
  hs_rows(g, b, h, row0, n);
  const int t0 = blockIdx.x * ROWS;
  if (t0 >= n) return;
  const int cg = threadIdx.x % CG, rr = threadIdx.x / CG;
  const int64_t hs = (int64_t)b * g.H + h;
  v4i raw[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int t = t0 + rr + p * RPP;
    raw[p] = (t < n) ? *reinterpret_cast<const v4i*>(x16 + (row0 + t) * D + cg * 8) : v4i{0, 0, 0, 0};
  }
  float shift[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (SMOOTH) {
    __shared__ float km_s[D];
    if (threadIdx.x < D) {
      const float km = (float)((double)colsum[hs * D + threadIdx.x] * 0x1p-24 / (double)n);
      km_s[threadIdx.x] = km;
      if (blockIdx.x == 0) mean[hs * D + threadIdx.x] = km;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) shift[j] = km_s[cg * 8 + j];
  } else if (MODE == kShiftBlock) {
    static_assert(MODE != kShiftBlock || ROWS == kQBlock, "the block mean needs the whole Q block");
    // exact: fp64 sums of fp16 values (rows past n loaded as zeros), one
    // divide by the block's token count, one rounding to fp32
    double acc[8] = {0., 0., 0., 0., 0., 0., 0., 0.};
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = (uint32_t)raw[p][j];
        acc[2 * j] += (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
        acc[2 * j + 1] += (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
      }
    __shared__ double part[RPP][D];
    __shared__ float qm_s[D];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[rr][cg * 8 + j] = acc[j];
    __syncthreads();
    if (threadIdx.x < D) {
      double sum = 0.;
      for (int r = 0; r < RPP; ++r) sum += part[r][threadIdx.x];
      const float qm = (float)(sum / (double)min(ROWS, n - t0));
      qm_s[threadIdx.x] = qm;
      mean[(hs * ceil_div(g.N, ROWS) + blockIdx.x) * D + threadIdx.x] = qm;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) shift[j] = qm_s[cg * 8 + j];
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int t = t0 + rr + p * RPP;
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = (uint32_t)raw[p][j];
      x[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)) - shift[2 * j];
      x[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)) - shift[2 * j + 1];
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));  // the block's four lanes
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int X = mx_exponent(amax);
    const uint32_t w = mx_pack8(x, ldexpf(1.f, X));
    if (t < n) {
      *reinterpret_cast<uint32_t*>(codes + (row0 + t) * (D / 2) + cg * 4) = w;
      if ((cg & 3) == 0) {
        const int blk = cg >> 2, kk = blk >> 1, gsel = blk & 1;
        const uint8_t sb = (uint8_t)(X + 127);
        if (!SMOOTH)
          qscale[(row0 + t) * 8 + 4 * gsel + kk] = sb;
        else
          aux[vtile_index(g, b, h, t / kKBlock) * kMxAuxBytes + mx_krow_of_key(t % kKBlock) * 8 + 4 * gsel + kk] =
              sb;
      }
    }
  }
}

// V as MX FP4 along keys, one 64-key tile per workgroup: for each channel c
// and key half g, the block of keys 64t + 32g .. +31 (zeros past n).  Packed
// in the PV operand order: codes[tile][dt][lane] 16 bytes, lane = c%32 + 32g,
// dt = c/32, key 32g + j in nibble j; scale byte of (c, g) at aux offset
// 512 + 4·lane + dt.  Grid (ceil(Nmax/64), H, B).
template <int D>
__global__ __launch_bounds__(kThreads) void mx_v_prepare_kernel(const uint16_t* __restrict__ v, SeqGeom g,
                                                                uint8_t* __restrict__ vcodes,
                                                                uint8_t* __restrict__ aux) {
  const int b = blockIdx.z, h = blockIdx.y, kb = blockIdx.x;
  int64_t row0;
  int n;
  hs_rows(g, b, h, row0, n);
  const int t0 = kb * kKBlock;
  if (t0 >= n) return;
  __shared__ uint16_t tile[kKBlock][D + 2];
  constexpr int CPR = D / 8;
  for (int idx = threadIdx.x; idx < kKBlock * CPR; idx += kThreads) {
    const int r = idx / CPR, c = idx % CPR;
    v4i val = {0, 0, 0, 0};
    if (t0 + r < n) val = *reinterpret_cast<const v4i*>(v + (row0 + t0 + r) * D + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[r][c * 8 + 2 * j] = (uint16_t)((uint32_t)val[j] & 0xffffu);
      tile[r][c * 8 + 2 * j + 1] = (uint16_t)((uint32_t)val[j] >> 16);
    }
  }
  __syncthreads();
  const int64_t ti = vtile_index(g, b, h, kb);
  for (int u = threadIdx.x; u < 2 * D; u += kThreads) {
    const int c = u % D, gsel = u / D;
    float x[32];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      x[j] = (float)__builtin_bit_cast(_Float16, tile[32 * gsel + j][c]);
      amax = fmaxf(amax, fabsf(x[j]));
    }
    const int X = mx_exponent(amax);
    const float sc = ldexpf(1.f, X);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = x[8 * q + j];
      w[q] = mx_pack8(y, sc);
    }
    const int lane = (c & 31) + 32 * gsel, dt = c >> 5;
    *reinterpret_cast<v4i*>(vcodes + (ti * (D / 32) + dt) * 1024 + lane * 16) =
        v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    aux[ti * kMxAuxBytes + 512 + 4 * lane + dt] = (uint8_t)(X + 127);
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers.
static inline dim3 hs_grid(const SeqGeom& g, int rows) { return dim3(ceil_div(g.N, rows), g.H, g.B); }
constexpr int kRowsPerBlock = 64;  // rows per workgroup of the per-token quantiser

void launch_zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)ceil_div64(n16, 256)), dim3(256), 0, st,
                     reinterpret_cast<v4i*>(p), n16);
}

void launch_quant_qk(const SeqGeom& gq, const SeqGeom& gk, const void* q, const void* k, float sm_scale,
                     int8_t* q_int8, int8_t* k_int8, float* q_scale, float* k_scale, float* k_mean,
                     float* q_mean, bool q_per_token, long long* colsum, hipStream_t st) {
  // gq: Q's geometry (H query heads); gk: K's (its own head count), same
  // sequences.  q_mean != nullptr selects Q smoothing, q_per_token per-token
  // Q scales (not both); without smoothing, q_int8 == nullptr leaves Q to the
  // attention kernel (it quantises the fp16 Q itself).
  const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q);
  const uint16_t* k16 = reinterpret_cast<const uint16_t*>(k);
  launch_zero(colsum, sizeof(long long) * (size_t)gk.B * gk.H * gk.d, st);
  const dim3 gqb = hs_grid(gq, kQBlock), gkb = hs_grid(gk, kKBlock), blk(kThreads);
  const long long* cs = colsum;
#define SAGE_QUANT(DD)                                                                                          \
  do {                                                                                                         \
    hipLaunchKernelGGL((k_colsum_kernel<DD>), hs_grid(gk, kColsumChunk), blk, 0, st, k16, gk,                  \
                       reinterpret_cast<unsigned long long*>(colsum));                                         \
    if (q_mean)                                                                                                \
      hipLaunchKernelGGL((quant_block_kernel<DD, kQBlock, kShiftBlock>), gqb, blk, 0, st, q16, gq,             \
                         (const long long*)nullptr, sm_scale, q_int8, q_scale, q_mean);                        \
    else if (q_per_token && q_int8)                                                                            \
      hipLaunchKernelGGL((quant_row_kernel<DD, kRowsPerBlock>), hs_grid(gq, kRowsPerBlock), blk, 0, st, q16,   \
                         gq, sm_scale, q_int8, q_scale);                                                       \
    else if (!q_per_token && q_int8)                                                                           \
      hipLaunchKernelGGL((quant_block_kernel<DD, kQBlock, kShiftNone>), gqb, blk, 0, st, q16, gq,              \
                         (const long long*)nullptr, sm_scale, q_int8, q_scale, (float*)nullptr);               \
    hipLaunchKernelGGL((quant_block_kernel<DD, kKBlock, kShiftKMean>), gkb, blk, 0, st, k16, gk, cs, 1.0f,     \
                       k_int8, k_scale, k_mean);                                                               \
  } while (0)
  if (gq.d == 128)
    SAGE_QUANT(128);
  else
    SAGE_QUANT(64);
#undef SAGE_QUANT
}

void launch_mx_prepare(const SeqGeom& gq, const SeqGeom& gk, const void* q, const void* k, const void* v,
                       uint8_t* q_codes, uint8_t* q_scales, uint8_t* k_codes, uint8_t* aux, uint8_t* v_codes,
                       float* k_mean, float* q_mean, long long* colsum, hipStream_t st) {
  const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q);
  const uint16_t* k16 = reinterpret_cast<const uint16_t*>(k);
  const uint16_t* v16 = reinterpret_cast<const uint16_t*>(v);
  launch_zero(colsum, sizeof(long long) * (size_t)gk.B * gk.H * gk.d, st);
  const dim3 blk(kThreads);
#define SAGE_MXPREP(DD)                                                                                         \
  do {                                                                                                         \
    hipLaunchKernelGGL((k_colsum_kernel<DD>), hs_grid(gk, kColsumChunk), blk, 0, st, k16, gk,                  \
                       reinterpret_cast<unsigned long long*>(colsum));                                         \
    if (q_mean)                                                                                                \
      hipLaunchKernelGGL((mx_rows_kernel<DD, kQBlock, kShiftBlock>), hs_grid(gq, kQBlock), blk, 0, st, q16,     \
                         gq, (const long long*)nullptr, q_codes, q_scales, (uint8_t*)nullptr, q_mean);         \
    else                                                                                                       \
      hipLaunchKernelGGL((mx_rows_kernel<DD, kRowsPerBlock, kShiftNone>), hs_grid(gq, kRowsPerBlock), blk, 0,  \
                         st, q16, gq, (const long long*)nullptr, q_codes, q_scales, (uint8_t*)nullptr,         \
                         (float*)nullptr);                                                                     \
    hipLaunchKernelGGL((mx_rows_kernel<DD, kRowsPerBlock, kShiftKMean>), hs_grid(gk, kRowsPerBlock), blk, 0,   \
                       st, k16, gk, (const long long*)colsum, k_codes, (uint8_t*)nullptr, aux, k_mean);        \
    hipLaunchKernelGGL((mx_v_prepare_kernel<DD>), hs_grid(gk, kKBlock), blk, 0, st, v16, gk, v_codes, aux);     \
  } while (0)
  if (gq.d == 128)
    SAGE_MXPREP(128);
  else
    SAGE_MXPREP(64);
#undef SAGE_MXPREP
}

void launch_v_scale(const SeqGeom& g, const void* v, float* v_scale, hipStream_t st) {
  const uint16_t* v16 = reinterpret_cast<const uint16_t*>(v);
  const int64_t count = (int64_t)g.B * g.H * g.d;
  launch_zero(v_scale, sizeof(float) * (size_t)count, st);  // count is a multiple of 64
  if (g.d == 128)
    hipLaunchKernelGGL((v_absmax_kernel<128>), hs_grid(g, kColsumChunk), dim3(kThreads), 0, st, v16, g,
                       reinterpret_cast<unsigned*>(v_scale));
  else
    hipLaunchKernelGGL((v_absmax_kernel<64>), hs_grid(g, kColsumChunk), dim3(kThreads), 0, st, v16, g,
                       reinterpret_cast<unsigned*>(v_scale));
  hipLaunchKernelGGL(v_scale_finalize_kernel, dim3((unsigned)ceil_div64(count, 256)), dim3(256), 0, st, v_scale,
                     count);
}

void launch_v_prepare(const SeqGeom& g, const void* v, const float* v_scale, bool fp8, bool rowmajor,
                      void* out, hipStream_t st) {
  const uint16_t* v16 = reinterpret_cast<const uint16_t*>(v);
  uint8_t* o = reinterpret_cast<uint8_t*>(out);
  const dim3 grid = hs_grid(g, kKBlock);
#define SAGE_VPREP(DD, F8, RM) \
  hipLaunchKernelGGL((v_prepare_kernel<DD, F8, RM>), grid, dim3(kThreads), 0, st, v16, g, v_scale, o)
  if (g.d == 128) {
    if (!fp8) SAGE_VPREP(128, false, false);
    else if (!rowmajor) SAGE_VPREP(128, true, false);
    else SAGE_VPREP(128, true, true);
  } else {
    if (!fp8) SAGE_VPREP(64, false, false);
    else if (!rowmajor) SAGE_VPREP(64, true, false);
    else SAGE_VPREP(64, true, true);
  }
#undef SAGE_VPREP
}

}  // namespace sage
