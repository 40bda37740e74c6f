// Q smoothing, second half: the score term that the smoothed Q̂ leaves out.
//
// Pages (by title): dtcms.com SageAttention summary, section "SageAttention 2"
// (Q is smoothed as well, for a more accurate QKᵀ); "⚡️SageAttention — brand
// new attention" (postsniper.ru), SageAttention2 bullets (Q normalised too, so
// that the attention result is not distorted).  Q's block mean q̄ is taken out
// before the INT8 step (quant.hip); every score of a row of Q block b then
// lacks
//
//     Δ[b][j] = sm_scale · q̄_b · x_j,    x_j = fp32(k_j) − km,
//
// which this kernel forms for every (Q block, key) of a head-sequence and
// hands to the attention kernel in the form it consumes:
//
//   slots[hs][b][j] (int32): the initial value of the Q̂K̂ᵀ accumulator for
//     key j in rows of block b: the magic bias 1.5·2^23 plus rint(Δ·log2e / c)
//     with c = δQ_b·δK_t·log2e, i.e. Δ counted in units of the tile's
//     dequantisation step.  The accumulator read as fp32 stays exact while
//     |Q̂K̂ᵀ + that integer| < 2^22, so the integer must stay within
//     2^22 − 1 − 127²·d; a 32-key half tile where any key misses that range,
//     or whose c is not a normal float (δQ = 0 for a constant block), gets the
//     bias alone and
//   flags[hs][b][2t + s] = 1 (half s of tile t), with fix[hs][b][j] = Δ·log2e
//     (fp32) for its keys: the attention kernel then adds Δ in fp32.  any[hs][b]
//     (cleared before the launch) becomes nonzero when some half of block b
//     falls back, so the attention kernel reads the flags of that row only.
//
// raw (MXFP4 and FP8 PV): the term is used in fp32, with no integer form:
// slots[hs][b][j] holds q̄_b · x_j · sm_log2e (fp32 bits) for every key, and no
// flags are written.  MXFP4 passes sm_log2e = 1 (raw score units: its kernel
// applies the softmax scale to the whole score); FP8 PV passes the softmax
// scale times log2(e), so the value is the term in the kernel's log2 units.
//
// The contraction q̄_b · x_j runs on the fp16 MFMA.  Both operands are scaled
// by powers of two into [-1, 1] (q̄_b by 2^-eq_b from its largest channel, x_j
// by 2^-ek_t from its K block's scale, or in raw mode from its wave's largest
// |x|) and split into fp16 hi + lo parts (about 22 significant bits each);
// hi·hi + hi·lo + lo·hi, plus lo·lo in raw mode, with fp32 accumulation —
// far below the INT8 quantisation error of the scores, and in raw mode close
// to an fp32 evaluation.
#include "sage_common.h"
#include "sage_internal.h"

namespace sage {

constexpr int kMagicBias = 0x4B400000;  // fp32 bits of 1.5 * 2^23
constexpr float kLog2eF = 1.4426950408889634f;
constexpr int kQbBlocksPerGroup = 32;   // Q blocks per MFMA column group

// LDS layout of a group's B operand, in 16-byte chunks: run (kstep, hi/lo) at
// kBRun·(2·kstep + hi/lo), the lanes of column half cg at kBHalf·cg + block.
// The 16 lanes of one write (8 channel parts x 2 blocks) then land on 16
// distinct bank groups at d = 64 and d = 128 (a stride of 64 chunks put them
// all on one), and each read stays 16 consecutive chunks per 16 lanes.
constexpr int kBRun = 73;
constexpr int kBHalf = 40;

template <int D>
constexpr int kSlotLimit = (1 << 22) - 1 - 127 * 127 * D;

__device__ __forceinline__ v8h split_hi(const float (&x)[8]) {
  v8h h;
#pragma unroll
  for (int j = 0; j < 8; ++j) h[j] = (_Float16)x[j];
  return h;
}
__device__ __forceinline__ v8h split_lo(const float (&x)[8], const v8h& hi) {
  v8h l;
#pragma unroll
  for (int j = 0; j < 8; ++j) l[j] = (_Float16)(x[j] - (float)hi[j]);
  return l;
}

// Power-of-two exponent e with 2^e > v >= 0 (e = 0 for v = 0).
__device__ __forceinline__ int pow2_above(float v) {
  int e = 0;
  (void)frexpf(v, &e);
  return v > 0.f ? e : 0;
}

// Grid (ceil(Nmax/128), H, B), 4 waves.  Wave w handles keys
// 128·blockIdx.x + 32w .. +31 of head-sequence (b, h): half w%2 of tile
// 2·blockIdx.x + w/2, against every Q block of the head-sequence, 32 blocks
// (one MFMA column group) at a time.
template <int D>
__global__ __launch_bounds__(kThreads) void q_bias_kernel(QBiasArgs a) {
  constexpr int KS = D / 16;   // 16-channel MFMA steps
  constexpr int CPT = D / 8;   // q̄ channels per thread when building a group
  const SeqGeom& g = a.g;
  const int b = blockIdx.z, h = blockIdx.y;
  int64_t row0;
  int n;
  hs_rows(g, b, h, row0, n);
  if (128 * (int)blockIdx.x >= n) return;  // uniform over the workgroup
  const int nqb = ceil_div(g.N, kQBlock), nkb = ceil_div(g.N, kKBlock);
  const int npad = nkb * kKBlock;
  const int nqb_seq = ceil_div(n, kQBlock);
  const int hk = h / a.kv_group;
  SeqGeom gk = g;
  gk.H = g.H / a.kv_group;
  int64_t krow0;
  int kn;
  hs_rows(gk, b, hk, krow0, kn);
  const int64_t hs = (int64_t)b * g.H + h, hsk = (int64_t)b * gk.H + hk;

  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, gg = lane >> 5;
  const int w = tid >> 6;
  const int kw0 = 128 * blockIdx.x + 32 * w;  // first key of this wave
  const int t = kw0 / kKBlock, s = (kw0 / 32) & 1;
  // every half of every tile with a key below n is written (a half past n
  // still gets its flag: the attention kernel reads both halves of a tile)
  const bool wave_live = kKBlock * t < n;

  __shared__ float km_s[D];
  __shared__ v8h bfrag[KS * 2 * kBRun];  // B operand of one group: (kstep, hi/lo, lane)
  __shared__ int eq_s[kQbBlocksPerGroup];
  if (tid < D) km_s[tid] = a.k_mean[hsk * D + tid];
  __syncthreads();

  // A operand: x_j / 2^ek as fp16 hi/lo; lane holds key kw0 + r32, channels
  // 16·kk + 8·gg .. +7 (zeros past n).  2^ek > max|x|: from the K block's
  // INT8 scale (128·δK), or in raw mode from this wave's own keys.
  const int key = kw0 + r32;
  float xs[KS][8];
  {
    v4i raw[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      raw[kk] = (key < n) ? *reinterpret_cast<const v4i*>(a.k + (krow0 + key) * D + 16 * kk + 8 * gg)
                          : v4i{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t wd = (uint32_t)raw[kk][j];
        const int c = 16 * kk + 8 * gg + 2 * j;
        // the smoothed K exactly as the K quantiser forms it
        xs[kk][2 * j] = (key < n) ? (float)__builtin_bit_cast(_Float16, (uint16_t)(wd & 0xffffu)) - km_s[c] : 0.f;
        xs[kk][2 * j + 1] = (key < n) ? (float)__builtin_bit_cast(_Float16, (uint16_t)(wd >> 16)) - km_s[c + 1] : 0.f;
      }
  }
  float dk = 0.f;
  int ek;
  if (a.raw) {
    float mx = 0.f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(xs[kk][j]));
    ek = pow2_above(wave_max(mx));
  } else {
    dk = wave_live ? a.k_scale[hsk * nkb + t] : 0.f;
    ek = pow2_above(128.f * dk);  // 128·δK > max|x| of the K block
  }
  const float kscale = ldexpf(1.f, -ek);
  v8h ahi[KS], alo[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = xs[kk][j] * kscale;
    ahi[kk] = split_hi(x);
    alo[kk] = split_lo(x, ahi[kk]);
  }

  const int ngroups = ceil_div(nqb_seq, kQbBlocksPerGroup);
  for (int grp = 0; grp < ngroups; ++grp) {
    // --- B operand of 32 Q blocks: q̄_b / 2^eq_b as fp16 hi/lo in LDS
    {
      const int bl = tid >> 3, part = tid & 7;
      const int bb = grp * kQbBlocksPerGroup + bl;
      float qv[CPT];
      const float* src = a.q_mean + (hs * nqb + bb) * D + CPT * part;
#pragma unroll
      for (int c = 0; c < CPT; c += 4) {
        const float4 f = (bb < nqb_seq) ? *reinterpret_cast<const float4*>(src + c) : float4{0.f, 0.f, 0.f, 0.f};
        qv[c] = f.x;
        qv[c + 1] = f.y;
        qv[c + 2] = f.z;
        qv[c + 3] = f.w;
      }
      float mx = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) mx = fmaxf(mx, fabsf(qv[c]));
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      mx = fmaxf(mx, __shfl_xor(mx, 4));
      const int eq = pow2_above(mx);
      const float qscale = ldexpf(1.f, -eq);
      if (part == 0) eq_s[bl] = eq;
#pragma unroll
      for (int m = 0; m < CPT / 8; ++m) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = qv[8 * m + j] * qscale;
        const int c = CPT * part + 8 * m;
        const int kk = c / 16, cg = (c % 16) / 8;
        const v8h hi = split_hi(x);
        bfrag[(2 * kk) * kBRun + kBHalf * cg + bl] = hi;
        bfrag[(2 * kk + 1) * kBRun + kBHalf * cg + bl] = split_lo(x, hi);
      }
    }
    __syncthreads();
    if (wave_live) {
      v16f acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int bl = kBHalf * gg + r32;
        const v8h bhi = bfrag[(2 * kk) * kBRun + bl], blo = bfrag[(2 * kk + 1) * kBRun + bl];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[kk], bhi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[kk], blo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[kk], bhi, acc, 0, 0, 0);
        // fp32 terms (FP8 P codes, MXFP4 scores) keep the lo·lo part as well
        if (a.raw) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[kk], blo, acc, 0, 0, 0);
      }
      // lane holds Q block bb = 32·grp + r32 for keys kw0 + 8(i/4) + 4gg + i%4
      const int bb = grp * kQbBlocksPerGroup + r32;
      const bool blk_live = bb < nqb_seq && !(a.causal && kKBlock * t > kQBlock * bb + kQBlock - 1);
      const float f = ldexpf(a.sm_log2e, eq_s[r32] + ek);
      if (a.raw) {
        // q̄·x·sm_log2e, every key, no flags
        if (blk_live) {
          const int64_t rowoff = (hs * nqb + bb) * (int64_t)npad;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int key0 = kw0 + 8 * q4 + 4 * gg;
            float4 vv;
            vv.x = acc[4 * q4] * f;
            vv.y = acc[4 * q4 + 1] * f;
            vv.z = acc[4 * q4 + 2] * f;
            vv.w = acc[4 * q4 + 3] * f;
            *reinterpret_cast<float4*>(a.slots + rowoff + key0) = vv;
          }
        }
      } else {
        const float dq = bb < nqb_seq ? a.q_scale[hs * nqb + bb] : 0.f;
        const float c2 = dq * dk * kLog2eF;  // the attention kernel's per-tile factor
        const float inv = 1.f / c2;
        float dl[16];
        bool fits = c2 >= 1.17549435e-38f && c2 <= 3.0e38f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          dl[i] = acc[i] * f;
          const int key = kw0 + 8 * (i >> 2) + 4 * gg + (i & 3);
          fits = fits && (key >= n || __builtin_fabsf(dl[i] * inv) <= (float)kSlotLimit<D>);
        }
        // both lanes of the block (gg = 0, 1) hold half of the 32 keys
        const int other = __shfl_xor((int)fits, 32);
        fits = fits && other;
        if (blk_live) {
          const int64_t rowoff = (hs * nqb + bb) * (int64_t)npad;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int key0 = kw0 + 8 * q4 + 4 * gg;
            int sv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = 4 * q4 + j;
              sv[j] = (fits && key0 + j < n) ? kMagicBias + (int)__builtin_rintf(dl[i] * inv) : kMagicBias;
            }
            *reinterpret_cast<v4i*>(a.slots + rowoff + key0) = v4i{sv[0], sv[1], sv[2], sv[3]};
            if (!fits)
              *reinterpret_cast<float4*>(a.fix + rowoff + key0) =
                  float4{dl[4 * q4], dl[4 * q4 + 1], dl[4 * q4 + 2], dl[4 * q4 + 3]};
          }
          if (gg == 0) {
            a.flags[(hs * nqb + bb) * (int64_t)(2 * nkb) + 2 * t + s] = fits ? 0 : 1;
            if (!fits) atomicOr(a.any + hs * nqb + bb, 1);  // the row's summary (rare)
          }
        }
      }
    }
    __syncthreads();  // the next group overwrites the B operand
  }
}

void launch_q_bias(const QBiasArgs& a, hipStream_t st) {
  const dim3 grid(ceil_div(a.g.N, 128), a.g.H, a.g.B), block(kThreads);
  if (a.g.d == 128)
    hipLaunchKernelGGL((q_bias_kernel<128>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((q_bias_kernel<64>), grid, block, 0, st, a);
}

}  // namespace sage
