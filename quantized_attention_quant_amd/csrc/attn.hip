// Fused 8-bit attention forward for gfx950.
//
// Method (pages by title):
//   * S = int32(Q̂K̂ᵀ)·δQ·δK — "⚡️SageAttention — brand new attention"
//     (postsniper.ru), quantisation introduction step 3 (C ≈ (ÂB̂)(δAδB)) and
//     SageAttention bullets (QKᵀ in INT8, scaling fused with neighbours);
//   * tiling, one fused kernel, online softmax — intelliparadigm
//     "Attention机制优化：从FlashAttention到SageAttention的工程实践", §3.1;
//   * PV in FP16 (postsniper, SageAttention bullets) or P and V in FP8 with
//     two-level accumulation (dtcms.com SageAttention summary, section
//     "SageAttention 2"; postsniper, SageAttention2 bullets);
//   * causal mask (deepseek.csdn.net post: sageattn with is_causal=True).
//
// Design (CDNA4, 64-lane waves):
//   * One workgroup = 4 waves = 128 queries = one Q scale block; each wave owns
//     32 queries.  Keys are walked in 64-key tiles (= one K scale block), so
//     every tile pair has a single scalar δQ·δK.
//   * Sᵀ = K̂·Q̂ᵀ on v_mfma_i32_32x32x32_i8: A = K̂ tile from LDS, B = the
//     wave's Q̂ held in VGPRs.  The 32x32 output puts one query per lane
//     (lanes l and l+32 share query l%32, each holding 16 of every 32 keys),
//     so row max/sum are in-lane plus one xor-32 exchange, and the running
//     output rescale α is a per-lane scalar.
//   * The int32 accumulator starts at the bit pattern of 1.5·2^23: since
//     |Q̂K̂ᵀ| <= 128·127² < 2^22, the result read as fp32 is exactly
//     1.5·2^23 + acc, so dequantisation is one FMA per score:
//     s·log2e - m = fma(F, c, -(1.5·2^23·c + m)) with c = δQ·δK·log2e.
//   * PV as Oᵀ = Vᵀ·Pᵀ: the softmax output in the S layout is directly the B
//     operand; V comes pre-packed (pre-pass) in A-operand order, so LDS reads
//     are contiguous 16/32-byte lane vectors.  FP16: v_mfma_f32_32x32x16_f16.
//     FP8: v_mfma_f32_32x32x64_f8f6f4 contracts exactly one 64-key tile.
//   * K̂ and V tiles are double-buffered in LDS with one barrier per tile; the
//     K̂ rows use an XOR swizzle of their 16-byte chunks so that the 8 lanes
//     served together read 8 distinct bank groups.
//   * Workgroup ids are remapped so that one XCD runs consecutive q-blocks of
//     the same head (K̂/V reuse in that XCD's L2); heavier causal blocks go
//     first.
#include "sage_common.h"
#include "sage_internal.h"

namespace sage {

constexpr float kMagicF = 12582912.0f;  // 1.5 * 2^23
constexpr int kMagicI = 0x4B400000;     // its fp32 bit pattern
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2E4M3Max = 8.807354922057604f;  // log2(448)

// 16-byte chunk index of K̂ tile row r, chunk c inside LDS (XOR swizzle).
template <int D>
__device__ __forceinline__ int k_lds_chunk(int r, int c) {
  constexpr int CPR = D / 16;              // chunks per row: 8 (d=128) or 4 (d=64)
  constexpr int RSH = (CPR == 8) ? 0 : 1;  // rows sharing a 128-byte bank line
  return r * CPR + (c ^ ((r >> RSH) & (CPR - 1)));
}

template <int D>
struct KTileRegs {
  static constexpr int N = kKBlock * D / 16 / kThreads;  // 16-byte chunks per thread
  v4i r[N];
};

template <int D, bool FP8>
struct VTileRegs {
  static constexpr int BYTES = kKBlock * D * (FP8 ? 1 : 2);
  static constexpr int N = BYTES / 16 / kThreads;
  v4i r[N];
};

// Global -> registers for K̂ rows [k0, k0+64) of a head-sequence (zeros past n).
template <int D>
__device__ __forceinline__ void load_k_tile(KTileRegs<D>& kr, const int8_t* __restrict__ kbase, int k0, int n) {
  constexpr int CPR = D / 16;
#pragma unroll
  for (int i = 0; i < KTileRegs<D>::N; ++i) {
    const int idx = threadIdx.x + kThreads * i;
    const int r = idx / CPR, c = idx % CPR;
    kr.r[i] = (k0 + r < n) ? *reinterpret_cast<const v4i*>(kbase + (int64_t)(k0 + r) * D + c * 16)
                           : v4i{0, 0, 0, 0};
  }
}
template <int D>
__device__ __forceinline__ void store_k_tile(const KTileRegs<D>& kr, v4i* __restrict__ lds) {
  constexpr int CPR = D / 16;
#pragma unroll
  for (int i = 0; i < KTileRegs<D>::N; ++i) {
    const int idx = threadIdx.x + kThreads * i;
    lds[k_lds_chunk<D>(idx / CPR, idx % CPR)] = kr.r[i];
  }
}
template <int D, bool FP8>
__device__ __forceinline__ void load_v_tile(VTileRegs<D, FP8>& vr, const uint8_t* __restrict__ tile) {
#pragma unroll
  for (int i = 0; i < VTileRegs<D, FP8>::N; ++i)
    vr.r[i] = *reinterpret_cast<const v4i*>(tile + (int64_t)(threadIdx.x + kThreads * i) * 16);
}
template <int D, bool FP8>
__device__ __forceinline__ void store_v_tile(const VTileRegs<D, FP8>& vr, v4i* __restrict__ lds) {
#pragma unroll
  for (int i = 0; i < VTileRegs<D, FP8>::N; ++i) lds[threadIdx.x + kThreads * i] = vr.r[i];
}

// The wave's Q̂ as the B operand of Sᵀ = K̂Q̂ᵀ: lane holds query r32, channels
// 32ks + 16g .. +15 for each 32-channel step ks (zeros for rows past n).
template <int D>
__device__ __forceinline__ void load_q_frags(v4i (&qf)[D / 32], const int8_t* __restrict__ qbase, int qrow, int n,
                                             int g) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qf[ks] = (qrow < n) ? *reinterpret_cast<const v4i*>(qbase + (int64_t)qrow * D + 32 * ks + 16 * g)
                        : v4i{0, 0, 0, 0};
}

// Sᵀ for one 64-key tile: S[s] covers keys 32s..32s+31; lane (r32, g) reg i
// holds key 32s + 8(i/4) + 4g + i%4 of query r32, as magic + Σ q̂·k̂.
template <int D>
__device__ __forceinline__ void qk_tile(const v4i* __restrict__ lds_k, const v4i (&qf)[D / 32], v16i (&S)[2],
                                        int r32, int g) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    v16i acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = kMagicI;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const v4i a = lds_k[k_lds_chunk<D>(32 * s + r32, 2 * ks + g)];
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[ks], acc, 0, 0, 0);
    }
    S[s] = acc;
  }
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); }

template <int D, bool FP8, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int DT = D / 32;  // 32-wide d tiles of the output
  using VR = VTileRegs<D, FP8>;
  __shared__ v4i lds_k[2][kKBlock * D / 16];
  __shared__ v4i lds_v[2][VR::BYTES / 16];

  const SeqGeom& g = a.g;
  const int nqb = ceil_div(g.N, kQBlock);
  const int nkb = ceil_div(g.N, kKBlock);
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = nqb - 1 - logical % nqb;  // heavy (late) causal blocks first
  const int hb = logical / nqb;
  const int h = hb / g.B, b = hb % g.B;
  int64_t row0;
  int n;
  hs_rows(g, b, h, row0, n);
  const int q0 = qb * kQBlock;
  if (q0 >= n) return;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r32 = lane & 31, gg = lane >> 5;
  const int64_t hs = (int64_t)b * g.H + h;
  const int qrow = q0 + 32 * w + r32;
  const int wq_lo = q0 + 32 * w;
  const int wq_hi = min(wq_lo + 31, n - 1);
  const bool wave_rows = wq_lo < n;

  v4i qf[DT];
  load_q_frags<D>(qf, a.q + row0 * D, qrow, n, gg);
  const float dq = a.q_scale[hs * nqb + qb];
  const float* __restrict__ ksc = a.k_scale + hs * nkb;
  const int8_t* __restrict__ kbase = a.k + row0 * D;
  const uint8_t* __restrict__ vbase = a.v_packed + vtile_index(g, b, h, 0) * VR::BYTES;

  const int kend = CAUSAL ? min(n, q0 + kQBlock) : n;
  const int ntiles = ceil_div(kend, kKBlock);

  float m_run = -__builtin_inff();
  float l_run = 0.f;
  v16f O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[dt][i] = 0.f;

  {
    KTileRegs<D> kr;
    VR vr;
    load_k_tile<D>(kr, kbase, 0, n);
    load_v_tile<D, FP8>(vr, vbase);
    store_k_tile<D>(kr, lds_k[0]);
    store_v_tile<D, FP8>(vr, lds_v[0]);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool next = t + 1 < ntiles;
    KTileRegs<D> kr;
    VR vr;
    if (next) {
      load_k_tile<D>(kr, kbase, (t + 1) * kKBlock, n);
      load_v_tile<D, FP8>(vr, vbase + (int64_t)(t + 1) * VR::BYTES);
    }
    const int k0 = t * kKBlock;
    if (wave_rows && (!CAUSAL || k0 <= wq_hi)) {
      v16i S[2];
      qk_tile<D>(lds_k[buf], qf, S, r32, gg);
      const float c2 = dq * ksc[t] * kLog2e;
      const bool full = (k0 + kKBlock <= n) && (!CAUSAL || k0 + kKBlock - 1 <= wq_lo);
      float F[2][16];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // read the element by value first: a bit cast of an ext-vector element lvalue
          // compiles to a read of element 0
          const int bits = S[s][i];
          F[s][i] = __int_as_float(bits);
        }
      if (!full) {
        // masked scores -> 0.0f, below every real value (>= 2^23)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * s + 8 * (i >> 2) + 4 * gg + (i & 3);
            const bool vis = key < n && (!CAUSAL || key <= qrow);
            F[s][i] = vis ? F[s][i] : 0.f;
          }
      }
      float mx = 0.f;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = max3f(mx, F[s][i], F[s][i + 1]);
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
      const float m_tile = (mx == 0.f) ? -__builtin_inff() : (mx - kMagicF) * c2;
      float m_new = __builtin_fmaxf(m_run, m_tile);
      m_new = (m_new == -__builtin_inff()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      // FP16 PV: one FMA per score, p = 2^(F·c - K) with K = fl(1.5·2^23·c + m).  The
      // rounding of K shifts a whole row-tile by <= ulp(K)/2 in the exponent (a common
      // factor on that tile's p and its share of l); fp16 P rounding is relative, so its
      // codes do not depend on it.
      // FP8 PV: the e4m3 codes of 448·p must follow the running max itself, so the
      // exponent is taken from the exact difference F - max (both in [2^23, 2^24)):
      // p·448 = 2^((F - mx)·c + (m_tile - m) + log2 448).
      const float kb = __builtin_fmaf(kMagicF, c2, m_new);
      const float cterm = (m_tile - m_new) + kLog2E4M3Max;
      float P[2][16];
      float lsum = 0.f;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float arg = FP8 ? __builtin_fmaf(F[s][i] - mx, c2, cterm) : __builtin_fmaf(F[s][i], c2, -kb);
          float p = __builtin_amdgcn_exp2f(arg);
          if (!full) p = (F[s][i] == 0.f) ? 0.f : p;
          P[s][i] = p;
          lsum += p;
        }
      l_run = alpha * l_run + lsum;
      m_run = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[dt][i] *= alpha;
      }
      if (!FP8) {
        const v8h* __restrict__ lv = reinterpret_cast<const v8h*>(lds_v[buf]);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const int s = kc >> 1, hh = kc & 1;
          v8h pk;
#pragma unroll
          for (int j = 0; j < 8; ++j) pk[j] = (_Float16)P[s][8 * hh + j];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(lv[(kc * DT + dt) * 64 + lane], pk, O[dt], 0, 0, 0);
        }
      } else {
        // p·448 <= 448·2^(1e-5) < 464, so the conversion cannot overflow e4m3.
        v8i pk;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int s = q >> 2, i0 = 4 * (q & 3);
          int wv = __builtin_amdgcn_cvt_pk_fp8_f32(P[s][i0], P[s][i0 + 1], 0, false);
          wv = __builtin_amdgcn_cvt_pk_fp8_f32(P[s][i0 + 2], P[s][i0 + 3], wv, true);
          pk[q] = wv;
        }
        const v8i* __restrict__ lv = reinterpret_cast<const v8i*>(lds_v[buf]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          O[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(lv[dt * 64 + lane], pk, O[dt], 0, 0, 0, 0, 0, 0);
      }
    }
    if (next) {
      store_k_tile<D>(kr, lds_k[buf ^ 1]);
      store_v_tile<D, FP8>(vr, lds_v[buf ^ 1]);
    }
    __syncthreads();
  }

  // Epilogue: o = O / l (FP16) or O·δV / l with l holding 448·Σp (FP8).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!wave_rows || qrow >= n) return;
  const float inv = 1.f / l_tot;
  uint16_t* __restrict__ orow = a.o + (row0 + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * dt + 8 * q4 + 4 * gg;
      float f[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) f[j] = O[dt][4 * q4 + j] * inv;
      if (FP8) {
        const float4 vs = *reinterpret_cast<const float4*>(a.v_scale + hs * D + d);
        f[0] *= vs.x;
        f[1] *= vs.y;
        f[2] *= vs.z;
        f[3] *= vs.w;
      }
      v2h lo = {(_Float16)f[0], (_Float16)f[1]};
      v2h hi = {(_Float16)f[2], (_Float16)f[3]};
      uint2 st;
      st.x = __builtin_bit_cast(uint32_t, lo);
      st.y = __builtin_bit_cast(uint32_t, hi);
      *reinterpret_cast<uint2*>(orow + d) = st;
    }
}

// Test hook: the int32 Q̂K̂ᵀ tiles computed by the same device code as above.
template <int D>
__global__ __launch_bounds__(kThreads) void qk_tiles_kernel(const int8_t* __restrict__ q, const int8_t* __restrict__ k,
                                                            int B, int H, int N, const int32_t* __restrict__ list,
                                                            int32_t* __restrict__ out) {
  __shared__ v4i lds_k[kKBlock * D / 16];
  const int idx = blockIdx.x;
  const int b = list[4 * idx], h = list[4 * idx + 1], qb = list[4 * idx + 2], kb = list[4 * idx + 3];
  int32_t* o = out + (int64_t)idx * kQBlock * kKBlock;
  if (b < 0 || b >= B || h < 0 || h >= H || qb < 0 || qb * kQBlock >= N || kb < 0 || kb * kKBlock >= N) {
    for (int i = threadIdx.x; i < kQBlock * kKBlock; i += kThreads) o[i] = 0;  // out-of-range entry
    return;
  }
  const int64_t row0 = ((int64_t)b * H + h) * N;
  KTileRegs<D> kr;
  load_k_tile<D>(kr, k + row0 * D, kb * kKBlock, N);
  store_k_tile<D>(kr, lds_k);
  __syncthreads();
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r32 = lane & 31, gg = lane >> 5;
  v4i qf[D / 32];
  load_q_frags<D>(qf, q + row0 * D, qb * kQBlock + 32 * w + r32, N, gg);
  v16i S[2];
  qk_tile<D>(lds_k, qf, S, r32, gg);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 32 * s + 8 * (i >> 2) + 4 * gg + (i & 3);
      o[(32 * w + r32) * kKBlock + key] = S[s][i] - kMagicI;
    }
}

void launch_attn(const AttnArgs& a, bool causal, bool fp8, hipStream_t st) {
  const int64_t blocks = (int64_t)a.g.B * a.g.H * ceil_div(a.g.N, kQBlock);
  const dim3 grid((unsigned)blocks), block(kThreads);
#define SAGE_ATTN(DD, F8, CS) hipLaunchKernelGGL((attn_fwd_kernel<DD, F8, CS>), grid, block, 0, st, a)
  if (a.g.d == 128) {
    if (!fp8) { if (causal) SAGE_ATTN(128, false, true); else SAGE_ATTN(128, false, false); }
    else { if (causal) SAGE_ATTN(128, true, true); else SAGE_ATTN(128, true, false); }
  } else {
    if (!fp8) { if (causal) SAGE_ATTN(64, false, true); else SAGE_ATTN(64, false, false); }
    else { if (causal) SAGE_ATTN(64, true, true); else SAGE_ATTN(64, true, false); }
  }
#undef SAGE_ATTN
}

void launch_qk_tiles(const int8_t* q, const int8_t* k, int B, int H, int N, int d, const int32_t* list, int n,
                     int32_t* out, hipStream_t st) {
  if (d == 128)
    hipLaunchKernelGGL((qk_tiles_kernel<128>), dim3(n), dim3(kThreads), 0, st, q, k, B, H, N, list, out);
  else
    hipLaunchKernelGGL((qk_tiles_kernel<64>), dim3(n), dim3(kThreads), 0, st, q, k, B, H, N, list, out);
}

}  // namespace sage
