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
//   * One workgroup = 8 waves = 256 queries (two Q scale blocks), each wave
//     owning 32 queries; two waves per SIMD, so one wave's MFMAs run while the
//     other's softmax occupies the VALU.  Keys are walked in 64-key tiles
//     (= one K scale block), so every tile and Q block pair has one scalar
//     δQ·δK.  Every K̂/V tile streamed into LDS serves 256 queries.
//   * Sᵀ = K̂·Q̂ᵀ on v_mfma_i32_32x32x32_i8: A = K̂ tile from LDS, B = the
//     wave's Q̂ held in VGPRs.  The 32x32 output puts one query per lane
//     (lanes l and l+32 share query l%32, each holding 16 of every 32 keys),
//     so row max/sum are in-lane plus one xor-32 exchange, and the running
//     output rescale α is a per-lane scalar.
//   * The int32 accumulator starts at the bit pattern of 1.5·2^23: since
//     |Q̂K̂ᵀ| <= 128·127² < 2^22, the result read as fp32 is exactly
//     1.5·2^23 + acc, so no int->float conversion is needed.
//   * PV as Oᵀ = Vᵀ·Pᵀ: the softmax output in the S layout is directly the B
//     operand.  FP16: the input's V rows, read from LDS with the transposing
//     ds_read_b64_tr_b16 into v_mfma_f32_32x32x16_f16's A operand.  FP8: V
//     pre-packed (pre-pass) in A-operand order; v_mfma_f32_32x32x64_f8f6f4
//     contracts exactly one 64-key tile.
//   * K̂ and V tiles stream into a 4-stage LDS ring with buffer_load ... lds
//     (no staging registers; out-of-range K̂ rows read as zero through the
//     buffer descriptor's size).  Tile t+2 is requested while tile t is being
//     consumed, so each tile has two iterations to arrive; one barrier per tile.
//   * The K̂ rows in LDS use an XOR swizzle of their 16-byte chunks so that the
//     8 lanes served together read 8 distinct bank groups.
//   * Workgroup ids are remapped so that one XCD runs consecutive query blocks
//     of the same head (K̂/V reuse in that XCD's L2); heavier causal blocks go
//     first.
//   * Smoothed Q (dtcms summary, "SageAttention 2"; smooth_q.hip forms the
//     term): the part of each score that Q's block mean carries is streamed
//     into LDS with the tile.  FP16 PV: it enters as the accumulator's initial
//     value — magic bias plus that term in units of the tile's δQ·δK — so the
//     softmax does no extra work; half tiles whose term does not fit that
//     integer range add it in fp32 instead (rare: a flag per half tile).  FP8
//     PV: the softmax adds every key's term in fp32 (log2 units), since the P
//     codes follow the scores closely enough that a term rounded to one unit
//     of δQ·δK would move some of them.
#include "sage_common.h"
#include "sage_internal.h"

namespace sage {

constexpr float kMagicF = 12582912.0f;  // 1.5 * 2^23
constexpr int kMagicI = 0x4B400000;     // its fp32 bit pattern
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2E4M3Max = 8.807354922057604f;  // log2(448)
// FP16 PV: the exponent reference is only moved when a lane's row-tile sum of
// p exceeds kLazyLimit = 2^8, so p <= 2^8 and the output rescale is rare.
constexpr float kLazyLimit = 256.0f;
[[maybe_unused]] constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One LDS stage: K̂ tile, V tile (FP16 PV: the input's rows; FP8: packed e4m3) and, with a smoothed Q, the
// accumulator initial values of the tile's 64 keys for the workgroup's two Q
// blocks (four 256-byte quarters: quarter w holds block w/2, keys 32(w%2) ..
// +31 in its first 128 bytes).
template <int D, bool FP8, int NT = kThreads, bool SM = false>
struct TileGeom {
  static constexpr int KBYTES = kKBlock * D;                    // K̂ tile, int8
  static constexpr int VBYTES = kKBlock * D * (FP8 ? 1 : 2);    // V tile
  static constexpr int SBYTES = SM ? 1024 : 0;                  // accumulator initial values
  static constexpr int KCHUNKS = KBYTES / 16;
  static constexpr int VCHUNKS = VBYTES / 16;
  static constexpr int KI = KCHUNKS / NT;                       // DMA instructions per wave
  static constexpr int VI = VCHUNKS / NT;
  static constexpr int SI = SM ? 1 : 0;
  static constexpr int STAGE = KBYTES + VBYTES + SBYTES;
  static_assert(KI * NT == KCHUNKS && VI * NT == VCHUNKS, "tile must split evenly over the waves");
};

// Where a tile's accumulator initial values come from (smoothed Q only): the
// workgroup's first Q block's row of int32 values, `bytes` long (one or two
// rows of npad keys).
struct SlotSrc {
  const int32_t* base;
  int bytes;
  int npad;
};

// 16-byte chunk index of K̂ tile row r, chunk c inside LDS (XOR swizzle).  A
// 128-bit LDS read serves 16 lanes at a time from 64 banks x 4 bytes = 256
// bytes; the 16 lanes of a fragment read hold 16 consecutive rows at one chunk
// column, and 256/D rows share a 256-byte bank line.  XOR-ing the chunk with
// r / (256/D) gives the 16 lanes 16 distinct 16-byte bank groups.
template <int D>
struct KSwizzle {
  static constexpr int CPR = D / 16;               // chunks per row: 8 (d=128) or 4 (d=64)
  static constexpr int RSH = (D == 128) ? 1 : 2;   // log2 of rows per 256-byte bank line
  static __device__ __forceinline__ int chunk(int r, int c) { return c ^ ((r >> RSH) & (CPR - 1)); }
};

template <int D>
__device__ __forceinline__ int k_lds_chunk(int r, int c) {
  return r * KSwizzle<D>::CPR + KSwizzle<D>::chunk(r, c);
}

// FP16 PV reads V straight from the input's row-major rows ([key][d], 2D bytes
// per key).  In 16-key block kc the PV A operand needs, per lane l, channel
// 32dt + l%32 of keys 16kc + 4(l/32) + 0..3 and 16kc + 8 + 4(l/32) + 0..3 (the
// key order in which the Sᵀ accumulator hands P to the B operand).  gfx950's
// transposing LDS read (ds_read_b64_tr_b16) gathers four such keys: within
// each 16-lane group, lane 4q + c receives element c of the 8-byte chunks that
// lanes q, 4 + q, 8 + q, 12 + q address, in that order (probed on the
// hardware).  So lane (g = l/16, j = (l/4)%4, q = l%4) addresses key row
// 16kc + 8r + 4(g/2) + j (r = 0, 1: the two reads) at channels
// 32dt + 16(g%2) + 4q .. +3.  The hardware serves such a read 32 lanes at a
// time: four rows, 64 bytes of each.  The tile therefore sits in LDS as D/32
// column slabs [dt][key][32 channels] of 64-byte row segments, four segments
// to a 256-byte bank line: the four rows of one half-read cover all 64 banks
// once, and every fragment is the lane's one base plus a constant offset.
constexpr int kVSeg = 64;             // bytes of one key's 32 channels
constexpr int kVSlab = kKBlock * kVSeg;  // one 32-channel slab of a tile

typedef short v4s16 __attribute__((__vector_size__(8)));
typedef short v8s16 __attribute__((__vector_size__(16)));
typedef __attribute__((address_space(3))) v4s16* lds_v4s16_t;

// One PV A-operand fragment from the tile's V rows in LDS: p is this lane's
// address for the first four keys (the other four are 8 rows further on).
__device__ __forceinline__ v8h v_frag_tr(const char* __restrict__ p, int row_bytes) {
  const v4s16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16_t)p);
  const v4s16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16_t)(p + 8 * row_bytes));
  return __builtin_bit_cast(v8h, (v8s16)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// This lane's LDS byte offset inside a V tile's slab: key row 4(g/2) + j,
// channels 16(g%2) + 4q of the slab.
__device__ __forceinline__ int v_tr_base(int lane) {
  const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
  return (4 * (g >> 1) + j) * kVSeg + 32 * (g & 1) + 8 * q;
}

// Fragment (kc, dt): 16-key block kc, 32-channel step dt.
__device__ __forceinline__ v8h v_frag(const char* __restrict__ vstage, int base, int kc, int dt) {
  return v_frag_tr(vstage + base + dt * kVSlab + 16 * kc * kVSeg, kVSeg);
}

// FP8 PV: the pre-pass packs each d tile's A operands as 64 lanes x 32 bytes.
// In LDS the two 16-byte halves sit apart (bytes 0-15 of every lane, then
// bytes 16-31), so each 128-bit read covers 64 consecutive chunks: with the
// lanes 32 bytes apart, lanes i and i+8 of a 16-lane group would share banks.
__device__ __forceinline__ v8i v_frag_fp8(const char* __restrict__ vstage, int lane, int dt) {
  const v4i* p = reinterpret_cast<const v4i*>(vstage) + dt * 128 + lane;
  const v4i lo = p[0], hi = p[64];
  return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// Request K̂ tile t (rows 64t..64t+63 of the head-sequence, zeros past its end)
// and V tile t into one LDS stage.  kbase/kbytes bound the head-sequence's K̂
// rows; vbase/vbytes its fp16 V rows (FP16 PV, stored as 32-channel slabs) or
// packed e4m3 tiles (FP8); reads past them return zero.
// Lane i of a DMA instruction lands at the instruction's LDS base + 16·i, so
// each lane fetches the global chunk that belongs at its LDS position.
template <int D, bool FP8, int NT = kThreads, bool SM = false>
__device__ __forceinline__ void issue_tile(const void* kbase, int kbytes, const void* vbase, int vbytes, int t,
                                           char* stage, int w, int lane, const SlotSrc& ss = SlotSrc{}) {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer-descriptor type exists only for the GPU target
  using G = TileGeom<D, FP8, NT, SM>;
  constexpr int CPR = D / 16;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(kbase), (short)0, kbytes,
                                                                      kBufferFlags);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(vbase), (short)0, vbytes,
                                                                      kBufferFlags);
#pragma unroll
  for (int j = 0; j < G::KI; ++j) {
    const int base = (w * G::KI + j) * 64;  // wave-uniform chunk index
    const int p = base + lane;
    const int r = p / CPR;
    const int c = KSwizzle<D>::chunk(r, p % CPR);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(stage + base * 16), 16,
                                             (t * kKBlock + r) * D + c * 16, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < G::VI; ++j) {
    const int base = (w * G::VI + j) * 64;
    if (FP8) {
      // LDS chunk p: d tile p/128, half (p/64)%2 of lane p%64's operand
      const int p = base + lane;
      const int src = (p & ~127) + 2 * (p & 63) + ((p >> 6) & 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(stage + G::KBYTES + base * 16), 16,
                                               t * G::VBYTES + src * 16, 0, 0, 0);
    } else {
      // LDS chunk p: slab p/256, key (p/4)%64, 16-byte piece p%4 of its segment
      const int p = base + lane;
      const int r = (p >> 2) & (kKBlock - 1);
      const unsigned off = (unsigned)(t * kKBlock + r) * (2u * D) + (unsigned)((p >> 8) * kVSeg + 16 * (p & 3));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(stage + G::KBYTES + base * 16), 16, (int)off, 0, 0,
                                               0);
    }
  }
  if (SM) {
    // quarter w (w < 4): lanes 0-31 fetch block w/2, keys 64t + 32(w%2) + lane;
    // lanes 32-63 read past the range (zeros) into the quarter's unused half
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(ss.base), (short)0,
                                                                        ss.bytes, kBufferFlags);
    const int off = lane < 32 ? ((w >> 1) * ss.npad + t * kKBlock + 32 * (w & 1) + lane) * 4 : ss.bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(stage + G::KBYTES + G::VBYTES + w * 256), 4, off, 0,
                                             0, 0);
  }
#endif
}

// Workgroup barrier without a workgroup-scope memory fence.  __syncthreads()
// makes every wave wait for all its outstanding vector-memory loads — the tile
// DMA in flight included — before the barrier.  Here each wave that issued tile
// DMA waits for exactly the tile the next phase reads (wait_dma).  The
// wavefront-scope fences emit no wait; they keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void barrier_only() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wait until at most OUTSTANDING of this wave's vector-memory loads are in
// flight (tile DMA completes in issue order).
template <int OUTSTANDING>
__device__ __forceinline__ void wait_dma() {
  static_assert(OUTSTANDING >= 0 && OUTSTANDING < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | OUTSTANDING);
}

template <int OUTSTANDING>
__device__ __forceinline__ void wait_dma_and_sync() {
  wait_dma<OUTSTANDING>();
  barrier_only();
}

// Uniform loads of read-only scales through the scalar data cache (SMEM), so
// they never wait behind the vector-memory counter the tile DMA uses.
__device__ __forceinline__ float load_uniform(const float* p, int64_t i) {
  return ((const __attribute__((address_space(4))) float*)p)[i];
}
__device__ __forceinline__ int load_uniform_i(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}
typedef int v2i __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2i load_uniform2(const int32_t* p, int64_t i) {  // i even
  return ((const __attribute__((address_space(4))) v2i*)p)[i / 2];
}

// max / sum over the two lanes that hold the same query row (l and l ^ 32).
__device__ __forceinline__ float pair_max(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
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

// K̂ fragments of one 64-key tile (A operand of Sᵀ = K̂Q̂ᵀ): kf[s][ks] is the
// 16 bytes of key 32s + r32, channels 32ks + 16g .. +15.
template <int D>
__device__ __forceinline__ void load_k_frags(const v4i* __restrict__ lds_k, v4i (&kf)[2][D / 32], int r32, int g) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) kf[s][ks] = lds_k[k_lds_chunk<D>(32 * s + r32, 2 * ks + g)];
}

// This lane's byte offsets of its K̂ fragments inside a K̂ tile (row r32, chunk
// column 2ks + g); rows 32..63 sit 32·D bytes further (the swizzle key of
// row r + 32 equals that of row r).  Computed once, so a fragment address is
// one add of the tile's stage offset.
template <int D>
__device__ __forceinline__ void k_frag_offsets(int r32, int g, int (&ofs)[D / 32]) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) ofs[ks] = 16 * k_lds_chunk<D>(r32, 2 * ks + g);
}
template <int D>
__device__ __forceinline__ void load_k_frags_at(const char* __restrict__ kstage, const int (&ofs)[D / 32],
                                                v4i (&kf)[2][D / 32]) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      kf[s][ks] = *reinterpret_cast<const v4i*>(kstage + ofs[ks] + s * 32 * D);
}

// Sᵀ of one 32-query half for one 64-key tile: S[s] covers keys 32s..32s+31;
// lane (r32, g) reg i holds key 32s + 8(i/4) + 4g + i%4 of query r32, as
// magic + Σ q̂·k̂ — or, with a smoothed Q (SM), as the initial value of that
// key (lslots: the wave's Q block's 64 values in LDS) + Σ q̂·k̂.
template <int D, bool SM = false>
__device__ __forceinline__ void qk_half(const v4i (&kf)[2][D / 32], const v4i (&qf)[D / 32], v16i (&S)[2],
                                        const v4i* __restrict__ lslots = nullptr, int g = 0,
                                        const v16i* magic = nullptr) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    v16i acc;
    if (!SM && magic) {
      // the first MFMA reads the start value from the persistent registers
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[s][0], qf[0], *magic, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < D / 32; ++ks) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[s][ks], qf[ks], acc, 0, 0, 0);
      S[s] = acc;
      continue;
    }
    if (SM) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4i init = lslots[16 * s + 2 * q + g];  // keys 32s + 8q + 4g .. +3
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * q + j] = init[j];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = kMagicI;
    }
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[s][ks], qf[ks], acc, 0, 0, 0);
    S[s] = acc;
  }
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); }

// Masking of a tile that is not fully visible: keys past n or (causal) after
// the row's query get the bit pattern of -inf in place of the magic-biased
// score, so they fall out of the row max and give p = 0 below (c > 0).
constexpr int kNegInfBits = (int)0xFF800000u;

template <bool CAUSAL>
__device__ __forceinline__ void mask_scores(v16i (&S)[2], int k0, int n, int qrow, int gg) {
  // lane (r32, g) reg i of S[s] holds key k0 + 4g + (32s + 8(i/4) + i%4)
  const int lim = (CAUSAL ? min(n - 1, qrow) : n - 1) - k0 - 4 * gg;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int off = 32 * s + 8 * (i >> 2) + (i & 3);
      const int v = S[s][i];
      S[s][i] = (off <= lim) ? v : kNegInfBits;
    }
}

__device__ __forceinline__ float tile_max(float mx, float c2) {
  return (mx == 0.f) ? -__builtin_inff() : (mx - kMagicF) * c2;
}

// FP16 PV: p = 2^(F·c - K), K = fl(M·c + m_ref) — one FMA per score, M the
// bias of F (1.5·2^23, or 0 for scores already in log2 units).  Rounding K
// moves the tile's exponents by up to ulp(K)/2 ≈ 0.75·c (log2 units) against
// the reference the other tiles use, i.e. a relative weight error of up to
// ~0.5·c for the tile: at most 0.4 % while c < kExactC2 = 2^-7 (ordinary
// inputs: c from 1e-4 to 5e-3).  Tiles with a larger c (|q|·|k| in the
// hundreds or more) are first taken to exact log2 units, (F - M)·c with F - M
// the integer score, and come here with c = 1, M = 0.  P is packed as four B
// operands.
constexpr float kExactC2 = 1.0f / 128.0f;
__device__ __forceinline__ float exp_pack_fp16(const float (&F)[2][16], float c2, float m_ref, v8h (&pk)[4],
                                               float M = kMagicF) {
  const float kb = __builtin_fmaf(M, c2, m_ref);
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    const int s = kc >> 1, hh = kc & 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(F[s][8 * hh + j], c2, -kb));
      pk[kc][j] = (_Float16)p;
    }
  }
  // The lane's share of the row sum, from the fp16 P that enters the PV product:
  // a pairwise tree of packed fp16 adds (15 v_pk_add_f16 instead of 28 fp32
  // adds; four fp16 roundings, so within 4·2^-11 of the exact sum of the fp16
  // values; p <= 2^8 on an accepted tile keeps it far from fp16 overflow, and
  // an overflowing first pass gives inf, which fails the lazy check below).
  const v8h s8 = (pk[0] + pk[1]) + (pk[2] + pk[3]);
  const v4h s4 = __builtin_shufflevector(s8, s8, 0, 1, 2, 3) + __builtin_shufflevector(s8, s8, 4, 5, 6, 7);
  const v2h s2 = __builtin_shufflevector(s4, s4, 0, 1) + __builtin_shufflevector(s4, s4, 2, 3);
  return (float)s2[0] + (float)s2[1];
}

// FP8 PV: the e4m3 codes of 448·p follow the running max itself (the schedule
// the method fixes): p·448 = 2^((F - mx)·c + (m_tile - m) + log2 448), with
// F - mx exact (both in [2^23, 2^24)); p·448 <= 448·2^(2^-20) < 464, so the
// conversion cannot overflow.  P is packed as one 32-byte B operand.
__device__ __forceinline__ float exp_pack_fp8(const float (&F)[2][16], float mx, float c2, float cterm, v8i& pk) {
  float ls[4] = {-0.f, -0.f, -0.f, -0.f};  // four short add chains, not one of 32
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int s = q >> 2, i0 = 4 * (q & 3);
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(F[s][i0 + j] - mx, c2, cterm));
      ls[j] += p[j];
    }
    // the two conversions write the low and then the high half of the word:
    // starting from the old (dead) value saves clearing a register first
    int wv = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pk[q], false);
    pk[q] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wv, true);
  }
  return (ls[0] + ls[1]) + (ls[2] + ls[3]);
}

// FP8 PV with a smoothed Q: the scores X are already in log2 units (the
// smoothing term added in fp32); p·448 = 2^(X + cterm), cterm = log2 448 - m.
__device__ __forceinline__ float exp_pack_fp8_log2(const float (&X)[2][16], float cterm, v8i& pk) {
  float ls[4] = {-0.f, -0.f, -0.f, -0.f};  // four short add chains, not one of 32
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int s = q >> 2, i0 = 4 * (q & 3);
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = __builtin_amdgcn_exp2f(X[s][i0 + j] + cterm);
      ls[j] += p[j];
    }
    int wv = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pk[q], false);
    pk[q] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wv, true);
  }
  return (ls[0] + ls[1]) + (ls[2] + ls[3]);
}

// O += P·V for one group of 32 queries.  FP8: level 1 (one tile's 64 keys)
// and level 2 (the running output) are one fp32 MFMA per d tile.
template <int D, bool FP8>
__device__ __forceinline__ void pv_tile(const char* __restrict__ vstage, int lane, const v8h (&pk16)[4],
                                        const v8i& pk8, v16f (&O)[D / 32]) {
  constexpr int DT = D / 32;
  if (!FP8) {
    const int vb = v_tr_base(lane);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v_frag(vstage, vb, kc, dt), pk16[kc], O[dt], 0, 0, 0);
  } else {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      O[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v_frag_fp8(vstage, lane, dt), pk8, O[dt], 0, 0, 0, 0,
                                                              0, 0);
  }
}

// Matrix phase with both parts (the steady state): PV of the previous tile and
// QKᵀ of the current one in one scheduling region.  All K̂ fragment reads go
// first (FP16 PV without smoothing: behind a scheduling barrier, since the
// read-count groups below cannot tell them from V reads; measured −0.3 to
// −0.8 % against letting the compiler interleave them); then every MFMA is
// followed by one V fragment read (two 64-bit transposing reads for FP16)
// while any remain, so each LDS read has several MFMAs (>= 256 cycles) to
// land before its use.
template <int D, bool FP8, bool SM = false>
__device__ __forceinline__ void matrix_both(const char* __restrict__ kstage, const int (&kofs)[D / 32],
                                            const char* __restrict__ vstage, int lane, int gg,
                                            const v4i (&qf)[D / 32], v16i (&S)[2],
                                            const v8h (&pk16)[4], const v8i& pk8, v16f (&O)[D / 32],
                                            const v4i* __restrict__ lslots = nullptr,
                                            const v16i* magic = nullptr) {
  constexpr int DT = D / 32;
  constexpr int NK = 2 * DT + (SM ? 8 : 0);  // K̂ fragment (+ initial value) reads (128-bit)
  constexpr int NV = FP8 ? 2 * DT : 8 * DT;  // V fragment reads (FP8: 128-bit; FP16: 64-bit transposing)
  constexpr int RPM = FP8 ? 1 : 2;           // V reads placed after each MFMA
  constexpr int NQK = 2 * DT;                // QKᵀ MFMAs
  constexpr int NPV = FP8 ? DT : 4 * DT;     // PV MFMAs
  constexpr bool kKFirst = !FP8 && !SM;
  v4i kf[2][DT];
  load_k_frags_at<D>(kstage, kofs, kf);
  if (kKFirst) __builtin_amdgcn_sched_barrier(0);
  if (!FP8) {
    const int vb = v_tr_base(lane);
    v8h vf[4 * DT];
#pragma unroll
    for (int i = 0; i < 4 * DT; ++i) vf[i] = v_frag(vstage, vb, i / DT, i % DT);
    qk_half<D, SM>(kf, qf, S, lslots, gg, magic);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[kc * DT + dt], pk16[kc], O[dt], 0, 0, 0);
  } else {
    v8i vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[dt] = v_frag_fp8(vstage, lane, dt);
    qk_half<D, SM>(kf, qf, S, lslots, gg, magic);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      O[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[dt], pk8, O[dt], 0, 0, 0, 0, 0, 0);
  }
  // schedule: NK reads, then MFMA / read pairs, then the remaining MFMAs
  if (!kKFirst) __builtin_amdgcn_sched_group_barrier(0x100, NK, 0);
#pragma unroll
  for (int i = 0; i < NQK + NPV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < NV / RPM) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
  }
}

template <int D>
__device__ __forceinline__ void rescale_o(v16f (&O)[D / 32], float& l_run, float alpha) {
  l_run *= alpha;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[dt][i] *= alpha;
}

// Per-wave state of the 32-query attention pipeline.
template <int D, bool FP8>
struct WaveCtx {
  v4i qf[D / 32];   // Q̂ B operand
  v16f O[D / 32];   // Oᵀ accumulator (d tiles of 32)
  v16i S[2];        // Sᵀ of the current tile
  v8h pk16[4];      // P of the previous tile (fp16 PV)
  v8i pk8;          // P of the previous tile (fp8 PV)
  float m_run;      // exponent reference (log2 units)
  float l_run;      // this lane's share of the row sum
};

// Row max of the tile's scores over both lanes of the row.  Magic-biased
// scores are positive, so the neutral value 0 (nothing visible) is enough;
// with SIGNED scores (log2 units) it is -inf.
template <bool SIGNED = false>
__device__ __forceinline__ float row_max(const float (&F)[2][16]) {
  float mx = SIGNED ? -__builtin_inff() : 0.f;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = max3f(mx, F[s][i], F[s][i + 1]);
  return pair_max(mx);
}

// Softmax phase of one tile (masked entries already -inf): P for the next
// matrix phase, the row statistics and, when the exponent reference moves,
// the output rescale — O is rescaled in one place only.
//
// FP16: P is formed against the current reference m first.  If every lane's
// sum of p stays <= kLazyLimit, no p exceeds that bound and the tile is
// done without a row max; otherwise (a row max passed m by more than
// 8 (log2 units), or the first visible tile of a row) m moves to the row max,
// O and l are rescaled and P is formed again.  Softmax does not depend on the
// reference and fp16 rounding is relative, so this changes nothing but
// rounding.  FP8: the codes follow the running max exactly, tile by tile.
//
// SM (smoothed Q): F is either magic-biased (M = 1.5·2^23) or, in a tile that
// took the fp32 path, already the score in log2 units (c2 = 1, M = 0), so the
// row max starts from -inf and the tile max is (max F - M)·c2.
//
// FP8 with a smoothed Q (lterm != nullptr): the scores are magic-biased
// integers and lterm holds, for this lane's 32 keys, the smoothing term in
// log2 units (fp32); s = (F - M)·c2 + term, exact max per tile as above.
template <int D, bool FP8, bool SM = false>
__device__ __forceinline__ void softmax_phase(WaveCtx<D, FP8>& c, float c2, float M = kMagicF,
                                              const float4* __restrict__ lterm = nullptr) {
  float F[2][16];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // read the element by value first: a bit cast of an ext-vector element
      // lvalue compiles to a read of element 0
      const int bits = c.S[s][i];
      F[s][i] = __int_as_float(bits);
    }
  if (!FP8) {
    // a row that has seen no visible key keeps m = -inf: its p become +inf
    // (visible) or 0 (masked), and the check below moves m
    float lsum = exp_pack_fp16(F, c2, __builtin_fmaxf(c.m_run, -3.0e38f), c.pk16, SM ? M : kMagicF);
    if (__any(!(lsum <= kLazyLimit))) {
      const float mt = SM ? (row_max<true>(F) - M) * c2 : tile_max(row_max(F), c2);
      float m_new = __builtin_fmaxf(c.m_run, mt);
      m_new = (m_new == -__builtin_inff()) ? 0.f : m_new;
      rescale_o<D>(c.O, c.l_run, __builtin_amdgcn_exp2f(c.m_run - m_new));
      c.m_run = m_new;
      lsum = exp_pack_fp16(F, c2, m_new, c.pk16, SM ? M : kMagicF);
    }
    c.l_run += lsum;
  } else if (SM && lterm) {
    // lane (r32, g) reg 4q + j of S[s] is key 32s + 8q + 4g + j: lterm[16s + 2q]
    // (already offset by g) holds those four keys' terms
    float X[2][16];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 tv = lterm[16 * s + 2 * q];
        const float t4[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) X[s][4 * q + j] = __builtin_fmaf(F[s][4 * q + j] - M, c2, t4[j]);
      }
    float m_new = __builtin_fmaxf(c.m_run, row_max<true>(X));
    m_new = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(c.m_run - m_new);
    const float lsum = exp_pack_fp8_log2(X, kLog2E4M3Max - m_new, c.pk8);
    if (__any(alpha != 1.f)) rescale_o<D>(c.O, c.l_run, alpha);
    c.m_run = m_new;
    c.l_run += lsum;
  } else {
    float mx = SM ? row_max<true>(F) : row_max(F);
    const float mt = SM ? (mx - M) * c2 : tile_max(mx, c2);
    if (SM) mx = (mx == -__builtin_inff()) ? 0.f : mx;  // all masked: F - 0 = -inf gives p = 0
    float m_new = __builtin_fmaxf(c.m_run, mt);
    m_new = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(c.m_run - m_new);
    const float lsum = exp_pack_fp8(F, mx, c2, (mt - m_new) + kLog2E4M3Max, c.pk8);
    if (__any(alpha != 1.f)) rescale_o<D>(c.O, c.l_run, alpha);
    c.m_run = m_new;
    c.l_run += lsum;
  }
}

// Workgroup: 8 waves x 32 queries = 256 queries (two Q scale blocks), two waves
// per SIMD (waves w and w+4 share one).  Waves 0-3 (group A) and 4-7 (group B)
// run the same per-tile work in opposite orders, so that on every SIMD one
// wave's MFMAs overlap the other wave's softmax.  Group A streams the tiles.
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kAttnRows = 32 * kAttnWaves;
constexpr int kAhead = 2;                // tiles requested ahead of the one being read
constexpr int kRingStages = kAhead + 2;  // + tile t (group A) and tile t-1 (group B's PV)
static_assert(kAhead >= 1 && kAhead <= 3, "wait_tiles handles up to two tiles in flight");

// Wait until at most `pending` tiles (L DMA instructions each) of this wave
// are still in flight.
template <int L>
__device__ __forceinline__ void wait_tiles(int pending) {
  if (pending >= 2)
    wait_dma<2 * L>();
  else if (pending == 1)
    wait_dma<L>();
  else
    wait_dma<0>();
}

// d=64 fits 128 VGPRs, so two workgroups share a CU (four waves per SIMD) and
// their independent phases fill each other's stalls; d=128 needs ~180, and so
// does d=64 with a smoothed Q (its accumulator initial values would spill) or
// with per-token Q scales and FP8 PV (one or two spilled registers).
template <int D, bool LOW_OCCUPANCY>
constexpr int kAttnWavesPerSimd = (D == 64 && !LOW_OCCUPANCY) ? 4 : 2;

// How Q is scaled: per 128-token block, per block with the smoothing term, or
// per token (one scale per query row, so the per-tile factor is per lane).
enum { kQmBlock = 0, kQmSmooth = 1, kQmToken = 2 };

template <int D, bool FP8, bool CAUSAL, int QM>
__global__ __attribute__((amdgpu_flat_work_group_size(kAttnThreads, kAttnThreads),
                          amdgpu_waves_per_eu(kAttnWavesPerSimd<D, QM == kQmSmooth || (QM == kQmToken && FP8)>,
                                              kAttnWavesPerSimd<D, QM == kQmSmooth || (QM == kQmToken && FP8)>)))
void attn_fwd_kernel(AttnArgs a) {
  constexpr bool SM = QM == kQmSmooth;
  constexpr int DT = D / 32;  // 32-wide d tiles of the output
  using G = TileGeom<D, FP8, kThreads, SM>;  // tiles are streamed by the 4 waves of group A
  __shared__ __attribute__((aligned(1024))) char smem[kRingStages * G::STAGE];

  const SeqGeom& g = a.g;
  const int nqb = ceil_div(g.N, kQBlock);
  const int nkb = ceil_div(g.N, kKBlock);
  const int nwb = ceil_div(g.N, kAttnRows);
  // causal: pair head-sequences when two of them (K̂ + V per key) fit one L2
  const bool pair = CAUSAL && 2 * (int64_t)g.N * (D + G::VBYTES / kKBlock) <= kXcdL2Bytes;
  int wb, hb;
  work_item(xcd_remap(blockIdx.x, gridDim.x), nwb, g.H * g.B, pair, wb, hb);
  const int h = hb / g.B, b = hb % g.B;
  int64_t row0;
  int n;
  hs_rows(g, b, h, row0, n);
  const int q0 = wb * kAttnRows;
  if (q0 >= n) return;

  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, gg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = w < kAttnWaves / 2;  // group A
  const int64_t hs = (int64_t)b * g.H + h;
  const int wq_lo = q0 + 32 * w;  // first query of the wave
  const int qrow = wq_lo + r32;
  const int wq_hi = min(wq_lo + 31, n - 1);
  const bool wave_rows = wq_lo < n;

  // K/V head of this query head (grouped-query attention; kv_group = 1 otherwise)
  SeqGeom gk = g;
  gk.H = g.H / a.kv_group;
  const int hk = h / a.kv_group;
  const int64_t hsk = (int64_t)b * gk.H + hk;
  int64_t krow0;
  int kn;
  hs_rows(gk, b, hk, krow0, kn);  // kn == n: same sequence

  const int kend = CAUSAL ? min(n, q0 + kAttnRows) : n;
  const int ntiles = ceil_div(kend, kKBlock);
  const int8_t* kbase = a.k + krow0 * D;
  const int kbytes = n * D;
  // V: FP16 PV reads the input's rows of this head-sequence; FP8 its packed tiles
  const uint8_t* vbase = FP8 ? a.v + vtile_index(gk, b, hk, 0) * G::VBYTES : a.v + krow0 * D * 2;
  const int vbytes = FP8 ? ceil_div(n, kKBlock) * G::VBYTES : (int)((unsigned)n * 2u * D);
  constexpr int L = G::KI + G::VI + G::SI;  // DMA instructions per group-A wave per tile
  // smoothed Q: this workgroup's rows of accumulator initial values (Q blocks
  // q0/128 and, if it exists, the next), fallback flags and fp32 terms
  const int npad = nkb * kKBlock;
  const int wqb = wq_lo / kQBlock;  // this wave's Q block
  const int wqb_in = min(wqb, nqb - 1);  // the same, kept in range for waves past n
  SlotSrc ss{};
  if (SM) ss = SlotSrc{a.qb_slots + (hs * nqb + q0 / kQBlock) * (int64_t)npad, (q0 + kQBlock < n ? 2 : 1) * npad * 4,
                       npad};

  WaveCtx<D, FP8> c;
  int kofs[DT];
  k_frag_offsets<D>(r32, gg, kofs);
  // FP16 PV at d=128: the accumulator start value 1.5·2^23 kept in 16
  // registers for the whole loop (the first QKᵀ MFMA of each half reads it),
  // in place of 16 vector moves per tile; opaque to the compiler so that it is
  // not re-materialised.  Measured -0.8 % at 16K, -1.8 % at 16K causal, but
  // +2.6 % for the FP8 PV kernel, which keeps the moves; d=64 has no registers
  // to spare at four waves per SIMD.
  v16i mg;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int m = kMagicI;
    if (D == 128 && !FP8) asm volatile("" : "+v"(m));
    mg[i] = m;
  }
  // Q quantised here (q16 set): the lane's 16-channel runs of its query in
  // fp32; per block, the wave's largest |x| goes to LDS and the block's four
  // waves' maxima are combined after the barrier below; per token, the two
  // lanes of the row combine theirs.  The codes and scales are those of the Q
  // pre-pass (the same quantiser, in the same precision).
  const bool qfuse = (QM == kQmBlock || QM == kQmToken) && a.q16 != nullptr;
  __shared__ float qmax_s[kAttnWaves];
  float qx[DT][16];
  float qamax = 0.f;  // per-token Q: the lane's row maximum
  float dq = 0.f;
  if (qfuse) {
    float amax = 0.f;
#pragma unroll
    for (int ks = 0; ks < DT; ++ks) {
      v4i raw[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
      if (qrow < n) {
        const v4i* src = reinterpret_cast<const v4i*>(a.q16 + (row0 + qrow) * D + 32 * ks + 16 * gg);
        raw[0] = src[0];
        raw[1] = src[1];
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t wd = (uint32_t)raw[h2][j];
          qx[ks][8 * h2 + 2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd & 0xffffu));
          qx[ks][8 * h2 + 2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd >> 16));
        }
#pragma unroll
      for (int j = 0; j < 16; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(qx[ks][j]));
    }
    if (QM == kQmToken) {
      qamax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));  // the row: both lane halves
    } else {
      amax = wave_max(amax);
      if (lane == 0) qmax_s[w] = amax;
    }
  } else {
    load_q_frags<D>(c.qf, a.q + row0 * D, qrow, n, gg);
    // δQ: the wave's block scale (uniform), or this lane's query's own scale
    dq = QM == kQmToken ? (qrow < n ? a.q_scale[row0 + qrow] : 0.f) : load_uniform(a.q_scale, hs * nqb + wqb_in);
  }
  const float* __restrict__ ksc = a.k_scale + hsk * nkb;
  // smoothed Q: whether any half tile of this wave's Q block falls back (rare);
  // only then are the per-tile flags read
  // (FP16 PV only: with FP8 PV every key's term is fp32, staged with the tile)
  const bool row_fb = SM && !FP8 && load_uniform_i(a.qb_any, hs * nqb + wqb_in) != 0;
  c.m_run = -__builtin_inff();
  c.l_run = 0.f;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) c.pk16[kc] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
  c.pk8 = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) c.O[dt][i] = 0.f;

  // FP16: the largest δK of the tiles this workgroup reads (four independent
  // loads per lane and pass; 256 tiles, the 16K case, take one pass)
  float dkmax = 0.f;
  if (!FP8) {
    for (int i0 = lane; i0 < ntiles; i0 += 256) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (i0 + 64 * j < ntiles) ? ksc[i0 + 64 * j] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) dkmax = __builtin_fmaxf(dkmax, v[j]);
    }
  }
  if (lead) {
    const int first = min(kAhead, ntiles);
    for (int t = 0; t < first; ++t)
      issue_tile<D, FP8, kThreads, SM>(kbase, kbytes, vbase, vbytes, t, smem + t * G::STAGE, w, lane, ss);
  }
  // the first tiles and this wave's Q̂ fragments have landed; an empty queue
  // here also lets the compiler see that no later MFMA waits on the Q̂ loads
  wait_dma<0>();
  barrier_only();
  if (qfuse) {
    // the Q block of this wave: waves 4·(w/4) .. +3
    const int wb0 = w & ~3;
    const float amax = QM == kQmToken ? qamax
                                      : __builtin_fmaxf(__builtin_fmaxf(qmax_s[wb0], qmax_s[wb0 + 1]),
                                                        __builtin_fmaxf(qmax_s[wb0 + 2], qmax_s[wb0 + 3]));
    const float s = amax / kInt8Max;
    const float r = 1.0f / s;
#pragma unroll
    for (int ks = 0; ks < DT; ++ks) {
      uint32_t wv[4] = {0u, 0u, 0u, 0u};  // an all-zero block (s = 0) has all codes 0
      if (s > 0.f) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          wv[q4] = pack4_i8(int8_code(qx[ks][4 * q4], s, r), int8_code(qx[ks][4 * q4 + 1], s, r),
                            int8_code(qx[ks][4 * q4 + 2], s, r), int8_code(qx[ks][4 * q4 + 3], s, r));
      }
      c.qf[ks] = v4i{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
    }
    dq = s * a.sm_scale;
  }
  // FP16: can a tile's factor δQ·δK·log2(e) exceed kExactC2 in this wave?
  // Only then are its tiles checked one by one (rare inputs).
  const bool exact_wave = !FP8 && __any(dq * wave_max(dkmax) * kLog2e > kExactC2);

  // tiles this wave takes part in: 0..nact-1 (causal: keys up to its last query)
  const int nact = !wave_rows ? 0 : CAUSAL ? min(ntiles, wq_hi / kKBlock + 1) : ntiles;
  auto softmax_step = [&](int u) {
    if (u < nact) {
      const int k0 = u * kKBlock;
      // c > 0 keeps -inf·c = -inf for masked keys; a zero scale means all
      // scores of the tile are 0, for which the smallest normal gives the same
      float c2 = __builtin_fmaxf(dq * load_uniform(ksc, u) * kLog2e, 1.17549435e-38f);
      const bool full = (k0 + kKBlock <= n) && (!CAUSAL || k0 + kKBlock - 1 <= wq_lo);
      if (!full) mask_scores<CAUSAL>(c.S, k0, n, qrow, gg);
      float M = kMagicF;
      if (SM && !FP8 && row_fb) {
        const int64_t row = hs * nqb + wqb;
        const v2i fb = load_uniform2(a.qb_flags, row * (2 * nkb) + 2 * u);
        if (fb.x | fb.y) {
          // a half tile whose smoothing term did not fit the accumulator:
          // every score of the tile becomes fp32 log2 units, s = (F - M)·c2
          // (+ the fp32 term of a fallback half); F - M is exact
          const float* fx = a.qb_fix + row * npad + k0;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const bool fall = s ? fb.y : fb.x;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 add = fall ? *reinterpret_cast<const float4*>(fx + 32 * s + 8 * q + 4 * gg)
                                      : float4{0.f, 0.f, 0.f, 0.f};
              const float av[4] = {add.x, add.y, add.z, add.w};
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int bits = c.S[s][4 * q + j];
                c.S[s][4 * q + j] = __float_as_int(__builtin_fmaf(__int_as_float(bits) - kMagicF, c2, av[j]));
              }
            }
          }
          c2 = 1.f;
          M = 0.f;
        }
      }
      if (exact_wave && M != 0.f && __any(c2 > kExactC2)) {
        // a large factor (rare inputs): the scores to exact log2 units in
        // place, (F - M)·c2, and the softmax runs with c2 = 1, M = 0; the
        // laundered M keeps the conversion inside this branch
        float mz = kMagicF;
        asm volatile("" : "+v"(mz));
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int bits = c.S[s][i];
            c.S[s][i] = __float_as_int((__int_as_float(bits) - mz) * c2);
          }
        c2 = 1.f;
        M = 0.f;
      }
      // FP16 takes the scores' bias at run time (magic-biased, or log2 units)
      const float4* lterm = nullptr;
      if (SM && FP8)
        lterm = reinterpret_cast<const float4*>(smem + (u & (kRingStages - 1)) * G::STAGE + G::KBYTES + G::VBYTES) +
                32 * (wqb - q0 / kQBlock) + gg;
      softmax_phase<D, FP8, SM || !FP8>(c, c2, M, lterm);
    }
  };
  // One workgroup barrier per tile.  Group A runs matrix(t) then softmax(t),
  // group B softmax(t-1) then matrix(t), so on each SIMD one wave's MFMAs
  // overlap the other wave's exponentials; matrix(t) = PV of tile t-1 and QKᵀ
  // of tile t.  Where a softmax outlasts a matrix phase (FP8 PV, d = 64), the
  // two softmaxes of a SIMD overlap and share its VALU; group B's is the one
  // the barrier waits on (its matrix phase still follows), so it issues at a
  // raised wave priority and group A's softmax takes the slack.
  constexpr bool kRaiseSoftB = FP8 || D == 64;
  for (int t = 0; t < ntiles; ++t) {
    if (lead && t + kAhead < ntiles)
      issue_tile<D, FP8, kThreads, SM>(kbase, kbytes, vbase, vbytes, t + kAhead,
                                       smem + ((t + kAhead) % kRingStages) * G::STAGE, w, lane, ss);
    if (!lead && t > 0) {
      if (kRaiseSoftB) __builtin_amdgcn_s_setprio(1);
      softmax_step(t - 1);
      if (kRaiseSoftB) __builtin_amdgcn_s_setprio(0);
    }
    // One place for both MFMA parts keeps O and S in fixed registers.  At t = 0
    // the pending P is zero (O += 0·V of tile 0, which has landed); at t = nact
    // the QKᵀ result is not used.
    if (t <= nact && nact > 0) {
      // stage offsets are wave-uniform: scalar arithmetic, one vector add per address
      const int kst = __builtin_amdgcn_readfirstlane((t % kRingStages) * G::STAGE);
      static_assert((kRingStages & (kRingStages - 1)) == 0, "ring index by mask");
      const int vst = (t > 0 ? (t - 1) & (kRingStages - 1) : 0) * G::STAGE;
      // FP8 with a smoothed Q: the accumulator starts at the bias alone (its term is added in fp32)
      matrix_both<D, FP8, SM && !FP8>(smem + kst, kofs, smem + vst + G::KBYTES, lane, gg, c.qf, c.S, c.pk16, c.pk8,
                                      c.O,
                                      reinterpret_cast<const v4i*>(smem + kst + G::KBYTES + G::VBYTES) +
                                          32 * (wqb - q0 / kQBlock),
                                      (D == 128 && !FP8) ? &mg : nullptr);
    }
    if (lead) softmax_step(t);
    // tile t+1 landed before anyone's next matrix phase (later tiles may fly)
    if (lead) wait_tiles<L>(max(0, min(kAhead - 1, ntiles - 2 - t)));
    barrier_only();
  }
  if (!lead && ntiles > 0) softmax_step(ntiles - 1);
  if (nact == ntiles && ntiles > 0)
    pv_tile<D, FP8>(smem + ((ntiles - 1) % kRingStages) * G::STAGE + G::KBYTES, lane, c.pk16, c.pk8, c.O);

  // Epilogue: o = O / l (FP16) or O·δV / l with l holding 448·Σp (FP8).
  const float l_tot = pair_sum(c.l_run);
  if (!wave_rows || qrow >= n) return;
  const float inv = 1.f / l_tot;
  if (a.lse && gg == 0) {
    // natural-log sum of exp of the row's scaled scores: m is in log2 units
    const float log2_l = __builtin_log2f(l_tot) - (FP8 ? kLog2E4M3Max : 0.f);
    a.lse[row0 + qrow] = (c.m_run + log2_l) * 0.6931471805599453f;
  }
  uint16_t* __restrict__ orow = a.o + (row0 + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * dt + 8 * q4 + 4 * gg;
      float f[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) f[j] = c.O[dt][4 * q4 + j] * inv;
      if (FP8) {
        const float4 vs = *reinterpret_cast<const float4*>(a.v_scale + hsk * D + d);  // per-lane d
        f[0] *= vs.x;
        f[1] *= vs.y;
        f[2] *= vs.z;
        f[3] *= vs.w;
      }
      v2h lo = {(_Float16)f[0], (_Float16)f[1]};
      v2h hi = {(_Float16)f[2], (_Float16)f[3]};
      uint2 stv;
      stv.x = __builtin_bit_cast(uint32_t, lo);
      stv.y = __builtin_bit_cast(uint32_t, hi);
      *reinterpret_cast<uint2*>(orow + d) = stv;
    }
}

// ---------------------------------------------------------------------------
// MXFP4 attention (dtcms summary, section "SageAttention 3": microscaling FP4
// attention with two-level quantisation; operands prepared in quant.hip).
// The schedule is attn_fwd_kernel's (two wave groups, one barrier per tile,
// LDS DMA two tiles ahead); what differs:
//   * Sᵀ = K̂Q̂ᵀ and Oᵀ = VᵀPᵀ both run on v_mfma_scale_f32_32x32x64_f8f6f4 with
//     e2m1 operands: each lane supplies 32 elements of one 32-wide block along
//     the contraction and that block's E8M0 scale; the accumulator is fp32.
//   * The K̂ rows of a tile sit in LDS in the order that makes each lane
//     half's 32 scores the keys 32g .. 32g+31 of the tile, so a lane's P values
//     are exactly one 32-key MX block of its query: level one is the online
//     softmax's p = 2^(s - m) <= 1, level two the block's power-of-two scale
//     from the lane's own largest p, then the hardware e2m1 conversion.
//   * LDS stage: K̂ codes (rows of d/2 bytes, 16-byte chunks XOR-swizzled on
//     the 256-byte bank line), packed V codes, and 1 KB of scales (K: 8 bytes
//     per row; V: 4 bytes per lane).
template <int D, bool SM = false>
struct MxGeom {
  static constexpr int KBYTES = kKBlock * D / 2;  // K̂ codes of a tile
  static constexpr int VBYTES = kKBlock * D / 2;  // packed V codes
  static constexpr int SBYTES = SM ? 1024 : 0;    // smoothed Q: the term per key, two Q blocks
  static constexpr int STAGE = KBYTES + VBYTES + kMxAuxBytes + SBYTES;
  static constexpr int KCH = KBYTES / 16;
  static constexpr int CI = (KBYTES + VBYTES) / 16 / kThreads;  // 16-byte DMA instructions per group-A wave
  static constexpr int CPR = D / 32;                             // 16-byte chunks per K̂ row
  static constexpr int RSH = (D == 128) ? 2 : 3;                 // log2 of rows per 256-byte bank line
  static_assert(CI * kThreads * 16 == KBYTES + VBYTES, "tile must split evenly over the waves");
  static __device__ __forceinline__ int chunk(int r, int c) { return r * CPR + (c ^ ((r >> RSH) & (CPR - 1))); }
};

// Key of LDS row r of an MXFP4 K̂ tile: row 32s + 8q + 4g + t holds key
// 32g + 16s + 4q + t.
__device__ __forceinline__ int mx_key_of_row(int r) {
  return 32 * ((r >> 2) & 1) + 16 * (r >> 5) + 4 * ((r >> 3) & 3) + (r & 3);
}

template <int D, bool SM = false>
__device__ __forceinline__ void issue_mx_tile(const void* kbase, int kbytes, const void* vbase, int vbytes,
                                              const void* abase, int abytes, int t, char* stage, int w, int lane,
                                              const SlotSrc& ss = SlotSrc{}) {
#if defined(__HIP_DEVICE_COMPILE__)
  using G = MxGeom<D, SM>;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(kbase), (short)0, kbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(vbase), (short)0, vbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(abase), (short)0, abytes, kBufferFlags);
#pragma unroll
  for (int j = 0; j < G::CI; ++j) {
    const int base = (w * G::CI + j) * 64;  // wave-uniform chunk index
    if (base < G::KCH) {
      // LDS slot p holds logical chunk (slot ^ swizzle) of row p / CPR
      const int p = base + lane;
      const int r = p / G::CPR, cs = p % G::CPR;
      const int c = cs ^ ((r >> G::RSH) & (G::CPR - 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(stage + base * 16), 16,
                                               (t * kKBlock + mx_key_of_row(r)) * (D / 2) + c * 16, 0, 0, 0);
    } else {
      const int p = base - G::KCH;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(stage + G::KBYTES + p * 16), 16,
                                               t * G::VBYTES + (p + lane) * 16, 0, 0, 0);
    }
  }
  // scales: wave w (< 4) brings bytes 256w .. 256w+255 of the tile's 1 KB
  __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + G::KBYTES + G::VBYTES + w * 256), 4,
                                           t * kMxAuxBytes + w * 256 + lane * 4, 0, 0, 0);
  if (SM) {
    // the term per key, as for the INT8 path: quarter w holds block w/2, keys
    // 64t + 32(w%2) + lane (lanes 32-63 read zeros past the range)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(ss.base), (short)0,
                                                                        ss.bytes, kBufferFlags);
    const int off = lane < 32 ? ((w >> 1) * ss.npad + t * kKBlock + 32 * (w & 1) + lane) * 4 : ss.bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_ptr_t)(stage + G::KBYTES + G::VBYTES + kMxAuxBytes + w * 256), 4, off, 0, 0, 0);
  }
#endif
}

// One scaled e2m1 MFMA with constant byte selects for both scales.
template <int SA, int SB>
__device__ __forceinline__ v16f mx_mfma(const v4i& a, const v4i& b, const v16f& c, int sa, int sb) {
  const v8i A = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const v8i B = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, SA, sa, SB, sb);
}

template <int D>
struct MxWave {
  v4i qf[D / 64];   // Q̂ e2m1 codes: query r32, channels 64kk + 32g .. +31
  int qsc;          // its E8M0 scales, byte kk
  v16f O[D / 32];
  v16f S[2];        // Sᵀ of the current tile (fp32)
  v4i pk;           // P codes of the previous tile (one 32-key block per lane)
  int psc;          // their E8M0 scale (byte 0)
  float m_run;
  float l_run;
};

// Matrix phase: PV of the previous tile (its P in pk) and QKᵀ of this one.
// With a smoothed Q (lslots: the wave's Q block's 64 terms in LDS, quarter
// layout) the QKᵀ accumulator starts from the term of each key.
template <int D, bool SM = false>
__device__ __forceinline__ void mx_matrix(const char* __restrict__ kstage, const char* __restrict__ vstage,
                                          const char* __restrict__ astage, const char* __restrict__ avstage,
                                          int lane, int r32, int gg, MxWave<D>& c,
                                          const float4* __restrict__ lslots = nullptr) {
  using G = MxGeom<D>;
  constexpr int DT = D / 32;
  const v4i* lk = reinterpret_cast<const v4i*>(kstage);
  v4i kf[2][D / 64];
  int ks[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int r = 32 * s + r32;
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) kf[s][kk] = lk[G::chunk(r, 2 * kk + gg)];
    ks[s] = *reinterpret_cast<const int*>(astage + r * 8 + 4 * gg);
  }
  const v4i* lv = reinterpret_cast<const v4i*>(vstage);
  v4i vf[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) vf[dt] = lv[dt * 64 + lane];
  const int vsc = *reinterpret_cast<const int*>(avstage + 512 + 4 * lane);
  float4 init[2][4];
  if (SM) {
    // S[s] reg i is key 32gg + 16s + i: four runs of four consecutive keys
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) init[s][q] = lslots[16 * gg + 4 * s + q];
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    v16f acc;
    if (SM) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[4 * q] = init[s][q].x;
        acc[4 * q + 1] = init[s][q].y;
        acc[4 * q + 2] = init[s][q].z;
        acc[4 * q + 3] = init[s][q].w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    }
    acc = mx_mfma<0, 0>(kf[s][0], c.qf[0], acc, ks[s], c.qsc);
    if (D == 128) acc = mx_mfma<1, 1>(kf[s][D / 64 - 1], c.qf[D / 64 - 1], acc, ks[s], c.qsc);
    c.S[s] = acc;
  }
  c.O[0] = mx_mfma<0, 0>(vf[0], c.pk, c.O[0], vsc, c.psc);
  c.O[1] = mx_mfma<1, 0>(vf[1], c.pk, c.O[1], vsc, c.psc);
  if (D == 128) {
    c.O[DT - 2] = mx_mfma<2, 0>(vf[DT - 2], c.pk, c.O[DT - 2], vsc, c.psc);
    c.O[DT - 1] = mx_mfma<3, 0>(vf[DT - 1], c.pk, c.O[DT - 1], vsc, c.psc);
  }
  // schedule: every LDS read first, then the MFMAs (each read has the earlier
  // MFMAs to land behind)
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 64) + 2 + DT + 1 + (SM ? 8 : 0), 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * (D / 64) + DT, 0);
}

// Masking of a tile that is not fully visible, in place: lane half gg holds
// keys k0 + 32gg + 16s + i in S[s][i].
template <bool CAUSAL>
__device__ __forceinline__ void mx_mask(v16f (&S)[2], int k0, int n, int qrow, int gg) {
  const int lim = (CAUSAL ? min(n - 1, qrow) : n - 1) - k0 - 32 * gg;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = S[s][i];
      S[s][i] = (16 * s + i <= lim) ? v : -__builtin_inff();
    }
}

// Softmax phase of one tile (masked scores already -inf): exact per-tile max
// (the P codes follow it), the MX P block of this lane, the row sum of the
// unrounded p.
template <int D>
__device__ __forceinline__ void mx_softmax(MxWave<D>& c, float c2) {
  float F[2][16];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float f = c.S[s][i];
      F[s][i] = f;
    }
  float lmx = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 16; i += 2) lmx = max3f(lmx, F[s][i], F[s][i + 1]);
  const float mt = pair_max(lmx) * c2;
  float m_new = __builtin_fmaxf(c.m_run, mt);
  m_new = (m_new == -__builtin_inff()) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(c.m_run - m_new);
  if (__any(alpha != 1.f)) rescale_o<D>(c.O, c.l_run, alpha);
  c.m_run = m_new;
  // level two: this lane's 32 p are one block; its scale from its largest p
  const int X = mx_exponent(__builtin_amdgcn_exp2f(__builtin_fmaf(lmx, c2, -m_new)));
  const float sc = __builtin_ldexpf(1.f, X);
  // all exponentials first, then the sums and conversions: the transcendental
  // results are not waited on right after they are issued
  float p[4][8];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < 8; ++j) p[q][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(F[q >> 1][8 * (q & 1) + j], c2, -m_new));
  __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);   // the FMAs
  __builtin_amdgcn_sched_group_barrier(0x400, 32, 0);   // the exponentials
  float part[4] = {-0.f, -0.f, -0.f, -0.f};
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int j = 0; j < 8; ++j) part[q] += p[q][j];
    // d=128: start from the previous P, dead here (at d=64 keeping it live
    // that long costs a spill)
    w[q] = mx_pack8(p[q], sc, D == 128 ? c.pk[q] : 0);
  }
  const float lsum = (part[0] + part[1]) + (part[2] + part[3]);
  c.pk = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  c.psc = X + 127;
  c.l_run += lsum;
}

template <int D, bool CAUSAL, bool SM>
__global__ __attribute__((amdgpu_flat_work_group_size(kAttnThreads, kAttnThreads),
                          amdgpu_waves_per_eu(kAttnWavesPerSimd<D, SM>, kAttnWavesPerSimd<D, SM>)))
void attn_mx_kernel(MxArgs a) {
  constexpr int DT = D / 32;
  using G = MxGeom<D, SM>;
  __shared__ __attribute__((aligned(1024))) char smem[kRingStages * G::STAGE];

  const SeqGeom& g = a.g;
  const int nwb = ceil_div(g.N, kAttnRows);
  // causal: pair head-sequences when two of them (codes and scales per key) fit one L2
  const bool pair = CAUSAL && 2 * (int64_t)g.N * ((G::KBYTES + G::VBYTES + kMxAuxBytes) / kKBlock) <= kXcdL2Bytes;
  int wb, hb;
  work_item(xcd_remap(blockIdx.x, gridDim.x), nwb, g.H * g.B, pair, wb, hb);
  const int h = hb / g.B, b = hb % g.B;
  int64_t row0;
  int n;
  hs_rows(g, b, h, row0, n);
  const int q0 = wb * kAttnRows;
  if (q0 >= n) return;

  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, gg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = w < kAttnWaves / 2;
  const int wq_lo = q0 + 32 * w;
  const int qrow = wq_lo + r32;
  const int wq_hi = min(wq_lo + 31, n - 1);
  const bool wave_rows = wq_lo < n;

  SeqGeom gk = g;
  gk.H = g.H / a.kv_group;
  const int hk = h / a.kv_group;
  int64_t krow0;
  int kn;
  hs_rows(gk, b, hk, krow0, kn);

  const int kend = CAUSAL ? min(n, q0 + kAttnRows) : n;
  const int ntiles = ceil_div(kend, kKBlock);
  const int ntiles_seq = ceil_div(n, kKBlock);
  const uint8_t* kbase = a.k + krow0 * (D / 2);
  const int kbytes = n * (D / 2);
  const int64_t tile0 = vtile_index(gk, b, hk, 0);
  const uint8_t* vbase = a.v + tile0 * G::VBYTES;
  const int vbytes = ntiles_seq * G::VBYTES;
  const uint8_t* abase = a.aux + tile0 * kMxAuxBytes;
  const int abytes = ntiles_seq * kMxAuxBytes;
  constexpr int L = G::CI + 1 + (SM ? 1 : 0);
  const int nqb = ceil_div(g.N, kQBlock), npad = ceil_div(g.N, kKBlock) * kKBlock;
  const int64_t hs = (int64_t)b * g.H + h;
  SlotSrc ss{};
  if (SM)
    ss = SlotSrc{reinterpret_cast<const int32_t*>(a.qb_slots) + (hs * nqb + q0 / kQBlock) * (int64_t)npad,
                 (q0 + kQBlock < n ? 2 : 1) * npad * 4, npad};

  MxWave<D> c;
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk)
    c.qf[kk] = (qrow < n) ? *reinterpret_cast<const v4i*>(a.q + (row0 + qrow) * (D / 2) + 32 * kk + 16 * gg)
                          : v4i{0, 0, 0, 0};
  c.qsc = (qrow < n) ? *reinterpret_cast<const int*>(a.q_scale + (row0 + qrow) * 8 + 4 * gg) : 0;
  c.m_run = -__builtin_inff();
  c.l_run = 0.f;
  c.pk = v4i{0, 0, 0, 0};
  c.psc = 0;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) c.O[dt][i] = 0.f;

  if (lead) {
    const int first = min(kAhead, ntiles);
    for (int t = 0; t < first; ++t)
      issue_mx_tile<D, SM>(kbase, kbytes, vbase, vbytes, abase, abytes, t, smem + t * G::STAGE, w, lane, ss);
  }
  wait_dma<0>();
  barrier_only();

  const int nact = !wave_rows ? 0 : CAUSAL ? min(ntiles, wq_hi / kKBlock + 1) : ntiles;
  auto softmax_step = [&](int u) {
    if (u < nact) {
      const int k0 = u * kKBlock;
      const bool full = (k0 + kKBlock <= n) && (!CAUSAL || k0 + kKBlock - 1 <= wq_lo);
      if (!full) mx_mask<CAUSAL>(c.S, k0, n, qrow, gg);
      mx_softmax<D>(c, a.c2);
    }
  };
  // The MXFP4 softmax (exact tile max, per-block P scales) outlasts the
  // matrix phase: group B's softmax issues at a raised wave priority, as in
  // attn_fwd_kernel.
  for (int t = 0; t < ntiles; ++t) {
    if (lead && t + kAhead < ntiles)
      issue_mx_tile<D, SM>(kbase, kbytes, vbase, vbytes, abase, abytes, t + kAhead,
                           smem + ((t + kAhead) % kRingStages) * G::STAGE, w, lane, ss);
    if (!lead && t > 0) {
      __builtin_amdgcn_s_setprio(1);
      softmax_step(t - 1);
      __builtin_amdgcn_s_setprio(0);
    }
    if (t <= nact && nact > 0) {
      const char* cur = smem + (t % kRingStages) * G::STAGE;
      const char* prev = smem + ((t == 0 ? 0 : t - 1) % kRingStages) * G::STAGE;
      mx_matrix<D, SM>(cur, prev + G::KBYTES, cur + G::KBYTES + G::VBYTES, prev + G::KBYTES + G::VBYTES, lane,
                       r32, gg, c,
                       reinterpret_cast<const float4*>(cur + G::KBYTES + G::VBYTES + kMxAuxBytes) +
                           32 * (wq_lo / kQBlock - q0 / kQBlock));
    }
    if (lead) softmax_step(t);
    if (lead) wait_tiles<L>(max(0, min(kAhead - 1, ntiles - 2 - t)));
    barrier_only();
  }
  if (!lead && ntiles > 0) softmax_step(ntiles - 1);
  if (nact == ntiles && ntiles > 0) {
    // PV of the last tile (its QKᵀ part is not needed)
    const char* prev = smem + ((ntiles - 1) % kRingStages) * G::STAGE;
    const v4i* lv = reinterpret_cast<const v4i*>(prev + G::KBYTES);
    const int vsc = *reinterpret_cast<const int*>(prev + G::KBYTES + G::VBYTES + 512 + 4 * lane);
    c.O[0] = mx_mfma<0, 0>(lv[0 * 64 + lane], c.pk, c.O[0], vsc, c.psc);
    c.O[1] = mx_mfma<1, 0>(lv[1 * 64 + lane], c.pk, c.O[1], vsc, c.psc);
    if (D == 128) {
      c.O[DT - 2] = mx_mfma<2, 0>(lv[(DT - 2) * 64 + lane], c.pk, c.O[DT - 2], vsc, c.psc);
      c.O[DT - 1] = mx_mfma<3, 0>(lv[(DT - 1) * 64 + lane], c.pk, c.O[DT - 1], vsc, c.psc);
    }
  }

  const float l_tot = pair_sum(c.l_run);
  if (!wave_rows || qrow >= n) return;
  const float inv = 1.f / l_tot;
  if (a.lse && gg == 0) a.lse[row0 + qrow] = (c.m_run + __builtin_log2f(l_tot)) * 0.6931471805599453f;
  uint16_t* __restrict__ orow = a.o + (row0 + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * dt + 8 * q4 + 4 * gg;
      v2h lo = {(_Float16)(c.O[dt][4 * q4] * inv), (_Float16)(c.O[dt][4 * q4 + 1] * inv)};
      v2h hi = {(_Float16)(c.O[dt][4 * q4 + 2] * inv), (_Float16)(c.O[dt][4 * q4 + 3] * inv)};
      uint2 stv;
      stv.x = __builtin_bit_cast(uint32_t, lo);
      stv.y = __builtin_bit_cast(uint32_t, hi);
      *reinterpret_cast<uint2*>(orow + d) = stv;
    }
}

void launch_attn_mx(const MxArgs& a, bool causal, hipStream_t st) {
  const int64_t blocks = (int64_t)a.g.B * a.g.H * ceil_div(a.g.N, kAttnRows);
  const dim3 grid((unsigned)blocks), block(kAttnThreads);
  const bool sm = a.qb_slots != nullptr;
#define SAGE_MX(DD, CS)                                                                   \
  do {                                                                                    \
    if (sm)                                                                               \
      hipLaunchKernelGGL((attn_mx_kernel<DD, CS, true>), grid, block, 0, st, a);          \
    else                                                                                  \
      hipLaunchKernelGGL((attn_mx_kernel<DD, CS, false>), grid, block, 0, st, a);         \
  } while (0)
  if (a.g.d == 128) {
    if (causal) SAGE_MX(128, true); else SAGE_MX(128, false);
  } else {
    if (causal) SAGE_MX(64, true); else SAGE_MX(64, false);
  }
#undef SAGE_MX
}

// Test hook: the int32 Q̂K̂ᵀ tiles computed by the attention kernel's own tile
// DMA and matrix phase (matrix_both, FP16 PV: the K̂ fragment offsets computed
// once, the accumulator start value held in registers at d=128), with a zero
// P against the zero V half of the stage, so that only the QKᵀ part counts.
template <int D>
__global__ __launch_bounds__(kThreads) void qk_tiles_kernel(const int8_t* __restrict__ q, const int8_t* __restrict__ k,
                                                            int B, int H, int N, const int32_t* __restrict__ list,
                                                            int32_t* __restrict__ out) {
  using G = TileGeom<D, false>;
  __shared__ __attribute__((aligned(1024))) char smem[G::STAGE];
  const int idx = blockIdx.x;
  const int b = list[4 * idx], h = list[4 * idx + 1], qb = list[4 * idx + 2], kb = list[4 * idx + 3];
  int32_t* o = out + (int64_t)idx * kQBlock * kKBlock;
  if (b < 0 || b >= B || h < 0 || h >= H || qb < 0 || qb * kQBlock >= N || kb < 0 || kb * kKBlock >= N) {
    for (int i = threadIdx.x; i < kQBlock * kKBlock; i += kThreads) o[i] = 0;  // out-of-range entry
    return;
  }
  const int64_t row0 = ((int64_t)b * H + h) * N;
  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, gg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the V half of the stage is not used here: a zero-size range reads zeros
  issue_tile<D, false>(k + row0 * D, N * D, k, 0, kb, smem, w, lane);
  wait_dma_and_sync<0>();
  v4i qf[D / 32];
  load_q_frags<D>(qf, q + row0 * D, qb * kQBlock + 32 * w + r32, N, gg);
  int kofs[D / 32];
  k_frag_offsets<D>(r32, gg, kofs);
  v16i mg;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int m = kMagicI;
    if (D == 128) asm volatile("" : "+v"(m));
    mg[i] = m;
  }
  v8h pk16[4];
  v16f O[D / 32];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) pk16[kc] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[dt][i] = 0.f;
  const v8i pk8 = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  v16i S[2];
  matrix_both<D, false, false>(smem, kofs, smem + G::KBYTES, lane, gg, qf, S, pk16, pk8, O, nullptr,
                               D == 128 ? &mg : nullptr);
  // keep the whole (zero) PV result live so that the phase is compiled as in the forward
  float z = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) z += O[dt][i];
  if (z != 0.f) o[0] = -1;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 32 * s + 8 * (i >> 2) + 4 * gg + (i & 3);
      o[(32 * w + r32) * kKBlock + key] = S[s][i] - kMagicI;
    }
}

void launch_attn(const AttnArgs& a, bool causal, bool fp8, hipStream_t st) {
  const int64_t blocks = (int64_t)a.g.B * a.g.H * ceil_div(a.g.N, kAttnRows);
  const dim3 grid((unsigned)blocks), block(kAttnThreads);
  const int qm = a.qb_slots != nullptr ? kQmSmooth : a.q_per_token ? kQmToken : kQmBlock;
#define SAGE_ATTN(DD, F8, CS)                                                                  \
  do {                                                                                         \
    if (qm == kQmSmooth)                                                                       \
      hipLaunchKernelGGL((attn_fwd_kernel<DD, F8, CS, kQmSmooth>), grid, block, 0, st, a);     \
    else if (qm == kQmToken)                                                                   \
      hipLaunchKernelGGL((attn_fwd_kernel<DD, F8, CS, kQmToken>), grid, block, 0, st, a);      \
    else                                                                                       \
      hipLaunchKernelGGL((attn_fwd_kernel<DD, F8, CS, kQmBlock>), grid, block, 0, st, a);      \
  } while (0)
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
