// Device-side definitions shared by the pre-pass and attention kernels.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA matrix cores, 160 KB LDS/CU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

// Geometry of the method (dtcms SageAttention summary, "SageAttention（v1）":
// per-block quantisation; block sizes are this implementation's reading).
constexpr int kQBlock = 128;  // tokens per Q scale block == queries per workgroup
constexpr int kKBlock = 64;   // tokens per K scale block == keys per attention tile
constexpr int kThreads = 256; // 4 wavefronts of 64
constexpr float kInt8Max = 127.0f;
constexpr float kE4M3Max = 448.0f;
constexpr int kMxAuxBytes = 1024;  // MXFP4: per K/V tile, K scales (512 B) + V scales (256 B) + pad

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

// One "head-sequence": a (batch entry, head) of a dense [B,H,N,d] tensor or a
// (sequence, head) of a packed [H,T,d] tensor.  Everything the method does per
// block, mean or mask stays inside one head-sequence.
struct SeqGeom {
  const int32_t* cu;  // varlen offsets (device) or nullptr for dense
  int B;              // batch size (dense) or number of sequences (varlen)
  int H;
  int N;              // tokens per sequence (dense) or maximum length (varlen)
  int d;
  int64_t T;          // total packed tokens (varlen)
};

// First token row (in units of d elements) and length of head-sequence (b, h).
__device__ __forceinline__ void hs_rows(const SeqGeom& g, int b, int h, int64_t& row0, int& n) {
  if (g.cu) {
    const int s = g.cu[b], e = g.cu[b + 1];
    n = e - s;
    row0 = (int64_t)h * g.T + s;
  } else {
    n = g.N;
    row0 = ((int64_t)b * g.H + h) * g.N;
  }
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Packed-V tiles: one tile = 64 keys x d channels, laid out in the order the
// attention kernel's MFMA lanes consume it.  Dense: tiles of head-sequence
// (b,h) are contiguous.  Varlen: head-major; sequence i of head h starts at
// tile floor(cu[i]/64) + i, which never overlaps its neighbours and needs only
// cu[i] to compute.
__host__ __device__ __forceinline__ int64_t vtiles_per_head_varlen(int64_t T, int nseq) {
  return ceil_div64(T, kKBlock) + nseq;
}
__device__ __forceinline__ int64_t vtile_index(const SeqGeom& g, int b, int h, int kb) {
  if (g.cu) {
    return (int64_t)h * vtiles_per_head_varlen(g.T, g.B) + g.cu[b] / kKBlock + b + kb;
  }
  return ((int64_t)b * g.H + h) * ceil_div(g.N, kKBlock) + kb;
}

// Map a workgroup id onto a logical work index so that consecutive logical
// indices run on the same XCD.  Workgroups are dispatched round-robin over the
// 8 XCDs; XCD x receives ids x, x+8, ...; it is given the contiguous logical
// range [x*q + min(x, r), ...) where total = 8q + r.  A bijection on [0,total).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, r = total % kXcd;
  const int x = bid % kXcd, local = bid / kXcd;
  return x * q + (x < r ? x : r) + local;
}

// Query block wb (of nwb) and head-sequence hb (of nhb) of a logical work
// index.  By default the blocks of one head-sequence are consecutive,
// heaviest (last) first, so an XCD streams one head-sequence's K/V through
// its L2 at a time.  With `pair` (causal, where block wb costs wb + 1 units)
// the blocks of head-sequences 2p and 2p + 1 alternate, heaviest first: that
// evens out the end of each XCD's run (in a greedy-dispatch model at
// 4x32x4096, 16 % over the balanced time one head-sequence at a time, 6 % in
// pairs), at the price of two head-sequences' K/V in L2 at once, so callers
// pair only when both fit.  A bijection on [0, nwb·nhb).
__device__ __forceinline__ void work_item(int logical, int nwb, int nhb, bool pair, int& wb, int& hb) {
  if (!pair) {
    wb = nwb - 1 - logical % nwb;
    hb = logical / nwb;
    return;
  }
  const int p = logical / (2 * nwb), i = logical % (2 * nwb);
  if (2 * p + 1 < nhb) {
    wb = nwb - 1 - i / 2;
    hb = 2 * p + (i & 1);
  } else {  // the last head-sequence of an odd count
    wb = nwb - 1 - i;
    hb = 2 * p;
  }
}

// One XCD's L2 (MI355X: 4 MB): the bound for pairing head-sequences.
constexpr int64_t kXcdL2Bytes = int64_t(4) << 20;

// Symmetric INT8 code of x for a block scale s > 0: rint of the IEEE fp32
// quotient fl32(x/s), clamped to ±127.  The quotient is first formed as
// y = fl32(x·r) with r = fl32(1/s): since |x/s| <= 127·(1 + 2^-23), y lies
// within 2.3e-5 of fl32(x/s), so rint(y) is the same integer unless y is within
// that distance of a half-integer; only then is the exact quotient divided out.
constexpr float kTieGuard = 6.103515625e-05f;  // 2^-14 > 2.3e-5

static __device__ __attribute__((noinline)) float exact_code(float x, float s) { return __builtin_rintf(x / s); }

__device__ __forceinline__ int int8_code(float x, float s, float r) {
  const float y = x * r;
  float c = __builtin_rintf(y);
  if (__builtin_expect(__builtin_fabsf(__builtin_fabsf(y - c) - 0.5f) <= kTieGuard, 0)) c = exact_code(x, s);
  return (int)__builtin_amdgcn_fmed3f(c, -kInt8Max, kInt8Max);
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

// MXFP4 block exponent (OCP microscaling, E8M0 range): the smallest X with
// amax <= 6·2^X, 6 being e2m1's largest value.  With amax = f·2^e,
// f in [0.5, 1): X = e - 3 + (f > 0.75); clamped to [-127, 127]; amax = 0
// gives -127.
__device__ __forceinline__ int mx_exponent(float amax) {
  int e = 0;
  const float f = frexpf(amax, &e);
  const int X = e - 3 + (f > 0.75f ? 1 : 0);
  return amax > 0.f ? max(-127, min(127, X)) : -127;
}

// Eight values as e2m1 nibbles of fp4(x / scale) (value j at bits 4j; round to
// nearest even, saturating at ±6 — the hardware conversion).
// The four conversions fill all four bytes, so `init` (any value, e.g. a dead
// register) only spares clearing one first.
__device__ __forceinline__ uint32_t mx_pack8(const float (&x)[8], float scale, int init = 0) {
  int w = init;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0], x[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4], x[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6], x[7], scale, 3);
  return (uint32_t)w;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace sage
