// Host-side launchers shared between the C ABI and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "sage_common.h"

namespace sage {

struct AttnArgs {
  const int8_t* q;         // Q codes, same layout as the fp16 input
  const int8_t* k;         // K codes (H / kv_group heads)
  const float* q_scale;    // [B][H][nqb] (per token: indexed like the Q rows), softmax scale folded in
  const float* k_scale;    // [B][Hkv][nkb]
  const uint8_t* v;        // FP16 PV: the fp16 input V itself; FP8: packed e4m3 tiles (Hkv heads)
  const float* v_scale;    // [B][Hkv][d] (FP8 mode)
  uint16_t* o;             // fp16 output, same layout as the input
  float* lse;              // optional fp32 log-sum-exp per query row, or nullptr
  SeqGeom g;               // geometry of Q and O (H query heads)
  int kv_group;            // query heads per K/V head: K/V head of h is h / kv_group
  // smoothed Q (all nullptr otherwise): per (Q block, key) accumulator initial
  // values [B][H][nqb][npad], per (Q block, tile, half) fallback flags
  // [B][H][nqb][2*nkb], fp32 terms [B][H][nqb][npad] (npad = 64*nkb) and per
  // (Q block) row summaries [B][H][nqb] (nonzero: some half of the row falls back)
  const int32_t* qb_slots = nullptr;
  const float* qb_fix = nullptr;
  const int32_t* qb_flags = nullptr;
  const int32_t* qb_any = nullptr;
  bool q_per_token = false;  // q_scale holds one scale per query row
  // per-block Q (neither option): when set, the attention kernel quantises the
  // fp16 Q itself (q and q_scale unused) with the softmax scale sm_scale
  const uint16_t* q16 = nullptr;
  float sm_scale = 0.f;
};

// MXFP4 attention (the operands of launch_mx_prepare).
struct MxArgs {
  const uint8_t* q;        // e2m1 codes [rows][d/2]
  const uint8_t* q_scale;  // E8M0 bytes [rows][2 dwords]: dword g, byte kk = block 2kk + g
  const uint8_t* k;        // e2m1 codes of the smoothed K [Hkv rows][d/2]
  const uint8_t* v;        // packed V tiles (e2m1 codes)
  const uint8_t* aux;      // per K/V tile: K scales (by LDS row) and V scales
  uint16_t* o;
  float* lse;
  SeqGeom g;
  int kv_group;
  float c2;                // softmax scale times log2(e)
  const float* qb_slots = nullptr;  // smoothed Q: the term q̄·x per (Q block, key), [B][H][nqb][npad]
};

// Inputs and outputs of the Q-smoothing term kernel (smooth_q.hip).
struct QBiasArgs {
  const uint16_t* k;       // fp16 K, Hkv heads
  const float* k_mean;     // [B][Hkv][d]
  const float* k_scale;    // [B][Hkv][nkb]
  const float* q_mean;     // [B][H][nqb][d]
  const float* q_scale;    // [B][H][nqb], softmax scale folded in
  int32_t* slots;          // [B][H][nqb][npad]
  float* fix;              // [B][H][nqb][npad]
  int32_t* flags;          // [B][H][nqb][2*nkb]
  int32_t* any;            // [B][H][nqb], zero on entry: set where a half of the row falls back
  SeqGeom g;               // geometry of Q (H query heads)
  int kv_group;
  float sm_log2e;          // softmax scale times log2(e)
  int causal;              // skip (block, tile) pairs no query of the block sees
  int raw = 0;             // MXFP4: write q̄·x (fp32, raw score units) for every key; no flags
};

void launch_zero(void* p, size_t bytes, hipStream_t st);
void launch_quant_qk(const SeqGeom& gq, const SeqGeom& gk, const void* q, const void* k, float sm_scale,
                     int8_t* q_int8, int8_t* k_int8, float* q_scale, float* k_scale, float* k_mean,
                     float* q_mean, bool q_per_token, long long* colsum, hipStream_t st);
void launch_q_bias(const QBiasArgs& a, hipStream_t st);
void launch_v_scale(const SeqGeom& g, const void* v, float* v_scale, hipStream_t st);
void launch_mx_prepare(const SeqGeom& gq, const SeqGeom& gk, const void* q, const void* k, const void* v,
                       uint8_t* q_codes, uint8_t* q_scales, uint8_t* k_codes, uint8_t* aux, uint8_t* v_codes,
                       float* k_mean, float* q_mean, long long* colsum, hipStream_t st);
void launch_v_prepare(const SeqGeom& g, const void* v, const float* v_scale, bool fp8, bool rowmajor,
                      void* out, hipStream_t st);
void launch_attn(const AttnArgs& a, bool causal, bool fp8, hipStream_t st);
void launch_attn_mx(const MxArgs& a, bool causal, hipStream_t st);
void launch_qk_tiles(const int8_t* q, const int8_t* k, int B, int H, int N, int d, const int32_t* list,
                     int n, int32_t* out, hipStream_t st);

}  // namespace sage
