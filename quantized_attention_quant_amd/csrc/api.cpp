// C ABI of the 8-bit attention forward (declarations and contracts in
// include/sage.h).  Every argument is validated on the host before anything
// is enqueued; on error nothing is launched.
#include "sage.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "sage_internal.h"

// Scratch of the allocation-free forward (sage_attn_fwd_noalloc): a device
// array the library owns, one copy per GPU, living until the process ends.
// Host code never passes the array's name to a kernel (in host code it is only
// a stand-in for the symbol): it looks up each device's copy once with
// hipGetSymbolAddress and passes that address.
static __device__ __align__(256) unsigned char scratch[SAGE_NOALLOC_SCRATCH_BYTES];

namespace {

using sage::ceil_div64;
using sage::SeqGeom;

constexpr size_t kWsAlign = 256;
constexpr int64_t kMaxTokensPerSeq = int64_t(1) << 23;  // keeps the int64 fixed-point K sums exact

inline size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }
inline size_t align16(size_t x) { return (x + 15) / 16 * 16; }
// The per-row fallback summaries follow the flags inside region [11].
inline int32_t* row_summaries(char* flags, int B, int H, int N) {
  const size_t qblocks = (size_t)B * H * ceil_div64(N, sage::kQBlock);
  return reinterpret_cast<int32_t*>(flags + align16(sizeof(int32_t) * qblocks * (size_t)(2 * ceil_div64(N, sage::kKBlock))));
}
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("SAGE_DEBUG");
    return e && e[0] == '1';
  }();
  return on;
}

// Offsets inside the attention workspace:
// [0] q_int8 [1] k_int8 [2] q_scale [3] k_scale [4] k_mean [5] packed V (fp8)
// [6] v_scale (fp8) [7] int64 K column sums; with a smoothed Q [8] q_mean,
// [9] accumulator initial values, [10] fp32 fallback terms, [11] fallback
// flags; total returned separately.
constexpr int kWsRegions = 12;
struct WsLayout {
  size_t off[kWsRegions];
  size_t total;
};

WsLayout make_layout(bool varlen, int B, int H, int Hkv, int N, int64_t T, int d, sage_pv_mode_t pv_mode,
                     int options) {
  const bool fp8 = pv_mode == SAGE_PV_FP8_E4M3;
  const bool smooth_q = (options & SAGE_OPT_SMOOTH_Q) != 0;
  const bool q_per_token = (options & SAGE_OPT_Q_PER_TOKEN) != 0;
  const int64_t tokens = varlen ? (int64_t)H * T : (int64_t)B * H * N;
  const int64_t ktokens = varlen ? (int64_t)Hkv * T : (int64_t)B * Hkv * N;
  const int64_t nqb = ceil_div64(N, sage::kQBlock), nkb = ceil_div64(N, sage::kKBlock);
  const int64_t vtiles = varlen ? (int64_t)Hkv * sage::vtiles_per_head_varlen(T, B) : (int64_t)B * Hkv * nkb;
  if (pv_mode == SAGE_MXFP4) {
    // [0] Q e2m1 codes [1] K codes [2] Q scales (8 B per row) [3] per-tile
    // K/V scales [4] k_mean [5] packed V codes [7] K column sums; with a
    // smoothed Q [8] q_mean and [9] the fp32 score term per (Q block, key)
    const size_t qblocks = smooth_q ? (size_t)B * H * nqb : 0;
    const size_t sizes[kWsRegions] = {
        (size_t)(tokens * d / 2), (size_t)(ktokens * d / 2), (size_t)tokens * 8,
        (size_t)vtiles * sage::kMxAuxBytes, sizeof(float) * (size_t)B * Hkv * d,
        (size_t)vtiles * sage::kKBlock * d / 2, 0, sizeof(long long) * (size_t)B * Hkv * d,
        sizeof(float) * qblocks * d, sizeof(float) * qblocks * (size_t)(nkb * sage::kKBlock), 0, 0};
    WsLayout L;
    size_t cur = 0;
    for (int i = 0; i < kWsRegions; ++i) {
      L.off[i] = cur;
      cur = align_up(cur + sizes[i]);
    }
    L.total = cur;
    return L;
  }
  const size_t qblocks = (size_t)B * H * nqb;  // (sequence, head, Q block) rows
  const size_t sq = smooth_q ? 1 : 0;
  const size_t sizes[kWsRegions] = {
      (size_t)(tokens * d),
      (size_t)(ktokens * d),
      sizeof(float) * (q_per_token ? (size_t)tokens : (size_t)B * H * nqb),
      sizeof(float) * (size_t)B * Hkv * nkb,
      sizeof(float) * (size_t)B * Hkv * d,
      fp8 ? (size_t)vtiles * sage::kKBlock * d : 0,  // FP16 PV reads the input V itself
      fp8 ? sizeof(float) * (size_t)B * Hkv * d : 0,
      sizeof(long long) * (size_t)B * Hkv * d,
      sq * sizeof(float) * qblocks * d,
      sq * sizeof(int32_t) * qblocks * (size_t)(nkb * sage::kKBlock),
      sq * sizeof(float) * qblocks * (size_t)(nkb * sage::kKBlock),
      // fallback flags, then (16-byte aligned) the per-row summaries
      sq * (align16(sizeof(int32_t) * qblocks * (size_t)(2 * nkb)) + align16(sizeof(int32_t) * qblocks)),
  };
  WsLayout L;
  size_t cur = 0;
  for (int i = 0; i < kWsRegions; ++i) {
    L.off[i] = cur;
    cur = align_up(cur + sizes[i]);
  }
  L.total = cur;
  return L;
}

// K/V heads: 1 <= Hkv <= H and Hkv divides H (grouped-query / multi-query).
inline bool kv_heads_ok(int H, int Hkv) { return Hkv >= 1 && Hkv <= H && H % Hkv == 0; }

constexpr int kKnownOptions = SAGE_OPT_SMOOTH_Q | SAGE_OPT_Q_PER_TOKEN;
inline bool options_known(int o) { return (o & ~kKnownOptions) == 0; }
// Q smoothing carries its term in units of a per-block δQ: not with per-token scales.
inline bool options_supported(int o) { return (o & kKnownOptions) != kKnownOptions; }
inline bool pv_mode_ok(sage_pv_mode_t m) { return m == SAGE_PV_FP16 || m == SAGE_PV_FP8_E4M3 || m == SAGE_MXFP4; }
// MXFP4 has its own Q scales (E8M0 per 32 channels, one row each): Q smoothing
// only, no per-token option.
inline bool mode_options_supported(sage_pv_mode_t m, int o) {
  return options_supported(o) && (m != SAGE_MXFP4 || (o & SAGE_OPT_Q_PER_TOKEN) == 0);
}

sage_status_t check_dims(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return SAGE_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != 128) return SAGE_ERR_INVALID_ARGUMENT;
  if (B > 65535 || H > 65535 || N > kMaxTokensPerSeq) return SAGE_ERR_INVALID_ARGUMENT;
  const int64_t blocks = (int64_t)B * H * ceil_div64(N, sage::kQBlock);
  if (blocks > 0x7fffffffLL) return SAGE_ERR_INVALID_ARGUMENT;
  return SAGE_OK;
}

bool resolve_sm_scale(float in, int d, float* out) {
  if (std::isnan(in) || std::isinf(in)) return false;
  *out = in > 0.f ? in : (float)(1.0 / std::sqrt((double)d));
  return true;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

sage_status_t finish(hipStream_t st) {
  if (hipGetLastError() != hipSuccess) return SAGE_ERR_DEVICE;
  if (debug_sync()) {
    const hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
      std::fprintf(stderr, "sage: device error %s\n", hipGetErrorString(e));
      return SAGE_ERR_DEVICE;
    }
  }
  return SAGE_OK;
}

// Shared body of the dense and varlen forward.  g: geometry of Q and O; K and V
// have Hkv heads over the same sequences.
sage_status_t attn_forward(const void* q, const void* k, const void* v, void* o, float* lse, const SeqGeom& g,
                           int Hkv, bool varlen, int is_causal, sage_pv_mode_t pv_mode, int options,
                           float sm_scale, void* workspace, size_t workspace_bytes, sage_stream_t stream) noexcept {
  if (!q || !k || !v || !o || !workspace) return SAGE_ERR_INVALID_ARGUMENT;
  if (!kv_heads_ok(g.H, Hkv)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SAGE_ERR_INVALID_ARGUMENT;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return SAGE_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(workspace) % kWsAlign) != 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (!pv_mode_ok(pv_mode)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!options_known(options)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!mode_options_supported(pv_mode, options)) return SAGE_ERR_UNSUPPORTED;
  float sm;
  if (!resolve_sm_scale(sm_scale, g.d, &sm)) return SAGE_ERR_INVALID_ARGUMENT;
  const bool fp8 = pv_mode == SAGE_PV_FP8_E4M3;
  const bool sq = (options & SAGE_OPT_SMOOTH_Q) != 0;
  const bool qtok = (options & SAGE_OPT_Q_PER_TOKEN) != 0;
  const WsLayout L = make_layout(varlen, g.B, g.H, Hkv, g.N, g.T, g.d, pv_mode, options);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE_TOO_SMALL;
  const int64_t rows = varlen ? (int64_t)g.H * g.T : (int64_t)g.B * g.H * g.N;
  const size_t tensor_bytes = (size_t)rows * g.d * 2;
  const size_t kv_bytes = tensor_bytes / (size_t)g.H * (size_t)Hkv;
  const size_t lse_bytes = lse ? (size_t)rows * sizeof(float) : 0;
  if (overlaps(o, tensor_bytes, q, tensor_bytes) || overlaps(o, tensor_bytes, k, kv_bytes) ||
      overlaps(o, tensor_bytes, v, kv_bytes) || overlaps(o, tensor_bytes, workspace, L.total))
    return SAGE_ERR_INVALID_ARGUMENT;
  // the kernels read q, k and v after the pre-pass has written the workspace
  // (fp16 V in place, K again for the smoothing term, Q in the attention kernel)
  if (overlaps(workspace, L.total, q, tensor_bytes) || overlaps(workspace, L.total, k, kv_bytes) ||
      overlaps(workspace, L.total, v, kv_bytes))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (lse && (overlaps(lse, lse_bytes, o, tensor_bytes) || overlaps(lse, lse_bytes, q, tensor_bytes) ||
              overlaps(lse, lse_bytes, k, kv_bytes) || overlaps(lse, lse_bytes, v, kv_bytes) ||
              overlaps(lse, lse_bytes, workspace, L.total)))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (tensor_bytes == 0) return SAGE_OK;  // varlen with no tokens at all

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  SeqGeom gk = g;
  gk.H = Hkv;
  if (pv_mode == SAGE_MXFP4) {
    uint8_t* aux = reinterpret_cast<uint8_t*>(ws + L.off[3]);
    sage::launch_zero(aux, L.off[4] - L.off[3], st);  // K scales of rows past a sequence's end stay 0
    float* km = reinterpret_cast<float*>(ws + L.off[4]);
    float* qm = sq ? reinterpret_cast<float*>(ws + L.off[8]) : nullptr;
    float* terms = reinterpret_cast<float*>(ws + L.off[9]);
    sage::launch_mx_prepare(g, gk, q, k, v, reinterpret_cast<uint8_t*>(ws + L.off[0]),
                            reinterpret_cast<uint8_t*>(ws + L.off[2]), reinterpret_cast<uint8_t*>(ws + L.off[1]), aux,
                            reinterpret_cast<uint8_t*>(ws + L.off[5]), km, qm,
                            reinterpret_cast<long long*>(ws + L.off[7]), st);
    if (sq) {
      // q̄·x in raw score units: the kernel applies the softmax scale to the sum
      sage::QBiasArgs qa{static_cast<const uint16_t*>(k), km, nullptr, qm, nullptr,
                         reinterpret_cast<int32_t*>(terms), nullptr, nullptr, nullptr, g, g.H / Hkv, 1.0f,
                         is_causal != 0};
      qa.raw = 1;
      sage::launch_q_bias(qa, st);
    }
    sage::MxArgs a{reinterpret_cast<const uint8_t*>(ws + L.off[0]), reinterpret_cast<const uint8_t*>(ws + L.off[2]),
                   reinterpret_cast<const uint8_t*>(ws + L.off[1]), reinterpret_cast<const uint8_t*>(ws + L.off[5]),
                   aux, static_cast<uint16_t*>(o), lse, g, g.H / Hkv, (float)((double)sm * 1.4426950408889634)};
    if (sq) a.qb_slots = terms;
    sage::launch_attn_mx(a, is_causal != 0, st);
    return finish(st);
  }
  int8_t* q8 = reinterpret_cast<int8_t*>(ws + L.off[0]);
  int8_t* k8 = reinterpret_cast<int8_t*>(ws + L.off[1]);
  float* qs = reinterpret_cast<float*>(ws + L.off[2]);
  float* ks = reinterpret_cast<float*>(ws + L.off[3]);
  float* km = reinterpret_cast<float*>(ws + L.off[4]);
  uint8_t* vp = reinterpret_cast<uint8_t*>(ws + L.off[5]);
  float* vs = reinterpret_cast<float*>(ws + L.off[6]);
  long long* colsum = reinterpret_cast<long long*>(ws + L.off[7]);
  float* qm = sq ? reinterpret_cast<float*>(ws + L.off[8]) : nullptr;
  int32_t* slots = reinterpret_cast<int32_t*>(ws + L.off[9]);
  float* fix = reinterpret_cast<float*>(ws + L.off[10]);
  int32_t* flags = reinterpret_cast<int32_t*>(ws + L.off[11]);

  // Q without smoothing (per block or per token): the attention kernel
  // quantises the fp16 Q itself (the same quantiser), so the pre-pass neither
  // writes nor the kernel reads Q̂ and δQ
  const bool qfuse = !sq;
  sage::launch_quant_qk(g, gk, q, k, sm, qfuse ? nullptr : q8, k8, qfuse ? nullptr : qs, ks, km, qm, qtok, colsum,
                        st);
  int32_t* any = sq && !fp8 ? row_summaries(ws + L.off[11], g.B, g.H, g.N) : nullptr;
  if (sq && fp8) {
    // FP8 PV: every key's term in fp32, sm_scale·q̄·x·log2(e), in region [10]
    sage::QBiasArgs qa{static_cast<const uint16_t*>(k), km, nullptr, qm, nullptr, reinterpret_cast<int32_t*>(fix),
                       nullptr, nullptr, nullptr, g, g.H / Hkv, (float)((double)sm * 1.4426950408889634),
                       is_causal != 0};
    qa.raw = 1;
    sage::launch_q_bias(qa, st);
  } else if (sq) {
    sage::launch_zero(any, align16(sizeof(int32_t) * (size_t)g.B * g.H * ceil_div64(g.N, sage::kQBlock)), st);
    const sage::QBiasArgs qa{static_cast<const uint16_t*>(k), km, ks, qm, qs, slots, fix, flags, any, g, g.H / Hkv,
                             (float)((double)sm * 1.4426950408889634), is_causal != 0};
    sage::launch_q_bias(qa, st);
  }
  if (fp8) {
    sage::launch_v_scale(gk, v, vs, st);
    sage::launch_v_prepare(gk, v, vs, /*fp8=*/true, /*rowmajor=*/false, vp, st);
  }
  // FP16 PV: the kernel reads V's fp16 rows directly (no copy)
  sage::AttnArgs a{q8, k8, qs, ks, fp8 ? vp : static_cast<const uint8_t*>(v), vs, static_cast<uint16_t*>(o), lse, g,
                   g.H / Hkv};
  a.q_per_token = qtok;
  if (qfuse) {
    a.q16 = static_cast<const uint16_t*>(q);
    a.sm_scale = sm;
  }
  if (sq) {
    // FP8 PV streams the fp32 terms with the tiles in place of initial values
    a.qb_slots = fp8 ? reinterpret_cast<const int32_t*>(fix) : slots;
    a.qb_fix = fix;
    a.qb_flags = fp8 ? nullptr : flags;
    a.qb_any = any;
  }
  sage::launch_attn(a, is_causal != 0, fp8, st);
  return finish(st);
}

sage_status_t varlen_geom(const int32_t* cu, int nseq, int max_seqlen, int64_t total_tokens, int H, int d,
                          SeqGeom* g) {
  if (!cu) return SAGE_ERR_INVALID_ARGUMENT;
  if (nseq < 1 || total_tokens < 0) return SAGE_ERR_INVALID_ARGUMENT;
  const sage_status_t s = check_dims(nseq, H, max_seqlen, d);
  if (s != SAGE_OK) return s;
  if (total_tokens > (int64_t)nseq * max_seqlen) return SAGE_ERR_INVALID_ARGUMENT;
  if (total_tokens > 0x7fffffffLL) return SAGE_ERR_INVALID_ARGUMENT;  // cu_seqlens are int32
  *g = SeqGeom{cu, nseq, H, max_seqlen, d, total_tokens};
  return SAGE_OK;
}


// The attention kernel alone on a workspace a preceding forward filled (the
// sage_test_attn_*from_workspace hooks); g: geometry of Q and O.
sage_status_t attn_from_workspace(void* o, const void* q, const void* v, const SeqGeom& g, int H_kv, bool varlen,
                                  int is_causal, sage_pv_mode_t pv_mode, int options, const void* workspace,
                                  size_t workspace_bytes, sage_stream_t stream) {
  const int H = g.H, d = g.d;
  if (!kv_heads_ok(H, H_kv)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!o || !workspace || !aligned16(o) || (reinterpret_cast<uintptr_t>(workspace) % kWsAlign) != 0)
    return SAGE_ERR_INVALID_ARGUMENT;
  if (!pv_mode_ok(pv_mode)) return SAGE_ERR_INVALID_ARGUMENT;
  if (pv_mode == SAGE_PV_FP16 && (!v || !aligned16(v))) return SAGE_ERR_INVALID_ARGUMENT;
  if (!options_known(options)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!mode_options_supported(pv_mode, options)) return SAGE_ERR_UNSUPPORTED;
  // Q without smoothing: the attention kernel quantises q itself, or, with q
  // NULL, reads Q̂ and δQ from regions [0] and [2]
  const bool qfuse = pv_mode != SAGE_MXFP4 && (options & SAGE_OPT_SMOOTH_Q) == 0 && q != nullptr;
  if (qfuse && !aligned16(q)) return SAGE_ERR_INVALID_ARGUMENT;
  const bool fp8 = pv_mode == SAGE_PV_FP8_E4M3;
  const WsLayout L = make_layout(varlen, g.B, H, H_kv, g.N, g.T, d, pv_mode, options);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE_TOO_SMALL;
  const int64_t rows = varlen ? (int64_t)H * g.T : (int64_t)g.B * H * g.N;
  const size_t tensor_bytes = (size_t)rows * d * 2;
  const size_t kv_bytes = tensor_bytes / (size_t)H * (size_t)H_kv;
  if (overlaps(o, tensor_bytes, workspace, L.total)) return SAGE_ERR_INVALID_ARGUMENT;
  if (pv_mode == SAGE_PV_FP16 && (overlaps(o, tensor_bytes, v, kv_bytes) || overlaps(workspace, L.total, v, kv_bytes)))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (qfuse && (overlaps(o, tensor_bytes, q, tensor_bytes) || overlaps(workspace, L.total, q, tensor_bytes)))
    return SAGE_ERR_INVALID_ARGUMENT;
  const char* ws = static_cast<const char*>(workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (pv_mode == SAGE_MXFP4) {
    float sm;
    resolve_sm_scale(0.f, d, &sm);
    sage::MxArgs a{reinterpret_cast<const uint8_t*>(ws + L.off[0]), reinterpret_cast<const uint8_t*>(ws + L.off[2]),
                   reinterpret_cast<const uint8_t*>(ws + L.off[1]), reinterpret_cast<const uint8_t*>(ws + L.off[5]),
                   reinterpret_cast<const uint8_t*>(ws + L.off[3]), static_cast<uint16_t*>(o), nullptr, g,
                   H / H_kv, (float)((double)sm * 1.4426950408889634)};
    if (options & SAGE_OPT_SMOOTH_Q) a.qb_slots = reinterpret_cast<const float*>(ws + L.off[9]);
    sage::launch_attn_mx(a, is_causal != 0, st);
    return finish(st);
  }
  sage::AttnArgs a{reinterpret_cast<const int8_t*>(ws + L.off[0]), reinterpret_cast<const int8_t*>(ws + L.off[1]),
                   reinterpret_cast<const float*>(ws + L.off[2]), reinterpret_cast<const float*>(ws + L.off[3]),
                   fp8 ? reinterpret_cast<const uint8_t*>(ws + L.off[5]) : static_cast<const uint8_t*>(v),
                   reinterpret_cast<const float*>(ws + L.off[6]), static_cast<uint16_t*>(o), nullptr, g, H / H_kv};
  a.q_per_token = (options & SAGE_OPT_Q_PER_TOKEN) != 0;
  if (qfuse) {
    a.q16 = static_cast<const uint16_t*>(q);
    resolve_sm_scale(0.f, d, &a.sm_scale);
  }
  if (options & SAGE_OPT_SMOOTH_Q) {
    a.qb_slots = reinterpret_cast<const int32_t*>(ws + L.off[fp8 ? 10 : 9]);
    a.qb_fix = reinterpret_cast<const float*>(ws + L.off[10]);
    a.qb_flags = fp8 ? nullptr : reinterpret_cast<const int32_t*>(ws + L.off[11]);
    a.qb_any = fp8 ? nullptr : row_summaries(const_cast<char*>(ws) + L.off[11], g.B, H, g.N);
  }
  sage::launch_attn(a, is_causal != 0, fp8, st);
  return finish(st);
}

// Device address of this device's copy of the scratch array, looked up once
// per device (with that device current) and kept; nullptr if the lookup fails.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_ptr[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
  });
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* sage_status_string(sage_status_t s) {
  switch (s) {
    case SAGE_OK: return "ok";
    case SAGE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SAGE_ERR_UNSUPPORTED: return "unsupported";
    case SAGE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SAGE_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

size_t sage_quant_qk_workspace_size(int B, int H, int d) {
  if (B < 1 || H < 1 || (d != 64 && d != 128)) return 0;
  return align_up(sizeof(long long) * (size_t)B * H * d);
}

sage_status_t sage_quant_qk(const void* q, const void* k, int B, int H, int N, int d, sage_layout_t layout,
                            const int32_t* cu_seqlens, int64_t total_tokens, float sm_scale, int8_t* q_int8,
                            int8_t* k_int8, float* q_scale, float* k_scale, float* k_mean, float* q_mean,
                            int options, void* workspace, size_t workspace_bytes, sage_stream_t stream) {
  if (layout != SAGE_LAYOUT_HND) return layout < 0 ? SAGE_ERR_INVALID_ARGUMENT : SAGE_ERR_UNSUPPORTED;
  SeqGeom g;
  if (cu_seqlens) {
    const sage_status_t s = varlen_geom(cu_seqlens, B, N, total_tokens, H, d, &g);
    if (s != SAGE_OK) return s;
  } else {
    const sage_status_t s = check_dims(B, H, N, d);
    if (s != SAGE_OK) return s;
    g = SeqGeom{nullptr, B, H, N, d, 0};
  }
  if (!q || !k || !q_int8 || !k_int8 || !q_scale || !k_scale || !k_mean || !workspace)
    return SAGE_ERR_INVALID_ARGUMENT;
  if (!options_known(options)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!options_supported(options)) return SAGE_ERR_UNSUPPORTED;
  if (((options & SAGE_OPT_SMOOTH_Q) != 0) != (q_mean != nullptr)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_int8) || !aligned16(k_int8) || !aligned16(q_scale) ||
      !aligned16(k_scale) || !aligned16(k_mean) || !aligned16(q_mean) ||
      (reinterpret_cast<uintptr_t>(workspace) % kWsAlign) != 0)
    return SAGE_ERR_INVALID_ARGUMENT;
  float sm;
  if (!resolve_sm_scale(sm_scale, d, &sm)) return SAGE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < sage_quant_qk_workspace_size(g.B, H, d)) return SAGE_ERR_WORKSPACE_TOO_SMALL;
  {
    // the pre-pass reads q and k while it writes the codes, scales and means
    const bool qtok = (options & SAGE_OPT_Q_PER_TOKEN) != 0;
    const int64_t rows = cu_seqlens ? (int64_t)H * total_tokens : (int64_t)B * H * N;
    const size_t nq = (size_t)B * H * ceil_div64(N, sage::kQBlock), nk = (size_t)B * H * ceil_div64(N, sage::kKBlock);
    const struct {
      const void* p;
      size_t n;
    } r[] = {{q, (size_t)rows * d * 2},
             {k, (size_t)rows * d * 2},
             {q_int8, (size_t)rows * d},
             {k_int8, (size_t)rows * d},
             {q_scale, sizeof(float) * (qtok ? (size_t)rows : nq)},
             {k_scale, sizeof(float) * nk},
             {k_mean, sizeof(float) * (size_t)B * H * d},
             {q_mean, q_mean ? sizeof(float) * nq * d : 0},
             {workspace, sage_quant_qk_workspace_size(g.B, H, d)}};
    constexpr int kRegions = sizeof(r) / sizeof(r[0]);
    for (int i = 2; i < kRegions; ++i)  // every output and the workspace against everything before it
      for (int j = 0; j < i; ++j)
        if (r[i].n && r[j].n && overlaps(r[i].p, r[i].n, r[j].p, r[j].n)) return SAGE_ERR_INVALID_ARGUMENT;
  }
  if (cu_seqlens && total_tokens == 0) return SAGE_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  sage::launch_quant_qk(g, g, q, k, sm, q_int8, k_int8, q_scale, k_scale, k_mean, q_mean,
                        (options & SAGE_OPT_Q_PER_TOKEN) != 0, static_cast<long long*>(workspace), st);
  return finish(st);
}

sage_status_t sage_quant_v_fp8(const void* v, int B, int H, int N, int d, sage_layout_t layout,
                               const int32_t* cu_seqlens, int64_t total_tokens, uint8_t* v_fp8, float* v_scale,
                               sage_stream_t stream) {
  if (layout != SAGE_LAYOUT_HND) return layout < 0 ? SAGE_ERR_INVALID_ARGUMENT : SAGE_ERR_UNSUPPORTED;
  SeqGeom g;
  if (cu_seqlens) {
    const sage_status_t s = varlen_geom(cu_seqlens, B, N, total_tokens, H, d, &g);
    if (s != SAGE_OK) return s;
  } else {
    const sage_status_t s = check_dims(B, H, N, d);
    if (s != SAGE_OK) return s;
    g = SeqGeom{nullptr, B, H, N, d, 0};
  }
  if (!v || !v_fp8 || !v_scale) return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned16(v) || !aligned16(v_fp8) || !aligned16(v_scale)) return SAGE_ERR_INVALID_ARGUMENT;
  if (cu_seqlens && total_tokens == 0) return SAGE_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  sage::launch_v_scale(g, v, v_scale, st);
  sage::launch_v_prepare(g, v, v_scale, /*fp8=*/true, /*rowmajor=*/true, v_fp8, st);
  return finish(st);
}

size_t sage_attn_workspace_size(int B, int H, int H_kv, int N, int d, sage_pv_mode_t pv_mode, int options) {
  if (check_dims(B, H, N, d) != SAGE_OK || !kv_heads_ok(H, H_kv)) return 0;
  if (!pv_mode_ok(pv_mode)) return 0;
  if (!options_known(options) || !mode_options_supported(pv_mode, options)) return 0;
  return make_layout(false, B, H, H_kv, N, 0, d, pv_mode, options).total;
}

sage_status_t sage_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                            int H_kv, int N, int d, sage_layout_t layout, int is_causal, sage_pv_mode_t pv_mode,
                            int options, float sm_scale, void* workspace, size_t workspace_bytes,
                            sage_stream_t stream) {
  if (layout != SAGE_LAYOUT_HND) return layout < 0 ? SAGE_ERR_INVALID_ARGUMENT : SAGE_ERR_UNSUPPORTED;
  const sage_status_t s = check_dims(B, H, N, d);
  if (s != SAGE_OK) return s;
  const SeqGeom g{nullptr, B, H, N, d, 0};
  return attn_forward(q, k, v, o, lse, g, H_kv, false, is_causal, pv_mode, options, sm_scale, workspace,
                      workspace_bytes, stream);
}

sage_status_t sage_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                    int H_kv, int N, int d, sage_layout_t layout, int is_causal,
                                    sage_pv_mode_t pv_mode, int options, float sm_scale, sage_stream_t stream) {
  if (layout != SAGE_LAYOUT_HND) return layout < 0 ? SAGE_ERR_INVALID_ARGUMENT : SAGE_ERR_UNSUPPORTED;
  const sage_status_t s = check_dims(B, H, N, d);
  if (s != SAGE_OK) return s;
  if (!kv_heads_ok(H, H_kv) || !pv_mode_ok(pv_mode) || !options_known(options)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!mode_options_supported(pv_mode, options)) return SAGE_ERR_UNSUPPORTED;
  if (make_layout(false, B, H, H_kv, N, 0, d, pv_mode, options).total > (size_t)SAGE_NOALLOC_SCRATCH_BYTES)
    return SAGE_ERR_WORKSPACE_TOO_SMALL;  // beyond the scratch array: use sage_attn_fwd with a workspace
  void* ws = scratch_for_current_device();
  if (!ws) return SAGE_ERR_DEVICE;
  const SeqGeom g{nullptr, B, H, N, d, 0};
  return attn_forward(q, k, v, o, lse, g, H_kv, false, is_causal, pv_mode, options, sm_scale, ws,
                      (size_t)SAGE_NOALLOC_SCRATCH_BYTES, stream);
}

size_t sage_attn_varlen_workspace_size(int nseq, int max_seqlen, int64_t total_tokens, int H, int H_kv, int d,
                                       sage_pv_mode_t pv_mode, int options) {
  if (nseq < 1 || total_tokens < 0 || check_dims(nseq, H, max_seqlen, d) != SAGE_OK || !kv_heads_ok(H, H_kv))
    return 0;
  if (!pv_mode_ok(pv_mode)) return 0;
  if (!options_known(options) || !mode_options_supported(pv_mode, options)) return 0;
  return make_layout(true, nseq, H, H_kv, max_seqlen, total_tokens, d, pv_mode, options).total;
}

sage_status_t sage_attn_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                   const int32_t* cu_seqlens, int nseq, int max_seqlen, int64_t total_tokens, int H,
                                   int H_kv, int d, int is_causal, sage_pv_mode_t pv_mode, int options,
                                   float sm_scale, void* workspace, size_t workspace_bytes, sage_stream_t stream) {
  SeqGeom g;
  const sage_status_t s = varlen_geom(cu_seqlens, nseq, max_seqlen, total_tokens, H, d, &g);
  if (s != SAGE_OK) return s;
  return attn_forward(q, k, v, o, lse, g, H_kv, true, is_causal, pv_mode, options, sm_scale, workspace,
                      workspace_bytes, stream);
}

sage_status_t sage_test_workspace_layout(int varlen, int B, int H, int H_kv, int N, int64_t total_tokens, int d,
                                         sage_pv_mode_t pv_mode, int options, size_t offsets_out[12]) {
  if (!offsets_out) return SAGE_ERR_INVALID_ARGUMENT;
  if (check_dims(B, H, N, d) != SAGE_OK || !kv_heads_ok(H, H_kv)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!pv_mode_ok(pv_mode)) return SAGE_ERR_INVALID_ARGUMENT;
  if (varlen && total_tokens < 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (!options_known(options)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!mode_options_supported(pv_mode, options)) return SAGE_ERR_UNSUPPORTED;
  const WsLayout L = make_layout(varlen != 0, B, H, H_kv, N, total_tokens, d, pv_mode, options);
  for (int i = 0; i < 7; ++i) offsets_out[i] = L.off[i];
  for (int i = 8; i < kWsRegions; ++i) offsets_out[i - 1] = L.off[i];
  offsets_out[11] = L.total;
  return SAGE_OK;
}

sage_status_t sage_test_attn_from_workspace(void* o, const void* q, const void* v, int B, int H, int H_kv, int N,
                                            int d,
                                            int is_causal, sage_pv_mode_t pv_mode, int options,
                                            const void* workspace, size_t workspace_bytes, sage_stream_t stream) {
  const sage_status_t s = check_dims(B, H, N, d);
  if (s != SAGE_OK) return s;
  return attn_from_workspace(o, q, v, SeqGeom{nullptr, B, H, N, d, 0}, H_kv, false, is_causal, pv_mode, options,
                             workspace, workspace_bytes, stream);
}

sage_status_t sage_test_attn_varlen_from_workspace(void* o, const void* q, const void* v, const int32_t* cu_seqlens,
                                                   int nseq, int max_seqlen, int64_t total_tokens, int H, int H_kv,
                                                   int d, int is_causal, sage_pv_mode_t pv_mode, int options,
                                                   const void* workspace, size_t workspace_bytes,
                                                   sage_stream_t stream) {
  SeqGeom g;
  const sage_status_t s = varlen_geom(cu_seqlens, nseq, max_seqlen, total_tokens, H, d, &g);
  if (s != SAGE_OK) return s;
  if (total_tokens == 0) return SAGE_OK;
  return attn_from_workspace(o, q, v, g, H_kv, true, is_causal, pv_mode, options, workspace, workspace_bytes, stream);
}

sage_status_t sage_test_qk_tiles(const int8_t* q_int8, const int8_t* k_int8, int B, int H, int N, int d,
                                 const int32_t* tile_list, int n_tiles, int32_t* out, sage_stream_t stream) {
  const sage_status_t s = check_dims(B, H, N, d);
  if (s != SAGE_OK) return s;
  if (!q_int8 || !k_int8 || !tile_list || !out || n_tiles < 1) return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_int8) || !aligned16(k_int8) || !aligned16(tile_list) || !aligned16(out))
    return SAGE_ERR_INVALID_ARGUMENT;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  sage::launch_qk_tiles(q_int8, k_int8, B, H, N, d, tile_list, n_tiles, out, st);
  return finish(st);
}

}  // extern "C"
