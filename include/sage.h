/*
 * sage.h — C ABI of the MI355X (gfx950) 8-bit quantised attention forward.
 *
 * What is computed (pages cited by title and section):
 *   - K smoothing: K minus its per-channel token mean, which leaves softmax
 *     unchanged (dtcms.com SageAttention summary, section "SageAttention（v1）";
 *     "⚡️SageAttention — brand new attention", SageAttention bullets).
 *   - Per-block symmetric INT8 quantisation of Q (128-token blocks) and of the
 *     smoothed K (64-token blocks): scale = max|x|/127, code = round(x/scale)
 *     ("⚡️SageAttention — brand new attention", quantisation introduction;
 *     dtcms summary "SageAttention（v1）", per-block quantisation).  The softmax
 *     scale is folded into Q's scale (same page, "fuse scaling and unscaling").
 *   - A tiled, fused attention (intelliparadigm "Attention机制优化", §3.1:
 *     tiling, fusion, online softmax): S = int32(Q̂K̂ᵀ)·δQ·δK, online fp32
 *     softmax, PV in FP16 with fp32 accumulation, or FP8 (e4m3) PV with
 *     per-channel V scales and two-level accumulation (dtcms summary, section
 *     "SageAttention 2"; postsniper page, SageAttention2 bullets).
 *   - Causal masking and variable-length packed batches (deepseek.csdn.net
 *     post: sageattn called with is_causal=True on [B,H,N,d] tensors;
 *     jsqmd "SageAttention完全指南", API list: sageattn_varlen).
 *   - Optional Q smoothing (dtcms summary, section "SageAttention 2": Q is
 *     smoothed as well, for a more accurate QKᵀ; postsniper page,
 *     SageAttention2 bullets: Q normalised too, without distorting the
 *     result): each 128-token Q block's channel mean q̄ is subtracted before
 *     the INT8 step and the score term it carries, sm_scale·q̄·(k − km), is
 *     added back to every score of the block's rows.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers (HIP global memory) unless stated.
 *     fp16 is IEEE binary16; the last dimension (d) is contiguous.
 *   - Layout HND: dense tensors are [B, H, N, d]; varlen tensors are packed
 *     [H, T, d] with sequence i on tokens [cu_seqlens[i], cu_seqlens[i+1]).
 *   - Supported head dims: d = 64 or d = 128.
 *   - Ownership: the caller allocates and frees every buffer, the workspace
 *     included.  The library never allocates or frees device memory and keeps
 *     no pointer after a call returns; its only device memory of its own is
 *     the static scratch array of sage_attn_fwd_noalloc.
 *   - Asynchrony: calls only enqueue work on `stream` (a hipStream_t; NULL is
 *     the null stream) and return without synchronising.  Buffers must stay
 *     valid until the stream has completed the work.
 *   - Errors: all validation happens on the host before anything is enqueued;
 *     on an error nothing is launched and outputs are untouched.  Null or
 *     misaligned (not 16-byte aligned) pointers, non-positive sizes, d not in
 *     {64,128}, unknown enum values -> SAGE_ERR_INVALID_ARGUMENT; a layout the
 *     library does not implement -> SAGE_ERR_UNSUPPORTED; a workspace smaller
 *     than the size query -> SAGE_ERR_WORKSPACE_TOO_SMALL; a failed launch ->
 *     SAGE_ERR_DEVICE.  No C++ exception crosses this boundary.
 *   - Inputs must be finite; the contents of cu_seqlens must satisfy the
 *     documented constraints (they live on the device and are not checked).
 *   - Calls are reentrant; the library holds no mutable global state, apart
 *     from the per-GPU scratch array of sage_attn_fwd_noalloc (see there).
 */
#ifndef SAGE_H_
#define SAGE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAGE_OK = 0,
  SAGE_ERR_INVALID_ARGUMENT = 1,
  SAGE_ERR_UNSUPPORTED = 2,
  SAGE_ERR_WORKSPACE_TOO_SMALL = 3,
  SAGE_ERR_DEVICE = 4
} sage_status_t;

/* SAGE_MXFP4: QKᵀ and PV both in OCP microscaling FP4 (dtcms summary, section
 * "SageAttention 3": microscaling FP4 attention, two-level quantisation):
 * e2m1 elements in blocks of 32 along the contracted axis (channels for Q and
 * the smoothed K, keys for P and V) with one E8M0 power-of-two scale each, the
 * smallest under which the block maximum fits e2m1's largest value 6; P is the
 * online softmax's p = e^(s - m) <= 1 (level one) microscaled per 32-key block
 * (level two).  Takes SAGE_OPT_SMOOTH_Q (not SAGE_OPT_Q_PER_TOKEN: its Q
 * scales are per row already).  Far coarser than the INT8 path (3-bit
 * elements): about 0.97 cosine to exact attention on Gaussian inputs. */
typedef enum { SAGE_PV_FP16 = 0, SAGE_PV_FP8_E4M3 = 1, SAGE_MXFP4 = 2 } sage_pv_mode_t;

/* Options, OR-ed into the `options` argument (0 = the default method).
 *   SAGE_OPT_SMOOTH_Q: Q smoothing — each 128-token Q block's channel mean q̄
 *     is subtracted before the INT8 step and the score term it carries,
 *     sm_scale·q̄·(k − km), is added back to every score of the block's rows
 *     (dtcms summary, section "SageAttention 2"; postsniper SageAttention2
 *     bullets).
 *   SAGE_OPT_Q_PER_TOKEN: one Q scale per token instead of per 128-token block
 *     (dtcms summary: per-token q/k quantisation in "SageAttention（v1）", finer
 *     granularity in "SageAttention 2"); q_scale is then indexed like the Q
 *     rows: [B,H,N] dense, [H,T] varlen.
 * The two are exclusive (SAGE_ERR_UNSUPPORTED): the smoothing term is carried
 * in units of a per-block δQ.  With SAGE_MXFP4 the smoothed Q is MX-quantised
 * and the term, q̄·(k − km) in fp32, starts the score accumulator of every key.
 * Unknown bits -> SAGE_ERR_INVALID_ARGUMENT. */
typedef enum { SAGE_OPT_SMOOTH_Q = 1, SAGE_OPT_Q_PER_TOKEN = 2 } sage_option_t;
typedef enum { SAGE_LAYOUT_HND = 0 } sage_layout_t;

/* A hipStream_t passed as an opaque pointer. */
typedef void* sage_stream_t;

/* Human-readable text for a status code (static storage; never NULL). */
const char* sage_status_string(sage_status_t s);

/* ------------------------------------------------------------------------
 * sage_quant_qk — K smoothing + per-block INT8 quantisation of Q and K.
 *   (postsniper page, quantisation introduction and SageAttention bullets;
 *    dtcms summary, section "SageAttention（v1）")
 *
 * cu_seqlens == NULL: dense. q, k fp16 [B,H,N,d]; outputs q_int8, k_int8
 *   int8 [B,H,N,d]; q_scale fp32 [B,H,ceil(N/128)]; k_scale fp32
 *   [B,H,ceil(N/64)]; k_mean fp32 [B,H,d].  total_tokens is ignored.
 * cu_seqlens != NULL: varlen.  B = number of sequences, N = max sequence
 *   length (>= every length), total_tokens = T = cu_seqlens[B].  q, k, q_int8,
 *   k_int8 are packed [H,T,d]; q_scale [B,H,ceil(N/128)], k_scale
 *   [B,H,ceil(N/64)] and k_mean [B,H,d] are indexed by sequence, entries past
 *   a sequence's own block count are left unwritten.  cu_seqlens is int32
 *   [B+1] on the device, cu[0]=0, non-decreasing, cu[B]=T, each length <= N.
 * sm_scale <= 0 selects the default fp32(1/sqrt(d)).  q_scale holds the block
 *   scale times sm_scale (fp32 product).
 * Semantics (bit-exact contract): km = fp32(exact int64 fixed-point column sum
 *   * 2^-24 / n) per (sequence, head, channel); x = fp32(k) - km in fp32;
 *   scale = fp32(max|x| / 127) (IEEE division); code = clamp(rint(fp32(x /
 *   scale)), -127, 127); an all-zero block has scale 0 and codes 0.  Q the same
 *   without the mean, or — options SAGE_OPT_SMOOTH_Q, which requires q_mean !=
 *   NULL (and NULL otherwise) — with the mean of each 128-token block by the
 *   same exact rule over the block's own tokens, written to q_mean fp32
 *   [B,H,ceil(N/128),d] (varlen: indexed by sequence); with
 *   SAGE_OPT_Q_PER_TOKEN each Q row is its own block and q_scale is [B,H,N]
 *   (varlen [H,T]).
 * workspace: device scratch of at least sage_quant_qk_workspace_size(B,H,d)
 *   bytes, 256-byte aligned; its contents on entry do not matter.
 */
size_t sage_quant_qk_workspace_size(int B, int H, int d);
sage_status_t sage_quant_qk(const void* q, const void* k, int B, int H, int N, int d,
                            sage_layout_t layout, const int32_t* cu_seqlens, int64_t total_tokens,
                            float sm_scale, int8_t* q_int8, int8_t* k_int8, float* q_scale,
                            float* k_scale, float* k_mean, float* q_mean, int options,
                            void* workspace, size_t workspace_bytes, sage_stream_t stream);

/* ------------------------------------------------------------------------
 * sage_quant_v_fp8 — per-channel e4m3 quantisation of V (the FP8-PV input).
 *   (dtcms summary, section "SageAttention 2": P and V in FP8)
 * Dense (cu_seqlens == NULL): v fp16 [B,H,N,d] -> v_fp8 e4m3 bytes [B,H,N,d],
 *   v_scale fp32 [B,H,d].  Varlen: v, v_fp8 packed [H,T,d], v_scale [B,H,d]
 *   per sequence.  scale = fp32(max_t |v| / 448); code = e4m3 of
 *   fp32(v / scale), round to nearest even, saturating at ±448 (OCP E4M3FN);
 *   a zero channel has scale 0 and codes 0.  No workspace.
 */
sage_status_t sage_quant_v_fp8(const void* v, int B, int H, int N, int d, sage_layout_t layout,
                               const int32_t* cu_seqlens, int64_t total_tokens, uint8_t* v_fp8,
                               float* v_scale, sage_stream_t stream);

/* ------------------------------------------------------------------------
 * sage_attn_fwd — full forward on dense [B,H,N,d] fp16 tensors.
 *   q fp16 [B,H,N,d]; k, v fp16 [B,H_kv,N,d]; o output fp16 [B,H,N,d] (may not
 *   alias the inputs).  H_kv divides H: query head h attends with K/V head
 *   h / (H / H_kv) (grouped-query or multi-query attention; H_kv = H is plain
 *   multi-head attention, and K smoothing and K blocks are per K/V head).
 *   lse: NULL, or fp32 [B,H,N] receiving, per query row, the natural-log sum
 *   of exp of the row's scaled scores s = δQ·δK·(q̂·k̂) over the visible keys
 *   (smoothed K: exact attention shifted by the row constant q·km·sm_scale),
 *   for merging partial results over key ranges; 4-byte aligned, no overlap.
 *   is_causal != 0 masks key j > query i (deepseek.csdn.net post: is_causal).
 *   pv_mode selects FP16 PV, FP8-e4m3 PV, or SAGE_MXFP4 (QKᵀ and PV in MXFP4;
 *   SAGE_OPT_Q_PER_TOKEN -> SAGE_ERR_UNSUPPORTED).  options (sage_option_t bits):
 *   SAGE_OPT_SMOOTH_Q — Q̂ and δQ come from Q minus its block mean and every
 *   score of a row of block b gets sm_scale·q̄_b·(k_j − km) added back
 *   (FP16 PV: carried within one unit of δQ·δK in the accumulator's start
 *   value, in fp32 for the rare half tiles it does not fit; FP8 PV and MXFP4:
 *   added in fp32 to every score; the workspace is then larger);
 *   SAGE_OPT_Q_PER_TOKEN — one Q scale per query row.  sm_scale <= 0 ->
 *   1/sqrt(d).
 *   The pre-pass (smoothing, quantisation, V packing) writes into the
 *   caller's workspace of at least sage_attn_workspace_size(...) bytes; its
 *   layout is internal (see sage_test_workspace_layout).
 *   Errors: SAGE_ERR_INVALID_ARGUMENT for null or misaligned (16-byte) tensor
 *   pointers, a workspace not 256-byte aligned, overlapping outputs, H_kv not
 *   dividing H, d not in {64, 128}, N > 2^23, B or H > 65535, or a NaN/Inf
 *   sm_scale; SAGE_ERR_WORKSPACE_TOO_SMALL; SAGE_ERR_DEVICE if a launch fails.
 *   Nothing is launched on error.  Asynchronous on `stream`.
 */
size_t sage_attn_workspace_size(int B, int H, int H_kv, int N, int d, sage_pv_mode_t pv_mode,
                                int options);
sage_status_t sage_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int H_kv, int N, int d, sage_layout_t layout,
                            int is_causal, sage_pv_mode_t pv_mode, int options, float sm_scale,
                            void* workspace, size_t workspace_bytes, sage_stream_t stream);

/* ------------------------------------------------------------------------
 * sage_attn_fwd_noalloc — sage_attn_fwd without a workspace argument, for
 *   callers that cannot allocate device memory (code under HIP graph capture,
 *   tight serving loops, harnesses that forbid allocation).  Same arguments,
 *   semantics, outputs and validation as sage_attn_fwd; the pre-pass results
 *   go to a scratch array the library owns: SAGE_NOALLOC_SCRATCH_BYTES of
 *   device memory per GPU, reserved when the library's code is loaded on that
 *   GPU and held until the process ends.  Problems whose
 *   sage_attn_workspace_size exceeds it -> SAGE_ERR_WORKSPACE_TOO_SMALL
 *   (call sage_attn_fwd with a workspace instead); SAGE_ERR_DEVICE if the
 *   scratch array cannot be located on the current device.  The call
 *   allocates and frees nothing.  Every call on one GPU shares that GPU's
 *   array (the pre-pass rewrites it; nothing is assumed about its contents on
 *   entry): calls that overlap on one GPU — on different streams, or from
 *   different host threads without ordering — race, and their results are
 *   undefined; calls on one stream are ordered and safe.
 */
#define SAGE_NOALLOC_SCRATCH_BYTES (256u << 20)
sage_status_t sage_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                    int B, int H, int H_kv, int N, int d, sage_layout_t layout,
                                    int is_causal, sage_pv_mode_t pv_mode, int options, float sm_scale,
                                    sage_stream_t stream);

/* ------------------------------------------------------------------------
 * sage_attn_varlen_fwd — forward on packed variable-length sequences.
 *   (jsqmd "SageAttention完全指南", API list: sageattn_varlen)
 *   q, o packed fp16 [H,T,d]; k, v packed fp16 [H_kv,T,d] (H_kv divides H, as
 *   for sage_attn_fwd); lse NULL or fp32 [H,T].  cu_seqlens device int32
 *   [nseq+1] with cu[0]=0, non-decreasing, cu[nseq]=total_tokens, every
 *   length <= max_seqlen.  Means, quantisation blocks (Q smoothing's included)
 *   and the causal mask are per sequence.  Empty sequences are allowed.
 */
size_t sage_attn_varlen_workspace_size(int nseq, int max_seqlen, int64_t total_tokens, int H,
                                       int H_kv, int d, sage_pv_mode_t pv_mode, int options);
sage_status_t sage_attn_varlen_fwd(const void* q, const void* k, const void* v, void* o,
                                   float* lse, const int32_t* cu_seqlens, int nseq,
                                   int max_seqlen, int64_t total_tokens, int H, int H_kv, int d,
                                   int is_causal, sage_pv_mode_t pv_mode, int options,
                                   float sm_scale, void* workspace, size_t workspace_bytes,
                                   sage_stream_t stream);

/* ------------------------------------------------------------------------
 * Test hooks (stable; prefix sage_test_).
 *
 * sage_test_workspace_layout: byte offsets, inside the sage_attn_fwd
 *   (varlen == 0) or sage_attn_varlen_fwd (varlen != 0) workspace, of
 *   [0] q_int8, [1] k_int8, [2] q_scale, [3] k_scale, [4] k_mean ([0] and [2]
 *   are left unwritten without SAGE_OPT_SMOOTH_Q in SAGE_PV_FP16 /
 *   SAGE_PV_FP8_E4M3 mode: the attention kernel quantises Q itself, with the
 *   same quantiser),
 *   [5] packed e4m3 V and [6] v_scale (fp8 mode; both empty in fp16 mode, whose
 *   kernel reads the caller's V directly),
 *   and, with SAGE_OPT_SMOOTH_Q (empty regions otherwise), [7] q_mean fp32
 *   [B,H,nqb,d], [8] accumulator initial values int32 [B,H,nqb,npad],
 *   [9] fp32 fallback terms [B,H,nqb,npad], [10] fallback flags int32
 *   [B,H,nqb,2·nkb] (nqb = ceil(N/128), nkb = ceil(N/64), npad = 64·nkb;
 *   entry [.,.,b,2t+s] = 1 where half s of key tile t carries the term in
 *   fp32 — then [9] holds it, as sm_scale·q̄_b·x_j·log2(e) — else [8] holds
 *   1.5·2^23 bits + rint(that / (δQ_b·δK_t·log2 e)); the flags are followed, at
 *   the next 16-byte boundary, by one int32 per (b, h, Q block), nonzero when
 *   some half of that block's row falls back), [11] total size
 *   (internal scratch sits between [6] and [7]).
 *   With SAGE_MXFP4 the regions are instead [0] Q e2m1 codes [rows][d/2]
 *   (channel c in nibble c%2 of byte c/2), [1] the smoothed K's codes, [2] Q
 *   E8M0 scale bytes [rows][8] (byte 4g + kk: channel block 2kk + g), [3] per
 *   K/V tile 1 KB of scales (K: 8 bytes per key in the kernel's row order;
 *   V: at 512 + 4·lane + dt), [4] k_mean, [5] packed V codes per tile
 *   ([dt][lane] 16 bytes: channel 32dt + lane%32, keys 32(lane/32) + j in
 *   nibble j), [6] empty, and with SAGE_OPT_SMOOTH_Q [7] q_mean fp32
 *   [B,H,nqb,d] and [8] the score term fp32 [B,H,nqb,npad], q̄_b·x_j before
 *   the softmax scale (keys past a sequence's end: 0; causal: blocks that
 *   see no key of a tile are not written), else [7]-[8] empty; [9]-[10] empty.
 *   For dense calls pass B,H,H_kv,N,d (total_tokens ignored); for varlen pass
 *   B = nseq, N = max_seqlen and total_tokens.  offsets_out is HOST memory.
 *   The int8/scale/mean regions use the same layouts as sage_quant_qk, with
 *   H_kv heads for K.
 *
 * sage_test_qk_tiles: int32 tiles of Q̂K̂ᵀ (128 queries x 64 keys each, row =
 *   query) for a list of (b, h, q_block, k_block) quadruples (device int32
 *   [n,4]) on dense int8 [B,H,N,d] inputs, computed by the attention kernel's
 *   own QKᵀ device code; entries outside [0,N) read as zero codes.  out is
 *   device int32 [n,128,64].
 */
/*
 * sage_test_attn_from_workspace: launch only the fused attention kernel on a
 *   workspace that a preceding sage_attn_fwd call with the same B,H,H_kv,N,d,
 *   is_causal, pv_mode and options has filled (its pre-pass results are reused
 *   as they are); writes o fp16 [B,H,N,d] (no LSE).  q: that call's fp16 Q
 *   [B,H,N,d] — without SAGE_OPT_SMOOTH_Q, in SAGE_PV_FP16 or
 *   SAGE_PV_FP8_E4M3 mode, the attention kernel quantises Q itself (the
 *   pre-pass then leaves regions [0] and [2] unwritten), with the default
 *   softmax scale; with q NULL in that mode the kernel instead reads Q̂ and δQ
 *   from regions [0] and [2], which the caller has filled (e.g. with
 *   sage_quant_qk's results); ignored, may be NULL, with SAGE_OPT_SMOOTH_Q.  v: that call's fp16 V [B,H_kv,N,d] (SAGE_PV_FP16 reads it
 *   directly; ignored, may be NULL, in the other modes).  Used to time the
 *   attention kernel alone.  Same validation as sage_attn_fwd.  SAGE_MXFP4
 *   uses the default softmax scale.
 */
sage_status_t sage_test_attn_from_workspace(void* o, const void* q, const void* v, int B, int H, int H_kv,
                                            int N, int d, int is_causal, sage_pv_mode_t pv_mode, int options,
                                            const void* workspace, size_t workspace_bytes,
                                            sage_stream_t stream);
/*
 * sage_test_attn_varlen_from_workspace: the same for packed variable-length
 *   sequences (jsqmd "SageAttention完全指南", API list: sageattn_varlen):
 *   launch only the fused attention kernel on a workspace that a preceding
 *   sage_attn_varlen_fwd call with the same cu_seqlens, nseq, max_seqlen,
 *   total_tokens, H, H_kv, d, is_causal, pv_mode and options has filled; o, q
 *   packed fp16 [H,T,d], v packed fp16 [H_kv,T,d] (q and v with the meaning
 *   they have above).  Same validation as sage_attn_varlen_fwd; with
 *   total_tokens = 0 nothing is launched.  Used to time the attention kernel
 *   alone on the varlen workload.
 */
sage_status_t sage_test_attn_varlen_from_workspace(void* o, const void* q, const void* v,
                                                   const int32_t* cu_seqlens, int nseq, int max_seqlen,
                                                   int64_t total_tokens, int H, int H_kv, int d,
                                                   int is_causal, sage_pv_mode_t pv_mode, int options,
                                                   const void* workspace, size_t workspace_bytes,
                                                   sage_stream_t stream);
sage_status_t sage_test_workspace_layout(int varlen, int B, int H, int H_kv, int N,
                                         int64_t total_tokens, int d, sage_pv_mode_t pv_mode,
                                         int options, size_t offsets_out[12]);
sage_status_t sage_test_qk_tiles(const int8_t* q_int8, const int8_t* k_int8, int B, int H, int N,
                                 int d, const int32_t* tile_list, int n_tiles, int32_t* out,
                                 sage_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SAGE_H_ */
