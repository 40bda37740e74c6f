"""CPU oracle for the SageAttention-style 8-bit attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (``quantized_attention_quant_amd``) never imports it and shares
no code with it: the two agree only because both follow the same pages.

The oracle is deliberately plain: numpy, no blocking or fusion beyond what the
method itself defines, fp64 for the attention arithmetic.  Where floating point
decides an integer (the INT8 and e4m3 codes of Q, K and V) the decision is
taken in fp32, the precision the GPU path uses, so those codes are comparable
bit for bit.

Pages cited (by title; sections as they appear on each page)
  [PS]  "⚡️SageAttention — brand new attention" (postsniper.ru): the
        quantisation introduction (scale = max|A|/127, round(A/scale),
        C ≈ (ÂB̂)(δAδB)), the outlier example, the SageAttention bullets
        (INT8 QKᵀ with K normalisation, fused scaling, FP16 PV) and the
        SageAttention2 bullets (FP8 PV stabilised with FP32 double buffering).
  [DT]  dtcms.com SageAttention summary: section "SageAttention（v1）"
        (smooth K by subtracting its mean; per-block or per-token Q/K
        quantisation) and section "SageAttention 2" (P and V in FP8, two-level
        accumulation for FP8 PV).
  [IP]  "Attention机制优化：从FlashAttention到SageAttention的工程实践"
        (intelliparadigm.com): §2.1 (Attn = softmax(QKᵀ/√d)V) and §3.1
        (tiling, kernel fusion, online softmax).
  [CS]  deepseek.csdn.net post on using sageattn in DeepSeek-VL2: the attention
        forward that transposes to [B, H, N, d] and calls sageattn with
        is_causal=True.

Readings where the pages are silent (each listed in the design notes):
  * block geometry: Q blocks of 128 tokens, K blocks of 64 tokens, all d
    channels, never crossing a sequence; the last block is partial;
  * K mean: exact int64 fixed-point column sum (every fp16 is a multiple of
    2^-24), one fp64 divide by n, one rounding to fp32; domain = one
    (sequence, head);
  * smoothed K stays in fp32 (not re-rounded to fp16);
  * round = round-half-to-even; clamp to ±127; an all-zero block has scale 0
    and codes 0;
  * the softmax scale (fp32 of 1/sqrt(d) computed in fp64) is multiplied into
    Q's emitted block scale after quantisation;
  * online softmax walks 64-key tiles in ascending order, updating the row max
    once per tile (the FP8 P codes depend on this schedule);
  * FP8 mode: V per-channel scale amax/448, codes OCP e4m3 (bias 7, max 448,
    round to nearest even, saturate to ±448); P codes are e4m3(p * 448);
    level 1 sums one tile's P̂V̂, level 2 is the running output;
  * the row sum l is taken from the unrounded p;
  * Q smoothing (optional): the mean of each 128-token Q block (the K-mean
    rule applied to that block) is subtracted before the INT8 step, and the
    part of the score it carries, sm_scale * q̄ · (k - km) with the smoothed K
    in fp32, is added back exactly (fp64) to every score of the block's rows;
  * per-token Q scales (optional, finer granularity): a Q "block" of one
    token, the same quantiser on each row alone;
  * MXFP4 mode (optional, [DT] "SageAttention 3"): Q, smoothed K, P and V as
    OCP microscaling FP4 — e2m1 elements in blocks of 32 with one
    power-of-two (E8M0) scale each, the scale chosen as the smallest power of
    two that fits the block maximum under e2m1's largest value 6 (no
    saturation); blocks run along the contracted axis (channels for Q and K,
    keys for P and V, 32-key blocks aligned within the sequence); P is first
    normalised by the running max (level one), then microscaled (level two).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

Q_BLOCK = 128      # tokens per Q quantisation block
K_BLOCK = 64       # tokens per K quantisation block
KV_TILE = 64       # keys per online-softmax step
INT8_MAX = 127
E4M3_MAX = 448.0
E2M1_MAX = 6.0     # largest OCP FP4 (e2m1) value
MX_BLOCK = 32      # elements per microscaling block
FIXED_POINT_SHIFT = 24   # fp16 values are integer multiples of 2^-24

__all__ = [
    "Q_BLOCK", "K_BLOCK", "KV_TILE", "default_sm_scale", "k_token_mean", "smooth_k",
    "quantize_int8_blocks", "quant_q", "quant_k", "quant_qk_dense", "quant_qk_varlen",
    "e4m3_decode", "e4m3_encode", "quant_v_fp8",
    "qk_int", "sage_attention_rows", "sdpa_fp64_rows", "head_views_dense",
    "head_views_varlen", "q_block_mean", "quant_q_smooth", "q_smooth_bias", "quant_q_per_token",
    "E2M1_MAX", "MX_BLOCK", "e2m1_decode", "e2m1_encode", "mx_block_exponent", "mx_quantize",
    "quant_mxfp4_qk", "quant_mxfp4_v", "mxfp4_decode", "mxfp4_attention_rows", "quant_mxfp4_q_smooth",
    "mxfp4_open_code_bound", "score_lse_rows",
]


# ----------------------------------------------------------------------------
# Scale of the softmax
# ----------------------------------------------------------------------------
def default_sm_scale(d: int) -> np.float32:
    """Softmax scale 1/sqrt(d) of [IP] §2.1, computed in fp64 and rounded once to fp32."""
    return np.float32(1.0 / math.sqrt(d))


# ----------------------------------------------------------------------------
# K smoothing ([DT] "SageAttention（v1）" first bullet; [PS] SageAttention bullets)
# ----------------------------------------------------------------------------
def k_token_mean(k: np.ndarray) -> np.ndarray:
    """Mean of K over its tokens, per channel: k fp16 [..., n, d] -> fp32 [..., d].

    [DT] "SageAttention（v1）": K is smoothed by subtracting its mean.  The sum
    is exact: each fp16 value times 2^24 is an integer, summed in int64, then
    divided by n once in fp64 and rounded once to fp32.
    """
    if k.dtype != np.float16:
        raise TypeError("k must be fp16")
    n = k.shape[-2]
    if n == 0:
        raise ValueError("empty sequence")
    fixed = (k.astype(np.float64) * float(2 ** FIXED_POINT_SHIFT)).astype(np.int64)
    total = fixed.sum(axis=-2, dtype=np.int64)
    mean64 = total.astype(np.float64) * (2.0 ** -FIXED_POINT_SHIFT) / float(n)
    return mean64.astype(np.float32)


def smooth_k(k: np.ndarray, km: np.ndarray) -> np.ndarray:
    """x = fp32(k) - km, in fp32 ([DT] "SageAttention（v1）"); broadcast over tokens."""
    return k.astype(np.float32) - km[..., None, :].astype(np.float32)


# ----------------------------------------------------------------------------
# Symmetric absmax INT8 quantiser ([PS] quantisation introduction, steps 1-2)
# ----------------------------------------------------------------------------
def quantize_int8_blocks(x: np.ndarray, block: int):
    """Per-block symmetric INT8 quantisation of fp32 x [..., n, d].

    [PS] quantisation introduction: scale = max|A| / 127, Â = round(A / scale).
    A block is ``block`` consecutive tokens times all d channels ([DT]
    "SageAttention（v1）": per-block quantisation of q and k); the last block
    may be partial.  Division and rounding are fp32 (round half to even);
    codes are clamped to [-127, 127]; an all-zero block gets scale 0, codes 0.

    Returns (codes int8 [..., n, d], scales fp32 [..., ceil(n/block)]).
    """
    if x.dtype != np.float32:
        raise TypeError("x must be fp32")
    *lead, n, d = x.shape
    nb = -(-n // block)
    pad = nb * block - n
    xp = x
    if pad:
        widths = [(0, 0)] * len(lead) + [(0, pad), (0, 0)]
        xp = np.pad(x, widths)          # zeros never raise the block max
    xb = xp.reshape(*lead, nb, block, d)
    amax = np.abs(xb).max(axis=(-2, -1))                       # fp32, exact
    scale = (amax / np.float32(INT8_MAX)).astype(np.float32)   # fp32 divide
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    ratio = (xb / safe[..., None, None]).astype(np.float32)    # fp32 divide
    codes = np.clip(np.rint(ratio), -INT8_MAX, INT8_MAX)
    codes = np.where((scale > 0)[..., None, None], codes, 0).astype(np.int8)
    codes = codes.reshape(*lead, nb * block, d)[..., :n, :]
    return np.ascontiguousarray(codes), scale


def quant_q(q: np.ndarray, sm_scale: np.float32):
    """Q per 128-token block, softmax scale folded into the emitted scale.

    [PS] SageAttention bullets: scaling is fused with the neighbouring
    operations; here the 1/sqrt(d) of [IP] §2.1 is multiplied (fp32) into δQ
    after the codes are taken from the unfolded scale.
    """
    codes, scale = quantize_int8_blocks(q.astype(np.float32), Q_BLOCK)
    return codes, (scale * np.float32(sm_scale)).astype(np.float32)


def quant_k(k: np.ndarray):
    """K smoothed by its token mean, then per 64-token block INT8.

    Returns (codes int8, scale fp32 per block, mean fp32 [.., d]).
    """
    km = k_token_mean(k)
    codes, scale = quantize_int8_blocks(smooth_k(k, km), K_BLOCK)
    return codes, scale, km


# ----------------------------------------------------------------------------
# Q smoothing ([DT] "SageAttention 2": Q is smoothed too, for a more accurate
# QKᵀ; [PS] SageAttention2 bullets: Q is normalised as well so that the
# attention result is not distorted)
# ----------------------------------------------------------------------------
def q_block_mean(q: np.ndarray) -> np.ndarray:
    """Per 128-token block channel mean of Q: fp16 [..., n, d] -> fp32
    [..., ceil(n/128), d].  Each block (the last one partial) uses the exact
    mean rule of the K mean over its own tokens."""
    n = q.shape[-2]
    return np.stack([k_token_mean(q[..., b0:min(n, b0 + Q_BLOCK), :]) for b0 in range(0, n, Q_BLOCK)], axis=-2)


def quant_q_per_token(q: np.ndarray, sm_scale: np.float32):
    """Q with one scale per token ([DT] "SageAttention（v1）": per-block or
    per-token quantisation of q and k; [DT] "SageAttention 2": finer, per
    thread, granularity): the quantiser of ``quantize_int8_blocks`` with a
    block of one row; sm_scale folded in.  Returns (codes, scale [..., n])."""
    codes, scale = quantize_int8_blocks(q.astype(np.float32), 1)
    return codes, (scale * np.float32(sm_scale)).astype(np.float32)


def quant_q_smooth(q: np.ndarray, sm_scale: np.float32):
    """Q smoothed by its block mean, then per 128-token block INT8.

    x = fp32(q) - q̄ (fp32, the block's own mean), quantised like Q without
    smoothing; sm_scale is folded into the emitted scale.  Returns (codes
    int8, scale fp32 per block, q̄ fp32 [..., nqb, d]).
    """
    n = q.shape[-2]
    qm = q_block_mean(q)
    x = q.astype(np.float32) - np.repeat(qm, Q_BLOCK, axis=-2)[..., :n, :]
    codes, scale = quantize_int8_blocks(x.astype(np.float32), Q_BLOCK)
    return codes, (scale * np.float32(sm_scale)).astype(np.float32), qm


def q_smooth_bias(q_mean: np.ndarray, k: np.ndarray, k_mean: np.ndarray, sm_scale: float) -> np.ndarray:
    """The score term the smoothed Q̂ leaves out, per (Q block, key), in fp64:

        bias[b, j] = sm_scale · Σ_c q̄[b, c] · x[j, c],   x = fp32(k) - km,

    the smoothed K in fp32 exactly as the K path forms it.  One (sequence,
    head): q_mean [nqb, d], k fp16 [n, d], k_mean [d] -> [nqb, n].  Every
    score of a row in block b gets bias[b, j] added before the softmax.
    """
    x = smooth_k(k, k_mean).astype(np.float64)
    return float(sm_scale) * (q_mean.astype(np.float64) @ x.T)


def quant_qk_dense(q: np.ndarray, k: np.ndarray, sm_scale: Optional[float] = None,
                   smooth_q: bool = False, q_per_token: bool = False) -> Dict[str, np.ndarray]:
    """Dense [B, H, N, d] fp16 inputs ([CS]: HND layout) -> INT8 tensors and scales.

    Output shapes: q_int8, k_int8 [B,H,N,d]; q_scale [B,H,ceil(N/128)] (with
    q_per_token [B,H,N]); k_scale [B,H,ceil(N/64)]; k_mean [B,H,d]; with
    smooth_q also q_mean [B,H,ceil(N/128),d].  K may have fewer heads than Q
    (its own shape).
    """
    d = q.shape[-1]
    sm = default_sm_scale(d) if not sm_scale or sm_scale <= 0 else np.float32(sm_scale)
    out = {}
    if smooth_q and q_per_token:
        raise ValueError("Q smoothing uses 128-token Q blocks")
    if smooth_q:
        qi, qs, out["q_mean"] = quant_q_smooth(q, sm)
    elif q_per_token:
        qi, qs = quant_q_per_token(q, sm)
    else:
        qi, qs = quant_q(q, sm)
    ki, ks, km = quant_k(k)
    out.update(q_int8=qi, q_scale=qs, k_int8=ki, k_scale=ks, k_mean=km)
    return out


def quant_qk_varlen(q: np.ndarray, k: np.ndarray, cu_seqlens: Sequence[int],
                    sm_scale: Optional[float] = None, smooth_q: bool = False,
                    q_per_token: bool = False) -> Dict[str, np.ndarray]:
    """Packed [H, T, d] inputs with sequence i on tokens [cu[i], cu[i+1]).

    Blocks and means never cross a sequence.  Scales and means are returned
    padded per sequence: q_scale [nseq,H,ceil(max/128)], k_scale
    [nseq,H,ceil(max/64)], k_mean [nseq,H,d], with smooth_q also q_mean
    [nseq,H,ceil(max/128),d]; padding entries are NaN (no value is defined
    there).  With q_per_token q_scale is per packed token, [H, T].  K may have
    fewer heads than Q (its own shape).
    """
    H, T, d = q.shape
    Hk = k.shape[0]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    nseq = len(cu) - 1
    lens = np.diff(cu)
    mx = max(int(lens.max()), 1)
    sm = default_sm_scale(d) if not sm_scale or sm_scale <= 0 else np.float32(sm_scale)
    qi = np.zeros((H, T, d), np.int8)
    ki = np.zeros((Hk, T, d), np.int8)
    qs = np.full((H, T) if q_per_token else (nseq, H, -(-mx // Q_BLOCK)), np.nan, np.float32)
    ks = np.full((nseq, Hk, -(-mx // K_BLOCK)), np.nan, np.float32)
    km = np.zeros((nseq, Hk, d), np.float32)
    qm = np.full((nseq, H, -(-mx // Q_BLOCK), d), np.nan, np.float32)
    for i in range(nseq):
        a, b = int(cu[i]), int(cu[i + 1])
        if b == a:
            continue
        if smooth_q:
            c, s, m = quant_q_smooth(q[:, a:b], sm)
            qm[i, :, : m.shape[-2]] = m
        elif q_per_token:
            c, s = quant_q_per_token(q[:, a:b], sm)
        else:
            c, s = quant_q(q[:, a:b], sm)
        qi[:, a:b] = c
        if q_per_token:
            qs[:, a:b] = s
        else:
            qs[i, :, : s.shape[-1]] = s
        c, s, m = quant_k(k[:, a:b])
        ki[:, a:b] = c
        ks[i, :, : s.shape[-1]] = s
        km[i] = m
    out = dict(q_int8=qi, q_scale=qs, k_int8=ki, k_scale=ks, k_mean=km)
    if smooth_q:
        out["q_mean"] = qm
    return out


# ----------------------------------------------------------------------------
# OCP FP8 E4M3 (e4m3fn) from its definition: 1 sign bit, 4 exponent bits with
# bias 7, 3 mantissa bits, subnormals at exponent field 0 (spacing 2^-9), the
# single NaN pattern S.1111.111, largest finite 448.
# ----------------------------------------------------------------------------
def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """e4m3 byte codes -> fp64 values (NaN for the NaN patterns)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), (e - 10).astype(np.int64)))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3 value, ties to even mantissa, saturating at ±448."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    neg = np.signbit(np.asarray(x, dtype=np.float64))
    a = np.minimum(a, E4M3_MAX)
    # exponent of the leading bit: a = f * 2^E, f in [0.5, 1) -> floor(log2 a) = E - 1
    _, E = np.frexp(a)
    e_unb = np.maximum(E - 1, -6)                 # below 2^-6: subnormal spacing 2^-9
    quantum_exp = e_unb - 3
    mant = np.rint(np.ldexp(a, -quantum_exp))     # exact scaling by a power of two
    # mantissa overflow (e.g. 15.5 -> 16) moves to the next binade
    carry = mant >= 16
    mant = np.where(carry, mant / 2, mant)
    e_unb = np.where(carry, e_unb + 1, e_unb)
    normal = mant >= 8
    efield = np.where(normal, e_unb + 7, 0)
    mfield = np.where(normal, mant - 8, mant)
    code = (efield.astype(np.int64) << 3) | mfield.astype(np.int64)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def quant_v_fp8(v: np.ndarray):
    """V per channel to e4m3 ([DT] "SageAttention 2": P and V in FP8; per-channel
    V scale = amax over tokens / 448).  v fp16 [..., n, d] ->
    (codes uint8 [..., n, d], scale fp32 [..., d]).  Division is fp32."""
    vf = v.astype(np.float32)
    amax = np.abs(vf).max(axis=-2)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    ratio = (vf / safe[..., None, :]).astype(np.float32)
    codes = e4m3_encode(ratio)
    codes = np.where((scale > 0)[..., None, :], codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


# ----------------------------------------------------------------------------
# OCP FP4 (e2m1) and microscaling (MX) blocks ([DT] "SageAttention 3":
# microscaling FP4 attention with two-level quantisation).  e2m1: 1 sign bit,
# 2 exponent bits with bias 1, 1 mantissa bit, exponent field 0 subnormal
# (spacing 0.5); magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no inf or NaN.
# ----------------------------------------------------------------------------
def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit e2m1 codes (low nibble of each byte) -> fp64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int64)))
    return np.where(c & 0x8, -mag, mag)


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """Nearest e2m1 value, ties to the even mantissa, saturating at ±6; the
    sign bit follows x (a negative value that rounds to zero gives -0)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    # spacing of the binade: 0.5 below 2, 1 in [2, 4), 2 in [4, 6]
    q = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    k = np.rint(a / q)                      # ties to even multiple = even mantissa
    v = np.minimum(k * q, E2M1_MAX)
    # value -> code: exponent field and mantissa bit of v
    code = np.select([v == 0, v == 0.5, v == 1, v == 1.5, v == 2, v == 3, v == 4],
                     [0, 1, 2, 3, 4, 5, 6], 7)
    code = np.where(np.signbit(x), code | 0x8, code)   # the sign is kept, -0 included
    return code.astype(np.uint8)


def mx_block_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer X with amax <= 6·2^X (the block maximum fits e2m1's
    largest value), within E8M0's [-127, 127]; amax = 0 gives -127.  Exact:
    with amax = f·2^e, f in [0.5, 1), X = e - 3 + (f > 0.75)."""
    amax = np.asarray(amax, dtype=np.float64)
    f, e = np.frexp(amax)
    X = e.astype(np.int64) - 3 + (f > 0.75)
    return np.where(amax > 0, np.clip(X, -127, 127), -127).astype(np.int64)


def mx_quantize(x: np.ndarray, axis: int):
    """MX FP4 of fp32 x in blocks of 32 along ``axis`` (the last block may be
    partial): per block X = mx_block_exponent(max|x|), codes = e2m1(x / 2^X)
    (an exact scaling).  Returns (codes uint8, same shape as x; X int64 with
    ``axis`` replaced by the block count)."""
    x = np.moveaxis(np.asarray(x, dtype=np.float32), axis, -1).astype(np.float64)
    *lead, n = x.shape
    nb = -(-n // MX_BLOCK)
    xp = np.zeros((*lead, nb * MX_BLOCK))
    xp[..., :n] = x
    xb = xp.reshape(*lead, nb, MX_BLOCK)
    X = mx_block_exponent(np.abs(xb).max(axis=-1))
    codes = e2m1_encode(xb * np.ldexp(1.0, -X)[..., None]).reshape(*lead, nb * MX_BLOCK)[..., :n]
    return np.moveaxis(codes, -1, axis), np.moveaxis(X, -1, axis)


def mxfp4_decode(codes: np.ndarray, X: np.ndarray, axis: int) -> np.ndarray:
    """Values of MX FP4 data: e2m1(code) · 2^X of its block (fp64)."""
    c = np.moveaxis(e2m1_decode(codes), axis, -1)
    sc = np.repeat(np.ldexp(1.0, np.moveaxis(X, axis, -1)), MX_BLOCK, axis=-1)[..., :c.shape[-1]]
    return np.moveaxis(c * sc, -1, axis)


def quant_mxfp4_qk(q: np.ndarray, k: np.ndarray):
    """Q and the smoothed K as MX FP4 along channels (32-channel blocks of each
    token).  Returns (q_codes, q_X [..., n, d/32], k_codes, k_X, k_mean); the
    softmax scale stays outside (a power-of-two scale cannot hold it)."""
    qc, qx = mx_quantize(q.astype(np.float32), -1)
    km = k_token_mean(k)
    kc, kx = mx_quantize(smooth_k(k, km), -1)
    return qc, qx, kc, kx, km


def quant_mxfp4_q_smooth(q: np.ndarray):
    """Q smoothed by its 128-token block mean (the rule of ``q_block_mean``),
    then MX FP4 along channels: x = fp32(q) - q̄.  Returns (codes, X, q_mean);
    the score term the mean carries is ``q_smooth_bias``, added to the scores
    of the block's rows as for the INT8 path."""
    n = q.shape[-2]
    qm = q_block_mean(q)
    x = q.astype(np.float32) - np.repeat(qm, Q_BLOCK, axis=-2)[..., :n, :]
    codes, X = mx_quantize(x.astype(np.float32), -1)
    return codes, X, qm


def quant_mxfp4_v(v: np.ndarray):
    """V as MX FP4 along keys: per channel, blocks of 32 consecutive keys of
    the sequence.  Returns (codes [..., n, d], X [..., ceil(n/32), d])."""
    return mx_quantize(v.astype(np.float32), -2)


def mxfp4_attention_rows(q_codes, q_X, k_codes, k_X, v_codes, v_X, rows: Sequence[int], causal: bool,
                         sm_scale: float, tile: int = KV_TILE, score_bias: Optional[np.ndarray] = None):
    """Output rows of the MXFP4 attention for one (sequence, head).

    S = (Q̃ K̃ᵀ)·sm_scale with Q̃, K̃ the decoded MX FP4 values; online softmax
    over 64-key tiles in ascending order (exact per-tile max, [IP] §3.1);
    level one: p = e^(s - m) <= 1; level two: per query and 32-key block,
    p̃ = e2m1(p / 2^X)·2^X with X from the block's largest p; O = αO + P̃·Ṽ;
    out = fp16(O / l), l from the unrounded p.  fp64 arithmetic.
    ``score_bias`` [ceil(n/128), n]: a term added to the scores of each Q
    block's rows, as in ``sage_attention_rows``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    n, d = k_codes.shape
    R = len(rows)
    qv = mxfp4_decode(q_codes[rows], q_X[rows], -1)
    kv = mxfp4_decode(k_codes, k_X, -1)
    vv = mxfp4_decode(v_codes, v_X, -2)
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    O = np.zeros((R, d))
    last_row = int(rows.max()) if R else -1
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        for t0 in range(0, n, tile):
            if causal and t0 > last_row:
                break
            keys = np.arange(t0, min(n, t0 + tile))
            s = (qv @ kv[keys].T) * float(sm_scale)
            if score_bias is not None:
                s = s + score_bias[rows // Q_BLOCK][:, keys]
            if causal:
                s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            live = m_new > -np.inf
            alpha = np.where(live, np.exp(m - m_new), 1.0)
            alpha = np.where(np.isneginf(m) & live, 0.0, alpha)
            p = np.where(live[:, None], np.exp(s - m_new[:, None]), 0.0)
            l = alpha * l + p.sum(axis=1)
            pq = np.zeros_like(p)
            for b0 in range(0, len(keys), MX_BLOCK):       # 32-key blocks of the tile
                sl = slice(b0, b0 + MX_BLOCK)
                X = mx_block_exponent(p[:, sl].max(axis=1))[:, None]
                pq[:, sl] = e2m1_decode(e2m1_encode(p[:, sl] * np.ldexp(1.0, -X))) * np.ldexp(1.0, X)
            O = alpha[:, None] * O + pq @ vv[keys]
            m = m_new
    return (O / l[:, None]).astype(np.float16)


def mxfp4_open_code_bound(q_codes, q_X, k_codes, k_X, v_codes, v_X, rows: Sequence[int], causal: bool,
                          sm_scale: float, score_eps: np.ndarray, tile: int = KV_TILE,
                          score_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Per output element of ``mxfp4_attention_rows``, the largest change that
    another correct evaluation of the scores can make through the P codes.

    P is quantised to 3-bit e2m1 elements with a per-block power-of-two scale
    taken from the block's largest p, so a score moved by a rounding-size ε (an
    fp32 evaluation against this fp64 one) can move a code, or a block's
    exponent, to a neighbour — each such choice is the method.  With ε per key
    (``score_eps`` [n], natural-log units), p moves by at most e^(±2ε) (ε from
    the score and ε from the tile max it is taken against); e2m1 rounding and
    the exponent choice are monotone, so every code lies between those of the
    two ends.  Returns fp64 [len(rows), d]: (W + γ·(W + 2·Wabs)) / l with W the
    running sum of |code change|·|Ṽ|, Wabs of |P̃|·|Ṽ| and γ = e^(4ε_max) - 1
    for the row sums.  Test infrastructure: the reference itself is
    ``mxfp4_attention_rows``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    n, d = k_codes.shape
    R = len(rows)
    qv = mxfp4_decode(q_codes[rows], q_X[rows], -1)
    kv = mxfp4_decode(k_codes, k_X, -1)
    vv = np.abs(mxfp4_decode(v_codes, v_X, -2))
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    W = np.zeros((R, d))
    Wabs = np.zeros((R, d))
    last_row = int(rows.max()) if R else -1
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        for t0 in range(0, n, tile):
            if causal and t0 > last_row:
                break
            keys = np.arange(t0, min(n, t0 + tile))
            s = (qv @ kv[keys].T) * float(sm_scale)
            if score_bias is not None:
                s = s + score_bias[rows // Q_BLOCK][:, keys]
            if causal:
                s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            live = m_new > -np.inf
            alpha = np.where(live, np.exp(m - m_new), 1.0)
            alpha = np.where(np.isneginf(m) & live, 0.0, alpha)
            p = np.where(live[:, None], np.exp(s - m_new[:, None]), 0.0)
            l = alpha * l + p.sum(axis=1)
            pq = np.zeros_like(p)
            dcode = np.zeros_like(p)
            for b0 in range(0, len(keys), MX_BLOCK):
                sl = slice(b0, b0 + MX_BLOCK)
                pb = p[:, sl]
                X = mx_block_exponent(pb.max(axis=1))[:, None]
                pq[:, sl] = e2m1_decode(e2m1_encode(pb * np.ldexp(1.0, -X))) * np.ldexp(1.0, X)
                e2 = 2.0 * score_eps[keys[sl]][None, :]
                lo, hi = pb * np.exp(-e2), pb * np.exp(e2)
                cands = []
                for ps in (lo, hi):
                    for Xc in (mx_block_exponent(ps.max(axis=1))[:, None],
                               mx_block_exponent(lo.max(axis=1))[:, None],
                               mx_block_exponent(hi.max(axis=1))[:, None]):
                        cands.append(e2m1_decode(e2m1_encode(ps * np.ldexp(1.0, -Xc))) * np.ldexp(1.0, Xc))
                dcode[:, sl] = np.max([np.abs(c - pq[:, sl]) for c in cands], axis=0)
            W = alpha[:, None] * W + dcode @ vv[keys]
            Wabs = alpha[:, None] * Wabs + pq @ vv[keys]
            m = m_new
    gamma = np.expm1(4.0 * np.max(score_eps))
    return (W + gamma * (W + 2.0 * Wabs)) / l[:, None]


# ----------------------------------------------------------------------------
# Integer QKᵀ ([PS] SageAttention bullets: QKᵀ in INT8)
# ----------------------------------------------------------------------------
def qk_int(q_int8: np.ndarray, k_int8: np.ndarray) -> np.ndarray:
    """Exact integer Q̂K̂ᵀ: [m, d] x [n, d] -> int64 [m, n].

    Computed as an fp64 matrix product of the small integers; every partial
    sum is an integer below 2^53, so the result is exact.
    """
    r = q_int8.astype(np.float64) @ k_int8.astype(np.float64).T
    return r.astype(np.int64)


# ----------------------------------------------------------------------------
# The method's attention for selected query rows of one (sequence, head)
# ----------------------------------------------------------------------------
def sage_attention_rows(q_int8: np.ndarray, q_scale: np.ndarray, k_int8: np.ndarray,
                        k_scale: np.ndarray, v: np.ndarray, rows: Sequence[int], causal: bool,
                        pv_mode: str = "fp16", v_scale: Optional[np.ndarray] = None,
                        tile: int = KV_TILE, score_bias: Optional[np.ndarray] = None,
                        q_block: int = Q_BLOCK):
    """Output rows of the quantised attention for one (sequence, head).

    Inputs: q_int8/k_int8 [n, d] codes, q_scale [ceil(n/q_block)] (softmax
    scale folded in; q_block = 1 for per-token Q scales), k_scale [ceil(n/64)];
    v fp16 [n, d] (fp16 mode) or e4m3 codes [n, d] with v_scale [d] (fp8
    mode).  ``rows``: query indices.  ``score_bias``: with a smoothed Q, the
    [ceil(n/128), n] term of ``q_smooth_bias``, added to every score of a row
    of that Q block.

    Steps:
      * S = int(Q̂K̂ᵀ) · δQ · δK  ([PS] quantisation step 3, C ≈ (ÂB̂)(δAδB)),
        plus the Q-smoothing term when given;
      * causal: key j > query i is masked ([CS]: is_causal=True);
      * online softmax over 64-key tiles in ascending order ([IP] §3.1):
        m' = max(m, max_j s), α = e^(m-m'), p = e^(s-m'), l = αl + Σp;
      * fp16 mode ([PS] SageAttention bullets, PV in FP16):
        O = αO + fp16(p)·V, out = fp16(O / l);
      * fp8 mode ([DT] "SageAttention 2"; [PS] SageAttention2 bullets):
        level 1: A = e4m3(448 p)·V̂ for this tile alone; level 2: O = αO + A;
        out = fp16(O · δV / (448 l)).
    Arithmetic in fp64.  Returns fp16 [len(rows), d].
    """
    rows = np.asarray(rows, dtype=np.int64)
    n, d = k_int8.shape
    R = len(rows)
    if pv_mode not in ("fp16", "fp8"):
        raise ValueError(pv_mode)
    qf = q_int8[rows].astype(np.float64)
    dq = q_scale[rows // q_block].astype(np.float64)
    if pv_mode == "fp8":
        if v_scale is None:
            raise ValueError("fp8 mode needs v_scale")
        vv = e4m3_decode(v)
    else:
        vv = v.astype(np.float64)
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    O = np.zeros((R, d))
    last_row = int(rows.max()) if R else -1
    with np.errstate(invalid="ignore", over="ignore"):
        for t0 in range(0, n, tile):
            if causal and t0 > last_row:
                break                                   # no visible key for any row
            keys = np.arange(t0, min(n, t0 + tile))
            acc = qf @ k_int8[keys].astype(np.float64).T
            dk = k_scale[keys // K_BLOCK].astype(np.float64)
            s = acc * dq[:, None] * dk[None, :]
            if score_bias is not None:
                s = s + score_bias[rows // Q_BLOCK][:, keys]
            if causal:
                s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            live = m_new > -np.inf
            alpha = np.where(live, np.exp(m - m_new), 1.0)
            alpha = np.where(np.isneginf(m) & live, 0.0, alpha)
            p = np.where(live[:, None], np.exp(s - m_new[:, None]), 0.0)
            l = alpha * l + p.sum(axis=1)
            if pv_mode == "fp16":
                pq = p.astype(np.float16).astype(np.float64)
                O = alpha[:, None] * O + pq @ vv[keys]
            else:
                pq = e4m3_decode(e4m3_encode(p * E4M3_MAX))
                A = pq @ vv[keys]                       # level 1: this tile only
                O = alpha[:, None] * O + A              # level 2: running output
            m = m_new
    if pv_mode == "fp16":
        out = O / l[:, None]
    else:
        out = O * v_scale.astype(np.float64)[None, :] / (E4M3_MAX * l[:, None])
    return out.astype(np.float16)


def score_lse_rows(q_int8: np.ndarray, q_scale: np.ndarray, k_int8: np.ndarray, k_scale: np.ndarray,
                   rows: Sequence[int], causal: bool, score_bias: Optional[np.ndarray] = None,
                   q_block: int = Q_BLOCK) -> np.ndarray:
    """Natural-log sum of exp of each row's dequantised scores over its visible
    keys, the quantity that merges partial softmax results over key ranges
    ([IP] §3.1 online softmax keeps it as (m, l): lse = m + log l):

        lse_i = log Σ_{j visible} exp(δQ_i · δK_j · (q̂_i · k̂_j) [+ bias]).

    ``score_bias`` as for ``sage_attention_rows`` (smoothed Q).  Plain
    definition in fp64 (shifted by the row max before exp).  Returns fp64
    [len(rows)]."""
    rows = np.asarray(rows, dtype=np.int64)
    n = k_int8.shape[0]
    keys = np.arange(n)
    acc = q_int8[rows].astype(np.float64) @ k_int8.astype(np.float64).T
    s = acc * q_scale[rows // q_block].astype(np.float64)[:, None] * k_scale[keys // K_BLOCK].astype(np.float64)[None, :]
    if score_bias is not None:
        s = s + score_bias[rows // Q_BLOCK]
    if causal:
        s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
    mx = s.max(axis=1)
    return mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))


# ----------------------------------------------------------------------------
# Plain definition: fp64 scaled-dot-product attention ([IP] §2.1)
# ----------------------------------------------------------------------------
def sdpa_fp64_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: Sequence[int],
                   causal: bool, sm_scale: Optional[float] = None) -> np.ndarray:
    """softmax(q kᵀ · sm_scale) v for the given query rows, in fp64, no
    quantisation and no smoothing.  q, k, v [n, d] (any float dtype)."""
    rows = np.asarray(rows, dtype=np.int64)
    n, d = k.shape
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    s = (q[rows].astype(np.float64) @ k.astype(np.float64).T) * scale
    if causal:
        s = np.where(np.arange(n)[None, :] > rows[:, None], -np.inf, s)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v.astype(np.float64)


# ----------------------------------------------------------------------------
# Convenience views: one (sequence, head) slice of the ABI-layout arrays
# ----------------------------------------------------------------------------
def head_views_dense(quant: Dict[str, np.ndarray], b: int, h: int):
    return (quant["q_int8"][b, h], quant["q_scale"][b, h], quant["k_int8"][b, h],
            quant["k_scale"][b, h])


def head_views_varlen(quant: Dict[str, np.ndarray], cu_seqlens, i: int, h: int):
    a, b = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
    n = b - a
    qs = quant["q_scale"]
    return (quant["q_int8"][h, a:b], qs[h, a:b] if qs.ndim == 2 else qs[i, h, : -(-n // Q_BLOCK)],
            quant["k_int8"][h, a:b], quant["k_scale"][i, h, : -(-n // K_BLOCK)])
