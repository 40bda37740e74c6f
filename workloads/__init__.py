"""Seeded synthetic inputs for the 8-bit attention forward.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantisation, no softmax, no scaling).  Both the CPU
oracle and the GPU path are fed from the same bytes produced here.

Shapes follow the workloads the pages describe: LLM prefill with a causal mask,
video-DiT-shaped long sequences with head dim 64, 32K long context, and packed
variable-length batches.  K carries a per-(head, channel) bias shared over
tokens: the token-shared channel offset that K smoothing targets (page
"SageAttention — brand new attention", paragraph on K normalisation; dtcms
summary, section "SageAttention（v1）", first bullet).

Recipe
------
* Generator: ``numpy.random.default_rng([seed, stream])``; fp32 draws rounded
  to fp16 with round-to-nearest-even (numpy ``astype``).
* ``seed = 1000 * cfg_index``; streams: q=0, k=1, v=2, q-bias=3, k-bias=4,
  outlier channels=5, sequence lengths=6.
* ``N(0, s)`` means ``s * standard_normal`` (s is the standard deviation).
* Biases have shape ``[H, d]`` and are added to every batch entry and token.
* bf16 inputs (the video-DiT workload) are drawn in fp32, rounded to bf16 with
  round-to-nearest-even, then cast to fp16 (exact at these magnitudes).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "generate", "Inputs", "generate_custom"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int              # seed = 1000 * index
    B: int                  # batch (dense) or number of sequences (varlen)
    H: int
    N: int                  # tokens per sequence (dense); max length bound (varlen)
    d: int
    causal: bool
    pv_mode: str            # "fp16" or "fp8"
    q_bias: float = 0.0     # std of the per-(head, channel) Q bias, 0 = none
    k_bias: float = 3.0     # std of the per-(head, channel) K bias
    outlier_frac: float = 0.0   # fraction of the H*d K channels scaled
    outlier_scale: float = 1.0
    outlier_bias_only: bool = False  # scale only the bias part of the outlier channels
    bf16: bool = False
    varlen: bool = False
    len_lo: int = 0
    len_hi: int = 0
    description: str = ""

    @property
    def seed(self) -> int:
        return 1000 * self.index


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, 1, 2, 256, 64, False, "fp16", k_bias=3.0,
                 description="B=1,H=2,N=256,d=64 non-causal, K bias N(0,3), fp16 PV"),
        Workload("llm_prefill", 2, 4, 32, 4096, 128, True, "fp16", k_bias=3.0,
                 description="LLM prefill B=4,H=32,N=4096,d=128 causal, fp16 PV"),
        Workload("video_dit", 3, 2, 24, 16384, 64, False, "fp16", k_bias=4.0,
                 outlier_frac=0.01, outlier_scale=20.0, bf16=True,
                 description="video-DiT B=2,H=24,N=16384,d=64 bf16->fp16, K bias N(0,4), "
                             "1% of K channels x20 (whole channel)"),
        Workload("video_dit_biasx20", 3, 2, 24, 16384, 64, False, "fp16", k_bias=4.0,
                 outlier_frac=0.01, outlier_scale=20.0, outlier_bias_only=True, bf16=True,
                 description="video-DiT variant: x20 applied to the bias of 1% of K channels only"),
        Workload("long_fp8", 4, 1, 40, 32768, 128, False, "fp8", q_bias=3.0, k_bias=3.0,
                 description="long context B=1,H=40,N=32768,d=128, Q and K bias N(0,3), FP8 PV"),
        Workload("varlen", 5, 16, 32, 8192, 128, True, "fp16", k_bias=3.0, varlen=True,
                 len_lo=512, len_hi=8192,
                 description="16 packed sequences, lengths U[512,8192], H=32,d=128 causal, fp16 PV"),
        Workload("seq16k", 6, 1, 40, 16384, 128, False, "fp16", k_bias=3.0,
                 description="B=1,H=40,N=16384,d=128 non-causal, fp16 PV (16K, d=128 point)"),
        Workload("seq16k_causal", 7, 1, 40, 16384, 128, True, "fp16", k_bias=3.0,
                 description="B=1,H=40,N=16384,d=128 causal, fp16 PV (the 16K point's causal variant)"),
        Workload("long_fp8_shard8", 8, 1, 5, 32768, 128, False, "fp8", q_bias=3.0, k_bias=3.0,
                 description="one GPU's head share of long_fp8 on 8 GPUs: B=1,H=5,N=32768,d=128, FP8 PV"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


@dataclasses.dataclass
class Inputs:
    """fp16 numpy arrays. Dense: q,k,v [B,H,N,d]. Varlen: q,k,v [H,T,d] + cu_seqlens."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_seqlens: Optional[np.ndarray] = None  # int32 [nseq+1]
    lengths: Optional[np.ndarray] = None


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _to_bf16_grid(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns fp32 holding bf16 values."""
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)
    return r


def _finish(x: np.ndarray, bf16: bool) -> np.ndarray:
    if bf16:
        x = _to_bf16_grid(x)
    return x.astype(np.float16)


def sequence_lengths(w: Workload) -> np.ndarray:
    rng = _rng(w.seed, 6)
    return rng.integers(w.len_lo, w.len_hi, size=w.B, endpoint=True).astype(np.int64)


def generate(w: Workload, heads: Optional[int] = None) -> Inputs:
    """Draw the workload's inputs.  ``heads`` (<= H) keeps only the first heads
    (the draws are made for all H and sliced, so values do not depend on it)."""
    H, d = w.H, w.d
    if w.varlen:
        lengths = sequence_lengths(w)
        T = int(lengths.sum())
        shape = (H, T, d)
        bshape = (H, 1, d)
    else:
        lengths = None
        shape = (w.B, H, w.N, d)
        bshape = (1, H, 1, d)
    q = _normal(_rng(w.seed, 0), shape)
    k = _normal(_rng(w.seed, 1), shape)
    v = _normal(_rng(w.seed, 2), shape)
    if w.q_bias:
        q += _normal(_rng(w.seed, 3), (H, d), w.q_bias).reshape(bshape)
    kb = _normal(_rng(w.seed, 4), (H, d), w.k_bias) if w.k_bias else np.zeros((H, d), np.float32)
    if w.outlier_frac > 0:
        n_out = int(round(w.outlier_frac * H * d))
        pick = _rng(w.seed, 5).choice(H * d, size=n_out, replace=False)
        if w.outlier_bias_only:
            kbf = kb.reshape(-1)
            kbf[pick] *= np.float32(w.outlier_scale)
            k += kb.reshape(bshape)
        else:
            k += kb.reshape(bshape)
            hh, cc = np.divmod(pick, d)
            for h, c in zip(hh.tolist(), cc.tolist()):
                if w.varlen:
                    k[h, :, c] *= np.float32(w.outlier_scale)
                else:
                    k[:, h, :, c] *= np.float32(w.outlier_scale)
    else:
        k += kb.reshape(bshape)
    if heads is not None and heads < H:
        if w.varlen:
            q, k, v = q[:heads], k[:heads], v[:heads]
        else:
            q, k, v = q[:, :heads], k[:, :heads], v[:, :heads]
    out = Inputs(_finish(np.ascontiguousarray(q), w.bf16),
                 _finish(np.ascontiguousarray(k), w.bf16),
                 _finish(np.ascontiguousarray(v), w.bf16))
    if w.varlen:
        out.lengths = lengths
        out.cu_seqlens = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return out


def generate_custom(seed: int, B: int, H: int, N: int, d: int, k_bias: float = 3.0,
                    q_bias: float = 0.0, lengths=None) -> Inputs:
    """Small ad-hoc shapes for edge-case tests (ragged N, tiny sequences...).
    With ``lengths`` the result is varlen-packed [H, T, d]."""
    w = Workload("custom", 0, B if lengths is None else len(lengths), H, N, d, False, "fp16",
                 q_bias=q_bias, k_bias=k_bias, varlen=lengths is not None)
    H_, d_ = H, d
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        T = int(lengths.sum())
        shape, bshape = (H_, T, d_), (H_, 1, d_)
    else:
        shape, bshape = (B, H_, N, d_), (1, H_, 1, d_)
    q = _normal(_rng(seed, 0), shape)
    k = _normal(_rng(seed, 1), shape)
    v = _normal(_rng(seed, 2), shape)
    if q_bias:
        q += _normal(_rng(seed, 3), (H_, d_), q_bias).reshape(bshape)
    if k_bias:
        k += _normal(_rng(seed, 4), (H_, d_), k_bias).reshape(bshape)
    out = Inputs(q.astype(np.float16), k.astype(np.float16), v.astype(np.float16))
    if lengths is not None:
        out.lengths = lengths
        out.cu_seqlens = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    del w
    return out
