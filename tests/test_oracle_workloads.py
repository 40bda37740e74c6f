"""The method (oracle O1) against fp64 exact attention (O2) at the workloads'
real shapes: one head per workload, sampled query rows.  CPU only.

Bar: cosine >= 0.998, the per-layer similarity the dtcms summary's section
"SageAttention（v1）" uses to accept a variant.  The video-DiT workload under
the literal reading (whole K channels scaled x20) is below that bar for the
method itself; it is held to the looser floor recorded next to it.
"""
import numpy as np
import pytest

from oracle import sage_oracle as O
import workloads


def cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


# literal-reading floor for video_dit: the method's own cosine there is ~0.995
FLOORS = {"video_dit": 0.99}


def _head_inputs(w, h):
    x = workloads.generate(w, heads=h + 1)
    if w.varlen:
        a, b = int(x.cu_seqlens[0]), int(x.cu_seqlens[1])
        return x.q[h, a:b], x.k[h, a:b], x.v[h, a:b]
    return x.q[0, h], x.k[0, h], x.v[0, h]


@pytest.mark.parametrize("name", ["tiny", "llm_prefill", "video_dit", "video_dit_biasx20",
                                  "long_fp8", "varlen", "seq16k", "seq16k_causal"])
def test_method_vs_exact_at_workload_shape(name):
    w = workloads.get(name)
    h = 1
    q, k, v = _head_inputs(w, h)
    n = q.shape[0]
    rng = np.random.default_rng(w.seed + 99)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(n, 96), replace=False)]))
    quant = O.quant_qk_dense(q[None, None], k[None, None])
    qi, qs, ki, ks = O.head_views_dense(quant, 0, 0)
    if w.pv_mode == "fp8":
        vc, vs = O.quant_v_fp8(v)
        ours = O.sage_attention_rows(qi, qs, ki, ks, vc, rows, w.causal, "fp8", vs)
    else:
        ours = O.sage_attention_rows(qi, qs, ki, ks, v, rows, w.causal, "fp16")
    ref = O.sdpa_fp64_rows(q, k, v, rows, w.causal)
    c = cos(ours, ref)
    assert c >= FLOORS.get(name, 0.998), (name, c)
