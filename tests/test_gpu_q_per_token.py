"""GPU parity of per-token Q scales (q_per_token) against the CPU oracle.

Bars as for the rest of the path: Q̂ codes and the per-token scales bit-exact
(whole tensors); outputs against the method with per-token Q scales (O1):
max-abs <= 2e-2, cosine >= 0.9995; against fp64 exact attention (O2): cosine
>= 0.998; the LSE within 2e-3.
"""
import sys

import numpy as np
import pytest
import torch

import quantized_attention_quant_amd as sage
import margins
import workloads
from oracle import sage_oracle as O

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
COS_O1 = 0.9995
COS_O2 = 0.998
LSE_ABS = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    return t.cpu().numpy()


def check_out(ours, o1, o2, label):
    ours = np.asarray(ours, np.float64)
    assert np.isfinite(ours).all(), label
    err = np.abs(ours - o1.astype(np.float64)).max()
    c1, c2 = cos(ours, o1), cos(ours, o2)
    say(f"{label}: max_abs_vs_O1={err:.3e} cos_O1={c1:.6f} cos_O2={c2:.6f}")
    margins.record(label, err, c1, c2)
    assert err <= MAX_ABS, (label, err)
    assert c1 >= COS_O1, (label, c1)
    assert c2 >= COS_O2, (label, c2)


def o1(views, v_head, rows, causal, pv_mode, vq=None):
    qi, qs, ki, ks = views
    if pv_mode == "fp8":
        vc, vs = vq if vq is not None else O.quant_v_fp8(v_head)
        return O.sage_attention_rows(qi, qs, ki, ks, vc, rows, causal, "fp8", vs, q_block=1)
    return O.sage_attention_rows(qi, qs, ki, ks, v_head, rows, causal, "fp16", q_block=1)


SMALL = [(n, d) for d in (64, 128) for n in (1, 63, 65, 129, 257)]


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", SMALL)
def test_q_per_token_small_all_rows(n, d, causal, pv_mode):
    say(f"case q_per_token small n={n} d={d} causal={causal} pv={pv_mode}")
    B, H = 2, 3
    x = workloads.generate_custom(700 + n + d, B, H, n, d, k_bias=3.0, q_bias=1.0)
    ws = torch.empty(sage.sage_attn_workspace_size(B, H, n, d, pv_mode, q_per_token=True), dtype=torch.uint8,
                     device="cuda")
    o, lse = sage.sage_attn_fwd(dev(x.q), dev(x.k), dev(x.v), is_causal=causal, pv_mode=pv_mode, workspace=ws,
                                return_lse=True, q_per_token=True)
    o, lse, wsn = host(o), host(lse), host(ws)
    quant = O.quant_qk_dense(x.q, x.k, q_per_token=True)
    offs = sage.sage_test_workspace_layout(False, B, H, n, 0, d, pv_mode, q_per_token=True)
    # Q̂ and the per-token scales are formed inside the attention kernel (bit
    # identity with the pre-pass: test_gpu_parity.test_in_kernel_q_quantisation_bit_exact)
    rows = np.arange(n)
    for b in range(B):
        for h in range(H):
            views = O.head_views_dense(quant, b, h)
            ref1 = o1(views, x.v[b, h], rows, causal, pv_mode)
            ref2 = O.sdpa_fp64_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, causal)
            check_out(o[b, h], ref1, ref2, f"q_per_token n={n} d={d} b={b} h={h}")
            want = O.score_lse_rows(*views, rows, causal, q_block=1)
            assert np.abs(lse[b, h].astype(np.float64) - want).max() <= LSE_ABS


def test_q_per_token_quant_entry_bit_exact():
    for n, d in ((1, 64), (129, 128), (1000, 64)):
        say(f"case q_per_token quant n={n} d={d}")
        x = workloads.generate_custom(720 + n, 2, 3, n, d, k_bias=3.0, q_bias=1.0)
        # rows of very different magnitudes: per-token scales differ from the block's
        x.q[:] = (x.q.astype(np.float32) * np.exp2(np.random.default_rng(n).integers(-6, 6, (2, 3, n, 1)))
                  ).astype(np.float16)
        got = {k2: host(v2) for k2, v2 in sage.sage_quant_qk(dev(x.q), dev(x.k), q_per_token=True).items()}
        ref = O.quant_qk_dense(x.q, x.k, q_per_token=True)
        for key in ("q_int8", "k_int8", "q_scale", "k_scale", "k_mean"):
            assert got[key].shape == ref[key].shape, key
            assert (got[key].view(np.uint8) == ref[key].view(np.uint8)).all(), key


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
def test_q_per_token_gqa(pv_mode):
    B, H, H_kv, n, d = 2, 4, 1, 200, 64
    x = workloads.generate_custom(730, B, H, n, d, k_bias=3.0, q_bias=1.0)
    k = np.ascontiguousarray(x.k[:, :H_kv])
    v = np.ascontiguousarray(x.v[:, :H_kv])
    for causal in (False, True):
        say(f"case q_per_token gqa pv={pv_mode} causal={causal}")
        o, lse = sage.sage_attn_fwd(dev(x.q), dev(k), dev(v), is_causal=causal, pv_mode=pv_mode, return_lse=True,
                                    q_per_token=True)
        o, lse = host(o), host(lse)
        k_rep, v_rep = np.repeat(k, H, axis=1), np.repeat(v, H, axis=1)
        quant = O.quant_qk_dense(x.q, k_rep, q_per_token=True)
        vq = O.quant_v_fp8(v_rep)
        rows = np.arange(n)
        for b in range(B):
            for h in range(H):
                views = O.head_views_dense(quant, b, h)
                ref1 = o1(views, v_rep[b, h], rows, causal, pv_mode, (vq[0][b, h], vq[1][b, h]))
                ref2 = O.sdpa_fp64_rows(x.q[b, h], k_rep[b, h], v_rep[b, h], rows, causal)
                check_out(o[b, h], ref1, ref2, f"q_per_token gqa b={b} h={h}")
                want = O.score_lse_rows(*views, rows, causal, q_block=1)
                assert np.abs(lse[b, h].astype(np.float64) - want).max() <= LSE_ABS


def test_q_per_token_varlen():
    lens = [1, 65, 300, 0, 129]
    H, d = 2, 128
    x = workloads.generate_custom(740, 0, H, 0, d, k_bias=3.0, q_bias=1.0, lengths=lens)
    cu = dev(x.cu_seqlens)
    mx = max(lens)
    got = {k2: host(v2) for k2, v2 in sage.sage_quant_qk(dev(x.q), dev(x.k), cu_seqlens=cu, max_seqlen=mx,
                                                         q_per_token=True).items()}
    quant = O.quant_qk_varlen(x.q, x.k, x.cu_seqlens, q_per_token=True)
    assert (got["q_int8"] == quant["q_int8"]).all()
    assert (got["q_scale"].view(np.uint32) == quant["q_scale"].view(np.uint32)).all()
    for pv_mode in ("fp16", "fp8"):
        for causal in (False, True):
            say(f"case q_per_token varlen pv={pv_mode} causal={causal}")
            o, lse = sage.sage_attn_varlen_fwd(dev(x.q), dev(x.k), dev(x.v), cu, mx, is_causal=causal,
                                               pv_mode=pv_mode, return_lse=True, q_per_token=True)
            o, lse = host(o), host(lse)
            for i, n in enumerate(lens):
                if n == 0:
                    continue
                a0 = int(x.cu_seqlens[i])
                rows = np.arange(n)
                for h in range(H):
                    views = O.head_views_varlen(quant, x.cu_seqlens, i, h)
                    vv = x.v[h, a0:a0 + n]
                    ref1 = o1(views, vv, rows, causal, pv_mode)
                    ref2 = O.sdpa_fp64_rows(x.q[h, a0:a0 + n], x.k[h, a0:a0 + n], vv, rows, causal)
                    check_out(o[h, a0:a0 + n], ref1, ref2, f"q_per_token varlen seq={i} h={h}")
                    want = O.score_lse_rows(*views, rows, causal, q_block=1)
                    assert np.abs(lse[h, a0:a0 + n].astype(np.float64) - want).max() <= LSE_ABS


def _sample_rows(n, rng, k=40):
    return np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, n - 1], rng.choice(n, size=min(n, k), replace=False)]))


@pytest.mark.parametrize("name", ["seq16k", "video_dit_biasx20", "llm_prefill"])
def test_q_per_token_workload(name):
    """Full-size workloads with per-token Q scales, in the benchmark's launch shape."""
    w = workloads.get(name)
    say(f"case q_per_token workload {name} {w.description}")
    x = workloads.generate(w)
    B, H, N, d = x.q.shape
    q = dev(x.q)
    k = dev(x.k)
    got = host(sage.sage_quant_qk(q, k, q_per_token=True)["q_scale"])
    ref = O.quant_qk_dense(x.q, x.k, q_per_token=True)
    assert (got.view(np.uint32) == ref["q_scale"].view(np.uint32)).all()
    o = host(sage.sage_attn_fwd(q, k, dev(x.v), is_causal=w.causal, pv_mode=w.pv_mode, q_per_token=True))
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 11)
    heads = [(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))]
    for b, h in heads:
        rows = _sample_rows(N, rng)
        views = O.head_views_dense(ref, b, h)
        ref1 = o1(views, x.v[b, h], rows, w.causal, w.pv_mode)
        ref2 = O.sdpa_fp64_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, w.causal)
        check_out(o[b, h, rows], ref1, ref2, f"q_per_token {name} b={b} h={h}")


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_q_per_token_large_magnitude(causal, d, pv_mode):
    """Inputs ×30: per-lane factors δQ_i·δK·log2(e) well above 2^-7, so the
    FP16 path's exact-log2 conversion decides lane by lane."""
    say(f"case q_per_token large magnitude d={d} causal={causal} pv={pv_mode}")
    B, H, n = 1, 2, 300
    x = workloads.generate_custom(760 + d, B, H, n, d, k_bias=3.0, q_bias=1.0)
    q = (x.q.astype(np.float32) * np.float32(30.0)).astype(np.float16)
    k = (x.k.astype(np.float32) * np.float32(30.0)).astype(np.float16)
    o = host(sage.sage_attn_fwd(dev(q), dev(k), dev(x.v), is_causal=causal, pv_mode=pv_mode, q_per_token=True))
    quant = O.quant_qk_dense(q, k, q_per_token=True)
    c2 = float(quant["q_scale"].max()) * float(quant["k_scale"].max()) * 1.4426950408889634
    assert c2 > 2.0 ** -7, c2
    rows = np.arange(n)
    for h in range(H):
        views = O.head_views_dense(quant, 0, h)
        ref1 = o1(views, x.v[0, h], rows, causal, pv_mode)
        ref2 = O.sdpa_fp64_rows(q[0, h], k[0, h], x.v[0, h], rows, causal)
        ours = np.asarray(o[0, h], np.float64)
        assert np.isfinite(ours).all()
        err = np.abs(ours - ref1).max()
        c1, c2o = cos(ours, ref1), cos(ours, ref2)
        say(f"  h={h}: max_abs_vs_O1={err:.3e} cos_O1={c1:.6f} cos_O2={c2o:.6f}")
        margins.record(f"x-scaled h={h}", err, c1, c2o)
        assert err <= MAX_ABS and c1 >= COS_O1, (h, err, c1)
        # at this magnitude the method itself is further from exact attention
        assert c2o >= min(COS_O2, cos(ref1, ref2) - 1e-4), (h, c2o)
