"""GPU parity of Q smoothing (smooth_q) against the CPU oracle.

Bars, as for the rest of the path: the Q block means, the residual INT8 codes
and their scales are bit-exact; the per-(Q block, key) smoothing term the
pre-pass hands to the attention kernel is checked against the oracle's fp64
term — FP16 PV: within one unit of the tile's dequantisation step δQ·δK plus
1e-5 of the term's absolute sum, or in fp32 where a half tile takes the
fallback; FP8 PV: in fp32 for every key, within the error of its split-fp16
evaluation; outputs against the method with the term (O1): max-abs <= 2e-2,
cosine >= 0.9995; against fp64 exact attention (O2): cosine >= 0.998; the LSE
within 2e-3.  The same bars hold for both PV modes.
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
MAGIC = 0x4B400000
LOG2E = np.float32(1.4426950408889634)


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


def o1_rows(quant, k_head, v_head, b, h, rows, causal, pv_mode, vq=None):
    """The method with the smoothing term for one (batch, head) of a dense call
    (K/V already repeated to the query heads)."""
    qi, qs, ki, ks = O.head_views_dense(quant, b, h)
    d = qi.shape[-1]
    sm = O.default_sm_scale(d)
    bias = O.q_smooth_bias(quant["q_mean"][b, h], k_head, quant["k_mean"][b, h], sm)
    if pv_mode == "fp8":
        vc, vs = vq if vq is not None else O.quant_v_fp8(v_head)
        o = O.sage_attention_rows(qi, qs, ki, ks, vc, rows, causal, "fp8", vs, score_bias=bias)
    else:
        o = O.sage_attention_rows(qi, qs, ki, ks, v_head, rows, causal, "fp16", score_bias=bias)
    return o, bias, (qi, qs, ki, ks)


def fit_decisions(quant, k_head, b, h, n, d):
    """Per (Q block, tile, half): the halves whose integer terms surely fit
    (every |Δ·log2e / c2| at least 1e-4 below the limit, c2 normal) and those
    that surely do not, from the oracle's fp64 terms; [nqb, nkb, 2] each."""
    nqb, nkb = -(-n // 128), -(-n // 64)
    sm = O.default_sm_scale(d)
    bias = O.q_smooth_bias(quant["q_mean"][b, h], k_head, quant["k_mean"][b, h], sm)
    c2 = (quant["q_scale"][b, h].astype(np.float32)[:, None] * quant["k_scale"][b, h].astype(np.float32)[None, :])
    c2 = (c2.astype(np.float32) * np.float32(LOG2E)).astype(np.float32).astype(np.float64)
    normal = (c2 >= np.finfo(np.float32).tiny) & (c2 <= 3.0e38)
    ratio = np.zeros((nqb, 64 * nkb))
    keys = np.arange(n)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio[:, :n] = np.abs(bias) * float(LOG2E) / c2[:, keys // 64]
    hmax = np.nan_to_num(ratio, nan=np.inf).reshape(nqb, nkb, 2, 32).max(axis=-1)
    limit = (1 << 22) - 1 - 127 * 127 * d
    sure_fit = normal[:, :, None] & (hmax < limit * (1 - 1e-4))
    sure_fb = ~normal[:, :, None] | (hmax > limit * (1 + 1e-4))
    return sure_fit, sure_fb


def check_terms(wsn, offs, quant, k, B, H, n, d, causal, expect_fallback=None):
    """The workspace's smoothing terms against the oracle's (dense, H_kv = H)."""
    nqb, nkb = -(-n // 128), -(-n // 64)
    npad = 64 * nkb
    slots = wsn[offs[8]:offs[8] + 4 * B * H * nqb * npad].view(np.int32).reshape(B, H, nqb, npad)
    fix = wsn[offs[9]:offs[9] + 4 * B * H * nqb * npad].view(np.float32).reshape(B, H, nqb, npad)
    flags = wsn[offs[10]:offs[10] + 4 * B * H * nqb * 2 * nkb].view(np.int32).reshape(B, H, nqb, nkb, 2)
    # per-row summaries after the flags (16-byte aligned): nonzero iff a written half falls back
    so = offs[10] + -(-4 * B * H * nqb * 2 * nkb // 16) * 16
    summary = wsn[so:so + 4 * B * H * nqb].view(np.int32).reshape(B, H, nqb)
    live = np.ones((nqb, nkb), bool)
    if causal:
        live = 64 * np.arange(nkb)[None, :] <= 128 * np.arange(nqb)[:, None] + 127
    for blk in range(nqb):
        want_any = (flags[:, :, blk][:, :, live[blk]] != 0).any(axis=(2, 3))
        assert ((summary[:, :, blk] != 0) == want_any).all(), ("row summary", blk)
    sm = O.default_sm_scale(d)
    seen_fb = 0
    for b in range(B):
        for h in range(H):
            bias = O.q_smooth_bias(quant["q_mean"][b, h], k[b, h], quant["k_mean"][b, h], sm)
            x = O.smooth_k(k[b, h], quant["k_mean"][b, h]).astype(np.float64)
            absum = np.abs(quant["q_mean"][b, h].astype(np.float64)) @ np.abs(x).T * float(sm)
            for qb in range(nqb):
                for t in range(nkb):
                    if causal and 64 * t > 128 * qb + 127:
                        continue  # no query of the block sees the tile: not written
                    c2 = np.float32(np.float32(quant["q_scale"][b, h, qb]) * np.float32(quant["k_scale"][b, h, t]))
                    c2 = np.float32(c2 * LOG2E)
                    for s in range(2):
                        keys = np.arange(64 * t + 32 * s, min(n, 64 * t + 32 * s + 32))
                        if len(keys) == 0:
                            continue
                        want = bias[qb, keys] * float(LOG2E)
                        scale = absum[qb, keys] * float(LOG2E)
                        if flags[b, h, qb, t, s] == 0:
                            assert c2 >= np.finfo(np.float32).tiny
                            got = (slots[b, h, qb, keys].astype(np.int64) - MAGIC).astype(np.float64)
                            err = np.abs(got - want / float(c2))
                            tol = 1.0 + 1e-5 * scale / float(c2)
                            assert (err <= tol).all(), (b, h, qb, t, s, err.max())
                        else:
                            seen_fb += 1
                            assert (slots[b, h, qb, keys] == MAGIC).all()
                            err = np.abs(fix[b, h, qb, keys].astype(np.float64) - want)
                            assert (err <= 1e-5 * scale + 1e-30).all(), (b, h, qb, t, s, err.max())
                            # the fallback is taken only when the integer would not fit
                            if c2 >= np.finfo(np.float32).tiny:
                                assert np.abs(want / float(c2)).max() > (1 << 22) - 1 - 127 * 127 * d - 4
    if expect_fallback is not None:
        assert (seen_fb > 0) == expect_fallback, seen_fb
    return seen_fb


def check_terms_fp32(wsn, offs, quant, k, B, H, n, d, causal):
    """FP8 PV: the workspace holds every key's term in fp32, sm_scale·q̄·x·log2(e)
    (region [9]), against the oracle's fp64 term.  The pre-pass splits q̄ and x,
    each scaled by a power of two below twice its largest magnitude, into fp16
    hi + lo parts (hi + lo within 2^-22 of the value, plus 2^-25 of the scale
    where lo is subnormal) and sums the four products of each channel in fp32
    (32 accumulations at d = 128): the bound is 2^-21·|q̄_c·x_c| and 2^-25 of
    the scales per channel, 2^-19 of Σ|q̄_c·x_c| for the accumulation, and
    the final rounding."""
    nqb, nkb = -(-n // 128), -(-n // 64)
    npad = 64 * nkb
    fix = wsn[offs[9]:offs[9] + 4 * B * H * nqb * npad].view(np.float32).reshape(B, H, nqb, npad)
    sm = float(O.default_sm_scale(d))
    for b in range(B):
        for h in range(H):
            bias = O.q_smooth_bias(quant["q_mean"][b, h], k[b, h], quant["k_mean"][b, h], sm)
            x = np.abs(O.smooth_k(k[b, h], quant["k_mean"][b, h]).astype(np.float64))
            qm = np.abs(quant["q_mean"][b, h].astype(np.float64))
            for qb in range(nqb):
                seen = n if not causal else min(n, 64 * ((128 * qb + 127) // 64 + 1))
                keys = np.arange(seen)
                want = bias[qb, keys] * float(LOG2E)
                absum = x[keys] @ qm[qb]
                scale = 2.0 * x.max() * qm[qb].sum() + 2.0 * qm[qb].max() * x[keys].sum(axis=1)
                tol = ((2.0 ** -21 * absum + 2.0 ** -25 * scale + 2.0 ** -19 * absum) * sm * float(LOG2E)
                       + 2.0 ** -22 * np.abs(want) + 1e-30)
                err = np.abs(fix[b, h, qb, keys].astype(np.float64) - want)
                assert (err <= tol).all(), (b, h, qb, float(err.max()), float((err / tol).max()))


# ---------------------------------------------------------------------------
SMALL = [(n, d) for d in (64, 128) for n in (1, 65, 129, 200, 257)]


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", SMALL)
def test_smooth_q_small_all_rows(n, d, causal, pv_mode):
    say(f"case smooth_q small n={n} d={d} causal={causal} pv={pv_mode}")
    B, H = 2, 3
    x = workloads.generate_custom(500 + n + d, B, H, n, d, k_bias=3.0, q_bias=3.0)
    ws = torch.empty(sage.sage_attn_workspace_size(B, H, n, d, pv_mode, smooth_q=True), dtype=torch.uint8,
                     device="cuda")
    o, lse = sage.sage_attn_fwd(dev(x.q), dev(x.k), dev(x.v), is_causal=causal, pv_mode=pv_mode, workspace=ws,
                                return_lse=True, smooth_q=True)
    o, lse, wsn = host(o), host(lse), host(ws)
    quant = O.quant_qk_dense(x.q, x.k, smooth_q=True)
    offs = sage.sage_test_workspace_layout(False, B, H, n, 0, d, pv_mode, smooth_q=True)
    n8 = B * H * n * d
    assert (wsn[offs[0]:offs[0] + n8].view(np.int8) == quant["q_int8"].ravel()).all()
    nqb = -(-n // 128)
    assert (wsn[offs[2]:offs[2] + 4 * B * H * nqb].view(np.uint32) == quant["q_scale"].view(np.uint32).ravel()).all()
    assert (wsn[offs[7]:offs[7] + 4 * B * H * nqb * d].view(np.uint32) ==
            quant["q_mean"].view(np.uint32).ravel()).all()
    if pv_mode == "fp8":
        check_terms_fp32(wsn, offs, quant, x.k, B, H, n, d, causal)
    else:
        # a last Q block of one token has a zero residual (δQ = 0): its half
        # tiles take the fp32 fallback; the others fit the accumulator
        check_terms(wsn, offs, quant, x.k, B, H, n, d, causal, expect_fallback=(n % 128 == 1))
    rows = np.arange(n)
    for b in range(B):
        for h in range(H):
            o1, bias, (qi, qs, ki, ks) = o1_rows(quant, x.k[b, h], x.v[b, h], b, h, rows, causal, pv_mode)
            o2 = O.sdpa_fp64_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, causal)
            check_out(o[b, h], o1, o2, f"smooth n={n} d={d} b={b} h={h}")
            want = O.score_lse_rows(qi, qs, ki, ks, rows, causal, score_bias=bias)
            assert np.abs(lse[b, h].astype(np.float64) - want).max() <= LSE_ABS


def test_smooth_q_quant_entry_bit_exact():
    for n, d in ((1, 64), (129, 128), (300, 64), (1000, 128)):
        say(f"case smooth_q quant n={n} d={d}")
        x = workloads.generate_custom(600 + n, 2, 3, n, d, k_bias=3.0, q_bias=3.0)
        got = {k2: host(v2) for k2, v2 in sage.sage_quant_qk(dev(x.q), dev(x.k), smooth_q=True).items()}
        ref = O.quant_qk_dense(x.q, x.k, smooth_q=True)
        for key in ("q_int8", "k_int8", "q_scale", "k_scale", "k_mean", "q_mean"):
            assert got[key].shape == ref[key].shape, key
            assert (got[key].view(np.uint8) == ref[key].view(np.uint8)).all(), key


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
def test_smooth_q_fallback_halves(pv_mode):
    """Blocks whose term does not fit the integer accumulator: a constant Q
    block (δQ = 0), a nearly constant one (tiny δQ) and one with a large mean
    and a small spread, against keys whose first half tile sits at the K mean
    (small term, fits) and whose second half does not."""
    n, d = 384, 64
    rng = np.random.default_rng(61)
    c = rng.standard_normal((3, d))
    q = np.empty((n, d))
    q[0:128] = c[0] * 2.0                                       # constant block
    q[128:256] = c[1] * 2.0 + rng.standard_normal((128, d)) * 1e-3
    q[256:384] = c[2] * 8.0 + rng.standard_normal((128, d)) * 0.05
    k = rng.standard_normal((n, d))
    k[0:32] = 0.0
    k[64:96] = 0.0
    v = rng.standard_normal((n, d))
    q16, k16, v16 = (a.astype(np.float16)[None, None] for a in (q, k, v))
    for causal in (False, True):
        say(f"case smooth_q fallback pv={pv_mode} causal={causal}")
        ws = torch.empty(sage.sage_attn_workspace_size(1, 1, n, d, pv_mode, smooth_q=True), dtype=torch.uint8,
                         device="cuda")
        o, lse = sage.sage_attn_fwd(dev(q16), dev(k16), dev(v16), is_causal=causal, pv_mode=pv_mode, workspace=ws,
                                    return_lse=True, smooth_q=True)
        o, lse, wsn = host(o), host(lse), host(ws)
        quant = O.quant_qk_dense(q16, k16, smooth_q=True)
        assert quant["q_scale"][0, 0, 0] == 0
        offs = sage.sage_test_workspace_layout(False, 1, 1, n, 0, d, pv_mode, smooth_q=True)
        if pv_mode == "fp8":
            check_terms_fp32(wsn, offs, quant, k16, 1, 1, n, d, causal)   # every key in fp32
        else:
            nfb = check_terms(wsn, offs, quant, k16, 1, 1, n, d, causal, expect_fallback=True)
            nqb, nkb = 3, 6
            flags = wsn[offs[10]:offs[10] + 4 * nqb * 2 * nkb].view(np.int32).reshape(nqb, nkb, 2)
            seen = 2 if causal else nkb             # tiles the constant block's queries see
            assert (flags[0, :seen] == 1).all()     # δQ = 0: every half tile of the constant block
            assert nfb > nkb * 2
        rows = np.arange(n)
        o1, bias, (qi, qs, ki, ks) = o1_rows(quant, k16[0, 0], v16[0, 0], 0, 0, rows, causal, pv_mode)
        o2 = O.sdpa_fp64_rows(q16[0, 0], k16[0, 0], v16[0, 0], rows, causal)
        check_out(o[0, 0], o1, o2, f"fallback pv={pv_mode} causal={causal}")
        want = O.score_lse_rows(qi, qs, ki, ks, rows, causal, score_bias=bias)
        assert np.abs(lse[0, 0].astype(np.float64) - want).max() <= LSE_ABS


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
def test_smooth_q_gqa(pv_mode):
    B, H, H_kv, n, d = 2, 4, 2, 257, 128
    x = workloads.generate_custom(620, B, H, n, d, k_bias=3.0, q_bias=3.0)
    k = np.ascontiguousarray(x.k[:, :H_kv])
    v = np.ascontiguousarray(x.v[:, :H_kv])
    for causal in (False, True):
        say(f"case smooth_q gqa pv={pv_mode} causal={causal}")
        o, lse = sage.sage_attn_fwd(dev(x.q), dev(k), dev(v), is_causal=causal, pv_mode=pv_mode, return_lse=True,
                                    smooth_q=True)
        o, lse = host(o), host(lse)
        k_rep, v_rep = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
        quant = O.quant_qk_dense(x.q, k_rep, smooth_q=True)
        vq = O.quant_v_fp8(v_rep)
        rows = np.arange(n)
        for b in range(B):
            for h in range(H):
                o1, bias, (qi, qs, ki, ks) = o1_rows(quant, k_rep[b, h], v_rep[b, h], b, h, rows, causal,
                                                     pv_mode, (vq[0][b, h], vq[1][b, h]))
                o2 = O.sdpa_fp64_rows(x.q[b, h], k_rep[b, h], v_rep[b, h], rows, causal)
                check_out(o[b, h], o1, o2, f"smooth gqa b={b} h={h}")
                want = O.score_lse_rows(qi, qs, ki, ks, rows, causal, score_bias=bias)
                assert np.abs(lse[b, h].astype(np.float64) - want).max() <= LSE_ABS


def test_smooth_q_varlen():
    lens = [1, 65, 300, 0, 129]
    H, d = 2, 128
    x = workloads.generate_custom(630, 0, H, 0, d, k_bias=3.0, q_bias=3.0, lengths=lens)
    cu = dev(x.cu_seqlens)
    mx = max(lens)
    got = {k2: host(v2) for k2, v2 in sage.sage_quant_qk(dev(x.q), dev(x.k), cu_seqlens=cu, max_seqlen=mx,
                                                         smooth_q=True).items()}
    quant = O.quant_qk_varlen(x.q, x.k, x.cu_seqlens, smooth_q=True)
    assert (got["q_int8"] == quant["q_int8"]).all()
    for i, n in enumerate(lens):
        nq = -(-n // 128)
        assert (got["q_scale"][i, :, :nq].view(np.uint32) == quant["q_scale"][i, :, :nq].view(np.uint32)).all()
        assert (got["q_mean"][i, :, :nq].view(np.uint32) == quant["q_mean"][i, :, :nq].view(np.uint32)).all()
    for pv_mode in ("fp16", "fp8"):
        for causal in (False, True):
            say(f"case smooth_q varlen pv={pv_mode} causal={causal}")
            o, lse = sage.sage_attn_varlen_fwd(dev(x.q), dev(x.k), dev(x.v), cu, mx, is_causal=causal,
                                               pv_mode=pv_mode, return_lse=True, smooth_q=True)
            o, lse = host(o), host(lse)
            sm = O.default_sm_scale(d)
            for i, n in enumerate(lens):
                if n == 0:
                    continue
                a0 = int(x.cu_seqlens[i])
                rows = np.arange(n)
                for h in range(H):
                    qi, qs, ki, ks = O.head_views_varlen(quant, x.cu_seqlens, i, h)
                    nq = -(-n // 128)
                    kk, vv = x.k[h, a0:a0 + n], x.v[h, a0:a0 + n]
                    bias = O.q_smooth_bias(quant["q_mean"][i, h, :nq], kk, quant["k_mean"][i, h], sm)
                    if pv_mode == "fp8":
                        vc, vs = O.quant_v_fp8(vv)
                        o1 = O.sage_attention_rows(qi, qs, ki, ks, vc, rows, causal, "fp8", vs, score_bias=bias)
                    else:
                        o1 = O.sage_attention_rows(qi, qs, ki, ks, vv, rows, causal, "fp16", score_bias=bias)
                    o2 = O.sdpa_fp64_rows(x.q[h, a0:a0 + n], kk, vv, rows, causal)
                    check_out(o[h, a0:a0 + n], o1, o2, f"smooth varlen seq={i} h={h} pv={pv_mode}")
                    want = O.score_lse_rows(qi, qs, ki, ks, rows, causal, score_bias=bias)
                    assert np.abs(lse[h, a0:a0 + n].astype(np.float64) - want).max() <= LSE_ABS


def _sample_rows(n, rng, k=40):
    return np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, n - 1], rng.choice(n, size=min(n, k), replace=False)]))


@pytest.mark.parametrize("name", ["long_fp8", "seq16k", "llm_prefill"])
def test_smooth_q_workload(name):
    """Full-size workloads with Q smoothing, in the benchmark's launch shape."""
    w = workloads.get(name)
    say(f"case smooth_q workload {name} {w.description}")
    x = workloads.generate(w)
    B, H, N, d = x.q.shape
    ws = torch.empty(sage.sage_attn_workspace_size(B, H, N, d, w.pv_mode, smooth_q=True), dtype=torch.uint8,
                     device="cuda")
    o = host(sage.sage_attn_fwd(dev(x.q), dev(x.k), dev(x.v), is_causal=w.causal, pv_mode=w.pv_mode,
                                smooth_q=True, workspace=ws))
    torch.cuda.synchronize()
    offs = sage.sage_test_workspace_layout(False, B, H, N, 0, d, w.pv_mode, smooth_q=True)
    nqb, nkb = -(-N // 128), -(-N // 64)
    rng = np.random.default_rng(w.seed + 9)
    heads = [(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))]
    ref = O.quant_qk_dense(x.q[:, :, :, :], x.k, smooth_q=True)
    if w.pv_mode != "fp8":
        # FP16 PV: integer initial values, with flags where a half falls back
        flags = host(ws[offs[10]:offs[10] + 4 * B * H * nqb * 2 * nkb]).view(np.int32).reshape(B, H, nqb, nkb, 2)
        live = np.ones((nqb, nkb), bool)
        if w.causal:
            live = 64 * np.arange(nkb)[None, :] <= 128 * np.arange(nqb)[:, None] + 127
        say(f"  fallback halves: {int(flags[:, :, live].sum())} of {B * H * int(live.sum()) * 2}")
        for b, h in heads:
            sure_fit, sure_fb = fit_decisions(ref, x.k[b, h], b, h, N, d)
            got = flags[b, h]
            assert (got[sure_fit & live[:, :, None]] == 0).all(), ("flag set on a fitting half", b, h)
            assert (got[sure_fb & live[:, :, None]] == 1).all(), ("flag missing", b, h)
    vq = O.quant_v_fp8(x.v) if w.pv_mode == "fp8" else None
    for b, h in heads:
        rows = _sample_rows(N, rng)
        o1, _, _ = o1_rows(ref, x.k[b, h], x.v[b, h], b, h, rows, w.causal, w.pv_mode,
                           None if vq is None else (vq[0][b, h], vq[1][b, h]))
        o2 = O.sdpa_fp64_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, w.causal)
        check_out(o[b, h, rows], o1, o2, f"smooth {name} b={b} h={h}")


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_smooth_q_large_magnitude(causal, d, pv_mode):
    """Inputs ×30: large per-tile factors (the FP16 path's exact-log2
    conversion) together with smoothing terms that may not fit the integer
    accumulator (the fp32 fallback halves); every row against the method."""
    say(f"case smooth_q large magnitude d={d} causal={causal} pv={pv_mode}")
    B, H, n = 1, 2, 300
    x = workloads.generate_custom(560 + d, B, H, n, d, k_bias=3.0, q_bias=3.0)
    q = (x.q.astype(np.float32) * np.float32(30.0)).astype(np.float16)
    k = (x.k.astype(np.float32) * np.float32(30.0)).astype(np.float16)
    o = host(sage.sage_attn_fwd(dev(q), dev(k), dev(x.v), is_causal=causal, pv_mode=pv_mode, smooth_q=True))
    quant = O.quant_qk_dense(q, k, smooth_q=True)
    c2 = float(quant["q_scale"].max()) * float(quant["k_scale"].max()) * float(LOG2E)
    assert c2 > 2.0 ** -7, c2
    rows = np.arange(n)
    for h in range(H):
        ref1, _, _ = o1_rows(quant, k[0, h], x.v[0, h], 0, h, rows, causal, pv_mode)
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
