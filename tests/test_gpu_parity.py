"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars
  * INT8 Q̂/K̂, their block scales, the K means, e4m3 V̂ and its per-channel
    scales, and the int32 Q̂K̂ᵀ tiles: bit-exact.
  * fp16 output vs the method (oracle O1): max-abs <= 2e-2 and cosine >=
    0.9995; vs fp64 exact attention (O2): cosine >= 0.998 (the pages' per-layer
    bar), except the video-DiT literal reading, held to min(0.998, cos_O1 - 1e-4).
Small shapes compare every row; the full-size workloads compare sampled rows
of sampled heads, in the same launch configuration the benchmark times.
"""
import functools
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


@functools.lru_cache(maxsize=2)
def inputs(name):
    return workloads.generate(workloads.get(name))


def check_out(ours, o1, o2, label, o2_floor=COS_O2):
    ours = np.asarray(ours, np.float64)
    assert np.isfinite(ours).all(), label
    err = np.abs(ours - o1.astype(np.float64)).max()
    c1 = cos(ours, o1)
    c2 = cos(ours, o2)
    say(f"{label}: max_abs_vs_O1={err:.3e} cos_O1={c1:.6f} cos_O2={c2:.6f}")
    margins.record(label, err, c1, c2)
    assert err <= MAX_ABS, (label, err)
    assert c1 >= COS_O1, (label, c1)
    assert c2 >= o2_floor, (label, c2)


# ---------------------------------------------------------------------------
# Small shapes: every row, ragged tails, both head dims, both PV modes
# ---------------------------------------------------------------------------
SMALL = [(n, d) for d in (64, 128) for n in (1, 63, 64, 65, 127, 129, 200, 257)]


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", SMALL)
def test_small_all_rows(n, d, causal, pv_mode):
    say(f"case small n={n} d={d} causal={causal} pv={pv_mode}")
    x = workloads.generate_custom(100 + n + d, 2, 3, n, d, k_bias=3.0, q_bias=1.0)
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    o = host(sage.sage_attn_fwd(q, k, v, is_causal=causal, pv_mode=pv_mode))
    quant = O.quant_qk_dense(x.q, x.k)
    vc, vs = O.quant_v_fp8(x.v)
    rows = np.arange(n)
    for b in range(2):
        for h in range(3):
            qi, qs, ki, ks = O.head_views_dense(quant, b, h)
            if pv_mode == "fp8":
                o1 = O.sage_attention_rows(qi, qs, ki, ks, vc[b, h], rows, causal, "fp8", vs[b, h])
            else:
                o1 = O.sage_attention_rows(qi, qs, ki, ks, x.v[b, h], rows, causal, "fp16")
            o2 = O.sdpa_fp64_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, causal)
            check_out(o[b, h], o1, o2, f"n={n} d={d} b={b} h={h}")
            if n == 1 or causal:
                # one visible key: the output is V itself (fp16 PV, bit-exact) or its e4m3
                # dequantisation (fp8 PV; within one fp16 ulp, since the kernel's row sum is
                # 448*2^e with |e| ~ 1e-6 from fp32 rounding of the running max)
                if pv_mode == "fp16":
                    assert (o[b, h, 0].view(np.uint16) == x.v[b, h, 0].view(np.uint16)).all()
                else:
                    want = (O.e4m3_decode(vc[b, h, 0]) * vs[b, h].astype(np.float64)).astype(np.float16)
                    ulp = np.spacing(np.abs(want)).astype(np.float64)
                    assert (np.abs(o[b, h, 0].astype(np.float64) - want) <= ulp).all()


@pytest.mark.parametrize("n,d", [(1, 64), (65, 128), (300, 64), (1000, 128)])
def test_quant_qk_bit_exact_small(n, d):
    say(f"case quant small n={n} d={d}")
    x = workloads.generate_custom(7 + n, 2, 2, n, d, k_bias=3.0)
    got = {k2: host(v2) for k2, v2 in sage.sage_quant_qk(dev(x.q), dev(x.k)).items()}
    ref = O.quant_qk_dense(x.q, x.k)
    for key in ("q_int8", "k_int8", "q_scale", "k_scale", "k_mean"):
        assert got[key].shape == ref[key].shape, key
        assert (got[key].view(np.uint8) == ref[key].view(np.uint8)).all(), key
    # custom softmax scale is folded the same way
    got2 = host(sage.sage_quant_qk(dev(x.q), dev(x.k), sm_scale=0.3)["q_scale"])
    ref2 = O.quant_qk_dense(x.q, x.k, sm_scale=0.3)["q_scale"]
    assert (got2.view(np.uint32) == ref2.view(np.uint32)).all()


def test_quant_rounding_boundaries():
    """Quotients at and next to half-integers: the kernel's reciprocal path must
    hand these to the exact fp32 division and round ties to even, exactly as the
    oracle does."""
    say("case quant rounding boundaries")
    rng = np.random.default_rng(5)
    n, d = 256, 64
    half = np.arange(-126, 126) + 0.5                      # exact ties (delta = 1)
    near = np.concatenate([half + 2.0 ** -9, half - 2.0 ** -9, half + 2.0 ** -6])
    vals = np.concatenate([half, near, rng.uniform(-127, 127, 4096)])
    q = rng.choice(vals, size=(1, 2, n, d)).astype(np.float16)
    q[..., 0, 0] = 127.0                                   # every block attains 127 -> delta = 1
    q[..., 128, 0] = -127.0
    # K: token pairs of opposite sign give an exactly zero column mean, so the
    # smoothed values are the fp16 inputs themselves
    kh = rng.choice(vals, size=(1, 2, n // 2, d)).astype(np.float16)
    kh[..., ::32, 1] = 127.0                               # every 64-token block attains 127
    k = np.empty((1, 2, n, d), np.float16)
    k[..., 0::2, :] = kh
    k[..., 1::2, :] = -kh
    got = {k2: host(v2) for k2, v2 in sage.sage_quant_qk(dev(q), dev(k)).items()}
    ref = O.quant_qk_dense(q, k)
    assert (ref["k_mean"] == 0).all()
    ties = np.abs(np.abs(q.astype(np.float64)) % 1.0 - 0.5) == 0
    assert ties.sum() > 1000
    for key in ("q_int8", "k_int8", "q_scale", "k_scale", "k_mean"):
        assert (got[key].view(np.uint8) == ref[key].view(np.uint8)).all(), key


def test_quant_zero_blocks_and_constant_k():
    say("case quant zero blocks")
    q = np.zeros((1, 1, 300, 64), np.float16)
    q[0, 0, 128:256] = 2.0
    k = np.full((1, 1, 300, 64), 1.5, np.float16)   # smoothing makes K exactly zero
    got = {k2: host(v2) for k2, v2 in sage.sage_quant_qk(dev(q), dev(k)).items()}
    ref = O.quant_qk_dense(q, k)
    for key in ref:
        assert (got[key].view(np.uint8) == ref[key].view(np.uint8)).all(), key
    assert (got["k_scale"] == 0).all() and (got["k_int8"] == 0).all()
    v = np.random.default_rng(1).standard_normal((1, 1, 300, 64)).astype(np.float16)
    o = host(sage.sage_attn_fwd(dev(q), dev(k), dev(v)))
    assert np.isfinite(o.astype(np.float64)).all()
    want = v[0, 0].astype(np.float64).mean(axis=0)
    assert np.abs(o[0, 0].astype(np.float64) - want).max() < 2e-3


def _zero_scale_inputs(seed, n=320, d=128, H=2):
    """K whose token mean is exactly c, with keys 64..127 equal to c (after
    smoothing that block is zero: δK = 0), and Q with its second 128-row block
    zero (δQ = 0).  Values are multiples of 1/16 below 8 in magnitude, so every
    sum is exact in fp16 and fp64."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, H, n, d)).astype(np.float16)
    q[:, :, 128:256] = 0
    k = np.empty((1, H, n, d), np.float16)
    others = np.concatenate([np.arange(64), np.arange(128, n)])
    for h in range(H):
        c = rng.integers(-16, 17, d) / 4.0
        k[0, h, 64:128] = c
        e = rng.integers(-32, 33, (len(others) // 2, d)) / 16.0
        pairs = np.concatenate([c + e, c - e])
        k[0, h, others] = pairs[rng.permutation(len(others))]
    v = rng.standard_normal((1, H, n, d)).astype(np.float16)
    return q, k, v


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_blocks_in_attention(causal, pv_mode):
    # a K block with δK = 0 and a Q block with δQ = 0 among ordinary blocks:
    # their scores are exactly 0, which the kernel forms with the smallest
    # normal factor in place of a zero one
    say(f"case zero-scale blocks causal={causal} pv={pv_mode}")
    q, k, v = _zero_scale_inputs(11 + causal)
    n = q.shape[2]
    quant = O.quant_qk_dense(q, k)
    assert (quant["k_scale"][0, :, 1] == 0).all() and (quant["q_scale"][0, :, 1] == 0).all()
    o = host(sage.sage_attn_fwd(dev(q), dev(k), dev(v), is_causal=causal, pv_mode=pv_mode))
    vc, vs = O.quant_v_fp8(v)
    rows = np.arange(n)
    for h in range(q.shape[1]):
        qi, qs, ki, ks = O.head_views_dense(quant, 0, h)
        if pv_mode == "fp8":
            o1 = O.sage_attention_rows(qi, qs, ki, ks, vc[0, h], rows, causal, "fp8", vs[0, h])
        else:
            o1 = O.sage_attention_rows(qi, qs, ki, ks, v[0, h], rows, causal, "fp16")
        o2 = O.sdpa_fp64_rows(q[0, h], k[0, h], v[0, h], rows, causal)
        check_out(o[0, h], o1, o2, f"zero-scale blocks h={h}")


@pytest.mark.parametrize("sm_scale", [0.02, 0.3])
@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(200, 64), (257, 128)])
def test_caller_softmax_scale(n, d, causal, pv_mode, sm_scale):
    # a softmax scale other than 1/sqrt(d): folded into δQ by the kernel's own
    # Q quantisation, as the oracle folds it into the pre-pass scale
    say(f"case sm_scale={sm_scale} n={n} d={d} causal={causal} pv={pv_mode}")
    x = workloads.generate_custom(300 + n + d, 1, 2, n, d, k_bias=3.0, q_bias=1.0)
    o = host(sage.sage_attn_fwd(dev(x.q), dev(x.k), dev(x.v), is_causal=causal, pv_mode=pv_mode,
                                sm_scale=sm_scale))
    quant = O.quant_qk_dense(x.q, x.k, sm_scale=sm_scale)
    vc, vs = O.quant_v_fp8(x.v)
    rows = np.arange(n)
    for h in range(2):
        qi, qs, ki, ks = O.head_views_dense(quant, 0, h)
        if pv_mode == "fp8":
            o1 = O.sage_attention_rows(qi, qs, ki, ks, vc[0, h], rows, causal, "fp8", vs[0, h])
        else:
            o1 = O.sage_attention_rows(qi, qs, ki, ks, x.v[0, h], rows, causal, "fp16")
        o2 = O.sdpa_fp64_rows(x.q[0, h], x.k[0, h], x.v[0, h], rows, causal, sm_scale=sm_scale)
        check_out(o[0, h], o1, o2, f"sm_scale={sm_scale} n={n} d={d} h={h}")


def test_quant_v_fp8_bit_exact_small():
    say("case quant v fp8 small")
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((2, 3, 131, 128)) * rng.choice([0.01, 1, 40], size=(1, 3, 1, 128))).astype(np.float16)
    v[0, 1, :, 5] = 0
    codes, scale = sage.sage_quant_v_fp8(dev(v))
    rc, rs = O.quant_v_fp8(v)
    assert (host(scale).view(np.uint32) == rs.view(np.uint32)).all()
    assert (host(codes) == rc).all()


@pytest.mark.parametrize("d", [64, 128])
def test_qk_tiles_bit_exact(d):
    say(f"case qk tiles d={d}")
    x = workloads.generate_custom(55 + d, 2, 2, 300, d, k_bias=3.0)
    quant = sage.sage_quant_qk(dev(x.q), dev(x.k))
    qi, ki = host(quant["q_int8"]), host(quant["k_int8"])
    tiles = np.array([(b, h, qb, kb) for b in range(2) for h in range(2) for qb in range(3) for kb in range(5)]
                     + [(0, 0, 5, 0), (0, 9, 0, 0)], np.int32)
    got = host(sage.sage_test_qk_tiles(quant["q_int8"], quant["k_int8"], dev(tiles)))
    for t, (b, h, qb, kb) in enumerate(tiles.tolist()):
        want = np.zeros((128, 64), np.int64)
        if h < 2 and qb < 3:
            qa = np.zeros((128, d), np.int8)
            ka = np.zeros((64, d), np.int8)
            qs = qi[b, h, qb * 128:(qb + 1) * 128]
            ks = ki[b, h, kb * 64:(kb + 1) * 64]
            qa[:len(qs)] = qs
            ka[:len(ks)] = ks
            want = O.qk_int(qa, ka)
        assert (got[t] == want).all(), (b, h, qb, kb)


def test_deterministic_and_workspace_matches_quant():
    say("case determinism")
    x = workloads.generate_custom(77, 1, 4, 1000, 128, k_bias=3.0)
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    for pv_mode in ("fp16", "fp8"):
        size = sage.sage_attn_workspace_size(1, 4, 1000, 128, pv_mode)
        ws = torch.empty(size, dtype=torch.uint8, device="cuda")
        outs = [host(sage.sage_attn_fwd(q, k, v, is_causal=True, pv_mode=pv_mode, workspace=ws)) for _ in range(3)]
        for o in outs[1:]:
            assert (o.view(np.uint16) == outs[0].view(np.uint16)).all()
        offs = sage.sage_test_workspace_layout(False, 1, 4, 1000, 0, 128, pv_mode)
        ref = sage.sage_quant_qk(q, k)
        wsn = host(ws)
        n8 = 4 * 1000 * 128
        # Q̂ and δQ are formed inside the attention kernel in this mode (see
        # test_in_kernel_q_quantisation_bit_exact); K̂, δK from the pre-pass
        assert (wsn[offs[1]:offs[1] + n8].view(np.int8) == host(ref["k_int8"]).ravel()).all()
        nk = 4 * 16
        assert (wsn[offs[3]:offs[3] + 4 * nk].view(np.float32) == host(ref["k_scale"]).ravel()).all()
        if pv_mode == "fp8":
            _, vs = sage.sage_quant_v_fp8(v)
            assert (wsn[offs[6]:offs[6] + 4 * 512].view(np.float32) == host(vs).ravel()).all()


LSE_ABS = 2e-3  # natural-log units; the kernel keeps m and l in fp32


# Grouped-query heads (H_kv < H) and the log-sum-exp output, against the oracle
# run on K/V repeated to H heads (the same computation per query head).
GQA = [(4, 2, 65, 64), (4, 1, 257, 128), (6, 3, 200, 64), (2, 2, 129, 128)]


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv,n,d", GQA)
def test_gqa_and_lse(H, H_kv, n, d, causal, pv_mode):
    say(f"case gqa H={H} H_kv={H_kv} n={n} d={d} causal={causal} pv={pv_mode}")
    B, grp = 2, H // H_kv
    x = workloads.generate_custom(300 + H * 10 + H_kv + n, B, H, n, d, k_bias=3.0, q_bias=1.0)
    q = x.q
    k = np.ascontiguousarray(x.k[:, :H_kv])
    v = np.ascontiguousarray(x.v[:, :H_kv])
    ws = torch.empty(sage.sage_attn_workspace_size(B, H, n, d, pv_mode, H_kv=H_kv), dtype=torch.uint8,
                     device="cuda")
    o, lse = sage.sage_attn_fwd(dev(q), dev(k), dev(v), is_causal=causal, pv_mode=pv_mode, workspace=ws,
                                return_lse=True)
    o, lse, wsn = host(o), host(lse), host(ws)
    # K codes per K/V head, bit-exact (smoothing and blocks per K/V head)
    ref = O.quant_qk_dense(q, k)
    offs = sage.sage_test_workspace_layout(False, B, H, n, 0, d, pv_mode, H_kv=H_kv)
    nk8 = B * H_kv * n * d
    assert (wsn[offs[1]:offs[1] + nk8].view(np.int8) == ref["k_int8"].ravel()).all()
    k_rep, v_rep = np.repeat(k, grp, axis=1), np.repeat(v, grp, axis=1)
    quant = O.quant_qk_dense(q, k_rep)
    vc, vs = O.quant_v_fp8(v_rep)
    rows = np.arange(n)
    for b in range(B):
        for h in range(H):
            qi, qs, ki, ks = O.head_views_dense(quant, b, h)
            if pv_mode == "fp8":
                o1 = O.sage_attention_rows(qi, qs, ki, ks, vc[b, h], rows, causal, "fp8", vs[b, h])
            else:
                o1 = O.sage_attention_rows(qi, qs, ki, ks, v_rep[b, h], rows, causal, "fp16")
            o2 = O.sdpa_fp64_rows(q[b, h], k_rep[b, h], v_rep[b, h], rows, causal)
            check_out(o[b, h], o1, o2, f"gqa b={b} h={h}")
            want = O.score_lse_rows(qi, qs, ki, ks, rows, causal)
            err = np.abs(lse[b, h].astype(np.float64) - want).max()
            assert err <= LSE_ABS, (b, h, err)


def test_gqa_varlen_with_lse():
    lens = [1, 65, 300, 0, 129]
    H, H_kv, d = 4, 2, 128
    cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, mx = int(cu_h[-1]), max(lens)
    x = workloads.generate_custom(55, 1, H, T, d, k_bias=3.0, q_bias=1.0)
    q = np.ascontiguousarray(x.q[0])
    k = np.ascontiguousarray(x.k[0, :H_kv])
    v = np.ascontiguousarray(x.v[0, :H_kv])
    cu = dev(cu_h)
    for pv_mode in ("fp16", "fp8"):
        for causal in (False, True):
            say(f"case gqa varlen pv={pv_mode} causal={causal}")
            o, lse = sage.sage_attn_varlen_fwd(dev(q), dev(k), dev(v), cu, mx, is_causal=causal, pv_mode=pv_mode,
                                               return_lse=True)
            o, lse = host(o), host(lse)
            k_rep, v_rep = np.repeat(k, 2, axis=0), np.repeat(v, 2, axis=0)
            quant = O.quant_qk_varlen(q, k_rep, cu_h)
            for i, n in enumerate(lens):
                if n == 0:
                    continue
                a0 = int(cu_h[i])
                rows = np.arange(n)
                for h in range(H):
                    qi, qs, ki, ks = O.head_views_varlen(quant, cu_h, i, h)
                    vv = v_rep[h, a0:a0 + n]
                    if pv_mode == "fp8":
                        vc, vs = O.quant_v_fp8(vv)
                        o1 = O.sage_attention_rows(qi, qs, ki, ks, vc, rows, causal, "fp8", vs)
                    else:
                        o1 = O.sage_attention_rows(qi, qs, ki, ks, vv, rows, causal, "fp16")
                    o2 = O.sdpa_fp64_rows(q[h, a0:a0 + n], k_rep[h, a0:a0 + n], vv, rows, causal)
                    check_out(o[h, a0:a0 + n], o1, o2, f"gqa varlen seq={i} h={h}")
                    want = O.score_lse_rows(qi, qs, ki, ks, rows, causal)
                    assert np.abs(lse[h, a0:a0 + n].astype(np.float64) - want).max() <= LSE_ABS


def test_varlen_small_all_rows():
    lens = [1, 63, 64, 65, 130, 0, 257]
    for d in (64, 128):
        for causal in (False, True):
            for pv_mode in ("fp16", "fp8"):
                say(f"case varlen small d={d} causal={causal} pv={pv_mode}")
                x = workloads.generate_custom(300 + d, 0, 2, 0, d, k_bias=3.0, lengths=lens)
                cu = dev(x.cu_seqlens)
                mx = max(lens)
                o = host(sage.sage_attn_varlen_fwd(dev(x.q), dev(x.k), dev(x.v), cu, mx, is_causal=causal,
                                                   pv_mode=pv_mode))
                quant = O.quant_qk_varlen(x.q, x.k, x.cu_seqlens)
                got = {k2: host(v2) for k2, v2 in sage.sage_quant_qk(dev(x.q), dev(x.k), cu_seqlens=cu,
                                                                     max_seqlen=mx).items()}
                assert (got["q_int8"] == quant["q_int8"]).all() and (got["k_int8"] == quant["k_int8"]).all()
                for i, n in enumerate(lens):
                    if n == 0:
                        continue
                    a = int(x.cu_seqlens[i])
                    nq, nk = -(-n // 128), -(-n // 64)
                    assert (got["q_scale"][i, :, :nq].view(np.uint32) == quant["q_scale"][i, :, :nq].view(np.uint32)).all()
                    assert (got["k_scale"][i, :, :nk].view(np.uint32) == quant["k_scale"][i, :, :nk].view(np.uint32)).all()
                    assert (got["k_mean"][i].view(np.uint32) == quant["k_mean"][i].view(np.uint32)).all()
                    for h in range(2):
                        qi, qs, ki, ks = O.head_views_varlen(quant, x.cu_seqlens, i, h)
                        vv = x.v[h, a:a + n]
                        rows = np.arange(n)
                        if pv_mode == "fp8":
                            vc, vs = O.quant_v_fp8(vv)
                            o1 = O.sage_attention_rows(qi, qs, ki, ks, vc, rows, causal, "fp8", vs)
                        else:
                            o1 = O.sage_attention_rows(qi, qs, ki, ks, vv, rows, causal, "fp16")
                        o2 = O.sdpa_fp64_rows(x.q[h, a:a + n], x.k[h, a:a + n], vv, rows, causal)
                        check_out(o[h, a:a + n], o1, o2, f"varlen seq={i} n={n} h={h}")


# ---------------------------------------------------------------------------
# Large magnitudes: with |q|·|k| in the hundreds the per-tile factor
# c = δQ·δK·log2(e) grows past 2^-7, where the FP16 path takes its scores to
# exact log2 units before the softmax; every row against the method.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("scale", [8.0, 30.0])
@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_large_magnitude_inputs(scale, pv_mode, d, causal):
    say(f"case large magnitude x{scale} pv={pv_mode} d={d} causal={causal}")
    B, H, n = 1, 2, 300
    x = workloads.generate_custom(555 + d, B, H, n, d, k_bias=3.0, q_bias=1.0)
    q = (x.q.astype(np.float32) * np.float32(scale)).astype(np.float16)
    k = (x.k.astype(np.float32) * np.float32(scale)).astype(np.float16)
    o = host(sage.sage_attn_fwd(dev(q), dev(k), dev(x.v), is_causal=causal, pv_mode=pv_mode))
    quant = O.quant_qk_dense(q, k)
    c2 = float(quant["q_scale"].max()) * float(quant["k_scale"].max()) * 1.4426950408889634
    assert c2 > 2.0 ** -7, c2  # the inputs do reach the exact-conversion range
    rows = np.arange(n)
    for h in range(H):
        qi, qs, ki, ks = O.head_views_dense(quant, 0, h)
        if pv_mode == "fp8":
            vc, vs = O.quant_v_fp8(x.v[0, h])
            o1 = O.sage_attention_rows(qi, qs, ki, ks, vc, rows, causal, "fp8", vs)
        else:
            o1 = O.sage_attention_rows(qi, qs, ki, ks, x.v[0, h], rows, causal, "fp16")
        o2 = O.sdpa_fp64_rows(q[0, h], k[0, h], x.v[0, h], rows, causal)
        check_out(o[0, h], o1, o2, f"x{scale} {pv_mode} d={d} h={h}", min(COS_O2, cos(o1, o2) - 1e-4))


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_mixed_magnitudes(d, pv_mode):
    """Sequences of ordinary and ×30 magnitude in one packed call: the
    exact-log2 conversion is on for some waves and off for others."""
    lens = [200, 130, 65, 300, 1, 257]
    mags = [1.0, 30.0, 1.0, 8.0, 30.0, 30.0]
    for causal in (False, True):
        say(f"case varlen mixed magnitudes d={d} causal={causal} pv={pv_mode}")
        x = workloads.generate_custom(330 + d, 0, 2, 0, d, k_bias=3.0, lengths=lens)
        q = x.q.astype(np.float32)
        k = x.k.astype(np.float32)
        for i, m in enumerate(mags):
            a, b = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
            q[:, a:b] *= np.float32(m)
            k[:, a:b] *= np.float32(m)
        q, k = q.astype(np.float16), k.astype(np.float16)
        cu = dev(x.cu_seqlens)
        o = host(sage.sage_attn_varlen_fwd(dev(q), dev(k), dev(x.v), cu, max(lens), is_causal=causal,
                                           pv_mode=pv_mode))
        quant = O.quant_qk_varlen(q, k, x.cu_seqlens)
        for i, n in enumerate(lens):
            a = int(x.cu_seqlens[i])
            for h in range(2):
                qi, qs, ki, ks = O.head_views_varlen(quant, x.cu_seqlens, i, h)
                vv = x.v[h, a:a + n]
                rows = np.arange(n)
                if pv_mode == "fp8":
                    vc, vs = O.quant_v_fp8(vv)
                    o1 = O.sage_attention_rows(qi, qs, ki, ks, vc, rows, causal, "fp8", vs)
                else:
                    o1 = O.sage_attention_rows(qi, qs, ki, ks, vv, rows, causal, "fp16")
                o2 = O.sdpa_fp64_rows(q[h, a:a + n], k[h, a:a + n], vv, rows, causal)
                check_out(o[h, a:a + n], o1, o2, f"x{mags[i]} seq={i} n={n} h={h}",
                          min(COS_O2, cos(o1, o2) - 1e-4))


# ---------------------------------------------------------------------------
# Full-size workloads: whole-tensor bit-exact quantisation, sampled output rows
# ---------------------------------------------------------------------------
def _sample_rows(n, rng, k=48):
    return np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, n - 1], rng.choice(n, size=min(n, k), replace=False)]))


@pytest.mark.parametrize("name", ["tiny", "llm_prefill", "video_dit", "video_dit_biasx20", "long_fp8", "seq16k",
                                  "seq16k_causal"])
def test_dense_workload(name):
    w = workloads.get(name)
    say(f"case workload {name} {w.description}")
    x = inputs(name)
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    got = {k2: host(v2) for k2, v2 in sage.sage_quant_qk(q, k).items()}
    ref = O.quant_qk_dense(x.q, x.k)
    for key in ("q_int8", "k_int8", "q_scale", "k_scale", "k_mean"):
        assert (got[key].view(np.uint8) == ref[key].view(np.uint8)).all(), key
    say(f"{name}: quantisation bit-exact over {x.q.size} elements")
    vc = vs = None
    if w.pv_mode == "fp8":
        gc, gs = sage.sage_quant_v_fp8(v)
        vc, vs = O.quant_v_fp8(x.v)
        assert (host(gs).view(np.uint32) == vs.view(np.uint32)).all()
        assert (host(gc) == vc).all()
        say(f"{name}: e4m3 V bit-exact")
    del got
    o = host(sage.sage_attn_fwd(q, k, v, is_causal=w.causal, pv_mode=w.pv_mode))
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 5)
    B, H, N, d = x.q.shape
    heads = [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(2)]
    if name == "tiny":
        heads = [(0, 0), (0, 1)]
    for b, h in heads:
        rows = np.arange(N) if name == "tiny" else _sample_rows(N, rng)
        qi, qs, ki, ks = O.head_views_dense(ref, b, h)
        if w.pv_mode == "fp8":
            o1 = O.sage_attention_rows(qi, qs, ki, ks, vc[b, h], rows, w.causal, "fp8", vs[b, h])
        else:
            o1 = O.sage_attention_rows(qi, qs, ki, ks, x.v[b, h], rows, w.causal, "fp16")
        o2 = O.sdpa_fp64_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, w.causal)
        floor = COS_O2
        if name == "video_dit":
            floor = min(COS_O2, cos(o1, o2) - 1e-4)
        check_out(o[b, h, rows], o1, o2, f"{name} b={b} h={h}", floor)
    # int32 tiles of this workload, computed by the attention kernel's QKᵀ code
    nq, nk = -(-N // 128), -(-N // 64)
    tl = np.array([(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(nq)), int(rng.integers(nk)))
                   for _ in range(64)], np.int32)
    tiles = host(sage.sage_test_qk_tiles(dev(ref["q_int8"]), dev(ref["k_int8"]), dev(tl)))
    for t, (b, h, qb, kb) in enumerate(tl.tolist()):
        want = O.qk_int(ref["q_int8"][b, h, qb * 128:(qb + 1) * 128], ref["k_int8"][b, h, kb * 64:(kb + 1) * 64])
        assert (tiles[t][:want.shape[0], :want.shape[1]] == want).all(), (b, h, qb, kb)


def test_varlen_workload():
    w = workloads.get("varlen")
    say(f"case workload varlen {w.description}")
    x = inputs("varlen")
    cu = dev(x.cu_seqlens)
    mx = int(x.lengths.max())
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    got = {k2: host(v2) for k2, v2 in sage.sage_quant_qk(q, k, cu_seqlens=cu, max_seqlen=mx).items()}
    ref = O.quant_qk_varlen(x.q, x.k, x.cu_seqlens)
    assert (got["q_int8"] == ref["q_int8"]).all() and (got["k_int8"] == ref["k_int8"]).all()
    for i, n in enumerate(x.lengths.tolist()):
        nq, nk = -(-n // 128), -(-n // 64)
        assert (got["q_scale"][i, :, :nq].view(np.uint32) == ref["q_scale"][i, :, :nq].view(np.uint32)).all()
        assert (got["k_scale"][i, :, :nk].view(np.uint32) == ref["k_scale"][i, :, :nk].view(np.uint32)).all()
        assert (got["k_mean"][i].view(np.uint32) == ref["k_mean"][i].view(np.uint32)).all()
    say("varlen: quantisation bit-exact")
    o = host(sage.sage_attn_varlen_fwd(q, k, v, cu, mx, is_causal=True))
    rng = np.random.default_rng(w.seed + 5)
    for i in [0, int(np.argmax(x.lengths)), int(np.argmin(x.lengths)), 7]:
        h = int(rng.integers(w.H))
        n = int(x.lengths[i])
        a = int(x.cu_seqlens[i])
        rows = _sample_rows(n, rng)
        qi, qs, ki, ks = O.head_views_varlen(ref, x.cu_seqlens, i, h)
        o1 = O.sage_attention_rows(qi, qs, ki, ks, x.v[h, a:a + n], rows, True, "fp16")
        o2 = O.sdpa_fp64_rows(x.q[h, a:a + n], x.k[h, a:a + n], x.v[h, a:a + n], rows, True)
        check_out(o[h, a + rows], o1, o2, f"varlen seq={i} n={n} h={h}")


@pytest.mark.parametrize("per_token", [False, True])
@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1000, 128), (333, 64), (129, 128)])
def test_in_kernel_q_quantisation_bit_exact(n, d, causal, pv_mode, per_token):
    """Without Q smoothing the attention kernel quantises Q itself (per block,
    or per token).  Its codes and scales are the pre-pass's: the same attention
    run on the pre-pass's Q̂ and δQ (placed in the workspace) gives a
    bit-identical output."""
    say(f"case in-kernel Q quantisation n={n} d={d} causal={causal} pv={pv_mode} per_token={per_token}")
    B, H = 2, 3
    x = workloads.generate_custom(880 + n + d, B, H, n, d, k_bias=3.0, q_bias=2.0)
    # a few rows of very different magnitude so that block maxima differ
    x.q[:, :, ::97] = (x.q[:, :, ::97].astype(np.float32) * np.float32(9.0)).astype(np.float16)
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    ws = torch.empty(sage.sage_attn_workspace_size(B, H, n, d, pv_mode, q_per_token=per_token), dtype=torch.uint8,
                     device="cuda")
    fused = sage.sage_attn_fwd(q, k, v, is_causal=causal, pv_mode=pv_mode, workspace=ws, q_per_token=per_token)
    ref = sage.sage_quant_qk(q, k, q_per_token=per_token)
    offs = sage.sage_test_workspace_layout(False, B, H, n, 0, d, pv_mode, q_per_token=per_token)
    n8, nq = B * H * n * d, B * H * (n if per_token else -(-n // 128))
    ws[offs[0]:offs[0] + n8].copy_(ref["q_int8"].reshape(-1).view(torch.uint8))
    ws[offs[2]:offs[2] + 4 * nq].copy_(ref["q_scale"].reshape(-1).view(torch.uint8))
    from_prepass = torch.empty_like(fused)
    sage.sage_test_attn_from_workspace(from_prepass, ws, v, is_causal=causal, pv_mode=pv_mode, q_per_token=per_token)
    torch.cuda.synchronize()
    same = torch.equal(fused.view(torch.int16), from_prepass.view(torch.int16))
    say(f"  bit-identical={same}")
    assert same
