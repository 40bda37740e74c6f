"""GPU parity of the MXFP4 mode (pv_mode "mxfp4") against the CPU oracle.

Bars: the e2m1 codes and E8M0 scales of Q, the smoothed K and V are
bit-exact in the workspace's packed layouts; outputs against the MXFP4 method
(O1): max-abs <= 2e-2 beyond the change the P codes the oracle leaves open can
make (the kernel forms p in fp32, the oracle in fp64; a code whose value lies
within that distance of an e4m1 rounding boundary may land on either
neighbour), cosine >= 0.9995; against fp64 exact attention (O2) no worse than
the method itself (cos(O1, O2) - 1e-3) — FP4's 3-bit elements keep it near
0.97 on these inputs, below the INT8 path's 0.998; the LSE within 2e-3.
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


def pack_nibbles(codes):
    """[..., m] nibbles -> [..., m/2] bytes, element 2i in the low nibble."""
    c = codes.astype(np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def krow_of_key(kappa):
    return 32 * ((kappa >> 4) & 1) + 8 * ((kappa >> 2) & 3) + 4 * (kappa >> 5) + (kappa & 3)


def check_workspace(wsn, offs, q, k, v, d):
    """Dense [B,H,n,d] inputs (H_kv = H): every code and scale byte the pre-pass
    wrote, against the oracle's MX quantisation."""
    B, H, n, _ = q.shape
    qc, qx, kc, kx, km = O.quant_mxfp4_qk(q, k)
    vc, vx = O.quant_mxfp4_v(v)
    rows = B * H * n
    assert (wsn[offs[0]:offs[0] + rows * d // 2] == pack_nibbles(qc).ravel()).all()
    assert (wsn[offs[1]:offs[1] + rows * d // 2] == pack_nibbles(kc).ravel()).all()
    qs = wsn[offs[2]:offs[2] + rows * 8].reshape(B, H, n, 8)
    for blk in range(d // 32):
        kk, g = blk // 2, blk % 2
        assert (qs[..., 4 * g + kk] == (qx[..., blk] + 127).astype(np.uint8)).all(), blk
    nt = -(-n // 64)
    aux = wsn[offs[3]:offs[3] + B * H * nt * 1024].reshape(B, H, nt, 1024)
    kappa = np.arange(n)
    for blk in range(d // 32):
        kk, g = blk // 2, blk % 2
        got = aux[:, :, kappa // 64, krow_of_key(kappa % 64) * 8 + 4 * g + kk]
        assert (got == (kx[..., blk] + 127).astype(np.uint8)).all(), ("k scale", blk)
    vt = wsn[offs[5]:offs[5] + B * H * nt * 32 * d].reshape(B, H, nt, d // 32, 64, 16)
    vpad = np.zeros((B, H, nt * 64, d), np.uint8)
    vpad[:, :, :n] = vc
    xpad = np.full((B, H, 2 * nt, d), -127, np.int64)
    xpad[:, :, :vx.shape[2]] = vx
    for dt in range(d // 32):
        for lane in range(64):
            c, g = 32 * dt + lane % 32, lane // 32
            keys = (np.arange(nt)[:, None] * 64 + 32 * g + np.arange(32)[None, :])   # [nt, 32]
            want = pack_nibbles(vpad[:, :, keys, c])                                   # [B,H,nt,16]
            assert (vt[:, :, :, dt, lane] == want).all(), ("v codes", dt, lane)
            sc = aux[:, :, :, 512 + 4 * lane + dt]
            assert (sc == (xpad[:, :, g::2, c][:, :, :nt] + 127).astype(np.uint8)).all(), ("v scale", dt, lane)
    return (qc, qx, kc, kx, km), (vc, vx)


def o1_rows(qq, vq, b, h, rows, causal, sm, v_rep_h=None):
    """The MXFP4 method for one (batch, head) with its open-code bound."""
    qc, qx, kc, kx, km = qq
    vc, vx = vq
    qv = O.mxfp4_decode(qc[b, h], qx[b, h], -1)
    kv = O.mxfp4_decode(kc[b, h], kx[b, h], -1)
    smax = np.abs(qv[rows]).sum(axis=1).max() * np.abs(kv).max() * sm
    eps = np.full(kc.shape[2], 4e-6 * (1.0 + smax))
    args = (qc[b, h], qx[b, h], kc[b, h], kx[b, h], vc[b, h], vx[b, h], rows, causal, sm)
    o1 = O.mxfp4_attention_rows(*args)
    bound = O.mxfp4_open_code_bound(*args, score_eps=eps)
    lse = O.score_lse_rows(qv, np.full(len(qv), sm), kv, np.ones(-(-len(kv) // 64)), rows, causal, q_block=1)
    return o1, bound, lse


def check_out(ours, o1, o2, label, bound):
    ours = np.asarray(ours, np.float64)
    assert np.isfinite(ours).all(), label
    diff = np.abs(ours - o1.astype(np.float64))
    over = (diff - bound).max()
    c1, c2, c12 = cos(ours, o1), cos(ours, o2), cos(o1, o2)
    say(f"{label}: max_abs_vs_O1={diff.max():.3e} (beyond open codes {over:.3e}) cos_O1={c1:.6f} "
        f"cos_O2={c2:.6f} (method {c12:.6f})")
    margins.record(label, diff.max(), c1, c2)
    assert over <= MAX_ABS, (label, over)
    assert c1 >= COS_O1, (label, c1)
    assert c2 >= c12 - 1e-3, (label, c2, c12)


SMALL = [(n, d) for d in (64, 128) for n in (1, 65, 129, 257)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", SMALL)
def test_mxfp4_small_all_rows(n, d, causal):
    say(f"case mxfp4 small n={n} d={d} causal={causal}")
    B, H = 2, 2
    x = workloads.generate_custom(800 + n + d, B, H, n, d, k_bias=3.0)
    ws = torch.empty(sage.sage_attn_workspace_size(B, H, n, d, "mxfp4"), dtype=torch.uint8, device="cuda")
    o, lse = sage.sage_attn_fwd(dev(x.q), dev(x.k), dev(x.v), is_causal=causal, pv_mode="mxfp4", workspace=ws,
                                return_lse=True)
    o, lse, wsn = host(o), host(lse), host(ws)
    offs = sage.sage_test_workspace_layout(False, B, H, n, 0, d, "mxfp4")
    qq, vq = check_workspace(wsn, offs, x.q, x.k, x.v, d)
    sm = float(O.default_sm_scale(d))
    rows = np.arange(n)
    for b in range(B):
        for h in range(H):
            o1, bound, want_lse = o1_rows(qq, vq, b, h, rows, causal, sm)
            o2 = O.sdpa_fp64_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, causal)
            check_out(o[b, h], o1, o2, f"mxfp4 n={n} d={d} b={b} h={h}", bound)
            assert np.abs(lse[b, h].astype(np.float64) - want_lse).max() <= LSE_ABS
            if n == 1 or causal:
                # row 0 sees one key: p = 1 exactly, the output is its decoded V row
                vv = O.mxfp4_decode(vq[0][b, h], vq[1][b, h], 0)
                assert (o[b, h, 0] == vv[0].astype(np.float16)).all()


def test_mxfp4_gqa_and_varlen():
    B, H, H_kv, n, d = 1, 4, 2, 200, 128
    x = workloads.generate_custom(830, B, H, n, d, k_bias=3.0)
    k = np.ascontiguousarray(x.k[:, :H_kv])
    v = np.ascontiguousarray(x.v[:, :H_kv])
    sm = float(O.default_sm_scale(d))
    for causal in (False, True):
        say(f"case mxfp4 gqa causal={causal}")
        o = host(sage.sage_attn_fwd(dev(x.q), dev(k), dev(v), is_causal=causal, pv_mode="mxfp4"))
        k_rep, v_rep = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
        qq = O.quant_mxfp4_qk(x.q, k_rep)
        vq = O.quant_mxfp4_v(v_rep)
        rows = np.arange(n)
        for h in range(H):
            o1, bound, _ = o1_rows(qq, vq, 0, h, rows, causal, sm)
            o2 = O.sdpa_fp64_rows(x.q[0, h], k_rep[0, h], v_rep[0, h], rows, causal)
            check_out(o[0, h], o1, o2, f"mxfp4 gqa h={h}", bound)
    lens = [1, 65, 300, 0, 129]
    xv = workloads.generate_custom(840, 0, 2, 0, 64, k_bias=3.0, lengths=lens)
    cu = dev(xv.cu_seqlens)
    sm = float(O.default_sm_scale(64))
    for causal in (False, True):
        say(f"case mxfp4 varlen causal={causal}")
        o, lse = sage.sage_attn_varlen_fwd(dev(xv.q), dev(xv.k), dev(xv.v), cu, max(lens), is_causal=causal,
                                           pv_mode="mxfp4", return_lse=True)
        o, lse = host(o), host(lse)
        for i, n in enumerate(lens):
            if n == 0:
                continue
            a0 = int(xv.cu_seqlens[i])
            qs, ks, vs = (t[:, a0:a0 + n][None] for t in (xv.q, xv.k, xv.v))
            qq = O.quant_mxfp4_qk(qs, ks)
            vq = O.quant_mxfp4_v(vs)
            rows = np.arange(n)
            for h in range(2):
                o1, bound, want_lse = o1_rows(qq, vq, 0, h, rows, causal, sm)
                o2 = O.sdpa_fp64_rows(xv.q[h, a0:a0 + n], xv.k[h, a0:a0 + n], xv.v[h, a0:a0 + n], rows, causal)
                check_out(o[h, a0:a0 + n], o1, o2, f"mxfp4 varlen seq={i} h={h}", bound)
                assert np.abs(lse[h, a0:a0 + n].astype(np.float64) - want_lse).max() <= LSE_ABS


def _sample_rows(n, rng, k=32):
    return np.unique(np.concatenate([[0, 1, 63, 64, 255, 256, n - 1], rng.choice(n, size=min(n, k), replace=False)]))


@pytest.mark.parametrize("name", ["seq16k", "video_dit_biasx20", "llm_prefill"])
def test_mxfp4_workload(name):
    """Full-size workloads in MXFP4 mode, in the benchmark's launch shape."""
    w = workloads.get(name)
    say(f"case mxfp4 workload {name} {w.description}")
    x = workloads.generate(w)
    B, H, N, d = x.q.shape
    o = host(sage.sage_attn_fwd(dev(x.q), dev(x.k), dev(x.v), is_causal=w.causal, pv_mode="mxfp4"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 13)
    sm = float(O.default_sm_scale(d))
    for b, h in [(0, 0), (B - 1, H - 1)]:
        qq = O.quant_mxfp4_qk(x.q[b:b + 1, h:h + 1], x.k[b:b + 1, h:h + 1])
        vq = O.quant_mxfp4_v(x.v[b:b + 1, h:h + 1])
        rows = _sample_rows(N, rng)
        o1, bound, _ = o1_rows(qq, vq, 0, 0, rows, w.causal, sm)
        o2 = O.sdpa_fp64_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, w.causal)
        check_out(o[b, h, rows], o1, o2, f"mxfp4 {name} b={b} h={h}", bound)


# --- Q smoothing in MXFP4 mode: Q minus its 128-token block mean is
# MX-quantised; the term q̄_b·x_j (raw units, fp32) starts every score's
# accumulator.  The term region is compared with the oracle's fp64 product
# within the error of its fp16 hi/lo split and fp32 sums:
# 1e-5·Σ|q̄||x| + 2^-22·Σ|q̄|·max|x|.

def term_tol(qm, k_head, km):
    x = O.smooth_k(k_head, km).astype(np.float64)
    qa = np.abs(qm.astype(np.float64))
    return 1e-5 * (qa @ np.abs(x).T) + 2.0 ** -22 * qa.sum(axis=1)[:, None] * np.abs(x).max()


def check_terms_mx(wsn, offs, qm, k, km, B, H, n, d, causal):
    nqb, npad = -(-n // 128), -(-n // 64) * 64
    assert (wsn[offs[7]:offs[7] + B * H * nqb * d * 4].view(np.float32).reshape(B, H, nqb, d) == qm).all(), "q_mean"
    terms = wsn[offs[8]:offs[8] + B * H * nqb * npad * 4].view(np.float32).reshape(B, H, nqb, npad)
    for b in range(B):
        for h in range(H):
            want = O.q_smooth_bias(qm[b, h], k[b, h], km[b, h], 1.0)
            tol = term_tol(qm[b, h], k[b, h], km[b, h])
            for blk in range(nqb):
                # causal: tiles past the block's last row are never read
                kend = min(n, 64 * (-(-min(n, 128 * blk + 128) // 64))) if causal else n
                got = terms[b, h, blk, :kend].astype(np.float64)
                assert (np.abs(got - want[blk, :kend]) <= tol[blk, :kend]).all(), ("term", b, h, blk)
                tend = min(npad, -(-kend // 64) * 64)
                assert (terms[b, h, blk, n:tend] == 0).all(), ("term past n", b, h, blk)


def o1_smooth_rows(qs, qsx, qm, kq, vq, k_head, b, h, rows, causal, sm):
    """The MXFP4 method with a smoothed Q for one (batch, head): output, the
    open-code bound and the LSE.  The score tolerance adds the term's."""
    kc, kx, km = kq
    vc, vx = vq
    qv = O.mxfp4_decode(qs, qsx, -1)
    kv = O.mxfp4_decode(kc, kx, -1)
    bias = O.q_smooth_bias(qm, k_head, km, sm)
    smax = np.abs(qv[rows]).sum(axis=1).max() * np.abs(kv).max() * sm
    tmax = sm * term_tol(qm, k_head, km).max()
    eps = np.full(kc.shape[0], 4e-6 * (1.0 + smax + np.abs(bias).max()) + tmax)
    o1 = O.mxfp4_attention_rows(qs, qsx, kc, kx, vc, vx, rows, causal, sm, score_bias=bias)
    bound = O.mxfp4_open_code_bound(qs, qsx, kc, kx, vc, vx, rows, causal, sm, score_eps=eps, score_bias=bias)
    lse = O.score_lse_rows(qv, np.full(len(qv), sm), kv, np.ones(-(-len(kv) // 64)), rows, causal,
                           score_bias=bias, q_block=1)
    return o1, bound, lse


SMALL_SQ = [(n, d) for d in (64, 128) for n in (1, 129, 257, 300)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", SMALL_SQ)
def test_mxfp4_smooth_q_small_all_rows(n, d, causal):
    say(f"case mxfp4 smooth_q small n={n} d={d} causal={causal}")
    B, H = 2, 2
    x = workloads.generate_custom(860 + n + d, B, H, n, d, k_bias=3.0, q_bias=2.0)
    ws = torch.empty(sage.sage_attn_workspace_size(B, H, n, d, "mxfp4", smooth_q=True), dtype=torch.uint8,
                     device="cuda")
    o, lse = sage.sage_attn_fwd(dev(x.q), dev(x.k), dev(x.v), is_causal=causal, pv_mode="mxfp4", workspace=ws,
                                return_lse=True, smooth_q=True)
    o, lse, wsn = host(o), host(lse), host(ws)
    offs = sage.sage_test_workspace_layout(False, B, H, n, 0, d, "mxfp4", smooth_q=True)
    qs, qsx, qm = O.quant_mxfp4_q_smooth(x.q)
    _, _, kc, kx, km = O.quant_mxfp4_qk(x.q, x.k)
    vc, vx = O.quant_mxfp4_v(x.v)
    rows_all = B * H * n
    assert (wsn[offs[0]:offs[0] + rows_all * d // 2] == pack_nibbles(qs).ravel()).all(), "q codes"
    assert (wsn[offs[1]:offs[1] + rows_all * d // 2] == pack_nibbles(kc).ravel()).all(), "k codes"
    qsc = wsn[offs[2]:offs[2] + rows_all * 8].reshape(B, H, n, 8)
    for blk in range(d // 32):
        assert (qsc[..., 4 * (blk % 2) + blk // 2] == (qsx[..., blk] + 127).astype(np.uint8)).all(), blk
    check_terms_mx(wsn, offs, qm, x.k, km, B, H, n, d, causal)
    sm = float(O.default_sm_scale(d))
    rows = np.arange(n)
    for b in range(B):
        for h in range(H):
            o1, bound, want_lse = o1_smooth_rows(qs[b, h], qsx[b, h], qm[b, h], (kc[b, h], kx[b, h], km[b, h]),
                                                 (vc[b, h], vx[b, h]), x.k[b, h], b, h, rows, causal, sm)
            o2 = O.sdpa_fp64_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, causal)
            check_out(o[b, h], o1, o2, f"mxfp4 smooth_q n={n} d={d} b={b} h={h}", bound)
            assert np.abs(lse[b, h].astype(np.float64) - want_lse).max() <= LSE_ABS


def test_mxfp4_smooth_q_gqa_and_varlen():
    B, H, H_kv, n, d = 1, 4, 2, 300, 128
    x = workloads.generate_custom(880, B, H, n, d, k_bias=3.0, q_bias=2.0)
    k = np.ascontiguousarray(x.k[:, :H_kv])
    v = np.ascontiguousarray(x.v[:, :H_kv])
    sm = float(O.default_sm_scale(d))
    k_rep, v_rep = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    qs, qsx, qm = O.quant_mxfp4_q_smooth(x.q)
    _, _, kc, kx, km = O.quant_mxfp4_qk(x.q, k_rep)
    vc, vx = O.quant_mxfp4_v(v_rep)
    rows = np.arange(n)
    for causal in (False, True):
        say(f"case mxfp4 smooth_q gqa causal={causal}")
        o = host(sage.sage_attn_fwd(dev(x.q), dev(k), dev(v), is_causal=causal, pv_mode="mxfp4", smooth_q=True))
        for h in range(H):
            o1, bound, _ = o1_smooth_rows(qs[0, h], qsx[0, h], qm[0, h], (kc[0, h], kx[0, h], km[0, h]),
                                          (vc[0, h], vx[0, h]), k_rep[0, h], 0, h, rows, causal, sm)
            o2 = O.sdpa_fp64_rows(x.q[0, h], k_rep[0, h], v_rep[0, h], rows, causal)
            check_out(o[0, h], o1, o2, f"mxfp4 smooth_q gqa h={h}", bound)
    lens = [1, 129, 300, 0, 128, 2]
    xv = workloads.generate_custom(890, 0, 2, 0, 64, k_bias=3.0, q_bias=2.0, lengths=lens)
    cu = dev(xv.cu_seqlens)
    sm = float(O.default_sm_scale(64))
    for causal in (False, True):
        say(f"case mxfp4 smooth_q varlen causal={causal}")
        o, lse = sage.sage_attn_varlen_fwd(dev(xv.q), dev(xv.k), dev(xv.v), cu, max(lens), is_causal=causal,
                                           pv_mode="mxfp4", return_lse=True, smooth_q=True)
        o, lse = host(o), host(lse)
        for i, n in enumerate(lens):
            if n == 0:
                continue
            a0 = int(xv.cu_seqlens[i])
            qq, kk_, vv = (t[:, a0:a0 + n][None] for t in (xv.q, xv.k, xv.v))
            qs, qsx, qm = O.quant_mxfp4_q_smooth(qq)
            _, _, kc, kx, km = O.quant_mxfp4_qk(qq, kk_)
            vc, vx = O.quant_mxfp4_v(vv)
            rows = np.arange(n)
            for h in range(2):
                o1, bound, want_lse = o1_smooth_rows(qs[0, h], qsx[0, h], qm[0, h], (kc[0, h], kx[0, h], km[0, h]),
                                                     (vc[0, h], vx[0, h]), kk_[0, h], 0, h, rows, causal, sm)
                o2 = O.sdpa_fp64_rows(qq[0, h], kk_[0, h], vv[0, h], rows, causal)
                check_out(o[h, a0:a0 + n], o1, o2, f"mxfp4 smooth_q varlen seq={i} h={h}", bound)
                assert np.abs(lse[h, a0:a0 + n].astype(np.float64) - want_lse).max() <= LSE_ABS


def test_mxfp4_smooth_q_workload_biased_q():
    """The biased-Q long-sequence workload (Q channel bias of std 3): sampled
    rows against the oracle, and smoothing must bring the output closer to
    exact attention than the plain MXFP4 path on the same inputs."""
    w = workloads.get("long_fp8")
    say(f"case mxfp4 smooth_q workload {w.name} {w.description}")
    x = workloads.generate(w)
    B, H, N, d = x.q.shape
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    o_s = host(sage.sage_attn_fwd(q, k, v, is_causal=w.causal, pv_mode="mxfp4", smooth_q=True))
    o_p = host(sage.sage_attn_fwd(q, k, v, is_causal=w.causal, pv_mode="mxfp4"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 17)
    sm = float(O.default_sm_scale(d))
    for b, h in [(0, 0), (B - 1, H - 1)]:
        qs, qsx, qm = O.quant_mxfp4_q_smooth(x.q[b:b + 1, h:h + 1])
        _, _, kc, kx, km = O.quant_mxfp4_qk(x.q[b:b + 1, h:h + 1], x.k[b:b + 1, h:h + 1])
        vc, vx = O.quant_mxfp4_v(x.v[b:b + 1, h:h + 1])
        rows = _sample_rows(N, rng)
        o1, bound, _ = o1_smooth_rows(qs[0, 0], qsx[0, 0], qm[0, 0], (kc[0, 0], kx[0, 0], km[0, 0]),
                                      (vc[0, 0], vx[0, 0]), x.k[b, h], 0, 0, rows, w.causal, sm)
        o2 = O.sdpa_fp64_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, w.causal)
        check_out(o_s[b, h, rows], o1, o2, f"mxfp4 smooth_q {w.name} b={b} h={h}", bound)
        c_s, c_p = cos(o_s[b, h, rows], o2), cos(o_p[b, h, rows], o2)
        say(f"  cos to exact: smoothed {c_s:.6f}, plain {c_p:.6f}")
        assert c_s > c_p, (c_s, c_p)
