"""The allocation-free forward, sage_attn_fwd_noalloc, through the C ABI,
against sage_attn_fwd with a caller workspace: the same kernels on the same
inputs, so the outputs (and LSE) are bit-identical.  Calls in a row on one
stream share the library's per-GPU scratch array; each later one is smaller
than the one before it, so any stale scratch contents would show."""
import sys

import numpy as np
import pytest
import torch

import quantized_attention_quant_amd as sage
import workloads

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    # B, H, H_kv, N, d, causal, pv_mode, smooth_q
    (2, 4, 2, 1000, 128, True, "fp16", False),
    (1, 3, 3, 300, 64, False, "fp8", False),
    (1, 2, 1, 129, 128, True, "fp8", True),
]


def test_noalloc_matches_workspace_forward():
    for i, (B, H, Hkv, N, d, causal, pv, sq) in enumerate(CASES):
        say(f"case noalloc #{i}: B={B} H={H} H_kv={Hkv} N={N} d={d} causal={causal} pv={pv} smooth_q={sq}")
        x = workloads.generate_custom(900 + i, B, H, N, d, k_bias=3.0, q_bias=1.0)
        q = torch.from_numpy(x.q).cuda()
        k = torch.from_numpy(np.ascontiguousarray(x.k[:, :Hkv])).cuda()
        v = torch.from_numpy(np.ascontiguousarray(x.v[:, :Hkv])).cuda()
        o_ref, lse_ref = sage.sage_attn_fwd(q, k, v, is_causal=causal, pv_mode=pv, smooth_q=sq, return_lse=True)
        o, lse = sage.sage_attn_fwd_noalloc(q, k, v, is_causal=causal, pv_mode=pv, smooth_q=sq, return_lse=True)
        torch.cuda.synchronize()
        a, b = o.cpu().numpy(), o_ref.cpu().numpy()
        assert (a.view(np.uint16) == b.view(np.uint16)).all(), (i, float(np.abs(a.astype(np.float64) - b).max()))
        assert (lse.cpu().numpy().view(np.uint32) == lse_ref.cpu().numpy().view(np.uint32)).all(), i


def test_noalloc_rejects_problems_beyond_the_scratch():
    q = torch.empty((1, 64, 32768, 128), dtype=torch.float16, device="cuda")
    assert sage.sage_attn_workspace_size(1, 64, 32768, 128) > sage.NOALLOC_SCRATCH_BYTES
    with pytest.raises(sage.SageError):
        sage.sage_attn_fwd_noalloc(q, q, q)
