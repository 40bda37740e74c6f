"""Head sharding on one GPU: a node of P GPUs runs the forward with no
collective by giving each GPU H/P heads (every (batch, head) is independent:
K smoothing, quantisation blocks and the softmax are all per head).  One GPU
shows that exactly: the forward over a slice of the heads equals, bit for bit,
the same heads of the full forward; and the full forward is deterministic
run to run.
"""
import sys

import pytest
import torch

import quantized_attention_quant_amd as sage
import workloads

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    ("llm_prefill", "fp16", {}),
    ("long_fp8", "fp8", {}),
    ("seq16k", "fp16", {"smooth_q": True}),
    ("seq16k", "mxfp4", {}),
]


@pytest.mark.parametrize("name,pv_mode,opts", CASES)
def test_head_shard_equals_full(name, pv_mode, opts):
    w = workloads.get(name)
    say(f"case shard {name} pv={pv_mode} {opts}")
    x = workloads.generate(w)
    B, H, N, d = x.q.shape
    q, k, v = (torch.from_numpy(a).cuda() for a in (x.q, x.k, x.v))
    full = sage.sage_attn_fwd(q, k, v, is_causal=w.causal, pv_mode=pv_mode, **opts)
    again = sage.sage_attn_fwd(q, k, v, is_causal=w.causal, pv_mode=pv_mode, **opts)
    torch.cuda.synchronize()
    assert torch.equal(full, again), "forward is not deterministic"
    P = 8
    per = H // P
    for r in (0, P - 1):
        h0, h1 = r * per, (r + 1) * per
        part = sage.sage_attn_fwd(q[:, h0:h1].contiguous(), k[:, h0:h1].contiguous(), v[:, h0:h1].contiguous(),
                                  is_causal=w.causal, pv_mode=pv_mode, **opts)
        torch.cuda.synchronize()
        same = torch.equal(part, full[:, h0:h1])
        say(f"  rank {r} heads {h0}..{h1 - 1}: bit-identical={same}")
        assert same, (name, r)
