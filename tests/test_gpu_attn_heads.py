"""The sparse attention with 64 or 128 heads against the same heads taken 16
at a time.  Heads do not interact: each wave of the attention kernel holds
its own 16 heads, and a call with 16 heads runs the same wave code over the
same splits of the selection (the split count depends on the token count and
the number of 64-head groups, equal here), so out and lse must agree bit for
bit whatever the head count of the call.
"""

import pytest
import torch

from sparse_attention_long_03_amd import binding as B
from sparse_attention_long_03_amd import inputs as I
from sparse_attention_long_03_amd.path import DSAPath

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    # decode, split over the selection (8 splits for every head count)
    "decode_h128": I.scaled(I.CONFIGS["decode128k"], B=4, L=20000),
    # ragged paged cache, short rows with -1 padding
    "paged_h64": I.scaled(I.CONFIGS["ragged_paged"], B=6, L=5000, min_len=100, H=64),
    # many tokens, one split for every head count
    "prefill_h128": I.scaled(I.CONFIGS["prefill64k"], L=300, k=256),
    # the decode batch at its full length
    "decode128k": I.CONFIGS["decode128k"],
}


@pytest.mark.parametrize("name", list(CASES))
def test_head_split_equals_sixteen_head_calls(name):
    x = I.make_inputs(CASES[name], DEV)
    c = x.cfg
    assert c.H % 64 == 0
    p = DSAPath(x)
    idx = I.random_selection(c, x.pos, c.k, DEV)
    out, lse = p.attn(idx)
    out, lse = out.clone(), lse.clone()
    ws = B.workspace(B.dsa_workspace_bytes(B.DSA_OP_ATTN, x.T, x.max_len, 16, c.k))
    for h in range(0, c.H, 16):
        q16 = x.q[:, h:h + 16, :].contiguous()
        o16 = torch.empty((x.T, 16, c.d_v), dtype=torch.bfloat16, device=DEV)
        l16 = torch.empty((x.T, 16), dtype=torch.float32, device=DEV)
        B.dsa_sparse_mla_attn(p.q, p.layout, 16, q16, x.kv, idx, c.k, c.scale, o16, l16, ws)
        torch.cuda.synchronize()
        assert torch.equal(out[:, h:h + 16].view(torch.int16), o16.view(torch.int16)), f"out, heads {h}..{h + 15}"
        assert torch.equal(lse[:, h:h + 16].view(torch.int32), l16.view(torch.int32)), f"lse, heads {h}..{h + 15}"
