"""The accumulation error of gfx950's FP8 matrix cores, measured through the
indexer entry point (dsa_indexer_logits).

Each query keeps one indexer head (one-hot head weights) and unit scales, so
its logit against key s is ReLU of one FP8 dot product as the matrix core
summed it.  Every query also appears with its codes negated, so that both
signs of each dot are seen.  The exact dot is a float64 sum over the decoded
codes; ReLU is 1-Lipschitz, so

    |logit - ReLU(exact dot)| <= |mfma dot - exact dot|,

and the test asserts this is at most FP8_ACC_BOUND times the sum of the
absolute values of the products.  The same bound sets the floor of the
indexer's parity tolerance (parity_util.check_logits) and of the KL signal's
natural-input tolerance.
"""

import numpy as np
import pytest
import torch

from sparse_attention_long_03_amd import binding as B
from sparse_attention_long_03_amd import inputs as I

from parity_util import FP8_ACC_BOUND, np_

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _decode(codes):
    """e4m3fn codes -> float64 through torch's own FP8 type (a library routine)."""
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("H_I,D_I", [(64, 128), (64, 64), (4, 128), (4, 64)])
def test_fp8_mfma_accumulation_bound(H_I, D_I):
    L = 4096
    cfg = I.scaled(I.CONFIGS["decode32k"], B=1, L=L, H_I=H_I, D_I=D_I, queries_per_seq=2 * H_I)
    x = I.make_inputs(cfg, DEV)
    T = 2 * H_I
    # query t keeps head t % H_I; queries H_I.. carry the negated codes of the first H_I
    q8 = x.iq8.clone()
    q8[H_I:] = q8[:H_I] ^ 0x80
    w = torch.zeros((T, H_I), dtype=torch.float32, device=DEV)
    w[torch.arange(T), torch.arange(T) % H_I] = 1.0
    ones_q = torch.ones(T, dtype=torch.float32, device=DEV)
    ones_k = torch.ones_like(x.iks)
    seq_id = torch.zeros(T, dtype=torch.int32, device=DEV)
    pos = torch.full((T,), L - 1, dtype=torch.int32, device=DEV)
    q = B.queries(seq_id, pos, 1, L)
    lay = B.contiguous_layout(L)
    logits = torch.empty((T, L), dtype=torch.float32, device=DEV)
    B.dsa_indexer_logits(q, lay, H_I, D_I, q8, ones_q, w, x.ik8, ones_k, logits)
    torch.cuda.synchronize()

    got = np_(logits).astype(np.float64)                       # [T, L]
    qd = _decode(np_(q8))                                       # [T, H_I, D_I]
    kd = _decode(np_(x.ik8[0]))                                 # [L, D_I]
    heads = np.arange(T) % H_I
    qh = qd[np.arange(T), heads]                                # [T, D_I]
    exact = qh @ kd.T                                           # float64, exact for these products
    mag = np.abs(qh) @ np.abs(kd).T
    err = np.abs(got - np.maximum(exact, 0.0))
    ratio = err / np.maximum(mag, 1e-300)
    worst = float(ratio.max())
    print(f"FP8 MFMA {H_I}x{D_I}: {ratio.size} dots, max |err|/sum|q*k| = {worst:.3e} "
          f"(mean {float(ratio.mean()):.3e}, {int((err > 0).sum())} inexact)", flush=True)
    assert worst <= FP8_ACC_BOUND, f"accumulation error {worst:.3e} above the bound {FP8_ACC_BOUND:.3e}"
