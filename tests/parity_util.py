"""Shared comparison helpers for the GPU parity tests (tolerances live here)."""

import numpy as np
import torch

import oracle as O
from sparse_attention_long_03_amd import inputs as I

# Indexer: 1e-3 relative per element, plus a floor proportional to the
# magnitude of the terms that make up the logit,
#   M[t,s] = qs[t] * ks[s] * sum_j |w[t,j]| * sum_d |q[t,j,d]| * |k[s,d]|.
# The gfx950 FP8 matrix cores do not accumulate exactly in fp32: a probe of
# 16x16x128 and 16x16x32 FP8 MFMAs on N(0,1) data quantised like ours showed
# errors up to 1.6e-5 (mean 1.4e-6) of sum_i |a_i b_i|, so a logit whose head
# dot products nearly cancel carries an absolute error of that order.  The
# floor 1e-4 * M is about six times the worst measured case.
IDX_RTOL = 1e-3
IDX_MAG = 1e-4
# Attention (bf16 output): max-abs 2e-2 / relative 1e-2 per element, and the
# relative Frobenius error of each query's output at most 1e-2.
ATT_ATOL = 2e-2
ATT_RTOL = 1e-2
ATT_FRO = 1e-2


def np_(t):
    return t.detach().cpu().numpy()


def host_inputs(x):
    """numpy views of a (small) DSAInputs for the oracle."""
    return dict(
        iq8=np_(x.iq8), iqs=np_(x.iqs).astype(np.float64), iw=np_(x.iw).astype(np.float64),
        ik8=np_(x.ik8), iks=np_(x.iks).astype(np.float64), q=I.bf16_bits(x.q), kv=I.bf16_bits(x.kv),
        seq_id=np_(x.seq_id), pos=np_(x.pos),
        bt=None if x.block_table is None else np_(x.block_table),
    )


def indexer_magnitude(q8_t, qs_t, w_t, k8_rows, ks_rows):
    """M[s] for one query: the sum of absolute values of every product term."""
    q = np.abs(O.decode_e4m3fn(np.asarray(q8_t)))
    k = np.abs(O.decode_e4m3fn(np.asarray(k8_rows)))
    return float(qs_t) * np.asarray(ks_rows, dtype=np.float64) * ((k @ q.T) @ np.abs(np.asarray(w_t, np.float64)))


def check_logits(gpu_row, ora_row, mag_row, what=""):
    g = np.asarray(gpu_row, dtype=np.float64)
    o = np.asarray(ora_row, dtype=np.float64)
    tol = IDX_RTOL * np.abs(o) + IDX_MAG * np.asarray(mag_row, dtype=np.float64)
    bad = np.abs(g - o) > tol
    assert not bad.any(), (f"{what}: {bad.sum()} logits out of tolerance; first at {np.argmax(bad)}: "
                           f"gpu {g[bad][0]} oracle {o[bad][0]}")


def check_attn(gpu_out, ora_out, what=""):
    g = np.asarray(gpu_out, dtype=np.float64)
    o = np.asarray(ora_out, dtype=np.float64)
    err = np.abs(g - o)
    bad = err > (ATT_ATOL + ATT_RTOL * np.abs(o))
    assert not bad.any(), f"{what}: {bad.sum()} outputs beyond atol/rtol; max err {err.max()}"
    for t in range(o.shape[0]):
        fro = np.linalg.norm(g[t] - o[t]) / max(np.linalg.norm(o[t]), 1e-30)
        assert fro <= ATT_FRO, f"{what}: query {t} relative Frobenius error {fro}"


def check_selection_valid(sel, ora_logits_row, n, k, mag_row):
    """GPU selection computed from GPU logits: the set is a valid top-k of the
    oracle logits up to the indexer tolerance (exact ties may resolve either
    way, values within tolerance of the k-th may swap)."""
    sel = np.asarray(sel)
    got = sel[sel >= 0]
    assert len(got) == min(k, n)
    assert len(np.unique(got)) == len(got)
    assert got.min() >= 0 and got.max() < n
    v = np.asarray(ora_logits_row[:n], dtype=np.float64)
    if n <= k:
        assert sorted(got.tolist()) == list(range(n))
        return
    tol = IDX_RTOL * np.abs(v) + IDX_MAG * np.asarray(mag_row[:n], dtype=np.float64)
    kth = np.sort(v)[::-1][k - 1]
    mask = np.zeros(n, bool)
    mask[got] = True
    # a selected value may sit below the k-th only by its own error plus the k-th's
    kth_tol = tol[np.argsort(-v, kind="stable")[k - 1]]
    assert np.all(v[mask] + tol[mask] >= kth - kth_tol)
    assert np.all(v[~mask] - tol[~mask] <= kth + kth_tol)


def bf16_to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def torch_seed_all(s=0):
    torch.manual_seed(s)
