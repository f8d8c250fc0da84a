"""GPU parity of the indexer's KL training signal: the target
(dsa_indexer_kl_target) and the loss with its gradients (dsa_indexer_kl)
against the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_long_03_amd import inputs as I
from sparse_attention_long_03_amd.path import DSAPath

from parity_util import KL_REL, check_bwd, exact_indexer_inputs, kl_magnitudes, np_

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    # 16 decode queries, 4K context, 16 attention heads, k = 256 (indexer 64 x 128)
    "decode_h16": I.scaled(I.CONFIGS["tiny"], H_I=64, D_I=128),
    # all 128 heads, k = 2048 of 3000 positions, three sequences
    "h128_k2048": I.scaled(I.CONFIGS["decode32k"], B=3, L=3000, queries_per_seq=3),
    # 64 heads over shuffled pages, ragged rows padded with -1
    "h64_paged": I.scaled(I.CONFIGS["ragged_paged"], B=4, L=2500, min_len=100, H=64, k=512),
    # prefill: 500 causal queries, rows shorter than k padded
    "h32_prefill": I.scaled(I.CONFIGS["prefill64k"], L=500, H=32, k=128),
}


def _bt(x):
    return None if x.block_table is None else np_(x.block_table)


@pytest.mark.parametrize("name", list(CASES))
def test_kl_target_matches_oracle(name):
    x = I.make_inputs(CASES[name], DEV)
    print(f"kl target {name}: T={x.T} H={x.cfg.H} k={x.cfg.k}", flush=True)
    p = DSAPath(x)
    _, _, idx = p.forward()
    tgt = np_(p.kl_target(idx))
    ref = O.indexer_kl_target(I.bf16_bits(x.q), I.bf16_bits(x.kv), np_(idx), np_(x.seq_id), x.cfg.scale, _bt(x))
    err = np.abs(tgt - ref)
    assert np.all(err <= 1e-3 * ref + 1e-7), f"{name}: max err {err.max()}"
    assert np.all(tgt[np_(idx) < 0] == 0)
    sums = tgt.sum(axis=1)
    has = (np_(idx) >= 0).any(axis=1)
    np.testing.assert_allclose(sums[has], 1.0, rtol=1e-4)


def _kl_oracle(x, idx, target):
    return O.indexer_kl(np_(x.iq8), np_(x.iqs).astype(np.float64), np_(x.iw).astype(np.float64), np_(x.ik8),
                        np_(x.iks).astype(np.float64), np_(idx), np_(x.seq_id), target, _bt(x))


def _check_kl(x, idx, target_np, loss, dq, dw, dk, what):
    rl, rdI, rdq, rdw, rdk = _kl_oracle(x, idx, target_np)
    np.testing.assert_allclose(np_(loss), rl, rtol=KL_REL, atol=1e-6, err_msg=f"{what} loss")
    m_dq, m_dk, m_dw = kl_magnitudes(np_(x.iq8), np_(x.iqs), np_(x.iw), np_(x.ik8), np_(x.iks), np_(idx),
                                     np_(x.seq_id), rdI, _bt(x))
    # dw: fp32 sums over exact dot products
    assert np.all(np.abs(np_(dw) - rdw) <= KL_REL * m_dw + 1e-7), f"{what} dw"
    check_bwd(np_(dq), rdq, m_dq, f"{what} dq")
    check_bwd(np_(dk), rdk, m_dk, f"{what} dk")


@pytest.mark.parametrize("name", list(CASES))
def test_kl_loss_and_gradients_match_oracle(name):
    x = exact_indexer_inputs(I.make_inputs(CASES[name], DEV))
    print(f"kl loss {name}: T={x.T} k={x.cfg.k}", flush=True)
    p = DSAPath(x)
    _, _, idx = p.forward()
    target = p.kl_target(idx)
    loss, dq, dw, dk = p.indexer_kl(idx, target)
    torch.cuda.synchronize()
    _check_kl(x, idx, np_(target).astype(np.float64), loss, dq, dw, dk, name)


def test_kl_edge_selections_and_accumulation():
    """Padding anywhere, a row twice in one query, a query with no selection,
    a zero target entry; dk accumulates over calls; paged equals contiguous."""
    cfg = I.scaled(I.CONFIGS["decode32k"], B=2, L=700, queries_per_seq=4, H=16, k=100)
    x = exact_indexer_inputs(I.make_inputs(cfg, DEV))
    g = np.random.default_rng(7)
    pos = np_(x.pos)
    idx = np.full((x.T, cfg.k), -1, dtype=np.int32)
    target = np.zeros((x.T, cfg.k))
    for t in range(x.T):
        n = [100, 37, 64, 1, 0, 99, 33, 65][t]
        if n:
            slots = g.choice(cfg.k, n, replace=False)
            idx[t, slots] = g.choice(int(pos[t]) + 1, n, replace=False)
            v = g.uniform(size=n)
            v[0] = 0.0 if n > 2 else v[0]
            target[t, slots] = v / v.sum()
    idx[1, 5] = idx[1, 6] = 17
    target[1, 5] = target[1, 6] = 0.01
    target[1] /= target[1].sum()
    idx_t = torch.from_numpy(idx).to(DEV)
    tgt_t = torch.from_numpy(target.astype(np.float32)).to(DEV)
    p = DSAPath(x)
    loss, dq, dw, dk = p.indexer_kl(idx_t, tgt_t)
    torch.cuda.synchronize()
    _check_kl(x, idx_t, np_(tgt_t).astype(np.float64), loss, dq, dw, dk, "edge")
    assert float(loss[4]) == 0.0 and torch.all(dq[4] == 0) and torch.all(dw[4] == 0)
    once = dk.clone()
    _, dq2, _, dk = p.indexer_kl(idx_t, tgt_t, dk=dk)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2)
    np.testing.assert_allclose(np_(dk), 2 * np_(once), rtol=1e-6, atol=1e-12)


def test_full_size_train_chunk_sampled():
    """4096 queries of a 64K sequence, H = 128, k = 2048: the target of sampled
    queries, and their loss, dq and dw against the oracle run on them."""
    cfg = I.CONFIGS["train64k_chunk4k"]
    x = exact_indexer_inputs(I.make_inputs(cfg, DEV))
    print(f"kl full size: T={x.T}", flush=True)
    p = DSAPath(x)
    _, _, idx = p.forward()
    target = p.kl_target(idx)
    loss, dq, dw, dk = p.indexer_kl(idx, target)
    torch.cuda.synchronize()
    idx_h, tgt_h = np_(idx), np_(target).astype(np.float64)
    for t in [0, 1, 2048, x.T - 1]:
        sl = slice(t, t + 1)
        rows = idx_h[sl]
        kv_sel = I.bf16_bits(x.kv[0][torch.as_tensor(rows[0], dtype=torch.int64, device=DEV)])[None]
        ref_t = O.indexer_kl_target(I.bf16_bits(x.q[sl]), kv_sel, np.arange(rows.shape[1])[None], np.zeros(1, int),
                                    cfg.scale)
        assert np.all(np.abs(tgt_h[sl] - ref_t) <= 1e-3 * ref_t + 1e-7), f"target {t}"
        rl, rdI, rdq, rdw, _ = O.indexer_kl(np_(x.iq8[sl]), np_(x.iqs[sl]).astype(np.float64),
                                            np_(x.iw[sl]).astype(np.float64), np_(x.ik8), np_(x.iks).astype(np.float64),
                                            rows, np.zeros(1, int), tgt_h[sl])
        np.testing.assert_allclose(float(loss[t]), rl[0], rtol=KL_REL, atol=1e-6)
        m_dq, _, m_dw = kl_magnitudes(np_(x.iq8[sl]), np_(x.iqs[sl]), np_(x.iw[sl]), np_(x.ik8), np_(x.iks), rows,
                                      np.zeros(1, int), rdI)
        assert np.all(np.abs(np_(dw[t]) - rdw[0]) <= KL_REL * m_dw[0] + 1e-7), f"dw {t}"
        check_bwd(np_(dq[t]), rdq[0], m_dq[0], f"full-size dq {t}")
    assert torch.all(torch.isfinite(dk)) and float(loss.min()) >= -1e-5
