"""GPU parity of the indexer's KL training signal: the target
(dsa_indexer_kl_target) and the loss with its gradients (dsa_indexer_kl)
against the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_long_03_amd import binding as B
from sparse_attention_long_03_amd import inputs as I
from sparse_attention_long_03_amd.path import DSAPath

from parity_util import (KL_BF16, KL_REL, check_bwd, exact_indexer_inputs, kl_exact_dI_error, kl_magnitudes,
                         kl_natural_tolerances, np_, oracle_selection)

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


def _oracle_target(x, sel):
    """The oracle's KL target over a selection, rounded to float32 (the form
    both sides take it in)."""
    t = O.indexer_kl_target(I.bf16_bits(x.q), I.bf16_bits(x.kv), sel, np_(x.seq_id), x.cfg.scale, _bt(x))
    return t.astype(np.float32)


@pytest.mark.parametrize("name", list(CASES))
def test_kl_target_matches_oracle(name):
    x = I.make_inputs(CASES[name], DEV)
    print(f"kl target {name}: T={x.T} H={x.cfg.H} k={x.cfg.k}", flush=True)
    sel = oracle_selection(x)
    idx = torch.from_numpy(sel).to(DEV)
    p = DSAPath(x)
    p.attn(idx)
    tgt = np_(p.kl_target(idx))
    ref = O.indexer_kl_target(I.bf16_bits(x.q), I.bf16_bits(x.kv), sel, np_(x.seq_id), x.cfg.scale, _bt(x))
    err = np.abs(tgt - ref)
    assert np.all(err <= 1e-3 * ref + 1e-7), f"{name}: max err {err.max()}"
    assert np.all(tgt[sel < 0] == 0)
    sums = tgt.sum(axis=1)
    has = (sel >= 0).any(axis=1)
    np.testing.assert_allclose(sums[has], 1.0, rtol=1e-4)


def _kl_oracle(x, idx, target):
    return O.indexer_kl(np_(x.iq8), np_(x.iqs).astype(np.float64), np_(x.iw).astype(np.float64), np_(x.ik8),
                        np_(x.iks).astype(np.float64), np_(idx), np_(x.seq_id), target, _bt(x))


def _check_kl(x, idx, target_np, loss, dq, dw, dk, what):
    rl, rdI, rdq, rdw, rdk = _kl_oracle(x, idx, target_np)
    np.testing.assert_allclose(np_(loss), rl, rtol=KL_REL, atol=1e-6, err_msg=f"{what} loss")
    args = (np_(x.iq8), np_(x.iqs), np_(x.iw), np_(x.ik8), np_(x.iks), np_(idx), np_(x.seq_id))
    m_dq, m_dk, m_dw = kl_magnitudes(*args, rdI, _bt(x))
    # the same sums over dI's own error bound: an absolute allowance per term
    e_dq, e_dk, e_dw = kl_magnitudes(*args, kl_exact_dI_error(*args, target_np, rdI, _bt(x)), _bt(x))
    # dw: fp32 sums over exact dot products
    assert np.all(np.abs(np_(dw) - rdw) <= KL_REL * m_dw + e_dw + 1e-7), f"{what} dw"
    check_bwd(np_(dq), rdq, m_dq + e_dq / KL_BF16, f"{what} dq", KL_BF16)
    check_bwd(np_(dk), rdk, m_dk + e_dk / KL_BF16, f"{what} dk", KL_BF16)


@pytest.mark.parametrize("name", list(CASES))
def test_kl_loss_and_gradients_match_oracle(name):
    x = exact_indexer_inputs(I.make_inputs(CASES[name], DEV))
    print(f"kl loss {name}: T={x.T} k={x.cfg.k}", flush=True)
    sel = oracle_selection(x)
    target = _oracle_target(x, sel)
    idx = torch.from_numpy(sel).to(DEV)
    p = DSAPath(x)
    loss, dq, dw, dk = p.indexer_kl(idx, torch.from_numpy(target).to(DEV))
    torch.cuda.synchronize()
    _check_kl(x, idx, target.astype(np.float64), loss, dq, dw, dk, name)


NATURAL = {
    # the generated FP8 codes and scales as they are: logits of order 100, a
    # sharply peaked indexer softmax
    "h128_k2048": (CASES["h128_k2048"], 1.0),
    # natural codes with the query scales divided by 16: logits of order 10
    "h64_paged_qs16": (CASES["h64_paged"], 1.0 / 16),
    "decode_h16_qs16": (CASES["decode_h16"], 1.0 / 16),
}


@pytest.mark.parametrize("name", list(NATURAL))
def test_kl_natural_fp8_inputs(name):
    """Loss and gradients on natural FP8 codes (not the integer-valued ones
    whose dot products are exact): every GPU value within the bound derived
    from the FP8 accumulation bound (parity_util.kl_natural_tolerances)."""
    cfg, qs_scale = NATURAL[name]
    x = I.make_inputs(cfg, DEV)
    x.iqs.mul_(qs_scale)
    print(f"kl natural {name}: T={x.T} k={x.cfg.k}", flush=True)
    sel = oracle_selection(x)
    target = _oracle_target(x, sel)
    idx = torch.from_numpy(sel).to(DEV)
    p = DSAPath(x)
    loss, dq, dw, dk = p.indexer_kl(idx, torch.from_numpy(target).to(DEV))
    torch.cuda.synchronize()
    t64 = target.astype(np.float64)
    rl, rdI, rdq, rdw, rdk = _kl_oracle(x, idx, t64)
    t_loss, t_dw, t_dq, t_dk = kl_natural_tolerances(np_(x.iq8), np_(x.iqs).astype(np.float64),
                                                     np_(x.iw).astype(np.float64), np_(x.ik8),
                                                     np_(x.iks).astype(np.float64), sel, np_(x.seq_id), t64, rdI,
                                                     _bt(x))
    for what, g, r, tol in (("loss", np_(loss), rl, t_loss), ("dw", np_(dw), rdw, t_dw), ("dq", np_(dq), rdq, t_dq),
                            ("dk", np_(dk), rdk, t_dk)):
        err = np.abs(np.asarray(g, np.float64) - r)
        ratio = err / np.maximum(tol, 1e-300)
        print(f"  {what}: max err/bound {ratio.max():.3g}, max |err| {err.max():.3g}", flush=True)
        assert np.all(err <= tol), f"{name} {what}: {int((err > tol).sum())} values beyond the derived bound"


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
    """4096 queries of a 64K sequence, H = 128, k = 2048, over a seeded random
    selection: the target of sampled queries, and their loss, dq and dw
    against the oracle run on them."""
    cfg = I.CONFIGS["train64k_chunk4k"]
    x = exact_indexer_inputs(I.make_inputs(cfg, DEV))
    print(f"kl full size: T={x.T}", flush=True)
    idx = I.random_selection(cfg, x.pos, cfg.k, DEV)
    idx_h = np_(idx)
    sample = [0, 1, 2048, x.T - 1]
    # the oracle's target on the sampled queries, a random distribution elsewhere
    target = I.random_distribution(cfg, idx)
    tgt_o = {}
    for t in sample:
        rows = idx_h[t:t + 1]
        kv_sel = I.bf16_bits(x.kv[0][torch.as_tensor(rows[0], dtype=torch.int64, device=DEV)])[None]
        tgt_o[t] = O.indexer_kl_target(I.bf16_bits(x.q[t:t + 1]), kv_sel, np.arange(rows.shape[1])[None],
                                       np.zeros(1, int), cfg.scale).astype(np.float32)
        target[t] = torch.from_numpy(tgt_o[t][0]).to(DEV)
    p = DSAPath(x)
    p.attn(idx)
    tgt_gpu = np_(p.kl_target(idx))
    loss, dq, dw, dk = p.indexer_kl(idx, target)
    torch.cuda.synchronize()
    for t in sample:
        ref_t = tgt_o[t][0].astype(np.float64)
        assert np.all(np.abs(tgt_gpu[t] - ref_t) <= 1e-3 * ref_t + 1e-7), f"target {t}"
        sl = slice(t, t + 1)
        rows = idx_h[sl]
        rl, rdI, rdq, rdw, _ = O.indexer_kl(np_(x.iq8[sl]), np_(x.iqs[sl]).astype(np.float64),
                                            np_(x.iw[sl]).astype(np.float64), np_(x.ik8), np_(x.iks).astype(np.float64),
                                            rows, np.zeros(1, int), tgt_o[t].astype(np.float64))
        np.testing.assert_allclose(float(loss[t]), rl[0], rtol=KL_REL, atol=1e-6)
        m_dq, _, m_dw = kl_magnitudes(np_(x.iq8[sl]), np_(x.iqs[sl]), np_(x.iw[sl]), np_(x.ik8), np_(x.iks), rows,
                                      np.zeros(1, int), rdI)
        assert np.all(np.abs(np_(dw[t]) - rdw[0]) <= KL_REL * m_dw[0] + 1e-7), f"dw {t}"
        check_bwd(np_(dq[t]), rdq[0], m_dq[0], f"full-size dq {t}", KL_BF16)
    assert torch.all(torch.isfinite(dk)) and float(loss.min()) >= -1e-5


DENSE = {
    # two sequences of 16421 positions (a ragged last chunk of 37), one query each, all 128 heads
    "decode_16k": I.scaled(I.CONFIGS["decode32k"], B=2, L=16421),
    # shuffled pages, ragged lengths, 1-2 queries per sequence, 64 heads
    "paged": I.scaled(I.CONFIGS["ragged_paged"], B=4, L=5000, min_len=100, H=64, k=512),
    # a 3000-token prefill: rows from 1 to 3000 positions, 16 heads
    "prefill_3000": I.scaled(I.CONFIGS["prefill64k"], L=3000, H=16, k=256),
}


def _dense_target(x):
    c = x.cfg
    p = DSAPath(x)
    ld = p.ld
    target = torch.full((x.T, ld), -7.0, dtype=torch.float32, device=DEV)
    lse = torch.empty((x.T, c.H), dtype=torch.float32, device=DEV)
    ws = B.workspace(B.dsa_workspace_bytes(B.DSA_OP_KL_TARGET_DENSE, x.T, x.max_len, c.H, 0))
    B.dsa_indexer_kl_target_dense(p.q, p.layout, c.H, x.q, x.kv, c.scale, target, lse, ws)
    torch.cuda.synchronize()
    return np_(target), np_(lse)


def _check_dense_row(x, t, tgt_row, lse_row, what):
    """Target and lse of query t against the oracle with every position 0..pos[t] selected."""
    n = int(x.pos[t]) + 1
    sel = np.arange(n, dtype=np.int32)[None]
    q_t, sid = I.bf16_bits(x.q[t:t + 1]), np.array([int(x.seq_id[t])])
    ref = O.indexer_kl_target(q_t, I.bf16_bits(x.kv), sel, sid, x.cfg.scale, _bt(x))[0]
    _, rl = O.sparse_mla_attention(q_t, I.bf16_bits(x.kv), sel, sid, x.cfg.scale, 512, _bt(x))
    err = np.abs(tgt_row[:n] - ref)
    assert np.all(err <= 1e-3 * ref + 1e-12), f"{what} query {t}: max relative err {np.max(err / ref):.3g}"
    assert np.all(tgt_row[n:] == -7.0), f"{what} query {t}: written past pos"
    np.testing.assert_allclose(tgt_row[:n].sum(), 1.0, rtol=1e-4)
    np.testing.assert_allclose(lse_row, rl[0], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("name", list(DENSE))
def test_dense_warmup_target_matches_oracle(name):
    x = I.make_inputs(DENSE[name], DEV)
    print(f"dense target {name}: T={x.T} H={x.cfg.H} max_len={x.max_len}", flush=True)
    tgt, lse = _dense_target(x)
    rows = range(x.T) if x.T <= 16 else sorted({0, 1, 2046, 2047, 2048, 2500, x.T - 1})
    for t in rows:
        _check_dense_row(x, t, tgt[t], lse[t], name)


def test_dense_warmup_target_at_128k():
    """One query over all 131072 positions of its sequence (64 chunks)."""
    cfg = I.scaled(I.CONFIGS["decode128k"], B=1, planted_frac=0.0)
    x = I.make_inputs(cfg, DEV)
    print(f"dense target 128K: T={x.T} max_len={x.max_len}", flush=True)
    tgt, lse = _dense_target(x)
    _check_dense_row(x, 0, tgt[0], lse[0], "128K")


def _dense_oracle_lse(x, t):
    n = int(x.pos[t]) + 1
    sel = np.arange(n, dtype=np.int32)[None]
    q_t, sid = I.bf16_bits(x.q[t:t + 1]), np.array([int(x.seq_id[t])])
    _, rl = O.sparse_mla_attention(q_t, I.bf16_bits(x.kv), sel, sid, x.cfg.scale, 512, _bt(x))
    return rl[0]


@pytest.mark.parametrize("name", ["decode_16k", "paged"])
def test_dense_target_given_lse_matches_oracle(name):
    """The one-pass dense target, given the oracle's dense lse (as a dense
    attention forward would return it), against the oracle's target."""
    x = I.make_inputs(DENSE[name], DEV)
    c = x.cfg
    p = DSAPath(x)
    print(f"dense target given lse {name}: T={x.T} H={c.H} max_len={x.max_len}", flush=True)
    lse = torch.from_numpy(np.stack([_dense_oracle_lse(x, t) for t in range(x.T)]).astype(np.float32)).to(DEV)
    target = torch.full((x.T, p.ld), -7.0, dtype=torch.float32, device=DEV)
    B.dsa_indexer_kl_target_dense_lse(p.q, p.layout, c.H, x.q, x.kv, c.scale, lse, target)
    torch.cuda.synchronize()
    tgt = np_(target)
    for t in range(x.T):
        n = int(x.pos[t]) + 1
        sel = np.arange(n, dtype=np.int32)[None]
        q_t, sid = I.bf16_bits(x.q[t:t + 1]), np.array([int(x.seq_id[t])])
        ref = O.indexer_kl_target(q_t, I.bf16_bits(x.kv), sel, sid, c.scale, _bt(x))[0]
        err = np.abs(tgt[t, :n] - ref)
        assert np.all(err <= 1e-3 * ref + 1e-12), f"query {t}: max relative err {np.max(err / ref):.3g}"
        assert np.all(tgt[t, n:] == -7.0), f"query {t}: written past pos"
        np.testing.assert_allclose(tgt[t, :n].sum(), 1.0, rtol=1e-4)


def test_dense_target_given_lse_at_128k():
    """The one-pass form over all 131072 positions of one sequence (64
    chunks), given the oracle's dense lse, against the oracle's target."""
    cfg = I.scaled(I.CONFIGS["decode128k"], B=1, planted_frac=0.0)
    x = I.make_inputs(cfg, DEV)
    p = DSAPath(x)
    print(f"dense target given lse 128K: T={x.T} max_len={x.max_len}", flush=True)
    lse = torch.from_numpy(_dense_oracle_lse(x, 0)[None].astype(np.float32)).to(DEV)
    target = torch.full((x.T, p.ld), -7.0, dtype=torch.float32, device=DEV)
    B.dsa_indexer_kl_target_dense_lse(p.q, p.layout, cfg.H, x.q, x.kv, cfg.scale, lse, target)
    torch.cuda.synchronize()
    n = int(x.pos[0]) + 1
    sel = np.arange(n, dtype=np.int32)[None]
    ref = O.indexer_kl_target(I.bf16_bits(x.q[0:1]), I.bf16_bits(x.kv), sel, np.array([int(x.seq_id[0])]), cfg.scale,
                              _bt(x))[0]
    tgt = np_(target)[0]
    err = np.abs(tgt[:n] - ref)
    assert np.all(err <= 1e-3 * ref + 1e-12), f"max relative err {np.max(err / ref):.3g}"
    np.testing.assert_allclose(tgt[:n].sum(), 1.0, rtol=1e-4)


def test_dense_target_one_pass_equals_two_pass():
    """Given the two-pass form's own lse, the one-pass form computes the same
    target (up to the lse's rounding through natural-log units)."""
    cfg = I.scaled(I.CONFIGS["decode32k"], B=2, L=9000, queries_per_seq=2, H=64, k=512)
    x = I.make_inputs(cfg, DEV)
    p = DSAPath(x)
    tgt2, lse = _dense_target(x)
    target = torch.full((x.T, p.ld), -7.0, dtype=torch.float32, device=DEV)
    B.dsa_indexer_kl_target_dense_lse(p.q, p.layout, cfg.H, x.q, x.kv, cfg.scale, torch.from_numpy(lse).to(DEV),
                                      target)
    torch.cuda.synchronize()
    tgt1 = np_(target)
    for t in range(x.T):
        n = int(x.pos[t]) + 1
        np.testing.assert_allclose(tgt1[t, :n], tgt2[t, :n], rtol=1e-5, atol=0)
        assert np.all(tgt1[t, n:] == -7.0)


def test_dense_warmup_target_equals_selected_target_with_every_position():
    """Below 2048 positions the sparse-stage target over a selection holding
    every position is the same computation: equal up to the lse rounding."""
    cfg = I.scaled(I.CONFIGS["decode32k"], B=3, L=1500, queries_per_seq=2, H=32, k=2048)
    x = I.make_inputs(cfg, DEV)
    tgt, lse = _dense_target(x)
    idx = torch.full((x.T, 2048), -1, dtype=torch.int32, device=DEV)
    for t in range(x.T):
        n = int(x.pos[t]) + 1
        idx[t, :n] = torch.arange(n, device=DEV, dtype=torch.int32)
    p = DSAPath(x)
    sel_tgt = np_(p.kl_target(idx, lse=torch.from_numpy(lse).to(DEV)))
    for t in range(x.T):
        n = int(x.pos[t]) + 1
        np.testing.assert_allclose(tgt[t, :n], sel_tgt[t, :n], rtol=1e-5, atol=0)
