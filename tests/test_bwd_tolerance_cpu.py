"""The backward's parity check has teeth: mistakes a kernel could plausibly
make (planted here in the oracle's result, on the CPU) fail it, while the
roundings the GPU is allowed (bf16 on P, dS and per-row gradients) pass."""

import numpy as np
import torch

import oracle as O
from sparse_attention_long_03_amd import inputs as I

from parity_util import attn_bwd_magnitudes, check_bwd


def _case():
    cfg = I.scaled(I.CONFIGS["tiny"], B=2, L=300, queries_per_seq=3, H=16, k=64)
    x = I.make_inputs(cfg)
    g = np.random.default_rng(3)
    idx = np.stack([g.choice(int(p) + 1, cfg.k, replace=False) for p in x.pos.numpy()])
    dO = I.output_grad(cfg, x.T).float().numpy().astype(np.float64)
    args = (I.bf16_bits(x.q), I.bf16_bits(x.kv), idx, x.seq_id.numpy(), cfg.scale)
    return x, cfg, idx, dO, args


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _variant(x, cfg, idx, dO, drop_D=False, no_scale=False, p_for_ds=False, bf16=False):
    """The backward with one planted mistake (same loop as the definition);
    bf16=True instead rounds what the GPU rounds: the output used for D, P,
    scale*dS and each selected row's gradient."""
    q = O.decode_bf16(I.bf16_bits(x.q))
    kv = O.decode_bf16(I.bf16_bits(x.kv))
    dq = np.zeros(q.shape)
    dkv = np.zeros(kv.shape)
    for t in range(x.T):
        b = int(x.seq_id[t])
        rows = kv[b, idx[t]]
        z = cfg.scale * q[t] @ rows.T
        p = np.exp(z - z.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        dP = dO[t] @ rows[:, :512].T
        o = p @ rows[:, :512]
        D = 0.0 if drop_D else np.sum(dO[t] * (_bf16(o) if bf16 else o), 1, keepdims=True)
        dS = p if p_for_ds else p * (dP - D)
        s = 1.0 if no_scale else cfg.scale
        sdS = _bf16(s * dS) if bf16 else s * dS
        pp = _bf16(p) if bf16 else p
        dq[t] = sdS @ rows
        gr = sdS.T @ q[t]
        gr[:, :512] += pp.T @ dO[t]
        if bf16:
            gr = _bf16(gr)
        for j, r in enumerate(idx[t]):
            dkv[b, r] += gr[j]
    return dq, dkv


def test_planted_mistakes_fail_and_roundings_pass():
    x, cfg, idx, dO, args = _case()
    dq, _, dkv = O.sparse_mla_attention_backward(*args, dO)
    m_dq, m_dkv = attn_bwd_magnitudes(*args, dO)

    def fails(fn):
        try:
            fn()
        except AssertionError:
            return True
        return False

    # allowed: the roundings the GPU makes
    bdq, bdkv = _variant(x, cfg, idx, dO, bf16=True)
    check_bwd(bdq, dq, m_dq)
    check_bwd(bdkv, dkv, m_dkv)
    assert not np.array_equal(bdq, dq)
    # planted: D dropped, softmax scale dropped, P used for dS
    for kw in (dict(drop_D=True), dict(no_scale=True), dict(p_for_ds=True)):
        wdq, wdkv = _variant(x, cfg, idx, dO, **kw)
        assert fails(lambda: check_bwd(wdq, dq, m_dq)), kw
        assert fails(lambda: check_bwd(wdkv, dkv, m_dkv)), kw
    # planted: the rope part of dkv or the value part (P^T dO) missing
    no_rope = dkv.copy()
    no_rope[..., 512:] = 0
    assert fails(lambda: check_bwd(no_rope, dkv, m_dkv))
    _, no_dv = _variant(x, cfg, idx, np.zeros_like(dO))
    assert fails(lambda: check_bwd(no_dv, dkv, m_dkv))
    # planted: a gradient added to the wrong row (off by one position)
    shifted = np.roll(dkv, 1, axis=1)
    assert fails(lambda: check_bwd(shifted, dkv, m_dkv))
    # the variant loop without a mistake reproduces the oracle
    rdq, rdkv = _variant(x, cfg, idx, dO)
    np.testing.assert_allclose(rdq, dq, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(rdkv, dkv, rtol=1e-12, atol=1e-15)


def test_kl_check_catches_planted_mistakes():
    """The KL gradients' check (2^-7 of the term magnitudes, Frobenius 1e-2)
    fails on plausible mistakes planted in the oracle's result."""
    from parity_util import KL_BF16, kl_exact_dI_error, kl_magnitudes
    g = np.random.default_rng(9)
    T, H_I, D_I, L, k = 3, 64, 128, 200, 40
    codes = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4, 0xC8], dtype=np.uint8)
    q8 = codes[g.integers(0, 9, size=(T, H_I, D_I))]
    k8 = codes[g.integers(0, 9, size=(1, L, D_I))]
    qs = np.full(T, 0.125)
    ks = 0.0625 + 0.0625 * g.uniform(size=(1, L))
    w = g.uniform(size=(T, H_I))
    idx = np.stack([g.choice(L, k, replace=False) for _ in range(T)])
    seq_id = np.zeros(T, int)
    tgt = g.uniform(size=(T, k))
    tgt /= tgt.sum(axis=1, keepdims=True)
    loss, dI, dq, dw, dk = O.indexer_kl(q8, qs, w, k8, ks, idx, seq_id, tgt)
    # the magnitudes as the GPU check takes them: dI's own error bound added per term
    args = (q8, qs, w, k8, ks, idx, seq_id)
    m_dq, m_dk, _ = kl_magnitudes(*args, dI)
    e_dq, e_dk, _ = kl_magnitudes(*args, kl_exact_dI_error(*args, tgt, dI))
    m_dq = m_dq + e_dq / KL_BF16
    m_dk = m_dk + e_dk / KL_BF16
    check_bwd(dq, dq, m_dq)
    check_bwd(dk, dk, m_dk)

    def fails(fn):
        try:
            fn()
        except AssertionError:
            return True
        return False

    # dq without the head weight; dI with the wrong sign
    assert fails(lambda: check_bwd(dq / w[:, :, None], dq, m_dq))
    assert fails(lambda: check_bwd(-dq, dq, m_dq))
    # dk without the query scale
    assert fails(lambda: check_bwd(dk / 0.125, dk, m_dk))
    # the ReLU's derivative dropped (every head counts), recomputed from the definition
    qd = O.decode_e4m3fn(q8) * qs[:, None, None]
    bad = np.zeros_like(dk)
    for t in range(T):
        gk = dI[t][:, None] * (np.ones((H_I, k)) * w[t][:, None]).T @ qd[t]
        for j, s in enumerate(idx[t]):
            bad[0, s] += gk[j]
    assert fails(lambda: check_bwd(bad, dk, m_dk))
