"""CPU-side bounds model of every workspace carve (no GPU).

Each entry point that takes a workspace computes its stated size
(dsa_workspace_bytes) and its pointers from one layout, which
dsa_workspace_layout reports.  Over a grid of shapes, including sizes whose
byte counts overflow 32 bits, every layout must

- start each region on a 256-byte boundary,
- tile [0, dsa_workspace_bytes) with its regions, each rounded up to 256
  bytes, in order and without overlap (so no region can reach into another or
  past the stated size), and
- give each region at least the bytes its kernel indexes, computed here with
  Python integers from the shapes the kernels are launched with.
"""

import itertools

import pytest

from sparse_attention_long_03_amd import binding as B

TK_CH = 4096        # top-k positions per chunk
TK_BINS = 2048      # top-k histogram bins
AT_TILE = 32        # attention rows per tile
FUSED_MIN_T = 2048  # dsa_forward fuses the indexer and the selection from here


def _a256(x):
    return (x + 255) // 256 * 256


def _cdiv(a, b):
    return (a + b - 1) // b


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libdsa.so not built")
    return B.lib()


def _check_tiling(op, T, L, H, k):
    total = B.dsa_workspace_bytes(op, T, L, H, k)
    regs = B.dsa_workspace_layout(op, T, L, H, k)
    if total == 0:
        assert regs == [], (op, T, L, H, k)
        return {}
    end = 0
    for parent, name, off, nbytes in regs:
        assert off % 256 == 0, (op, name, off)
        assert off == end, (op, T, L, H, k, name, off, end)  # in order, no gap, no overlap
        end = off + _a256(nbytes)
    assert end == total, (op, T, L, H, k, end, total)
    return {(p + "." if p else "") + n: b for p, n, _, b in regs}


def _topk_min(T, L, k, prefix=""):
    slots = T * max(1, _cdiv(L, TK_CH))
    return {prefix + "hist": T * TK_BINS * 4, prefix + "counts": slots * 8,
            prefix + "above": slots * min(k, TK_CH) * 4, prefix + "ckey": slots * TK_CH * 4,
            prefix + "cpos": slots * TK_CH * 4}


def _check_min(got, need, what):
    for name, b in need.items():
        assert name in got, (what, name, sorted(got))
        assert got[name] >= b, (what, name, got[name], b)


TS = [0, 1, 3, 16, 255, 256, 2047, 2048, 4097]
LS = [1, 100, 4095, 4096, 4097, 131072, 1 << 22]
HS = [16, 64, 128]
KS = [1, 256, 2048]


def test_topk_layout(lib):
    for T, L, k in itertools.product(TS, LS, KS):
        got = _check_tiling(B.DSA_OP_TOPK, T, L, 0, k)
        if T:
            _check_min(got, _topk_min(T, L, k), ("topk", T, L, k))


def test_forward_layout(lib):
    for T, L, H, k in itertools.product(TS, [100, 4097, 131072, 1 << 22], HS, KS):
        got = _check_tiling(B.DSA_OP_FORWARD, T, L, H, k)
        if not T:
            continue
        need = {"sel": T * k * 4}
        if T >= FUSED_MIN_T:
            # candidate lists of at least k + 320 entries per query token
            need.update({"fused.ckey": T * (k + 320) * 4, "fused.cpos": T * (k + 320) * 4})
        else:
            need["logits"] = T * ((L + 3) // 4 * 4) * 4
            need.update(_topk_min(T, L, k, "topk."))
        _check_min(got, need, ("forward", T, L, H, k))
        assert got.get("logits", 0) in (0, need.get("logits", 0)), "logits sized in full 64-bit arithmetic"


def test_forward_logits_past_32_bits(lib):
    # 2047 rows of 4M positions: 34 GB of logits, more than 32 bits can count
    T, L = 2047, 1 << 22
    got = _check_tiling(B.DSA_OP_FORWARD, T, L, 128, 2048)
    assert got["logits"] == T * L * 4 > 1 << 32


def test_attention_layouts(lib):
    for T, H, k in itertools.product(TS, HS, KS):
        got = _check_tiling(B.DSA_OP_ATTN, T, 0, H, k)
        if got:  # several splits: partials of every (token, split, head)
            _check_min(got, {"o": T * 2 * H * 512 * 2, "ml": T * 2 * H * 8}, ("attn", T, H, k))
    for T, L, H in itertools.product(TS, LS[:6], HS):
        got = _check_tiling(B.DSA_OP_DENSE_ATTN, T, L, H, 2048)
        if got:
            _check_min(got, {"o": T * 2 * H * 512 * 2, "ml": T * 2 * H * 8}, ("dense", T, L, H))


def test_backward_layout(lib):
    for T, H, k in itertools.product(TS, HS, KS):
        got = _check_tiling(B.DSA_OP_ATTN_BWD, T, 0, H, k)
        if not T:
            continue
        N = T * _cdiv(k, AT_TILE) * AT_TILE  # selected slots, each row padded to whole tiles
        _check_min(got, {"dsp": N * 2 * H * 2, "slot_grad": N * 576 * 2, "rows": N * 4, "cnt": T * 4,
                         "scatter.keys_b": N * 4, "scatter.vals_a": N * 4, "scatter.vals_b": N * 4,
                         "scatter.totals": 256 * 4}, ("bwd", T, H, k))


def test_kl_layouts(lib):
    for T, k in itertools.product(TS, KS):
        got = _check_tiling(B.DSA_OP_INDEXER_KL, T, 0, 0, k)
        if T:
            N = T * k
            _check_min(got, {"slot_dk": N * 128 * 2, "rows": N * 4, "scatter.keys_b": N * 4}, ("kl", T, k))
    for T, L, H in itertools.product(TS, LS, HS):
        got = _check_tiling(B.DSA_OP_KL_TARGET_DENSE, T, L, H, 0)
        if T:
            _check_min(got, {"ml": T * _cdiv(L, 2048) * H * 8}, ("kl dense", T, L, H))


def test_fused_selection_layout(lib):
    for T, L, k in itertools.product(TS, LS, KS):
        got = _check_tiling(B.DSA_OP_INDEXER_TOPK, T, L, 0, k)
        if T:
            _check_min(got, {"ckey": T * (k + 320) * 4, "cpos": T * (k + 320) * 4}, ("fused", T, L, k))


def test_projection_layout(lib):
    for T, d, (H_I, D_I) in itertools.product(TS, [256, 7168], [(64, 128), (64, 64), (4, 64)]):
        got = _check_tiling(B.DSA_OP_INDEXER_PROJ, T, d, H_I, D_I)
        if T:
            _check_min(got, {"part": T * (H_I * D_I + H_I + D_I) * 4}, ("proj", T, d, H_I, D_I))


def test_layout_rejects_bad_arguments(lib):
    f = lib.dsa_workspace_layout
    assert f(B.DSA_OP_TOPK, -1, 10, 0, 4, None, 0) == B.DSA_ERR_INVALID_ARG
    assert f(B.DSA_OP_TOPK, 4, 10, 0, 4, None, 3) == B.DSA_ERR_INVALID_ARG   # regions NULL, max_regions > 0
    assert f(B.DSA_OP_TOPK, 4, 10, 0, 4, None, -1) == B.DSA_ERR_INVALID_ARG
    assert f(99, 4, 10, 16, 4, None, 0) == 0   # no workspace for an unknown op (as dsa_workspace_bytes)
    assert f(B.DSA_OP_TOPK, 4, 10, 0, 4, None, 0) == 5   # the count, nothing written
