"""The streaming selection rule of the fused prefill kernel (indexer_topk.hip),
modelled on the CPU and checked against a stable top-k.

"DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
Consideration (DSA)", part (2): each query keeps the k keys with the highest
index scores; equal scores go to the lowest position first.

The kernel never holds a whole row: per query it appends (order key, position)
to a list whenever the key is above a threshold tau, and when the list could
overflow it keeps only the k best entries (in list order: those above the
k-th largest key K*, then the first entries equal to K*) and sets tau = K*.
This test replays that rule with the kernel's tile size (64 keys), check
interval (every 4 tiles), capacity bound and final selection, on rows that
force many compactions, and requires the result to equal the stable top-k.
It pins the rule, not the GPU code; the GPU tests compare the kernel with the
separate logits + top-k calls and with the oracle.
"""

import numpy as np
import pytest

TILE = 64       # keys per tile
AHEAD = 4       # tiles between two capacity checks
MARGIN = (AHEAD + 1) * TILE  # the smallest capacity is k + MARGIN


def _kth(keys, k):
    """K*, the k-th largest key of the list, and how many entries equal to
    K* are kept (k minus the number above it)."""
    kstar = np.sort(keys)[::-1][k - 1]
    return kstar, k - int(np.count_nonzero(keys > kstar))


def _keep(keys, pos, kstar, ties):
    """List order: entries above K*, and the first `ties` entries equal to K*."""
    eq = keys == kstar
    first_eq = eq & (np.cumsum(eq) <= ties)
    m = (keys > kstar) | first_eq
    return keys[m], pos[m]


def stream_select(keys, k, cap):
    assert cap >= k + MARGIN
    n = keys.shape[0]
    lk = np.zeros(0, dtype=np.int64)
    lp = np.zeros(0, dtype=np.int64)
    tau = 0  # every order key is above 0
    ntiles = -(-n // TILE)
    for g in range(0, max(ntiles, 1), AHEAD):
        for t in range(g, g + AHEAD):
            s = np.arange(t * TILE, min((t + 1) * TILE, n))
            if s.size == 0:
                continue
            take = keys[s] > tau
            lk = np.concatenate([lk, keys[s][take]])
            lp = np.concatenate([lp, s[take]])
        assert lk.size <= cap, "the list overflowed its capacity"
        if lk.size > cap - AHEAD * TILE:
            kstar, ties = _kth(lk, k)
            lk, lp = _keep(lk, lp, kstar, ties)
            assert lk.size == k
            tau = int(kstar)
    if lk.size <= k:
        return np.concatenate([lp, -np.ones(k - lp.size, dtype=np.int64)])
    kstar, ties = _kth(lk, k)
    return _keep(lk, lp, kstar, ties)[1]


def stable_topk(keys, k):
    """Positions of the k largest keys, lowest position first among equals,
    in ascending position order, padded with -1."""
    n = keys.shape[0]
    order = np.lexsort((np.arange(n), -keys))[:k]
    sel = np.sort(order)
    return np.concatenate([sel, -np.ones(k - sel.size, dtype=np.int64)])


def _rows(rng, n):
    yield "uniform", rng.integers(1, 1 << 32, size=n, dtype=np.int64)
    yield "five_values", rng.choice(np.array([7, 8, 9, 1 << 20, 1 << 31], dtype=np.int64), size=n)
    yield "increasing", np.arange(1, n + 1, dtype=np.int64) * 3
    yield "decreasing", np.arange(n, 0, -1, dtype=np.int64) * 3
    yield "constant", np.full(n, 12345, dtype=np.int64)
    # late large keys: every compaction's threshold is overtaken later
    yield "ramp_with_noise", (np.arange(n, dtype=np.int64) // 50) * 1000 + rng.integers(1, 900, size=n)
    # a few consecutive values: later keys one above K* must still enter
    yield "consecutive_values", rng.integers(1, 6, size=n).astype(np.int64)
    half = n // 2
    yield "second_half_one_higher", np.concatenate([rng.integers(10, 12, size=half),
                                                   rng.integers(11, 13, size=n - half)]).astype(np.int64)


@pytest.mark.parametrize("k", [1, 7, 64, 100])
@pytest.mark.parametrize("extra", [0, 64, 512])
def test_streaming_rule_equals_stable_topk(k, extra):
    rng = np.random.default_rng(1000 * k + extra)
    cap = k + MARGIN + extra
    for n in (1, k - 1 if k > 1 else 2, k, k + 1, 300, 1500, 3001):
        for name, keys in _rows(rng, n):
            got = stream_select(keys, k, cap)
            want = stable_topk(keys, k)
            assert np.array_equal(got, want), f"{name} n={n} k={k} cap={cap}"


def test_a_dropped_entry_never_returns():
    """The threshold only rises: after a compaction, no key at or below K*
    can enter, and the final answer still equals the stable top-k."""
    rng = np.random.default_rng(5)
    k, cap = 16, 16 + MARGIN
    keys = rng.integers(1, 50, size=5000).astype(np.int64)  # heavy ties
    assert np.array_equal(stream_select(keys, k, cap), stable_topk(keys, k))
