"""The C-ABI library loads, exports what include/dsa.h declares, and rejects
bad arguments before touching a device (these run without a GPU)."""

import ctypes
import os
import re

import pytest

from sparse_attention_long_03_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

FAKE = ctypes.c_void_p(1 << 20)  # non-null, 256-byte aligned; never dereferenced on a failing path


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(dsa_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libdsa.so not built")
    return B.lib()


def test_header_declares_the_entry_points():
    d = _declared()
    for name in B.EXPORTS:
        assert name in d, name
    assert set(d) == set(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert B.dsa_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5):
        assert B.dsa_status_str(code) != "unknown status"
    assert B.dsa_status_str(-99) == "unknown status"


def _q(T=4, Bn=1, max_len=100, seq=FAKE, pos=FAKE):
    return B.dsa_queries(T, Bn, seq, pos, max_len)


def _lay(cap=100):
    return B.contiguous_layout(cap)


def test_topk_validation(lib):
    f = lib.dsa_topk
    assert f(FAKE, 100, FAKE, 4, 100, 0, FAKE, FAKE, 1 << 30, None) == B.DSA_ERR_INVALID_ARG   # k = 0
    assert f(FAKE, 100, FAKE, 4, 100, 4096, FAKE, FAKE, 1 << 30, None) == B.DSA_ERR_UNSUPPORTED  # k > 2048
    big = 4 * 1024 * 1024  # the longest row the selection handles
    assert f(FAKE, big + 4, FAKE, 4, big + 1, 64, FAKE, FAKE, 1 << 40, None) == B.DSA_ERR_UNSUPPORTED
    assert f(FAKE, 100, FAKE, 4, 100, 64, FAKE, None, 0, None) == B.DSA_ERR_WORKSPACE
    assert f(FAKE, 100, FAKE, 4, 100, 64, FAKE, FAKE, 16, None) == B.DSA_ERR_WORKSPACE
    assert f(FAKE, 99, FAKE, 4, 100, 64, FAKE, FAKE, 1 << 30, None) == B.DSA_ERR_INVALID_ARG   # ld < max_len
    assert f(FAKE, 102, FAKE, 4, 100, 64, FAKE, FAKE, 1 << 30, None) == B.DSA_ERR_INVALID_ARG  # ld % 4
    assert f(None, 100, FAKE, 4, 100, 64, FAKE, FAKE, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    assert f(None, 100, None, 0, 100, 64, None, None, 0, None) == B.DSA_OK                    # T = 0: nothing to do


def test_indexer_validation(lib):
    f = lib.dsa_indexer_logits
    ok = dict(H_I=64, D_I=128)

    def call(q=None, lay=None, H_I=64, D_I=128, ptrs=(FAKE,) * 5, logits=FAKE, ld=100):
        q = q or _q()
        lay = lay or _lay()
        return f(ctypes.byref(q), ctypes.byref(lay), H_I, D_I, *ptrs, logits, ld, None)

    del ok
    assert call(H_I=8) == B.DSA_ERR_UNSUPPORTED
    assert call(D_I=96) == B.DSA_ERR_UNSUPPORTED
    assert call(H_I=0) == B.DSA_ERR_INVALID_ARG
    assert call(ld=98) == B.DSA_ERR_INVALID_ARG
    assert call(logits=None) == B.DSA_ERR_INVALID_ARG
    assert call(logits=ctypes.c_void_p((1 << 20) + 4)) == B.DSA_ERR_INVALID_ARG            # misaligned
    assert call(lay=_lay(cap=50)) == B.DSA_ERR_INVALID_ARG                                   # capacity < max_len
    assert call(q=_q(Bn=0)) == B.DSA_ERR_INVALID_ARG
    assert call(q=_q(seq=None)) == B.DSA_ERR_INVALID_ARG
    paged = B.dsa_kv_layout(1, 32, FAKE, 4, 10, 0)
    assert call(lay=paged) == B.DSA_ERR_UNSUPPORTED                                          # page size 32
    paged = B.dsa_kv_layout(1, 64, FAKE, 1, 10, 0)
    assert call(lay=paged) == B.DSA_ERR_INVALID_ARG                                          # 1 page < 100 tokens
    paged = B.dsa_kv_layout(1, 64, None, 4, 10, 0)
    assert call(lay=paged) == B.DSA_ERR_INVALID_ARG
    assert call(q=_q(T=0, seq=None, pos=None)) == B.DSA_OK


def test_attention_and_forward_validation(lib):
    q, lay = _q(), _lay()
    a = lib.dsa_sparse_mla_attn
    assert a(ctypes.byref(q), ctypes.byref(lay), 48, FAKE, FAKE, FAKE, 64, 0.1, FAKE, None, FAKE, 1 << 30, None) == B.DSA_ERR_UNSUPPORTED
    assert a(ctypes.byref(q), ctypes.byref(lay), 128, FAKE, FAKE, FAKE, 4096, 0.1, FAKE, None, FAKE, 1 << 30, None) == B.DSA_ERR_UNSUPPORTED
    assert a(ctypes.byref(q), ctypes.byref(lay), 128, FAKE, FAKE, FAKE, 64, 0.0, FAKE, None, FAKE, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    assert a(ctypes.byref(q), ctypes.byref(lay), 128, FAKE, FAKE, FAKE, 64, float("nan"), FAKE, None, FAKE, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    assert a(ctypes.byref(q), ctypes.byref(lay), 128, None, FAKE, FAKE, 64, 0.1, FAKE, None, FAKE, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    # a split-K shape needs a workspace
    qq = _q(T=2)
    need = B.dsa_workspace_bytes(B.DSA_OP_ATTN, 2, 100, 128, 2048)
    assert need > 0
    assert a(ctypes.byref(qq), ctypes.byref(lay), 128, FAKE, FAKE, FAKE, 2048, 0.1, FAKE, None, None, 0, None) == B.DSA_ERR_WORKSPACE
    assert a(ctypes.byref(qq), ctypes.byref(lay), 128, FAKE, FAKE, FAKE, 2048, 0.1, FAKE, None, FAKE, need - 1, None) == B.DSA_ERR_WORKSPACE
    fw = lib.dsa_forward
    args = [64, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 2048, 0.1, FAKE, None, None]
    need_f = B.dsa_workspace_bytes(B.DSA_OP_FORWARD, 4, 100, 128, 2048)
    assert fw(ctypes.byref(q), ctypes.byref(lay), *args, FAKE, need_f - 1, None) == B.DSA_ERR_WORKSPACE
    assert fw(ctypes.byref(q), ctypes.byref(lay), *args, None, 0, None) == B.DSA_ERR_WORKSPACE
    bad = list(args)
    bad[0] = 5
    assert fw(ctypes.byref(q), ctypes.byref(lay), *bad, FAKE, need_f, None) == B.DSA_ERR_UNSUPPORTED


def test_workspace_sizes_are_monotone(lib):
    a = B.dsa_workspace_bytes(B.DSA_OP_FORWARD, 16, 131072, 128, 2048)
    b = B.dsa_workspace_bytes(B.DSA_OP_FORWARD, 16, 65536, 128, 2048)
    assert a > b > 0
    assert B.dsa_workspace_bytes(B.DSA_OP_TOPK, 16, 131072, 0, 2048) >= 2 * 16 * 131072 * 4
    assert B.dsa_workspace_bytes(99, 16, 131072, 128, 2048) == 0
    assert B.dsa_workspace_bytes(B.DSA_OP_ATTN, -1, 10, 128, 2048) == 0


def test_fused_indexer_topk_validation(lib):
    f = lib.dsa_indexer_topk
    q, lay = _q(T=16), _lay()

    def call(k=256, ws=FAKE, nbytes=None, H_I=64, q_=None, idx=FAKE):
        nbytes = 8 * 16 * (k + 320) if nbytes is None else nbytes
        return f(ctypes.byref(q_ or q), ctypes.byref(lay), H_I, 128, FAKE, FAKE, FAKE, FAKE, FAKE, k, idx, ws, nbytes,
                 None)

    assert call(k=0) == B.DSA_ERR_INVALID_ARG
    assert call(k=4096) == B.DSA_ERR_UNSUPPORTED
    assert call(H_I=8) == B.DSA_ERR_UNSUPPORTED
    assert call(idx=None) == B.DSA_ERR_INVALID_ARG
    assert call(ws=None) == B.DSA_ERR_WORKSPACE
    assert call(nbytes=8 * 16 * (256 + 320) - 1) == B.DSA_ERR_WORKSPACE      # fewer than k + 320 slots
    assert call(ws=ctypes.c_void_p((1 << 20) + 64)) == B.DSA_ERR_WORKSPACE   # misaligned
    assert call(q_=_q(T=0, seq=None, pos=None)) == B.DSA_OK
    # the preferred size holds every position of the row plus 4 tiles (no
    # compaction), and at least k + 320 slots
    pref = B.dsa_workspace_bytes(B.DSA_OP_INDEXER_TOPK, 16, 100, 0, 256)
    assert pref == 8 * 16 * (256 + 320)
    assert B.dsa_workspace_bytes(B.DSA_OP_INDEXER_TOPK, 16, 5000, 0, 256) == 8 * 16 * (5056 + 256)
    assert B.dsa_workspace_bytes(B.DSA_OP_INDEXER_TOPK, 16, 1 << 20, 0, 2048) == 8 * 16 * 12288


def test_fused_preferred_workspace_is_accepted(lib):
    # The call takes the list capacity as the largest multiple of 64 slots that
    # the workspace holds per token and needs at least k + 320; the preferred
    # size must therefore be a whole number of 64-slot tiles per token.  (A
    # k + 320 minimum that is not a multiple of 64, e.g. k = 1 on a short row,
    # once gave a preferred size the call rejected.)
    for T in (1, 16, 55):
        for max_len in (1, 55, 64, 100, 4095, 20000, 1 << 20):
            for k in (1, 7, 32, 64, 100, 256, 300, 2047, 2048):
                pref = B.dsa_workspace_bytes(B.DSA_OP_INDEXER_TOPK, T, max_len, 0, k)
                assert pref % (8 * T * 64) == 0, (T, max_len, k, pref)
                cap = pref // (8 * T)
                assert k + 320 <= cap <= 12288, (T, max_len, k, cap)


def test_forward_workspace_switches_to_fused_selection(lib):
    # below 2048 query tokens the logits are stored; from 2048 on they are not
    small = B.dsa_workspace_bytes(B.DSA_OP_FORWARD, 2047, 65536, 128, 2048)
    big = B.dsa_workspace_bytes(B.DSA_OP_FORWARD, 2048, 65536, 128, 2048)
    assert small >= 2047 * 65536 * 4
    assert big < 2048 * 65536 * 4


def test_cache_write_validation(lib):
    f = lib.dsa_cache_write
    q, lay = _q(), _lay()
    assert f(ctypes.byref(q), ctypes.byref(lay), 96, FAKE, None, FAKE, FAKE, None, None) == B.DSA_ERR_UNSUPPORTED
    assert f(ctypes.byref(q), ctypes.byref(lay), 0, FAKE, None, FAKE, FAKE, None, None) == B.DSA_ERR_INVALID_ARG
    assert f(ctypes.byref(q), ctypes.byref(lay), 128, FAKE, FAKE, FAKE, FAKE, None, None) == B.DSA_ERR_INVALID_ARG
    assert f(ctypes.byref(q), ctypes.byref(lay), 128, None, None, FAKE, FAKE, None, None) == B.DSA_ERR_INVALID_ARG
    assert f(ctypes.byref(q), ctypes.byref(_lay(cap=50)), 128, FAKE, None, FAKE, FAKE, None, None) == B.DSA_ERR_INVALID_ARG
    q0 = _q(T=0, seq=None, pos=None)
    assert f(ctypes.byref(q0), ctypes.byref(lay), 128, None, None, None, None, None, None) == B.DSA_OK


def test_masked_dense_validation(lib):
    f = lib.dsa_masked_dense_attn
    q, lay = _q(max_len=100), _lay()
    assert f(ctypes.byref(q), ctypes.byref(lay), 48, FAKE, FAKE, FAKE, 64, 0.1, FAKE, None, FAKE, 1 << 30, None) == B.DSA_ERR_UNSUPPORTED
    big = _q(max_len=20000)
    assert f(ctypes.byref(big), ctypes.byref(_lay(cap=20000)), 128, FAKE, FAKE, FAKE, 64, 0.1, FAKE, None, FAKE, 1 << 30, None) == B.DSA_ERR_UNSUPPORTED
    need = B.dsa_workspace_bytes(B.DSA_OP_DENSE_ATTN, 4, 16384, 128, 2048)
    assert need > 0
    q16 = _q(max_len=16384)
    assert f(ctypes.byref(q16), ctypes.byref(_lay(cap=16384)), 128, FAKE, FAKE, FAKE, 2048, 0.1, FAKE, None, FAKE, need - 1, None) == B.DSA_ERR_WORKSPACE


def test_attention_backward_validation(lib):
    f = lib.dsa_sparse_mla_attn_bwd
    q, lay = _q(T=4), _lay()
    need = B.dsa_workspace_bytes(B.DSA_OP_ATTN_BWD, 4, 100, 128, 2048)
    # per token: P / dS rows, one bf16 gradient row per slot, four sort words per slot
    assert need >= 4 * 2048 * (4 * 128 + 1152 + 16)

    def call(H=128, k=2048, scale=0.1, ptrs=None, ws=FAKE, nbytes=need, q_=None, lay_=None):
        p = list(ptrs or (FAKE,) * 8)  # q, kv, idx, out, lse, d_out, dq, dkv
        return f(ctypes.byref(q_ or q), ctypes.byref(lay_ or lay), H, p[0], p[1], p[2], k, scale, p[3], p[4], p[5],
                 p[6], p[7], ws, nbytes, None)

    assert call(H=48) == B.DSA_ERR_UNSUPPORTED
    assert call(k=4096) == B.DSA_ERR_UNSUPPORTED
    assert call(scale=0.0) == B.DSA_ERR_INVALID_ARG
    for i in range(8):
        ptrs = [FAKE] * 8
        ptrs[i] = None
        assert call(ptrs=ptrs) == B.DSA_ERR_INVALID_ARG, i
    mis = [FAKE] * 8
    mis[7] = ctypes.c_void_p((1 << 20) + 4)  # dkv misaligned
    assert call(ptrs=mis) == B.DSA_ERR_INVALID_ARG
    assert call(ws=None) == B.DSA_ERR_WORKSPACE
    assert call(nbytes=need - 1) == B.DSA_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p((1 << 20) + 64)) == B.DSA_ERR_WORKSPACE
    # caches of 2^31 rows or more are not handled (row ids are 31-bit)
    assert call(lay_=B.contiguous_layout(1 << 31)) == B.DSA_ERR_UNSUPPORTED
    assert call(q_=_q(T=0, seq=None, pos=None), ptrs=[None] * 8, ws=None, nbytes=0) == B.DSA_OK
    assert B.dsa_workspace_bytes(B.DSA_OP_ATTN_BWD, 0, 100, 128, 2048) == 0
    # the two steps check their own arguments
    fdq, fdkv = lib.dsa_sparse_mla_attn_bwd_dq, lib.dsa_sparse_mla_attn_bwd_dkv
    a = [FAKE] * 7  # q, kv, idx, out, lse, d_out, dq
    assert fdq(ctypes.byref(q), ctypes.byref(lay), 128, a[0], None, a[2], 2048, 0.1, a[3], a[4], a[5], a[6], FAKE,
               need, None) == B.DSA_ERR_INVALID_ARG
    assert fdq(ctypes.byref(q), ctypes.byref(lay), 128, a[0], a[1], a[2], 2048, 0.1, a[3], a[4], a[5], None, FAKE,
               need, None) == B.DSA_ERR_INVALID_ARG
    assert fdq(ctypes.byref(q), ctypes.byref(lay), 128, a[0], a[1], a[2], 2048, 0.1, a[3], a[4], a[5], a[6], FAKE,
               need - 1, None) == B.DSA_ERR_WORKSPACE
    assert fdkv(ctypes.byref(q), ctypes.byref(lay), 128, FAKE, 2048, FAKE, None, FAKE, need, None) == B.DSA_ERR_INVALID_ARG
    assert fdkv(ctypes.byref(q), ctypes.byref(lay), 128, None, 2048, FAKE, FAKE, FAKE, need, None) == B.DSA_ERR_INVALID_ARG
    assert fdkv(ctypes.byref(q), ctypes.byref(lay), 48, FAKE, 2048, FAKE, FAKE, FAKE, need, None) == B.DSA_ERR_UNSUPPORTED
    assert fdkv(ctypes.byref(q), ctypes.byref(lay), 128, FAKE, 2048, FAKE, FAKE, FAKE, need - 1, None) == B.DSA_ERR_WORKSPACE
    assert B.dsa_workspace_bytes(B.DSA_OP_ATTN_BWD, 8, 100, 128, 2048) > need


def test_indexer_kl_validation(lib):
    q, lay = _q(T=4), _lay()
    ft, fk = lib.dsa_indexer_kl_target, lib.dsa_indexer_kl
    # target: as the attention's arguments, plus lse
    assert ft(ctypes.byref(q), ctypes.byref(lay), 48, FAKE, FAKE, FAKE, 64, 0.1, FAKE, FAKE, None) == B.DSA_ERR_UNSUPPORTED
    assert ft(ctypes.byref(q), ctypes.byref(lay), 128, FAKE, FAKE, FAKE, 64, 0.1, None, FAKE, None) == B.DSA_ERR_INVALID_ARG
    assert ft(ctypes.byref(q), ctypes.byref(lay), 128, FAKE, FAKE, FAKE, 64, 0.1, FAKE, None, None) == B.DSA_ERR_INVALID_ARG
    assert ft(ctypes.byref(q), ctypes.byref(lay), 128, FAKE, FAKE, FAKE, 4096, 0.1, FAKE, FAKE, None) == B.DSA_ERR_UNSUPPORTED
    need = B.dsa_workspace_bytes(B.DSA_OP_INDEXER_KL, 4, 100, 0, 2048)
    assert need >= 4 * 2048 * (128 * 2 + 4)

    def call(H_I=64, D_I=128, k=2048, ptrs=None, ws=FAKE, nbytes=need, q_=None):
        p = list(ptrs or (FAKE,) * 11)  # q8, qs, w, k8, ks, idx, target, loss, dq, dw, dk
        return fk(ctypes.byref(q_ or q), ctypes.byref(lay), H_I, D_I, p[0], p[1], p[2], p[3], p[4], p[5], k, p[6],
                  p[7], p[8], p[9], p[10], ws, nbytes, None)

    assert call(H_I=4) == B.DSA_ERR_UNSUPPORTED      # the KL kernel is built for 64 x 128
    assert call(D_I=64) == B.DSA_ERR_UNSUPPORTED
    assert call(k=0) == B.DSA_ERR_INVALID_ARG
    assert call(k=4096) == B.DSA_ERR_UNSUPPORTED
    for i in range(5, 11):
        ptrs = [FAKE] * 11
        ptrs[i] = None
        assert call(ptrs=ptrs) == B.DSA_ERR_INVALID_ARG, i
    assert call(ws=None) == B.DSA_ERR_WORKSPACE
    assert call(nbytes=need - 1) == B.DSA_ERR_WORKSPACE
    assert call(q_=_q(T=0, seq=None, pos=None), ptrs=[None] * 11, ws=None, nbytes=0) == B.DSA_OK


def test_forward_noalloc_validation(lib):
    """The no-allocation forward checks its arguments like dsa_forward and
    rejects a request larger than its static scratch before any HIP call."""
    f = lib.dsa_forward_noalloc
    lay = _lay(1 << 17)

    def call(q_=None, H_I=64, H=128, k=2048, out=FAKE, **kw):
        q_ = q_ or _q(T=4, max_len=1000)
        return f(ctypes.byref(q_), ctypes.byref(lay), H_I, 128, FAKE, FAKE, FAKE, FAKE, FAKE, H, FAKE, FAKE, k, 0.04,
                 out, None, None, None)

    assert call(H_I=8) == B.DSA_ERR_UNSUPPORTED
    assert call(k=0) == B.DSA_ERR_INVALID_ARG
    assert call(out=None) == B.DSA_ERR_INVALID_ARG
    assert call(q_=_q(T=0, seq=None, pos=None)) == B.DSA_OK
    # 64 decode queries of 128K positions need more than the 64 MiB scratch
    assert B.dsa_workspace_bytes(B.DSA_OP_FORWARD, 64, 1 << 17, 128, 2048) > (64 << 20)
    assert call(q_=_q(T=64, max_len=1 << 17)) == B.DSA_ERR_SCRATCH_LIMIT
    assert "static scratch" in B.dsa_status_str(B.DSA_ERR_SCRATCH_LIMIT)


def test_indexer_project_validation(lib):
    f = lib.dsa_indexer_project

    def call(T=4, d=512, H_I=64, D_I=128, wk=FAKE, kn=FAKE, ws=FAKE, nbytes=0, h=FAKE):
        return f(T, d, H_I, D_I, h, FAKE, FAKE, wk, FAKE, FAKE, FAKE, kn, ws, nbytes, None)

    need = B.dsa_workspace_bytes(B.DSA_OP_INDEXER_PROJ, 4, 512, 64, 128)
    assert need >= 4 * (64 * 128 + 64 + 128) * 4
    assert call(d=500) == B.DSA_ERR_UNSUPPORTED            # not a multiple of 64
    assert call(H_I=8) == B.DSA_ERR_UNSUPPORTED
    assert call(wk=None) == B.DSA_ERR_INVALID_ARG            # key weights without a key output
    assert call(kn=None) == B.DSA_ERR_INVALID_ARG
    assert call(h=None) == B.DSA_ERR_INVALID_ARG
    assert call(nbytes=need - 1) == B.DSA_ERR_WORKSPACE
    assert call(ws=None, nbytes=need) == B.DSA_ERR_WORKSPACE
    assert call(T=0) == B.DSA_OK
    assert B.dsa_workspace_bytes(B.DSA_OP_INDEXER_PROJ, 4, 500, 64, 128) == 0


def test_kl_target_dense_validation(lib):
    f = lib.dsa_indexer_kl_target_dense
    lay = _lay(5000)

    def call(q_=None, H=128, ld=5000, target=FAKE, ws=FAKE, nbytes=0, scale=0.04):
        q_ = q_ or _q(T=4, max_len=5000)
        return f(ctypes.byref(q_), ctypes.byref(lay), H, FAKE, FAKE, scale, target, ld, None, ws, nbytes, None)

    need = B.dsa_workspace_bytes(B.DSA_OP_KL_TARGET_DENSE, 4, 5000, 128, 0)
    assert need == 256 * ((4 * 3 * 128 * 8 + 255) // 256)   # 3 chunks of 2048 positions
    assert call(H=24) == B.DSA_ERR_UNSUPPORTED
    assert call(scale=0.0) == B.DSA_ERR_INVALID_ARG
    assert call(ld=4999) == B.DSA_ERR_INVALID_ARG
    assert call(target=None) == B.DSA_ERR_INVALID_ARG
    assert call(nbytes=need - 1) == B.DSA_ERR_WORKSPACE
    assert call(q_=_q(T=0, seq=None, pos=None)) == B.DSA_OK



def test_kl_target_dense_lse_validation(lib):
    f = lib.dsa_indexer_kl_target_dense_lse
    lay = _lay(5000)

    def call(q_=None, H=128, ld=5000, lse=FAKE, target=FAKE, scale=0.04):
        q_ = q_ or _q(T=4, max_len=5000)
        return f(ctypes.byref(q_), ctypes.byref(lay), H, FAKE, FAKE, scale, lse, target, ld, None)

    assert call(H=24) == B.DSA_ERR_UNSUPPORTED
    assert call(scale=0.0) == B.DSA_ERR_INVALID_ARG
    assert call(ld=4999) == B.DSA_ERR_INVALID_ARG
    assert call(lse=None) == B.DSA_ERR_INVALID_ARG
    assert call(lse=ctypes.c_void_p((1 << 20) + 2)) == B.DSA_ERR_INVALID_ARG   # misaligned
    assert call(target=None) == B.DSA_ERR_INVALID_ARG
    assert call(q_=_q(T=0, seq=None, pos=None)) == B.DSA_OK