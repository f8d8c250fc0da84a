"""Convenience wrapper: run the DSA path on a set of GPU-resident inputs.

Builds the C descriptors once, owns the outputs and the workspace, and calls
the C entry points through :mod:`.binding`.  No arithmetic happens here.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import binding as B
from .inputs import DSAInputs


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


class DSAPath:
    def __init__(self, x: DSAInputs):
        cfg = x.cfg
        self.x = x
        self.cfg = cfg
        self.T = x.T
        self.q = B.queries(x.seq_id, x.pos, cfg.B, x.max_len)
        if x.block_table is not None:
            self.layout = B.paged_layout(x.block_table, x.kv.shape[0], cfg.page_size)
        else:
            self.layout = B.contiguous_layout(x.kv.shape[1])
        self.ld = round_up(max(x.max_len, 1), 4)
        self.valid_len = (x.pos + 1).to(torch.int32)
        dev = x.q.device
        self.dev = dev
        self.out = torch.empty((self.T, cfg.H, cfg.d_v), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((self.T, cfg.H), dtype=torch.float32, device=dev)
        self.idx = torch.empty((self.T, cfg.k), dtype=torch.int32, device=dev)
        self._ws = {}

    def ws(self, op: int) -> torch.Tensor:
        if op not in self._ws:
            n = B.dsa_workspace_bytes(op, self.T, self.x.max_len, self.cfg.H, self.cfg.k)
            self._ws[op] = B.workspace(n, self.dev)
        return self._ws[op]

    def new_logits(self) -> torch.Tensor:
        return torch.empty((self.T, self.ld), dtype=torch.float32, device=self.dev)

    def indexer(self, logits: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        x, c = self.x, self.cfg
        if logits is None:
            logits = self.new_logits()
        B.dsa_indexer_logits(self.q, self.layout, c.H_I, c.D_I, x.iq8, x.iqs, x.iw, x.ik8, x.iks, logits, stream)
        return logits

    def topk(self, logits: torch.Tensor, idx: Optional[torch.Tensor] = None, valid_len=None, k=None,
             stream=None) -> torch.Tensor:
        k = self.cfg.k if k is None else k
        if idx is None:
            idx = torch.empty((logits.shape[0], k), dtype=torch.int32, device=self.dev)
        vl = self.valid_len if valid_len is None else valid_len
        ws = B.workspace(B.dsa_workspace_bytes(B.DSA_OP_TOPK, logits.shape[0], logits.shape[1], 0, k), self.dev)
        B.dsa_topk(logits, vl, logits.shape[1], k, idx, ws, stream)
        return idx

    def indexer_topk(self, idx: Optional[torch.Tensor] = None, k=None, ws_bytes=None, stream=None) -> torch.Tensor:
        """Fused indexer + selection (no logits); `ws_bytes` overrides the
        preferred workspace size (a smaller one compacts the candidate lists
        more often, with the same result)."""
        x, c = self.x, self.cfg
        k = c.k if k is None else k
        if idx is None:
            idx = torch.empty((self.T, k), dtype=torch.int32, device=self.dev)
        n = B.dsa_workspace_bytes(B.DSA_OP_INDEXER_TOPK, self.T, x.max_len, 0, k) if ws_bytes is None else ws_bytes
        ws = B.workspace(n, self.dev)
        B.dsa_indexer_topk(self.q, self.layout, c.H_I, c.D_I, x.iq8, x.iqs, x.iw, x.ik8, x.iks, k, idx, ws, stream)
        return idx

    def attn(self, idx: torch.Tensor, stream=None):
        x, c = self.x, self.cfg
        B.dsa_sparse_mla_attn(self.q, self.layout, c.H, x.q, x.kv, idx, idx.shape[1], c.scale, self.out, self.lse,
                              self.ws(B.DSA_OP_ATTN), stream)
        return self.out, self.lse

    def attn_bwd(self, idx: torch.Tensor, d_out: torch.Tensor, out=None, lse=None, dkv=None, stream=None):
        """Backward of the sparse attention for the selection `idx`, given the
        forward's out / lse (those of the last attn() call by default).
        Returns (dq float32[T, H, 576], dkv float32 in the cache's layout);
        the gradients are added into `dkv` when one is given."""
        x, c = self.x, self.cfg
        out = self.out if out is None else out
        lse = self.lse if lse is None else lse
        dq = torch.empty((self.T, c.H, c.D), dtype=torch.float32, device=self.dev)
        if dkv is None:
            dkv = torch.zeros(x.kv.shape, dtype=torch.float32, device=self.dev)
        k = idx.shape[1]
        n = B.dsa_workspace_bytes(B.DSA_OP_ATTN_BWD, self.T, x.max_len, c.H, k)
        if ("bwd", n) not in self._ws:
            self._ws[("bwd", n)] = B.workspace(n, self.dev)
        B.dsa_sparse_mla_attn_bwd(self.q, self.layout, c.H, x.q, x.kv, idx, k, c.scale, out, lse, d_out, dq, dkv,
                                  self._ws[("bwd", n)], stream)
        return dq, dkv

    def attn_bwd_steps(self, idx: torch.Tensor, d_out: torch.Tensor, dkv: torch.Tensor, stream=None):
        """The same backward as attn_bwd, as its two steps (dq, then dkv)."""
        x, c = self.x, self.cfg
        dq = torch.empty((self.T, c.H, c.D), dtype=torch.float32, device=self.dev)
        k = idx.shape[1]
        n = B.dsa_workspace_bytes(B.DSA_OP_ATTN_BWD, self.T, x.max_len, c.H, k)
        if ("bwd", n) not in self._ws:
            self._ws[("bwd", n)] = B.workspace(n, self.dev)
        ws = self._ws[("bwd", n)]
        B.dsa_sparse_mla_attn_bwd_dq(self.q, self.layout, c.H, x.q, x.kv, idx, k, c.scale, self.out, self.lse, d_out,
                                     dq, ws, stream)
        B.dsa_sparse_mla_attn_bwd_dkv(self.q, self.layout, c.H, x.q, k, d_out, dkv, ws, stream)
        return dq, dkv

    def kl_target(self, idx: torch.Tensor, lse=None, stream=None) -> torch.Tensor:
        """Head-mean attention probabilities of the selected entries (the
        indexer's KL target), from the forward's lse (the last attn() call's
        by default)."""
        x, c = self.x, self.cfg
        lse = self.lse if lse is None else lse
        target = torch.empty(idx.shape, dtype=torch.float32, device=self.dev)
        B.dsa_indexer_kl_target(self.q, self.layout, c.H, x.q, x.kv, idx, idx.shape[1], c.scale, lse, target, stream)
        return target

    def indexer_kl(self, idx: torch.Tensor, target: torch.Tensor, dk=None, stream=None):
        """KL loss of the indexer against `target` and its gradients:
        (loss [T], dq [T, H_I, D_I], dw [T, H_I], dk in the key cache's
        layout, added into `dk` when one is given)."""
        x, c = self.x, self.cfg
        k = idx.shape[1]
        loss = torch.empty((self.T,), dtype=torch.float32, device=self.dev)
        dq = torch.empty((self.T, c.H_I, c.D_I), dtype=torch.float32, device=self.dev)
        dw = torch.empty((self.T, c.H_I), dtype=torch.float32, device=self.dev)
        if dk is None:
            dk = torch.zeros(x.ik8.shape, dtype=torch.float32, device=self.dev)
        n = B.dsa_workspace_bytes(B.DSA_OP_INDEXER_KL, self.T, x.max_len, 0, k)
        if ("kl", n) not in self._ws:
            self._ws[("kl", n)] = B.workspace(n, self.dev)
        B.dsa_indexer_kl(self.q, self.layout, c.H_I, c.D_I, x.iq8, x.iqs, x.iw, x.ik8, x.iks, idx, k, target, loss, dq,
                         dw, dk, self._ws[("kl", n)], stream)
        return loss, dq, dw, dk

    def dense_attn(self, idx: torch.Tensor, out=None, lse=None, stream=None):
        """The masked dense variant over the same selection (contiguous rows)."""
        x, c = self.x, self.cfg
        out = torch.empty_like(self.out) if out is None else out
        lse = torch.empty_like(self.lse) if lse is None else lse
        n = B.dsa_workspace_bytes(B.DSA_OP_DENSE_ATTN, self.T, x.max_len, c.H, idx.shape[1])
        if ("dense", n) not in self._ws:
            self._ws[("dense", n)] = B.workspace(n, self.dev)
        B.dsa_masked_dense_attn(self.q, self.layout, c.H, x.q, x.kv, idx, idx.shape[1], c.scale, out, lse,
                                self._ws[("dense", n)], stream)
        return out, lse

    def forward(self, stream=None):
        x, c = self.x, self.cfg
        B.dsa_forward(self.q, self.layout, c.H_I, c.D_I, x.iq8, x.iqs, x.iw, x.ik8, x.iks, c.H, x.q, x.kv, c.k,
                      c.scale, self.out, self.lse, self.idx, self.ws(B.DSA_OP_FORWARD), stream)
        return self.out, self.lse, self.idx
