"""Seeded synthetic inputs for the DSA hot path.

This module only draws numbers and lays them out (FP8 / bf16 storage, page
tables, planted keys).  It holds none of the method's arithmetic, so both the
GPU library's tests and the CPU oracle's tests may use it.

Workload shapes follow the DeepSeek-V3.2-Exp DSA articles: an FP8 lightning
indexer with few heads, top-k = 2048, and MLA in MQA mode with a 576-wide
latent row (512 no-rope + 64 rope) shared by 128 query heads, served from
64-token pages.  Every tensor has its own seed so that any one of them can be
regenerated alone.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

FP8_MAX = 448.0
_MIN_SCALE = 2.0 ** -126

# tensor ids used to derive per-tensor seeds
_T_IQ, _T_IK, _T_W, _T_Q, _T_KV, _T_LEN, _T_PAGES, _T_PLANT, _T_NQ, _T_DOUT, _T_SEL, _T_DIST = range(12)


@dataclasses.dataclass(frozen=True)
class DSAConfig:
    name: str
    kind: str                    # "decode" | "prefill" | "ragged"
    B: int                       # sequences
    L: int                       # context length (max length for "ragged")
    H_I: int                     # indexer heads
    D_I: int                     # indexer head dim
    H: int                       # attention query heads
    k: int                       # tokens kept per query
    D: int = 576                 # latent row width (key)
    d_v: int = 512               # value width (leading part of the row)
    attn_std: float = 1.0        # std of attention q and latent kv entries
    scale: float = 1.0 / 24.0    # softmax scale, 1/sqrt(576)
    paged: bool = False
    page_size: int = 64
    planted_frac: float = 0.0    # fraction of planted far keys (long-context decode)
    min_len: int = 0             # "ragged": lengths uniform in [min_len, L]
    queries_per_seq: int = 1     # decode: trailing query tokens per sequence
    seed: int = 0


CONFIGS = {
    # tiny step, oracle in seconds
    "tiny": DSAConfig("tiny", "decode", B=1, L=4096, H_I=4, D_I=64, H=16, k=256,
                      attn_std=1.0 / 24.0, queries_per_seq=16, seed=1000),
    # batched decode, 32K context
    "decode32k": DSAConfig("decode32k", "decode", B=64, L=32768, H_I=64, D_I=128, H=128, k=2048, seed=1001),
    # long-context decode, 128K context with planted far keys
    "decode128k": DSAConfig("decode128k", "decode", B=16, L=131072, H_I=64, D_I=128, H=128, k=2048,
                            planted_frac=0.02, seed=1002),
    # prefill, 64K tokens all causal queries
    "prefill64k": DSAConfig("prefill64k", "prefill", B=1, L=65536, H_I=64, D_I=128, H=128, k=2048, seed=1003),
    # training-step backward: the last 4096 tokens of a 64K-token sequence as
    # queries (each keeps a full k = 2048 selection)
    "train64k_chunk4k": DSAConfig("train64k_chunk4k", "decode", B=1, L=65536, H_I=64, D_I=128, H=128, k=2048,
                                  queries_per_seq=4096, seed=1005),
    # ragged paged batch
    "ragged_paged": DSAConfig("ragged_paged", "ragged", B=128, L=131072, H_I=64, D_I=128, H=128, k=2048,
                              paged=True, min_len=2048, seed=1004),
}


def scaled(cfg: DSAConfig, **kw) -> DSAConfig:
    """A copy of a config with some fields replaced (smaller test variants)."""
    return dataclasses.replace(cfg, **kw)


def _gen(cfg_seed: int, tensor_id: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(cfg_seed * 1000003 + tensor_id * 7919 + 17)
    return g


def quantize_e4m3fn(x: torch.Tensor):
    """Per-token FP8 storage: one float32 scale per leading index.

    scale = max(amax / 448, 2^-126) over the trailing dims; the code is the
    e4m3fn rounding (to nearest even) of x / scale clamped to +-448.
    Returns (uint8 codes with x's shape, float32 scales with x.shape[:-ndim]).
    """
    flat = x.reshape(x.shape[0], -1).float()
    amax = flat.abs().amax(dim=1)
    scale = torch.clamp(amax / FP8_MAX, min=_MIN_SCALE)
    y = (flat / scale[:, None]).clamp(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(x.shape)
    return codes, scale.float()


@dataclasses.dataclass
class DSAInputs:
    cfg: DSAConfig
    # query side
    seq_id: torch.Tensor         # int32 [T]
    pos: torch.Tensor            # int32 [T]; query t sees keys 0..pos[t] of its sequence
    iq8: torch.Tensor            # uint8 [T, H_I, D_I]
    iqs: torch.Tensor            # f32 [T]
    iw: torch.Tensor             # f32 [T, H_I]
    q: torch.Tensor              # bf16 [T, H, D]
    # caches (contiguous [B, L_max, ...] or paged [P, page, ...])
    ik8: torch.Tensor            # uint8
    iks: torch.Tensor            # f32
    kv: torch.Tensor             # bf16
    block_table: Optional[torch.Tensor]   # int32 [B, max_pages] or None
    seq_lens: torch.Tensor       # int32 [B] (host)
    max_len: int                 # max over t of pos[t]+1
    planted: Optional[list] = None        # per sequence: int64 tensor of planted positions

    @property
    def T(self) -> int:
        return int(self.pos.shape[0])


def _workload(cfg: DSAConfig):
    """Sequence lengths and query positions (host int tensors)."""
    if cfg.kind == "prefill":
        lens = torch.tensor([cfg.L], dtype=torch.int32)
        seq_id = torch.zeros(cfg.L, dtype=torch.int32)
        pos = torch.arange(cfg.L, dtype=torch.int32)
        return lens, seq_id, pos
    if cfg.kind == "decode":
        lens = torch.full((cfg.B,), cfg.L, dtype=torch.int32)
        nq = torch.full((cfg.B,), cfg.queries_per_seq, dtype=torch.int32)
    else:  # ragged
        g = _gen(cfg.seed, _T_LEN, "cpu")
        lens = torch.randint(cfg.min_len, cfg.L + 1, (cfg.B,), generator=g, dtype=torch.int64).to(torch.int32)
        gq = _gen(cfg.seed, _T_NQ, "cpu")
        nq = torch.randint(1, 3, (cfg.B,), generator=gq, dtype=torch.int64).to(torch.int32)
    seq_id, pos = [], []
    for b in range(cfg.B):
        for j in range(int(nq[b])):
            seq_id.append(b)
            pos.append(int(lens[b]) - int(nq[b]) + j)
    return lens, torch.tensor(seq_id, dtype=torch.int32), torch.tensor(pos, dtype=torch.int32)


def _randn(shape, gen, device, dtype=torch.float32, chunk_rows: int = 1 << 16):
    """Normal draws filled in row chunks (bounded temporary memory)."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device).to(dtype)
    return out


def make_inputs(cfg: DSAConfig, device="cpu") -> DSAInputs:
    """Draw every tensor of a config on ``device`` (seeded, reproducible)."""
    lens, seq_id, pos = _workload(cfg)
    T = int(pos.shape[0])
    B = cfg.B
    L_max = int(lens.max())
    dev = torch.device(device)

    # indexer query side: q ~ N(0,1) quantised per token, w ~ U(0,1)
    xq = torch.randn((T, cfg.H_I, cfg.D_I), generator=_gen(cfg.seed, _T_IQ, dev), device=dev)
    iq8, iqs = quantize_e4m3fn(xq)
    iw = torch.rand((T, cfg.H_I), generator=_gen(cfg.seed, _T_W, dev), device=dev)

    # attention query
    q = _randn_bf16_scaled((T, cfg.H, cfg.D), _gen(cfg.seed, _T_Q, dev), dev, cfg.attn_std)

    # key-side tensors in logical order [B, L_max, ...]
    n_tok = B * L_max
    xk = _randn((n_tok, cfg.D_I), _gen(cfg.seed, _T_IK, dev), dev)
    planted = None
    if cfg.planted_frac > 0:
        planted = []
        gp = _gen(cfg.seed, _T_PLANT, "cpu")
        xk3 = xk.view(B, L_max, cfg.D_I)
        for b in range(B):
            L = int(lens[b])
            m = int(round(cfg.planted_frac * L))
            sel = torch.randperm(L // 2, generator=gp)[:m].sort().values
            planted.append(sel)
            # one decode query per sequence: point the planted keys along the
            # weighted sum of its indexer query heads (before quantisation)
            t = int((seq_id == b).nonzero()[0])
            v = (iw[t][:, None] * xq[t]).sum(0)
            v = v / v.norm()
            noise = torch.randn((m, cfg.D_I), generator=gp).to(dev) * 0.1
            xk3[b, sel.to(dev)] = 16.0 * v[None, :] + noise
    ik8_l, iks_l = quantize_e4m3fn(xk)
    ik8_l = ik8_l.view(B, L_max, cfg.D_I)
    iks_l = iks_l.view(B, L_max)
    kv_l = _randn_bf16_scaled((B, L_max, cfg.D), _gen(cfg.seed, _T_KV, dev), dev, cfg.attn_std)

    block_table = None
    if cfg.paged:
        ps = cfg.page_size
        pages_per = [-(-int(l) // ps) for l in lens]
        P = sum(pages_per)
        max_pages = max(pages_per)
        perm = torch.randperm(P, generator=_gen(cfg.seed, _T_PAGES, "cpu")).to(torch.int32)
        bt = torch.full((B, max_pages), -1, dtype=torch.int32)
        ik8 = torch.zeros((P, ps, cfg.D_I), dtype=torch.uint8, device=dev)
        iks = torch.zeros((P, ps), dtype=torch.float32, device=dev)
        kv = torch.zeros((P, ps, cfg.D), dtype=torch.bfloat16, device=dev)
        c = 0
        for b in range(B):
            n = pages_per[b]
            phys = perm[c:c + n]
            c += n
            bt[b, :n] = phys
            L = int(lens[b])
            padded = n * ps
            pk = torch.zeros((padded, cfg.D_I), dtype=torch.uint8, device=dev)
            ps_ = torch.zeros((padded,), dtype=torch.float32, device=dev)
            pv = torch.zeros((padded, cfg.D), dtype=torch.bfloat16, device=dev)
            pk[:L] = ik8_l[b, :L]
            ps_[:L] = iks_l[b, :L]
            pv[:L] = kv_l[b, :L]
            idx = phys.long().to(dev)
            ik8[idx] = pk.view(n, ps, cfg.D_I)
            iks[idx] = ps_.view(n, ps)
            kv[idx] = pv.view(n, ps, cfg.D)
        del ik8_l, iks_l, kv_l
        block_table = bt.to(dev)
    else:
        ik8, iks, kv = ik8_l, iks_l, kv_l

    return DSAInputs(cfg=cfg, seq_id=seq_id.to(dev), pos=pos.to(dev), iq8=iq8, iqs=iqs, iw=iw, q=q,
                     ik8=ik8, iks=iks, kv=kv, block_table=block_table, seq_lens=lens,
                     max_len=int(pos.max()) + 1, planted=planted)


def _randn_bf16_scaled(shape, gen, device, std: float, chunk_rows: int = 1 << 14) -> torch.Tensor:
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1, shape[-1])
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        flat[r0:r1] = (torch.randn((r1 - r0, shape[-1]), generator=gen, device=device) * std).to(torch.bfloat16)
    return out


def output_grad(cfg: DSAConfig, T: int, device="cpu") -> torch.Tensor:
    """Gradient of the attention output for the backward: bf16 [T, H, d_v],
    N(0, 1) entries (seeded per config)."""
    dev = torch.device(device)
    return _randn_bf16_scaled((T, cfg.H, cfg.d_v), _gen(cfg.seed, _T_DOUT, dev), dev, 1.0)


def random_selection(cfg: DSAConfig, pos: torch.Tensor, k: int, device="cpu") -> torch.Tensor:
    """int32 [T, k]: per query t, min(k, pos[t] + 1) distinct positions drawn
    uniformly from 0..pos[t], in random order, the rest -1 (seeded per
    config).  A stand-in selection for steps that take any selection."""
    dev = torch.device(device)
    pos = pos.to(dev).long()
    T = int(pos.shape[0])
    L = int(pos.max()) + 1 if T else 1
    g = _gen(cfg.seed, _T_SEL, dev)
    out = torch.full((T, k), -1, dtype=torch.int32, device=dev)
    for r0 in range(0, T, 256):
        r1 = min(T, r0 + 256)
        u = torch.rand((r1 - r0, L), generator=g, device=dev)
        u[torch.arange(L, device=dev)[None, :] > pos[r0:r1, None]] = -1.0
        kk = min(k, L)
        val, sel = torch.topk(u, kk, dim=1)
        sel = torch.where(val >= 0, sel, torch.full_like(sel, -1))
        out[r0:r1, :kk] = sel.to(torch.int32)
    return out


def random_distribution(cfg: DSAConfig, idx: torch.Tensor) -> torch.Tensor:
    """float32 [T, k]: a random probability distribution over each row's
    entries != -1 (0 on padding), seeded per config."""
    g = _gen(cfg.seed, _T_DIST, idx.device)
    v = torch.rand(idx.shape, generator=g, device=idx.device) * (idx >= 0)
    return (v / v.sum(dim=1, keepdim=True).clamp_min(1e-30)).float()


def tie_heavy_logits(T: int, n: int, levels: int = 256, seed: int = 7, device="cpu") -> torch.Tensor:
    """float32 [T, n] rows holding integers 0..levels-1: many equal values at
    any top-k boundary (the 256-level ragged-batch selection test)."""
    g = _gen(seed, 99, device)
    u = torch.rand((T, n), generator=g, device=device)
    return torch.floor(u * (levels - 0.001)).float()


def bf16_bits(x: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def math_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
