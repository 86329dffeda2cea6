"""Seeded synthetic workloads for index-selected sparse attention over a paged KV cache.

This module only draws inputs. It holds none of the method's arithmetic (no scores, no
selection, no attention); the HIP path and the CPU oracle both read what it produces.

Every tensor comes from its own ``torch.Generator('cpu')`` seeded with
``1000 * config_id + tensor_id + seed_offset`` (tensor ids: 0 page permutation, 1 indexer
queries, 2 indexer keys, 3 head weights, 4 attention queries, 5 K / latent KV rows, 6 V rows,
7 context lengths). Values are fp32 N(0, 1) draws rounded to bf16 (round-to-nearest-even), or
quantized to OCP E4M3 with one fp32 absmax scale per stored row, generated in physical-page
order. Blocked KV layout follows "Engineering Path for Day-0 Adaptation of Trillion-Scale
Sparse Models on Domestic AI Accelerators", §3.2 and "Adapting GPU Software Stacks for
Ultra-Large-Scale Sparse Attention Models: A Day-0 Engineering Guide", §3.2.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

E4M3_MAX = 448.0


@dataclass
class Workload:
    name: str
    config_id: int
    num_seqs: int
    ctx_lens: list            # host ints, one per sequence
    page_size: int
    pages_per_seq: int
    num_pages: int
    page_table: torch.Tensor  # int32 [num_seqs, pages_per_seq]
    q_lens: list              # query tokens per sequence (1 = decode)
    # indexer
    idx_heads: int
    idx_dim: int
    idx_dtype: str            # "bf16" | "fp8" | "mxfp8"
    q_idx: torch.Tensor       # bf16 [nq, idx_heads, idx_dim]
    w: torch.Tensor           # fp32 [nq, idx_heads]
    idx_keys: torch.Tensor    # bf16 [num_pages, page_size, idx_dim] or uint8 codes
    idx_scale: Optional[torch.Tensor]  # fp32 [num_pages, page_size] (fp8) else None
    pooled: Optional[torch.Tensor]     # bf16 [num_pages, idx_dim] block summaries, or None
    topk: int
    block_topk: int           # 0 = single-level selection
    # attention
    heads_q: int
    heads_kv: int
    dim_qk: int
    dim_v: int
    kv_dtype: str             # "bf16" | "fp8" (one scale per row) | "fp8t128" (per 128 entries)
    q: torch.Tensor           # bf16 [nq, heads_q, dim_qk]
    k_cache: torch.Tensor     # [num_pages, page_size, heads_kv, k_row] (bf16 or uint8 codes)
    v_cache: Optional[torch.Tensor]  # None when V is the first dim_v entries of each K row
    # fp32 [num_pages, page_size] (fp8), [num_pages, page_size, heads_kv, ceil(dim_qk / 128)]
    # (fp8t128), else None
    kv_scale: Optional[torch.Tensor]
    softmax_scale: float
    seeds: dict = field(default_factory=dict)
    # uint8 E8M0 bytes [num_pages, page_size, idx_dim / 32] (mxfp8 indexer keys) else None
    idx_mx_scale: Optional[torch.Tensor] = None

    # ---- derived views --------------------------------------------------------------
    @property
    def num_queries(self) -> int:
        return sum(self.q_lens)

    def q_seq(self) -> torch.Tensor:
        """int32 [nq]: sequence of each query row."""
        return torch.tensor([b for b, n in enumerate(self.q_lens) for _ in range(n)],
                            dtype=torch.int32)

    def q_pos(self) -> torch.Tensor:
        """int64 [nq]: absolute position of each query row (the last q_len tokens)."""
        out = []
        for b, n in enumerate(self.q_lens):
            out.extend(range(self.ctx_lens[b] - n, self.ctx_lens[b]))
        return torch.tensor(out, dtype=torch.int64)

    def q_indptr(self) -> torch.Tensor:
        out = [0]
        for n in self.q_lens:
            out.append(out[-1] + n)
        return torch.tensor(out, dtype=torch.int32)

    @property
    def v_aliases_k(self) -> bool:
        return self.v_cache is None

    @property
    def k_row(self) -> int:
        return self.k_cache.shape[-1]


# ---------------------------------------------------------------------------- helpers

def _gen(config_id: int, tensor_id: int, offset: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * config_id + tensor_id + offset)
    return g


def _randn_bf16(shape, g) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def quantize_rows_e4m3(x: torch.Tensor):
    """Quantize the rows (last dim) of fp32 ``x`` [..., row] to OCP E4M3.

    One scale per row: sigma = absmax / 448 (1 when the row is all zero) and
    code = RNE(clamp(x / sigma, -448, 448)). Returns (uint8 codes [..., row], fp32 sigma [...]).
    """
    amax = x.abs().amax(dim=-1)
    sigma = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    codes = (x / sigma.unsqueeze(-1)).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8), sigma.to(torch.float32)


def quantize_tiles_e4m3(x: torch.Tensor, tile: int = 128):
    """Quantize fp32 ``x`` [..., n] to OCP E4M3 with one scale per ``tile`` consecutive elements
    of the last dim (a shorter last tile keeps its own scale): sigma = tile absmax / 448 (1 for an
    all-zero tile), code = RNE(clamp(x / sigma, -448, 448)). Returns (uint8 codes [..., n], fp32
    sigma [..., ceil(n / tile)])."""
    n = x.shape[-1]
    nt = -(-n // tile)
    pad = torch.zeros(*x.shape[:-1], nt * tile - n, dtype=x.dtype)
    t = torch.cat([x, pad], dim=-1).reshape(*x.shape[:-1], nt, tile)
    amax = t.abs().amax(dim=-1)
    sigma = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    codes = (t / sigma.unsqueeze(-1)).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    codes = codes.view(torch.uint8).reshape(*x.shape[:-1], nt * tile)[..., :n].contiguous()
    return codes, sigma.to(torch.float32)


def quantize_rows_mxfp8(x: torch.Tensor):
    """Quantize fp32 ``x`` [..., n] (n a multiple of 32) to MXFP8: every 32 consecutive
    elements share one power-of-two scale 2^X, X = floor(log2(amax)) - 8 clamped to
    [-127, 127] (-127 for an all-zero block), stored as the E8M0 byte X + 127; elements are
    code = RNE(clamp(v / 2^X, -448, 448)) in OCP E4M3. Returns (uint8 codes [..., n],
    uint8 E8M0 [..., n / 32])."""
    n = x.shape[-1]
    blocks = x.reshape(*x.shape[:-1], n // 32, 32)
    amax = blocks.abs().amax(dim=-1)
    _, e = torch.frexp(amax)  # amax = f * 2^e, f in [0.5, 1)
    xexp = torch.where(amax > 0, e - 1 - 8, torch.full_like(e, -127)).clamp(-127, 127)
    scaled = blocks * torch.pow(2.0, -xexp.to(torch.float64)).to(torch.float32).unsqueeze(-1)
    codes = scaled.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.reshape(x.shape), (xexp + 127).to(torch.uint8)


def _page_table(num_seqs, ctx_lens, page_size, g):
    pages = [math.ceil(n / page_size) for n in ctx_lens]
    pages_per_seq = max(1, max(pages))
    num_pages = max(1, sum(pages))
    perm = torch.randperm(num_pages, generator=g).to(torch.int32)
    pt = torch.zeros((num_seqs, pages_per_seq), dtype=torch.int32)
    k = 0
    for b, np_ in enumerate(pages):
        pt[b, :np_] = perm[k:k + np_]
        k += np_
    return pt, pages_per_seq, num_pages


def _pooled_keys(keys_bf16, page_table, ctx_lens, page_size):
    """Block summaries: for every used physical page, the mean over its valid tokens of the
    indexer key rows, computed in fp64 and rounded to bf16. Pages not holding any valid
    token keep zeros."""
    num_pages, _, dim = keys_bf16.shape
    pooled = torch.zeros((num_pages, dim), dtype=torch.float64)
    kf = keys_bf16.to(torch.float64)
    for b, n in enumerate(ctx_lens):
        npg = math.ceil(n / page_size)
        phys = page_table[b, :npg].to(torch.int64)
        counts = torch.full((npg,), page_size, dtype=torch.float64)
        if npg:
            counts[-1] = n - (npg - 1) * page_size
        valid = torch.arange(page_size).unsqueeze(0) < counts.unsqueeze(1)  # [npg, P]
        sums = (kf[phys] * valid.unsqueeze(-1)).sum(dim=1)
        pooled[phys] = sums / counts.unsqueeze(1)
    return pooled.to(torch.bfloat16)


# ---------------------------------------------------------------------------- presets

PRESETS = {
    # name: (config_id, defaults)
    "tiny": (1, dict(num_seqs=1, ctx=4096, page_size=64, idx_heads=4, idx_dim=64,
                     weights="softmax", topk=256, heads_q=8, heads_kv=1, dim_qk=128, dim_v=128,
                     mla=False, dtype="bf16", q_len=1, block_topk=0)),
    "decode32k": (2, dict(num_seqs=32, ctx=32768, page_size=64, idx_heads=64, idx_dim=128,
                          weights="scaled", topk=2048, heads_q=128, heads_kv=1, dim_qk=576,
                          dim_v=512, mla=True, dtype="bf16", q_len=1, block_topk=0)),
    "prefill64k": (3, dict(num_seqs=1, ctx=65536, page_size=64, idx_heads=64, idx_dim=128,
                           weights="scaled", topk=2048, heads_q=128, heads_kv=1, dim_qk=576,
                           dim_v=512, mla=True, dtype="bf16", q_len=4096, block_topk=0)),
    "long1m": (4, dict(num_seqs=4, ctx=1048576, page_size=64, idx_heads=64, idx_dim=128,
                       weights="scaled", topk=2048, heads_q=128, heads_kv=1, dim_qk=576,
                       dim_v=512, mla=True, dtype="bf16", q_len=1, block_topk=512)),
    "fp8ragged": (5, dict(num_seqs=64, ctx="loguniform", ctx_lo=4096, ctx_hi=131072,
                          page_size=64, idx_heads=64, idx_dim=128, weights="scaled", topk=2048,
                          heads_q=128, heads_kv=1, dim_qk=576, dim_v=512, mla=True, dtype="fp8",
                          q_len=1, block_topk=0)),
    # the ragged batch in the pages' own FP8 granularities: the indexer in MXFP8 (groups of 32,
    # E8M0 scales) and the KV cache in E4M3 with one scale per 128 entries of each row
    "mxfp8ragged": (6, dict(num_seqs=64, ctx="loguniform", ctx_lo=4096, ctx_hi=131072,
                            page_size=64, idx_heads=64, idx_dim=128, weights="scaled", topk=2048,
                            heads_q=128, heads_kv=1, dim_qk=576, dim_v=512, mla=True,
                            dtype="fp8t128", idx_dtype="mxfp8", q_len=1, block_topk=0)),
}


def make(preset: str, seed_offset: int = 0, **overrides) -> Workload:
    """Draw the workload ``preset`` (see PRESETS), optionally with smaller shapes.

    overrides may replace any default, e.g. ``make("decode32k", num_seqs=2, ctx=5000)``;
    ``ctx`` may be an int, a list of per-sequence ints, or "loguniform".
    """
    config_id, defaults = PRESETS[preset]
    p = dict(defaults)
    p.update(overrides)
    B, P = p["num_seqs"], p["page_size"]
    off = seed_offset

    # context lengths
    if isinstance(p["ctx"], (list, tuple)):
        ctx_lens = [int(x) for x in p["ctx"]]
        assert len(ctx_lens) == B
    elif p["ctx"] == "loguniform":
        g = _gen(config_id, 7, off)
        u = torch.rand(B, generator=g, dtype=torch.float64)
        lo, hi = math.log(p["ctx_lo"]), math.log(p["ctx_hi"])
        ctx_lens = [int(math.floor(math.exp(lo + (hi - lo) * float(x)))) for x in u]
    else:
        ctx_lens = [int(p["ctx"])] * B

    q_len = p["q_len"]  # query rows per sequence: one count for all, or one per sequence
    ql = list(q_len) if isinstance(q_len, (list, tuple)) else [q_len] * B
    q_lens = [min(q, n) if n > 0 else 0 for q, n in zip(ql, ctx_lens)]
    if q_len == 1:
        q_lens = [1] * B  # decode: one query row per sequence even when empty
    nq = sum(q_lens)

    pt, pages_per_seq, num_pages = _page_table(B, ctx_lens, P, _gen(config_id, 0, off))

    H_I, d_I = p["idx_heads"], p["idx_dim"]
    q_idx = _randn_bf16((nq, H_I, d_I), _gen(config_id, 1, off))
    kf = torch.randn((num_pages, P, d_I), generator=_gen(config_id, 2, off), dtype=torch.float32)
    gw = _gen(config_id, 3, off)
    if p["weights"] == "softmax":
        w = torch.softmax(torch.randn((nq, H_I), generator=gw, dtype=torch.float32), dim=-1)
    else:
        w = torch.randn((nq, H_I), generator=gw, dtype=torch.float32) / 8.0

    dtype = p["dtype"]
    # the indexer keys follow the cache dtype unless given; tile scales are defined for latent KV
    # rows only, so with them the keys default to bf16
    idx_dtype = p.get("idx_dtype", dtype if dtype in ("bf16", "fp8") else "bf16")
    assert idx_dtype in ("bf16", "fp8", "mxfp8"), f"indexer key dtype {idx_dtype!r}"
    idx_mx_scale = None
    if idx_dtype == "mxfp8":
        idx_keys, idx_mx_scale = quantize_rows_mxfp8(kf)
        idx_scale, keys_bf16_for_pool = None, None
    elif idx_dtype == "fp8":
        idx_keys, idx_scale = quantize_rows_e4m3(kf)
        keys_bf16_for_pool = None
    else:
        idx_keys, idx_scale = kf.to(torch.bfloat16), None
        keys_bf16_for_pool = idx_keys
    del kf

    pooled = None
    if p["block_topk"]:
        assert idx_dtype == "bf16", "block summaries are defined over bf16 indexer keys"
        pooled = _pooled_keys(keys_bf16_for_pool, pt, ctx_lens, P)

    Hq, Hkv, dqk, dv = p["heads_q"], p["heads_kv"], p["dim_qk"], p["dim_v"]
    q = _randn_bf16((nq, Hq, dqk), _gen(config_id, 4, off))
    kvf = torch.randn((num_pages, P, Hkv, dqk), generator=_gen(config_id, 5, off),
                      dtype=torch.float32)
    v_cache = None
    kv_scale = None
    if dtype == "fp8":
        assert p["mla"] and Hkv == 1, "fp8 rows carry one scale per token row"
        k_cache, sc = quantize_rows_e4m3(kvf.reshape(num_pages, P, Hkv * dqk))
        k_cache = k_cache.reshape(num_pages, P, Hkv, dqk)
        kv_scale = sc
    elif dtype == "fp8t128":
        assert p["mla"], "tile scales are defined for latent rows (V inside K)"
        # scales [pages, P, Hkv, tiles]; in slices of pages to bound the temporaries
        parts = [quantize_tiles_e4m3(kvf[i:i + 2048], 128) for i in range(0, num_pages, 2048)]
        k_cache = torch.cat([c for c, _ in parts])
        kv_scale = torch.cat([t for _, t in parts])
        del parts
    else:
        k_cache = kvf.to(torch.bfloat16)
    del kvf
    if not p["mla"]:
        v_cache = _randn_bf16((num_pages, P, Hkv, dv), _gen(config_id, 6, off))

    scale = p.get("softmax_scale", 1.0 / math.sqrt(dqk))
    return Workload(
        name=preset, config_id=config_id, num_seqs=B, ctx_lens=ctx_lens, page_size=P,
        pages_per_seq=pages_per_seq, num_pages=num_pages, page_table=pt, q_lens=q_lens,
        idx_heads=H_I, idx_dim=d_I, idx_dtype=idx_dtype, q_idx=q_idx, w=w, idx_keys=idx_keys,
        idx_scale=idx_scale, pooled=pooled, topk=p["topk"], block_topk=p["block_topk"],
        heads_q=Hq, heads_kv=Hkv, dim_qk=dqk, dim_v=dv, kv_dtype=dtype, q=q, k_cache=k_cache,
        v_cache=v_cache, kv_scale=kv_scale, softmax_scale=float(scale),
        seeds={"config_id": config_id, "seed_offset": off}, idx_mx_scale=idx_mx_scale,
    )


# ---------------------------------------------------------------------------- indexer prolog

@dataclass
class PrologInputs:
    """Synthetic inputs of the indexer prolog (no trained weights): per new token a query
    latent x_q and a hidden state x; projection weights [out_features, in_features]."""
    x_q: torch.Tensor    # bf16 [rows, d_q]
    x: torch.Tensor      # bf16 [rows, d_model]
    w_q: torch.Tensor    # bf16 [H_I * d_I, d_q]
    w_k: torch.Tensor    # bf16 [d_I, d_model]
    w_w: torch.Tensor    # bf16 [H_I, d_model]
    gamma: torch.Tensor  # fp32 [d_I]
    beta: torch.Tensor   # fp32 [d_I]


def make_prolog(rows: int, heads: int, dim: int, d_q: int = 1536, d_model: int = 7168,
                seed: int = 0) -> PrologInputs:
    """Seeded prolog inputs: activations N(0,1); weights N(0,1)/sqrt(fan_in); LayerNorm weight
    1 + N(0, 0.1^2) and bias N(0, 0.1^2). All bf16 except the LayerNorm parameters."""
    g = lambda i: _gen(9, i, seed)
    bf = lambda shape, i, s=1.0: (torch.randn(shape, generator=g(i)) * s).to(torch.bfloat16)
    return PrologInputs(
        x_q=bf((rows, d_q), 1), x=bf((rows, d_model), 2),
        w_q=bf((heads * dim, d_q), 3, d_q ** -0.5), w_k=bf((dim, d_model), 4, d_model ** -0.5),
        w_w=bf((heads, d_model), 5, d_model ** -0.5),
        gamma=1.0 + 0.1 * torch.randn(dim, generator=g(6)),
        beta=0.1 * torch.randn(dim, generator=g(7)))
