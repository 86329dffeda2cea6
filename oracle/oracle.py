"""ctypes front end of the C oracle (``sa_oracle.c``). Test infrastructure only.

Each function takes a workload object (attributes as drawn by the shared input generator)
plus an optional subset of query rows, converts the tensors to numpy without changing any
value (bf16 and E4M3 stay as bit patterns / codes; the C code decodes them), calls the C
routine and returns numpy arrays. ``real`` picks the arithmetic: "f64" (default) or "f32".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sa_oracle.c")
_LIBS = {"f64": os.path.join(_HERE, "liboracle_f64.so"),
         "f32": os.path.join(_HERE, "liboracle_f32.so")}
_loaded = {}
NEG_INF = float("-inf")


def build(force: bool = True) -> None:
    """Compile both arithmetic variants with gcc (-O2 -fopenmp)."""
    for real, path in _LIBS.items():
        if not force and os.path.exists(path) and os.path.getmtime(path) >= os.path.getmtime(_SRC):
            continue
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-o",
               path + ".tmp", _SRC, "-lm"]
        if real == "f32":
            cmd.insert(1, "-DORACLE_FLOAT")
        subprocess.run(cmd, check=True)
        os.replace(path + ".tmp", path)


def load(real: str = "f64"):
    if real in _loaded:
        return _loaded[real]
    path = _LIBS[real]
    if not os.path.exists(path):
        build(force=False)
    lib = C.CDLL(path)
    rt = np.float64 if real == "f64" else np.float32
    assert lib.ora_real_bytes() == np.dtype(rt).itemsize
    lib.ora_max_threads.restype = C.c_int
    P = C.c_void_p
    i32, i64, f32 = C.c_int, C.c_int64, C.c_float
    lib.ora_index_scores.argtypes = [i32, P, P, i32, i32, P, P, i32, P, P, P, i32, i32, i64, P]
    lib.ora_block_scores.argtypes = [i32, P, P, i32, i32, P, P, P, P, i32, i32, i64, P]
    lib.ora_topk.argtypes = [i32, i64, P, P, i32, P]
    lib.ora_topk_in_blocks.argtypes = [i32, P, P, i32, i32, P, P, i32, P, P, P, i32, i32, P,
                                       i32, i32, P]
    lib.ora_sparse_attn.argtypes = [i32, P, P, i32, i32, i32, i32, P, i32, P, P, P, P, i64,
                                    i64, i64, i64, i32, i32, P, i32, i32, i32, P, f32, P]
    lib.ora_bf16.restype = C.c_double if real == "f64" else C.c_float
    lib.ora_bf16.argtypes = [C.c_uint16]
    lib.ora_e4m3.restype = C.c_double if real == "f64" else C.c_float
    lib.ora_e4m3.argtypes = [C.c_uint8]
    lib.ora_e4m3_encode.restype = C.c_uint8
    lib.ora_e4m3_encode.argtypes = [C.c_double]
    lib.ora_mx_exponent.restype = C.c_int
    lib.ora_mx_exponent.argtypes = [C.c_double]
    lib.ora_mx_quantize_bf16.restype = None
    lib.ora_mx_quantize_bf16.argtypes = [P, i32, P, P]
    lib.ora_index_scores_mx.argtypes = [i32, P, P, i32, i32, P, P, P, P, P, i32, i32, i64, P]
    lib.ora_index_scores_mx.restype = C.c_int
    lib.ora_cache_append.argtypes = [i32, P, P, P, i32, i32, P, i32, i32, P, P, P, P, P, i32,
                                     i32, i32, i32, P, P, P, P, P]
    for fn in ("ora_index_scores", "ora_block_scores", "ora_topk", "ora_topk_in_blocks",
               "ora_sparse_attn", "ora_cache_append"):
        getattr(lib, fn).restype = C.c_int
    lib.real_dtype = rt
    _loaded[real] = lib
    return lib


# ---------------------------------------------------------------------------- conversions

def _np(t, dtype=None):
    """torch tensor -> contiguous numpy array; bf16 becomes its uint16 bit patterns."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        a = t.view(torch.int16).numpy().view(np.uint16)
    elif t.dtype == torch.float8_e4m3fn:
        a = t.view(torch.uint8).numpy()
    else:
        a = t.numpy()
    if dtype is not None:
        a = a.astype(dtype, copy=False)
    return np.ascontiguousarray(a)


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _rows(wl, rows):
    nq = wl.num_queries
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    q_seq = _np(wl.q_seq(), np.int32)[rows].copy()
    q_pos = _np(wl.q_pos(), np.int64)[rows].copy()
    return rows, q_seq, q_pos


def _fmt(dtype: str) -> int:
    """Stored-vector formats: bf16; E4M3 with one fp32 scale per row; E4M3 with one fp32 scale
    per 128-entry tile of each token and head (KV only)."""
    return {"bf16": 0, "fp8": 1, "fp8t128": 2}[dtype]


def bf16_decode(bits: np.ndarray, real: str = "f64") -> np.ndarray:
    lib = load(real)
    return np.array([lib.ora_bf16(int(b)) for b in np.asarray(bits).ravel()],
                    dtype=lib.real_dtype).reshape(np.shape(bits))


def e4m3_encode(values) -> np.ndarray:
    """Nearest E4M3 codes (ties to even mantissa, saturating at +-448)."""
    lib = load("f64")
    v = np.asarray(values, dtype=np.float64)
    return np.array([lib.ora_e4m3_encode(float(x)) for x in v.ravel()], dtype=np.uint8).reshape(v.shape)


def mx_exponent(amax: float) -> int:
    """Shared exponent X of an MXFP8 block with largest magnitude ``amax``."""
    return int(load("f64").ora_mx_exponent(float(amax)))


def mx_quantize_bf16(bits: np.ndarray):
    """bf16 bit patterns [..., n] (n a multiple of 32) -> (E4M3 codes [..., n], E8M0 [..., n/32])."""
    lib = load("f64")
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    n = b.shape[-1]
    flat = b.reshape(-1, n)
    codes = np.empty(flat.shape, dtype=np.uint8)
    e8m0 = np.empty((flat.shape[0], n // 32), dtype=np.uint8)
    for r in range(flat.shape[0]):
        lib.ora_mx_quantize_bf16(_p(flat[r]), n, _p(codes[r]), _p(e8m0[r]))
    return codes.reshape(b.shape), e8m0.reshape(b.shape[:-1] + (n // 32,))


def e4m3_decode(codes: np.ndarray, real: str = "f64") -> np.ndarray:
    lib = load(real)
    return np.array([lib.ora_e4m3(int(c)) for c in np.asarray(codes).ravel()],
                    dtype=lib.real_dtype).reshape(np.shape(codes))


# ---------------------------------------------------------------------------- steps

def index_scores(wl, rows=None, ncols=None, real: str = "f64") -> np.ndarray:
    """Scores [len(rows), ncols]; column t holds the score of position t, -inf past q_pos."""
    lib = load(real)
    rows, q_seq, q_pos = _rows(wl, rows)
    if ncols is None:
        ncols = int(q_pos.max()) + 1 if len(rows) else 1
    q_idx = _np(wl.q_idx)[rows].copy()
    w = _np(wl.w, np.float32)[rows].copy()
    keys = _np(wl.idx_keys)
    pt = _np(wl.page_table, np.int32)
    out = np.empty((len(rows), ncols), dtype=lib.real_dtype)
    if wl.idx_dtype == "mxfp8":
        e8m0 = _np(wl.idx_mx_scale, np.uint8)
        rc = lib.ora_index_scores_mx(len(rows), _p(q_seq), _p(q_pos), wl.idx_heads, wl.idx_dim,
                                     _p(q_idx), _p(w), _p(keys), _p(e8m0), _p(pt),
                                     wl.pages_per_seq, wl.page_size, ncols, _p(out))
        assert rc == 0, "oracle index_scores_mx rejected its inputs"
        return out
    scale = None if wl.idx_scale is None else _np(wl.idx_scale, np.float32)
    rc = lib.ora_index_scores(len(rows), _p(q_seq), _p(q_pos), wl.idx_heads, wl.idx_dim,
                              _p(q_idx), _p(w), _fmt(wl.idx_dtype), _p(keys), _p(scale), _p(pt),
                              wl.pages_per_seq, wl.page_size, ncols, _p(out))
    assert rc == 0, "oracle index_scores rejected its inputs"
    return out


def block_scores(wl, rows=None, real: str = "f64") -> np.ndarray:
    """Coarse-stage block scores [len(rows), pages_per_seq] over the pooled summaries."""
    lib = load(real)
    rows, q_seq, q_pos = _rows(wl, rows)
    q_idx = _np(wl.q_idx)[rows].copy()
    w = _np(wl.w, np.float32)[rows].copy()
    pooled = _np(wl.pooled)
    pt = _np(wl.page_table, np.int32)
    ncols = wl.pages_per_seq
    out = np.empty((len(rows), ncols), dtype=lib.real_dtype)
    rc = lib.ora_block_scores(len(rows), _p(q_seq), _p(q_pos), wl.idx_heads, wl.idx_dim,
                              _p(q_idx), _p(w), _p(pooled), _p(pt), wl.pages_per_seq,
                              wl.page_size, ncols, _p(out))
    assert rc == 0
    return out


def topk(scores: np.ndarray, n_valid, k: int, real: str = "f64") -> np.ndarray:
    """Row-wise Top-k of ``scores`` over columns [0, n_valid[r]); ascending positions, -1 pad."""
    lib = load(real)
    s = np.ascontiguousarray(scores, dtype=lib.real_dtype)
    if s.ndim == 1:
        s = s[None, :]
    nv = np.ascontiguousarray(np.broadcast_to(np.asarray(n_valid, dtype=np.int64), (s.shape[0],)))
    out = np.empty((s.shape[0], k), dtype=np.int32)
    rc = lib.ora_topk(s.shape[0], s.shape[1], _p(s), _p(nv), k, _p(out))
    assert rc == 0, "oracle topk rejected its inputs (NaN score?)"
    return out


def topk_in_blocks(wl, blocks: np.ndarray, rows=None, k=None, real: str = "f64") -> np.ndarray:
    """Fine stage: Top-k among the visible tokens of the given blocks (one row per query)."""
    lib = load(real)
    assert wl.idx_dtype != "mxfp8", "two-level selection is defined over bf16 / E4M3 keys"
    rows, q_seq, q_pos = _rows(wl, rows)
    k = wl.topk if k is None else k
    blocks = np.ascontiguousarray(blocks, dtype=np.int32)
    q_idx = _np(wl.q_idx)[rows].copy()
    w = _np(wl.w, np.float32)[rows].copy()
    keys = _np(wl.idx_keys)
    scale = None if wl.idx_scale is None else _np(wl.idx_scale, np.float32)
    pt = _np(wl.page_table, np.int32)
    out = np.empty((len(rows), k), dtype=np.int32)
    rc = lib.ora_topk_in_blocks(len(rows), _p(q_seq), _p(q_pos), wl.idx_heads, wl.idx_dim,
                                _p(q_idx), _p(w), _fmt(wl.idx_dtype), _p(keys), _p(scale), _p(pt),
                                wl.pages_per_seq, wl.page_size, _p(blocks), blocks.shape[1], k,
                                _p(out))
    assert rc == 0
    return out


def sparse_attn(wl, idx: np.ndarray, rows=None, real: str = "f64") -> np.ndarray:
    """Attention over the selected positions ``idx`` [len(rows), K]; returns [rows, Hq, dv]."""
    lib = load(real)
    rows, q_seq, q_pos = _rows(wl, rows)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    k = idx.shape[1]
    q = _np(wl.q)[rows].copy()
    kc = _np(wl.k_cache)
    k_row = wl.k_cache.shape[-1]
    k_stride = wl.heads_kv * k_row
    if wl.v_cache is None:
        vc, v_stride, v_head_stride = kc, k_stride, k_row
    else:
        vc = _np(wl.v_cache)
        v_stride, v_head_stride = wl.heads_kv * wl.v_cache.shape[-1], wl.v_cache.shape[-1]
    sc = None if wl.kv_scale is None else _np(wl.kv_scale, np.float32)
    k_tiles = v_tiles = 0
    if wl.kv_dtype == "fp8t128":
        assert wl.v_cache is None, "tile scales are defined for latent rows (V inside K)"
        k_tiles = v_tiles = -(-wl.dim_qk // 128)
    pt = _np(wl.page_table, np.int32)
    out = np.empty((len(rows), wl.heads_q, wl.dim_v), dtype=lib.real_dtype)
    rc = lib.ora_sparse_attn(len(rows), _p(q_seq), _p(q_pos), wl.heads_q, wl.heads_kv,
                             wl.dim_qk, wl.dim_v, _p(q), _fmt(wl.kv_dtype), _p(kc), _p(vc),
                             _p(sc), _p(sc), k_stride, v_stride, k_row, v_head_stride, k_tiles,
                             v_tiles, _p(pt),
                             wl.pages_per_seq, wl.page_size, k, _p(idx),
                             float(wl.softmax_scale), _p(out))
    assert rc == 0, "oracle sparse_attn rejected its inputs"
    return out


def two_level_select(wl, rows=None, real: str = "f64"):
    """Hierarchical selection: block Top-(block_topk) over pooled summaries, then token Top-K
    inside the kept blocks. Returns (blocks [rows, block_topk], idx [rows, K], block_scores)."""
    rows, q_seq, q_pos = _rows(wl, rows)
    bs = block_scores(wl, rows, real)
    nblk = (q_pos // wl.page_size) + 1
    blocks = topk(bs, nblk, wl.block_topk, real)
    idx = topk_in_blocks(wl, blocks, rows, wl.topk, real)
    return blocks, idx, bs


def max_threads(real: str = "f64") -> int:
    """OpenMP threads the oracle's loops use (omp_get_max_threads of its library)."""
    return int(load(real).ora_max_threads())


def decode_step(wl, rows=None, real: str = "f64"):
    """Whole path for the given query rows: indexer scores -> Top-K (single- or two-level)
    -> sparse attention. Returns dict(idx, out, scores|block_scores, blocks)."""
    rows_arr, q_seq, q_pos = _rows(wl, rows)
    res = {}
    if wl.block_topk:
        blocks, idx, bs = two_level_select(wl, rows_arr, real)
        res.update(blocks=blocks, block_scores=bs)
    else:
        s = index_scores(wl, rows_arr, real=real)
        idx = topk(s, q_pos + 1, wl.topk, real)
        res["scores"] = s
    res["idx"] = idx
    res["out"] = sparse_attn(wl, idx, rows_arr, real)
    return res


def cache_append(wl, k_idx_new, kv_new, v_new=None, indexer=True, kv=True) -> dict:
    """The cache writes of the step before the path: the new token rows (one per query row of
    ``wl``, at the positions ``wl.q_pos()``) written into copies of the workload's caches.

    k_idx_new: bf16 [rows, d_I]; kv_new: bf16 [rows, heads_kv, dim_qk]; v_new: bf16
    [rows, heads_kv, dim_v] for separate V caches. Returns numpy copies of the caches after the
    append: idx_keys, idx_scale, idx_mx_scale, pooled, k_cache, v_cache, kv_scale (None where
    the workload has none)."""
    lib = load()
    rows, q_seq, q_pos = _rows(wl, None)
    ctx = np.asarray(wl.ctx_lens, dtype=np.int32)
    pt = _np(wl.page_table, np.int32)
    cp = lambda t, dt=None: None if t is None else _np(t, dt).copy()
    out = {
        "idx_keys": cp(wl.idx_keys), "idx_scale": cp(wl.idx_scale, np.float32),
        "idx_mx_scale": cp(wl.idx_mx_scale, np.uint8), "pooled": cp(wl.pooled),
        "k_cache": cp(wl.k_cache), "v_cache": cp(wl.v_cache), "kv_scale": cp(wl.kv_scale, np.float32),
    }
    kin = _np(k_idx_new).copy() if indexer else None
    kvin = _np(kv_new).copy() if kv else None
    vin = _np(v_new).copy() if (kv and v_new is not None) else None
    idx_fmt = {"bf16": 0, "fp8": 1, "mxfp8": 2}[wl.idx_dtype]
    kv_fmt = _fmt(wl.kv_dtype)
    rc = lib.ora_cache_append(
        len(rows), _p(q_seq), _p(q_pos), _p(pt), wl.pages_per_seq, wl.page_size, _p(ctx),
        wl.idx_dim if indexer else 0, idx_fmt, _p(kin), _p(out["idx_keys"]), _p(out["idx_scale"]),
        _p(out["idx_mx_scale"]), _p(out["pooled"]), wl.heads_kv if kv else 0, wl.dim_qk,
        wl.dim_v, kv_fmt, _p(kvin), _p(vin), _p(out["k_cache"]), _p(out["v_cache"]),
        _p(out["kv_scale"]))
    assert rc == 0, "oracle cache_append rejected its inputs"
    return out


# ---------------------------------------------------------------------------- indexer prolog

LN_EPS = 1e-6


def indexer_prolog(x_q, x, w_q, w_k, w_w, gamma, beta, eps: float = LN_EPS):
    """The indexer prolog ([CANN] §2.2: Q projection, K normalization, head-weight projection),
    in fp64 from the given (bf16) inputs, with the plain definitions:
        q_I = x_q W_q^T      (row r, head h: entries h*d_I .. h*d_I + d_I - 1)
        k_I = LayerNorm(x W_k^T) * gamma + beta   (mean and biased variance over d_I, eps)
        w   = x W_w^T
    Weights are [out_features, in_features]. Returns (q_I [rows, H_I*d_I], k_I [rows, d_I],
    w [rows, H_I]) as float64 numpy arrays. (Q quantization, the pages' fourth prolog operation,
    happens inside the MXFP8 indexer.)"""
    f = lambda t: np.asarray(t.float().numpy() if hasattr(t, "float") else t, dtype=np.float64)
    xq, xx = f(x_q), f(x)
    q = xq @ f(w_q).T
    y = xx @ f(w_k).T
    mu = y.mean(axis=1, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=1, keepdims=True)
    k = (y - mu) / np.sqrt(var + eps) * f(gamma)[None, :] + f(beta)[None, :]
    w = xx @ f(w_w).T
    return q, k, w
