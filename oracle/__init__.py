"""ctypes front-end of the plain C oracle (``dsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the product package.  The
functions take host numpy arrays (or CPU torch tensors) holding the same bytes
the GPU path consumes and return float64 results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, E4M3 = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, OpenMP over rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        vp, i32, i64, dp = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_e4m3_value.argtypes = [i32]
        L.orc_e4m3_value.restype = dp
        L.orc_e4m3_table.argtypes = [vp]
        L.orc_e4m3_table.restype = None
        L.orc_indexer.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, vp]
        L.orc_indexer.restype = i32
        L.orc_topk.argtypes = [vp, i64, vp, i32, i32, vp]
        L.orc_topk.restype = i32
        L.orc_sparse_attn.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, dp, vp, vp]
        L.orc_sparse_attn.restype = i32
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.restype = i32
        L.orc_quantize_e4m3.argtypes = [vp, i32, i64, i32, i32, ctypes.c_float, vp, vp]
        L.orc_quantize_e4m3.restype = i32
        L.orc_rope_rows.argtypes = [vp, vp, i64, i32, i32, i32, vp, dp, vp]
        L.orc_rope_rows.restype = i32
        L.orc_kv_pack_fp8.argtypes = [vp, i64, vp]
        L.orc_kv_pack_fp8.restype = i32
        L.orc_kv_unpack_fp8.argtypes = [vp, i64, vp]
        L.orc_kv_unpack_fp8.restype = i32
        L.orc_indexer_kl.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, dp, vp]
        L.orc_indexer_kl.restype = i32
        L.orc_sparse_attn_bwd.argtypes = [vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, dp, vp, vp]
        L.orc_sparse_attn_bwd.restype = i32
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = i32
        _lib = L
    return _lib


def _np(x, dtype=None) -> np.ndarray:
    """Host, C-contiguous numpy view of a numpy array or CPU torch tensor."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16 or x.dtype == torch.float8_e4m3fn:
                x = x.view(torch.uint16 if x.dtype == torch.bfloat16 else torch.uint8)
            x = x.contiguous().numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(x)
    if dtype is not None:
        a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().orc_num_threads())


def e4m3_value(code: int) -> float:
    return float(lib().orc_e4m3_value(int(code)))


def e4m3_table() -> np.ndarray:
    out = np.empty(256, dtype=np.float32)
    lib().orc_e4m3_table(_ptr(out))
    return out


def indexer(q_idx, q_scale, k_idx, k_scale, w, t_pos, dtype: int) -> np.ndarray:
    """Scores [n_rows, Lk] (float64, -inf where s > t_pos) for one batch entry.

    q_idx [n_rows,H,D], q_scale [n_rows,H] or None, k_idx [Lk,D],
    k_scale [Lk] or None, w [n_rows,H], t_pos [n_rows] int64.
    """
    q = _np(q_idx)
    k = _np(k_idx)
    n_rows, H, D = q.shape
    Lk = k.shape[0]
    assert k.shape[1] == D
    if dtype == E4M3:
        q = q.view(np.uint8)
        k = k.view(np.uint8)
    else:
        q = _np(q, np.float32)
        k = _np(k, np.float32)
    qs = None if q_scale is None else _np(q_scale, np.float32)
    ks = None if k_scale is None else _np(k_scale, np.float32)
    ww = _np(w, np.float32)
    tp = _np(t_pos, np.int64)
    assert ww.shape == (n_rows, H) and tp.shape == (n_rows,)
    out = np.empty((n_rows, Lk), dtype=np.float64)
    rc = lib().orc_indexer(_ptr(q), _ptr(qs), _ptr(k), _ptr(ks), _ptr(ww), dtype,
                           _ptr(tp), n_rows, Lk, H, D, _ptr(out))
    if rc != 0:
        raise ValueError("orc_indexer: bad arguments")
    return out


def indexer_abs_mass(q_idx, q_scale, k_idx, k_scale, w, t_pos, dtype: int) -> np.ndarray:
    """M[t,s] = sum_j |w_j| sum_d |qhat_jd| |khat_d|: the indexer evaluated on
    absolute values.  It bounds every partial sum of the score, so eps * M
    bounds accumulation error in any summation order (used for tolerances)."""
    if dtype == E4M3:
        qa = _np(q_idx).view(np.uint8) & 0x7F
        ka = _np(k_idx).view(np.uint8) & 0x7F
    else:
        qa = np.abs(_np(q_idx, np.float32))
        ka = np.abs(_np(k_idx, np.float32))
    return indexer(qa, q_scale, ka, k_scale, np.abs(_np(w, np.float32)), t_pos, dtype)


def topk(scores, t_pos, k: int) -> np.ndarray:
    """Top-k index sets [n_rows, k] int32 (ascending s, -1 padded)."""
    sc = _np(scores, np.float64)
    n_rows, ld = sc.shape
    tp = _np(t_pos, np.int64)
    out = np.empty((n_rows, k), dtype=np.int32)
    rc = lib().orc_topk(_ptr(sc), ld, _ptr(tp), n_rows, int(k), _ptr(out))
    if rc != 0:
        raise ValueError("orc_topk: bad arguments")
    return out


def sparse_attn(q, kv, idx, d_v: int, scale: float, dtype: int) -> Tuple[np.ndarray, np.ndarray]:
    """(out [n_rows,H,d_v], lse [n_rows,H]) float64 over the selected rows.

    q [n_rows,H,d_qk] and kv [Lk,d_qk] as fp32 or as bf16 bit patterns.
    """
    qq = _np(q)
    kk = _np(kv)
    if dtype == BF16:
        qq = qq.view(np.uint16)
        kk = kk.view(np.uint16)
    else:
        qq = _np(qq, np.float32)
        kk = _np(kk, np.float32)
    ii = _np(idx, np.int32)
    n_rows, H, d_qk = qq.shape
    Lk = kk.shape[0]
    k = ii.shape[1]
    out = np.empty((n_rows, H, d_v), dtype=np.float64)
    lse = np.empty((n_rows, H), dtype=np.float64)
    rc = lib().orc_sparse_attn(_ptr(qq), _ptr(kk), dtype, _ptr(ii), n_rows, k, Lk, H,
                               d_qk, int(d_v), float(scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("orc_sparse_attn: bad arguments")
    return out, lse


def e4m3_encode(y: float) -> int:
    """Nearest e4m3fn code to the fp32 value y (ties to even, saturating)."""
    return int(lib().orc_e4m3_encode(float(y)))


def quantize_e4m3(x, token_dims: int = 1, repeat: int = 1, margin: float = 1.0):
    """Per-token FP8 quantisation of x (fp32 array or bf16/fp32 torch tensor).

    A token is the trailing ``token_dims`` dimensions.  Returns (codes uint8
    with x's shape, scales float32 [n_tokens, repeat])."""
    dtype = F32
    try:
        import torch
        if isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16:
            dtype = BF16
    except ImportError:
        pass
    a = _np(x) if dtype == BF16 else _np(x, np.float32)
    shape = a.shape
    tok_len = int(np.prod(shape[len(shape) - token_dims:]))
    n_tok = int(a.size // tok_len) if tok_len else 0
    codes = np.empty(shape, dtype=np.uint8)
    scales = np.empty((n_tok, repeat), dtype=np.float32)
    rc = lib().orc_quantize_e4m3(_ptr(a), dtype, n_tok, tok_len, int(repeat), float(margin),
                                 _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("orc_quantize_e4m3: bad arguments")
    return codes, scales


def rope_rows(nope, rope, pos, base: float = 10000.0) -> np.ndarray:
    """Assembled rows [n_tok, heads, d_nope + d_rope] float64.

    nope [n_tok, heads, d_nope] and rope [n_tok, heads, d_rope] as bf16 bit
    patterns (or bf16 torch tensors); pos [n_tok] int64 positions."""
    nn = _np(nope).view(np.uint16)
    rr = _np(rope).view(np.uint16)
    n_tok, heads, d_nope = nn.shape
    d_rope = rr.shape[2]
    assert rr.shape[:2] == (n_tok, heads)
    pp = _np(pos, np.int64)
    out = np.empty((n_tok, heads, d_nope + d_rope), dtype=np.float64)
    rc = lib().orc_rope_rows(_ptr(nn), _ptr(rr), n_tok, heads, d_nope, d_rope, _ptr(pp), float(base),
                             _ptr(out))
    if rc != 0:
        raise ValueError("orc_rope_rows: bad arguments")
    return out


KV_FP8_ROW_BYTES = 656


def kv_pack_fp8(kv) -> np.ndarray:
    """Packed FP8 rows [..., 656] uint8 of bf16 latent rows [..., 576]."""
    a = _np(kv).view(np.uint16)
    assert a.shape[-1] == 576
    n = int(a.size // 576)
    out = np.empty(a.shape[:-1] + (KV_FP8_ROW_BYTES,), dtype=np.uint8)
    if lib().orc_kv_pack_fp8(_ptr(a), n, _ptr(out)) != 0:
        raise ValueError("orc_kv_pack_fp8: bad arguments")
    return out


def kv_unpack_fp8(packed) -> np.ndarray:
    """The fp32 values [..., 576] that packed FP8 rows [..., 656] stand for."""
    a = _np(packed).view(np.uint8)
    assert a.shape[-1] == KV_FP8_ROW_BYTES
    n = int(a.size // KV_FP8_ROW_BYTES)
    out = np.empty(a.shape[:-1] + (576,), dtype=np.float32)
    if lib().orc_kv_unpack_fp8(_ptr(a), n, _ptr(out)) != 0:
        raise ValueError("orc_kv_unpack_fp8: bad arguments")
    return out


def sparse_attn_fp8kv(q, packed, idx, d_v: int, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over packed FP8 latent rows: the rows' fp32 values (exact)
    and the bf16 queries widened to fp32 (exact), then ``sparse_attn``."""
    kvf = kv_unpack_fp8(packed)
    qf = _np(q).view(np.uint16).astype(np.uint32) << 16
    return sparse_attn(qf.view(np.float32), kvf, idx, d_v, scale, F32)


def indexer_kl(q, kv, scores, t_pos, scale: float, dtype: int) -> np.ndarray:
    """KL(p_t || Softmax(I_t)) per row, float64 [n_rows]: p_t = the mean over
    heads of the dense attention distributions of q [n_rows,H,d_qk] over
    kv [Lk,d_qk] (rows s <= t_pos), I = scores [n_rows,Lk]."""
    qq = _np(q)
    kk = _np(kv)
    if dtype == BF16:
        qq = qq.view(np.uint16)
        kk = kk.view(np.uint16)
    else:
        qq = _np(qq, np.float32)
        kk = _np(kk, np.float32)
    n_rows, H, d_qk = qq.shape
    Lk = kk.shape[0]
    sc = _np(scores, np.float64)
    assert sc.shape == (n_rows, Lk)
    tp = _np(t_pos, np.int64)
    out = np.empty(n_rows, dtype=np.float64)
    if lib().orc_indexer_kl(_ptr(qq), _ptr(kk), dtype, _ptr(sc), _ptr(tp), n_rows, Lk, H, d_qk, float(scale),
                            _ptr(out)) != 0:
        raise ValueError("orc_indexer_kl: bad arguments")
    return out


def sparse_attn_bwd(q, kv, dout, idx, d_v: int, scale: float, dtype: int) -> Tuple[np.ndarray, np.ndarray]:
    """(dq [n_rows,H,d_qk], dkv [Lk,d_qk]) float64: gradients of sum(out * dout)
    for out = sparse_attn(q, kv, idx, d_v, scale) (fp32 or bf16 inputs)."""
    def prep(x):
        a = _np(x)
        return a.view(np.uint16) if dtype == BF16 else _np(a, np.float32)
    qq, kk, gg = prep(q), prep(kv), prep(dout)
    ii = _np(idx, np.int32)
    n_rows, H, d_qk = qq.shape
    Lk = kk.shape[0]
    k = ii.shape[1]
    assert gg.shape == (n_rows, H, d_v)
    dq = np.empty((n_rows, H, d_qk), dtype=np.float64)
    dkv = np.empty((Lk, d_qk), dtype=np.float64)
    if lib().orc_sparse_attn_bwd(_ptr(qq), _ptr(kk), _ptr(gg), dtype, _ptr(ii), n_rows, k, Lk, H, d_qk, int(d_v),
                                 float(scale), _ptr(dq), _ptr(dkv)) != 0:
        raise ValueError("orc_sparse_attn_bwd: bad arguments")
    return dq, dkv


def forward_rows(inp: dict, cfg, rows, with_scores: bool = False):
    """End-to-end oracle (scores -> top-k -> attention) for flattened rows.

    ``inp`` is a dict of host tensors as drawn by ``dsa_inputs.make_inputs``
    (or row-subsets of the query-side tensors when ``rows`` is given as the
    explicit list they were taken from).  Returns dict with idx, out, lse and
    optionally scores, all for the listed rows in order.
    """
    rows = np.asarray(rows, dtype=np.int64)
    dt = E4M3 if cfg.idx_dtype == "fp8" else F32
    io = BF16 if cfg.io_dtype == "bf16" else F32
    res = {"idx": [], "out": [], "lse": [], "scores": []}
    for b in np.unique(rows // cfg.Lq):
        sel = rows[rows // cfg.Lq == b]
        t = sel % cfg.Lq
        t_pos = cfg.q_pos0 + t
        qi = inp["q_idx"][b][t]
        qs = inp["q_scale"][b][t] if dt == E4M3 else None
        ks = inp["k_scale"][b] if dt == E4M3 else None
        sc = indexer(qi, qs, inp["k_idx"][b], ks, inp["w"][b][t], t_pos, dt)
        ix = topk(sc, t_pos, cfg.k)
        o, l = sparse_attn(inp["q"][b][t], inp["kv"][b], ix, cfg.d_v, cfg.softmax_scale, io)
        res["idx"].append(ix)
        res["out"].append(o)
        res["lse"].append(l)
        if with_scores:
            res["scores"].append(sc)
    # restore the caller's row order
    order = np.concatenate([np.nonzero(rows // cfg.Lq == b)[0] for b in np.unique(rows // cfg.Lq)])
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    outd = {k: np.concatenate(v)[inv] for k, v in res.items() if v}
    return outd
