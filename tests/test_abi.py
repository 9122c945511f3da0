"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments with the documented status before any launch.

No test here reaches a kernel launch: every call either fails validation or is
an empty problem (B == 0 or Lq == 0), which returns before touching HIP.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

OK, NULL, SHAPE, DTYPE, UNSUP, ALIGN, WS, HIP = range(8)
F32, BF16, FP8 = 0, 1, 2


@pytest.fixture(scope="module")
def L():
    from sparse_attention_04_amd import lib
    return lib


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert {"dsa_indexer_scores", "dsa_topk", "dsa_sparse_attn", "dsa_forward",
            "dsa_forward_workspace_size", "dsa_status_string", "dsa_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_exports_are_the_declared_entry_points(L):
    """The product library exports exactly the header's entry points (the
    measurement probe lives in a library of its own)."""
    import subprocess
    path = L._name
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln and ln.split()[-1].startswith("dsa_")})
    assert exported == _declared(), (exported, _declared())


def test_status_strings(L):
    for s in range(8):
        assert L.dsa_status_string(s)
    assert L.dsa_status_string(0) == b"ok"


A = 0x10000           # a fake, 16-byte aligned "device address": never dereferenced here
MIS = A + 4


def idx_scores(L, **kw):
    a = dict(q=A, qs=A, k=A, ks=A, w=A, sc=A, B=1, Lq=8, Lk=8, q0=0, H=64, D=128, dt=FP8)
    a.update(kw)
    return L.dsa_indexer_scores(a["q"], a["qs"], a["k"], a["ks"], a["w"], a["sc"], a["B"], a["Lq"],
                                a["Lk"], a["q0"], a["H"], a["D"], a["dt"], None)


def test_indexer_validation(L):
    assert idx_scores(L, q=None) == NULL
    assert idx_scores(L, qs=None) == NULL
    assert idx_scores(L, sc=None) == NULL
    assert idx_scores(L, k=MIS) == ALIGN
    assert idx_scores(L, Lq=9) == SHAPE                    # q_pos0 + Lq > Lk
    assert idx_scores(L, q0=1) == SHAPE
    assert idx_scores(L, Lk=-1) == SHAPE
    assert idx_scores(L, H=32) == UNSUP                    # FP8 built for 64 x 128
    assert idx_scores(L, D=64) == UNSUP
    assert idx_scores(L, dt=BF16) == DTYPE
    assert idx_scores(L, dt=F32) == DTYPE                  # scales given for F32
    assert idx_scores(L, dt=F32, qs=None, ks=None, D=30, H=4) == UNSUP
    assert b"q_pos0" in L.dsa_last_error() or L.dsa_last_error() != b""
    # empty problems are valid and launch nothing
    assert idx_scores(L, B=0) == OK
    assert idx_scores(L, Lq=0) == OK and L.dsa_last_error() == b""


def test_topk_validation(L):
    f = L.dsa_topk
    assert f(None, A, 1, 4, 4, 0, 2, None) == NULL
    assert f(A, None, 1, 4, 4, 0, 2, None) == NULL
    assert f(A, MIS, 1, 4, 4, 0, 2, None) == ALIGN
    assert f(A, A, 1, 4, 4, 0, 0, None) == SHAPE           # k < 1
    assert f(A, A, 1, 4, 4, 0, 5, None) == SHAPE           # k > Lk
    assert f(A, A, 1, 4, 4, 2, 2, None) == SHAPE           # q_pos0 + Lq > Lk
    assert f(A, A, 70000, 1, 4, 0, 2, None) == UNSUP       # grid y limit
    assert f(A, A, 1, 0, 4, 0, 2, None) == OK


def attn(L, **kw):
    a = dict(q=A, kv=A, idx=A, out=A, lse=None, B=1, Lq=4, Lk=8, q0=0, H=128, dqk=576, dv=512,
             k=4, scale=0.1, dt=BF16)
    a.update(kw)
    return L.dsa_sparse_attn(a["q"], a["kv"], a["idx"], a["out"], a["lse"], a["B"], a["Lq"], a["Lk"],
                             a["q0"], a["H"], a["dqk"], a["dv"], a["k"], a["scale"], a["dt"], None, 0, None)


def test_attention_validation(L):
    assert attn(L, q=None) == NULL
    assert attn(L, idx=None) == NULL
    assert attn(L, lse=MIS) == ALIGN
    assert attn(L, dv=600) == SHAPE                        # d_v > d_qk
    assert attn(L, scale=0.0) == SHAPE
    assert attn(L, scale=float("nan")) == SHAPE
    assert attn(L, k=0) == SHAPE
    assert attn(L, H=24) == UNSUP                          # bf16 needs H % 16 == 0
    assert attn(L, H=144) == UNSUP
    assert attn(L, dqk=256, dv=256) == UNSUP
    assert attn(L, dt=FP8) == DTYPE
    assert attn(L, dt=F32, k=5000) == UNSUP
    assert attn(L, B=0) == OK


def test_attention_split_workspace(L):
    ws = L.dsa_sparse_attn_workspace_size
    part = lambda rows, ns, H=128, dv=512: rows * ns * H * (dv + 1) * 4
    assert ws(64, 1, 128, 576, 512, 2048, BF16) == part(64, 4)        # decode batch: 4 splits
    assert ws(1, 8, 128, 576, 512, 2048, BF16) == part(8, 8)          # at most 8 splits
    assert ws(1, 8, 32, 576, 512, 2048, BF16) == part(8, 8, H=32)
    assert ws(1, 8, 128, 576, 512, 256, BF16) == part(8, 2)           # at least 4 chunks of 32 per split
    assert ws(1, 128, 128, 576, 512, 2048, BF16) == 256               # enough rows: no split, the row counter
    assert ws(1, 8, 128, 576, 512, 64, BF16) == 256                   # too few chunks to split
    assert ws(1, 8, 128, 576, 512, 2048, F32) == 0
    assert ws(1, 8, 16, 576, 512, 2048, BF16) == 0
    assert ws(1, 8, 96, 576, 512, 2048, BF16) == 0
    assert ws(1, 8, 128, 128, 128, 2048, BF16) == 0
    assert ws(0, 8, 128, 576, 512, 2048, BF16) == 0


AUTO_TILE_BYTES = 4 << 30      # the forward's automatic query tile: score tile cap
SEL_AUTO, SEL_TILES, SEL_CAND = 0, 1, 2


def _r256(x):
    return (x + 255) // 256 * 256


def _cand_extra(B, Lq, Lk, k):
    """Candidate-route workspace beyond the score-tile route's: per row the
    sample scores (every 2^r-th key, r = max(0, floor(log2(k / 128))), padded
    to 4), tau, the list length, the flag and the list of 2k (score, s) pairs,
    and the list pass's 256-byte block counter."""
    r = 0
    while (128 << (r + 1)) <= k:
        r += 1
    ls_pad = ((((Lk - 1) >> r) + 1) + 3) // 4 * 4
    rows = B * Lq
    return _r256(rows * ls_pad * 4) + 3 * _r256(rows * 4) + _r256(rows * 2 * k * 8) + 256


def test_forward_workspace(L):
    ws = lambda B, Lq, Lk, k, T, sel=SEL_TILES: L.dsa_forward_workspace_size(B, Lq, Lk, k, 128, 576, 512, BF16,
                                                                            T, sel)
    # score tiles: one tile of scores plus the selected sets of every row (the
    # attention runs once over all rows after the last tile)
    # (plus 256 bytes: the attention's row counter)
    assert ws(1, 32768, 32768, 2048, 1024) == 1024 * 32768 * 4 + 32768 * 2048 * 4 + 256
    assert ws(1, 131072, 131072, 2048, 4096) == 4096 * 131072 * 4 + 131072 * 2048 * 4 + 256
    # auto tile: the largest score tile within AUTO_TILE_BYTES
    for Lk in (4096, 32768, 131072):
        T = min(Lk, AUTO_TILE_BYTES // (Lk * 4))
        tiles = T * Lk * 4 + Lk * 2048 * 4 + 256
        assert ws(1, Lk, Lk, 2048, 0) == tiles
        # candidates on top of the fallback tiles
        assert ws(1, Lk, Lk, 2048, 0, SEL_CAND) == tiles + _cand_extra(1, Lk, Lk, 2048)
        # AUTO takes candidates from 1024 blocks of 16 rows up (not at L = 4096)
        assert ws(1, Lk, Lk, 2048, 0, SEL_AUTO) == (tiles if Lk == 4096 else tiles + _cand_extra(1, Lk, Lk, 2048))
    assert ws(1, 32768, 32768, 512, 0, SEL_AUTO) == ws(1, 32768, 32768, 512, 0)      # k < 1024: tiles
    assert ws(1, 300, 300, 64, 0, SEL_CAND) == ws(1, 300, 300, 64, 0) + _cand_extra(1, 300, 300, 64)
    # decode batch: scores, indices and the attention's split partials (4 splits)
    assert ws(64, 1, 65536, 2048, 0) == 64 * 65536 * 4 + 64 * 2048 * 4 + 64 * 4 * 128 * 513 * 4
    assert ws(64, 1, 65536, 2048, 0, SEL_AUTO) == ws(64, 1, 65536, 2048, 0)
    # routes that do not take the problem, and unknown routes
    assert ws(64, 1, 65536, 2048, 0, SEL_CAND) == 0                 # Lq < 8
    assert ws(1, 8192, 8192, 3000, 0, SEL_CAND) == 0                # k > 2048
    assert ws(1, 1 << 14, 1 << 14, 64, 0, SEL_CAND) == 0            # a sample of 16384 keys
    assert ws(1, 131072, 131072, 2048, 4096, SEL_CAND) > 0         # a sample of 8192 keys
    assert ws(1, 8, 8, 4, 0, 3) == 0 and ws(1, 8, 8, 4, -1) == 0
    assert ws(0, 1, 1, 1, 0) == 0
    need = ws(1, 8, 8, 4, 0)

    def fwd(workspace, nbytes, **kw):
        a = dict(H=64, D=128, dt=FP8, Hq=128, dqk=576, dv=512, io=BF16, k=4, T=0, sel=SEL_AUTO)
        a.update(kw)
        return L.dsa_forward(A, A, A, A, A, a["H"], a["D"], a["dt"], A, A, a["Hq"], a["dqk"], a["dv"],
                             a["io"], 0.1, 1, 8, 8, 0, a["k"], None, A, None, a["T"], a["sel"], workspace,
                             nbytes, None)

    assert fwd(None, need) == WS
    assert fwd(A, need - 1) == WS
    assert fwd(A + 16, need) == WS                          # not 256-byte aligned
    assert fwd(A, need, k=9) == SHAPE
    assert fwd(A, need, T=-1) == SHAPE
    assert fwd(A, need, H=16) == UNSUP
    assert fwd(A, need, io=FP8) == DTYPE
    assert fwd(A, need, sel=3) == SHAPE
    assert fwd(A, need, sel=SEL_CAND) == WS                 # the candidate route needs more
    # the candidate route on fp32 indexer inputs (no scales)
    assert L.dsa_forward(A, None, A, None, A, 4, 32, F32, A, A, 128, 576, 512, BF16, 0.1, 1, 8, 8, 0, 4, None, A,
                         None, 0, SEL_CAND, A, ws(1, 8, 8, 4, 0, SEL_CAND), None) == UNSUP


def test_quantize_validation(L):
    def q(**kw):
        a = dict(x=A, dt=F32, c=A, s=A, n=4, t=128, r=1, m=1.0)
        a.update(kw)
        return L.dsa_quantize_e4m3(a["x"], a["dt"], a["c"], a["s"], a["n"], a["t"], a["r"], a["m"], None)
    assert q(x=None) == NULL and q(c=None) == NULL and q(s=None) == NULL
    assert q(x=MIS) == ALIGN
    assert q(dt=FP8) == DTYPE
    assert q(t=12) == UNSUP and q(t=0) == UNSUP and q(t=16392) == UNSUP
    assert q(r=0) == SHAPE and q(n=-1) == SHAPE
    assert q(m=0.0) == SHAPE and q(m=float("inf")) == SHAPE and q(m=float("nan")) == SHAPE
    assert q(n=0, x=None) == OK                     # empty: nothing to do


def test_rope_assemble_validation(L):
    def r(**kw):
        a = dict(n=A, r=A, o=A, B=1, L=4, h=1, dn=512, dr=64, p0=0, base=10000.0)
        a.update(kw)
        return L.dsa_rope_assemble(a["n"], a["r"], a["o"], a["B"], a["L"], a["h"], a["dn"], a["dr"], a["p0"],
                                   a["base"], None)
    assert r(r=None) == NULL and r(o=None) == NULL and r(n=None) == NULL
    assert r(n=None, dn=0, B=0) == OK               # no compressed part, empty problem
    assert r(o=MIS) == ALIGN
    assert r(dr=6) == UNSUP and r(dr=136) == UNSUP and r(dn=4) == UNSUP and r(dr=0) == UNSUP
    assert r(base=1.0) == SHAPE and r(base=float("nan")) == SHAPE
    assert r(h=0) == SHAPE and r(p0=-1) == SHAPE and r(B=-1) == SHAPE
    assert r(B=0) == OK and r(L=0) == OK
