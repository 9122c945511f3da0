"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a library routine, a closed form, an
invariant the definition implies, or brute force on tiny inputs, so that a
dropped term, a wrong sign or index, or a transposed operand fails at least
one of them.  The definitions pinned are those of "DeepseekV3.2 拆解", section
核心组件 (indexer score, top-k selection, attention over the selected set).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, E4M3, F32

rng = np.random.default_rng(1234)


# ---------------------------------------------------------------- e4m3 decode

def test_e4m3_table_matches_torch_cast():
    """All 256 codes against torch's float8_e4m3fn -> float32 conversion."""
    ours = oracle.e4m3_table()
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan_o, nan_r = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_o, nan_r)
    assert np.array_equal(ours[~nan_o], ref[~nan_r])
    # signed zero preserved
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_e4m3_closed_forms():
    assert oracle.e4m3_value(0x7E) == 448.0                # S.1111.110: 1.75 * 2^8
    assert oracle.e4m3_value(0xFE) == -448.0
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e4m3_value(0x01) == 2.0 ** -9              # smallest subnormal
    assert oracle.e4m3_value(0x08) == 2.0 ** -6              # smallest normal
    assert oracle.e4m3_value(0x38) == 1.0                    # exponent field = bias
    assert oracle.e4m3_value(0x3C) == 1.5


# ---------------------------------------------------------------- indexer

def _f32(*shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)


def test_indexer_hand_example():
    """Two heads, two dims, three tokens, small integers: exact by hand."""
    q = np.array([[[1, 2], [0, 1]],      # query row t=2: head0 (1,2), head1 (0,1)
                  ], dtype=np.float32)
    k = np.array([[3, -1], [-2, -2], [1, 1]], dtype=np.float32)
    w = np.array([[2.0, -3.0]], dtype=np.float32)
    s = oracle.indexer(q, None, k, None, w, np.array([2]), F32)
    # s=0: head0 dot 3-2=1 -> 2*1; head1 dot -1 -> relu 0        => 2
    # s=1: head0 dot -2-4=-6 -> 0;  head1 dot -2 -> 0             => 0
    # s=2: head0 dot 1+2=3 -> 6;    head1 dot 1 -> -3*1 = -3      => 3
    assert s.tolist() == [[2.0, 0.0, 3.0]]
    s1 = oracle.indexer(q, None, k, None, w, np.array([1]), F32)
    assert s1[0, 0] == 2.0 and s1[0, 1] == 0.0 and s1[0, 2] == -np.inf


def test_indexer_single_head_is_relu_gemm():
    """H^I = 1, w = 1: I = max(0, Q K^T) on the causal triangle."""
    L, D = 40, 32
    Q = _f32(L, 1, D)
    K = _f32(L, D)
    t_pos = np.arange(L)
    s = oracle.indexer(Q, None, K, None, np.ones((L, 1), np.float32), t_pos, F32)
    ref = np.maximum(Q[:, 0, :].astype(np.float64) @ K.astype(np.float64).T, 0.0)
    mask = np.tril(np.ones((L, L), bool))
    assert np.allclose(s[mask], ref[mask], rtol=1e-12, atol=1e-12)
    assert np.all(s[~mask] == -np.inf)


def test_indexer_two_heads_signed_weights():
    """w = (1, -1): difference of two ReLU GEMMs (catches a dropped sign/head)."""
    L, D = 33, 16
    Q = _f32(L, 2, D)
    K = _f32(L, D)
    w = np.tile(np.array([[1.0, -1.0]], np.float32), (L, 1))
    s = oracle.indexer(Q, None, K, None, w, np.arange(L), F32)
    Qd, Kd = Q.astype(np.float64), K.astype(np.float64)
    ref = np.maximum(Qd[:, 0] @ Kd.T, 0) - np.maximum(Qd[:, 1] @ Kd.T, 0)
    mask = np.tril(np.ones((L, L), bool))
    assert np.allclose(s[mask], ref[mask], rtol=1e-12, atol=1e-12)


def test_indexer_linear_in_w_and_head_permutation():
    L, H, D = 24, 5, 8
    Q = _f32(L, H, D)
    K = _f32(L, D)
    w1, w2 = _f32(L, H), _f32(L, H)
    tp = np.arange(L)
    a = oracle.indexer(Q, None, K, None, w1, tp, F32)
    b = oracle.indexer(Q, None, K, None, w2, tp, F32)
    c = oracle.indexer(Q, None, K, None, (2 * w1 + 3 * w2).astype(np.float32), tp, F32)
    m = np.tril(np.ones((L, L), bool))
    assert np.allclose(c[m], 2 * a[m] + 3 * b[m], rtol=1e-6, atol=1e-6)
    perm = rng.permutation(H)
    p = oracle.indexer(Q[:, perm], None, K, None, w1[:, perm], tp, F32)
    assert np.allclose(p[m], a[m], rtol=1e-12, atol=1e-12)


def test_indexer_all_negative_dots_give_zero():
    L, H, D = 10, 3, 4
    Q = np.abs(_f32(L, H, D)) + 0.1
    K = -(np.abs(_f32(L, D)) + 0.1)
    s = oracle.indexer(Q.astype(np.float32), None, K.astype(np.float32), None, _f32(L, H),
                       np.arange(L), F32)
    assert np.all(s[np.tril(np.ones((L, L), bool))] == 0.0)


def test_indexer_fp8_matches_torch_dequantised():
    """FP8 path = f32 path on inputs dequantised with torch's own cast."""
    L, H, D = 20, 4, 16
    qc = torch.randint(0, 256, (L, H, D), dtype=torch.uint8)
    kc = torch.randint(0, 256, (L, D), dtype=torch.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x11      # no NaN codes
    kc[(kc & 0x7F) == 0x7F] = 0x22
    qs = torch.rand(L, H) + 0.5
    ks = torch.rand(L) + 0.5
    w = torch.randn(L, H)
    tp = np.arange(L) + 3
    Lk = L + 3
    kc2 = torch.cat([kc, kc[:3]])
    ks2 = torch.cat([ks, ks[:3]])
    a = oracle.indexer(qc, qs, kc2, ks2, w, tp, E4M3)
    qhat = (qc.view(torch.float8_e4m3fn).float() * qs[:, :, None]).numpy()
    khat = (kc2.view(torch.float8_e4m3fn).float() * ks2[:, None]).numpy()
    b = oracle.indexer(qhat, None, khat, None, w, tp, F32)
    assert a.shape == (L, Lk)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- top-k

def _topk_bruteforce(row: np.ndarray, t_pos: int, k: int) -> np.ndarray:
    n = t_pos + 1
    v = row[:n].astype(np.float64)
    v = np.where(v == 0.0, 0.0, v)
    order = np.lexsort((np.arange(n), -v))        # score desc, then index asc
    sel = np.sort(order[:min(k, n)])
    out = -np.ones(k, np.int32)
    out[:sel.size] = sel
    return out


def test_topk_matches_lexsort_with_heavy_ties():
    L, k = 300, 37
    S = rng.integers(-4, 5, size=(L, L)).astype(np.float64)   # many exact ties
    tp = np.arange(L)
    got = oracle.topk(S, tp, k)
    for t in range(L):
        assert np.array_equal(got[t], _topk_bruteforce(S[t], t, k)), t


def test_topk_signed_zero_is_one_value():
    row = np.array([[-0.0, 0.0, -0.0, 1.0, 0.0, -1.0]])
    got = oracle.topk(row, np.array([5]), 3)
    assert got.tolist() == [[0, 1, 3]]            # 1.0 first, then zeros by index


def test_topk_invariants_random():
    L, k = 257, 64
    S = rng.standard_normal((L, L))
    tp = np.arange(L)
    got = oracle.topk(S, tp, k)
    for t in range(L):
        n = t + 1
        sel = got[t][got[t] >= 0]
        assert sel.size == min(k, n)
        assert np.all(got[t][sel.size:] == -1)
        assert np.all(np.diff(sel) > 0) and sel.max() <= t
        rest = np.setdiff1d(np.arange(n), sel)
        if rest.size:
            assert S[t, sel].min() >= S[t, rest].max()


def test_topk_planted_cases():
    k = 16
    const = np.full((1, 100), 0.5)
    assert oracle.topk(const, np.array([99]), k)[0].tolist() == list(range(k))
    short = rng.standard_normal((1, 100))
    assert oracle.topk(short, np.array([9]), k)[0].tolist() == list(range(10)) + [-1] * 6
    ramp = np.arange(100, dtype=np.float64)[None]
    assert oracle.topk(ramp, np.array([99]), k)[0].tolist() == list(range(84, 100))
    # only s <= t_pos may be read: huge values past t_pos are ignored
    spiky = np.zeros((1, 100)); spiky[0, 50:] = 1e9
    assert oracle.topk(spiky, np.array([40]), 4)[0].tolist() == [0, 1, 2, 3]


# ---------------------------------------------------------------- attention

def _sdpa_masked(q, kv, d_v, scale, mask):
    """torch SDPA in fp64 on the CPU: q [L,H,D], kv [Lk,D], mask [L,Lk] bool."""
    Q = torch.as_tensor(q, dtype=torch.float64).permute(1, 0, 2)           # H,L,D
    K = torch.as_tensor(kv, dtype=torch.float64)[None].expand(Q.shape[0], -1, -1)
    V = K[..., :d_v]
    o = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=torch.as_tensor(mask)[None], scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_attention_k_ge_L_is_causal_dense_attention():
    """With k >= L every preceding token is kept: DSA == causal attention."""
    L, H, D = 48, 4, 64
    q = _f32(L, H, D)
    kv = _f32(L, D)
    idx = np.tile(np.arange(L, dtype=np.int32), (L, 1))
    idx[np.triu(np.ones((L, L), bool), 1)] = -1           # row t keeps 0..t
    out, lse = oracle.sparse_attn(q, kv, idx, D, 0.125, F32)
    Q = torch.as_tensor(q, dtype=torch.float64).permute(1, 0, 2)
    K = torch.as_tensor(kv, dtype=torch.float64)[None].expand(H, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, K, is_causal=True, scale=0.125)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_attention_sparse_set_matches_masked_sdpa_and_value_prefix():
    L, H, Dqk, Dv, k = 40, 3, 48, 32, 7
    q = _f32(L, H, Dqk)
    kv = _f32(L, Dqk)
    idx = -np.ones((L, k), np.int32)
    mask = np.zeros((L, L), bool)
    for t in range(L):
        sel = np.sort(rng.choice(t + 1, size=min(k, t + 1), replace=False))
        idx[t, :sel.size] = sel
        mask[t, sel] = True
    out, lse = oracle.sparse_attn(q, kv, idx, Dv, 0.2, F32)
    ref = _sdpa_masked(q, kv, Dv, 0.2, mask)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12)
    # lse consistency: sum_s exp(z_s - lse) == 1, z computed independently
    z = 0.2 * np.einsum("thd,sd->ths", q.astype(np.float64), kv.astype(np.float64))
    tot = np.where(mask[:, None, :], np.exp(z - lse[:, :, None]), 0.0).sum(-1)
    assert np.allclose(tot, 1.0, rtol=1e-12)


def test_attention_single_row_returns_value_exactly_and_order_invariance():
    L, H, D = 20, 2, 32
    q = _f32(L, H, D)
    kv = _f32(L, D)
    idx = np.full((L, 4), -1, np.int32)
    idx[:, 0] = rng.integers(0, L, size=L)
    out, _ = oracle.sparse_attn(q, kv, idx, D, 1.0, F32)
    assert np.array_equal(out, np.broadcast_to(kv[idx[:, 0]][:, None, :].astype(np.float64), out.shape))
    idx2 = np.stack([rng.permutation(L)[:6] for _ in range(L)]).astype(np.int32)
    a, la = oracle.sparse_attn(q, kv, idx2, D, 0.3, F32)
    b, lb = oracle.sparse_attn(q, kv, idx2[:, ::-1].copy(), D, 0.3, F32)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14) and np.allclose(la, lb, rtol=1e-13)


def test_attention_bf16_decode_matches_torch_upcast():
    L, H, D = 16, 2, 32
    qb = torch.randn(L, H, D).to(torch.bfloat16)
    kvb = torch.randn(L, D).to(torch.bfloat16)
    idx = np.tile(np.arange(L, dtype=np.int32), (L, 1))
    a, la = oracle.sparse_attn(qb, kvb, idx, D, 0.25, BF16)
    b, lb = oracle.sparse_attn(qb.float().numpy(), kvb.float().numpy(), idx, D, 0.25, F32)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_attention_empty_set():
    q = _f32(1, 2, 16)
    kv = _f32(4, 16)
    out, lse = oracle.sparse_attn(q, kv, np.full((1, 3), -1, np.int32), 16, 1.0, F32)
    assert np.all(out == 0) and np.all(lse == -np.inf)


# ---------------------------------------------------------------- composition

def test_forward_rows_dense_special_case_on_tiny_config():
    """Tiny fp32 workload with k >= L: the end-to-end oracle ignores the
    indexer and equals causal dense attention."""
    from dsa_inputs import CONFIGS, make_inputs
    cfg = CONFIGS["tiny_fp32_L256"].with_(k=256)
    inp = make_inputs(cfg, seed=0)
    rows = np.arange(cfg.Lq)
    res = oracle.forward_rows(inp, cfg, rows)
    assert np.all(res["idx"][:, 0] == 0)
    Q = inp["q"][0].double().permute(1, 0, 2)
    K = inp["kv"][0].double()[None].expand(cfg.n_heads, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, K, is_causal=True,
                                                           scale=cfg.softmax_scale)
    assert np.allclose(res["out"], ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_forward_rows_selects_from_indexer_scores():
    from dsa_inputs import CONFIGS, make_inputs
    cfg = CONFIGS["tiny_fp32_L256"]
    inp = make_inputs(cfg, seed=0)
    rows = np.array([0, 5, 31, 32, 100, 255])
    res = oracle.forward_rows(inp, cfg, rows, with_scores=True)
    for i, r in enumerate(rows):
        sc = res["scores"][i]
        assert np.array_equal(res["idx"][i], _topk_bruteforce(sc, int(r), cfg.k))


def test_abs_mass_bounds_the_score():
    """M = sum_j |w_j| sum_d |q_jd k_d| >= |I| everywhere (triangle inequality),
    with equality when every term is non-negative."""
    L, H, D = 30, 4, 16
    Q, K, w = _f32(L, H, D), _f32(L, D), _f32(L, H)
    tp = np.arange(L)
    I = oracle.indexer(Q, None, K, None, w, tp, F32)
    M = oracle.indexer_abs_mass(Q, None, K, None, w, tp, F32)
    m = np.tril(np.ones((L, L), bool))
    assert np.all(M[m] >= np.abs(I[m]) - 1e-12)
    Qp, Kp, wp = np.abs(Q), np.abs(K), np.abs(w)
    assert np.allclose(oracle.indexer(Qp, None, Kp, None, wp, tp, F32)[m],
                       oracle.indexer_abs_mass(Q, None, K, None, w, tp, F32)[m], rtol=1e-12)
