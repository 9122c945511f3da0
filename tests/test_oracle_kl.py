"""Pins of the oracle's indexer distillation loss ("DeepseekV3.2 拆解",
section 预训练策略, dense warm-up stage: L^I = sum_t KL(p_t || Softmax(I_t))),
with p_t read as the mean over heads of the main attention's dense
distributions over the keys s <= t.

The loss is pinned to torch's own softmax / log_softmax / kl_div computed in
float64 from the raw inputs, to the invariants of a KL divergence (>= 0, zero
exactly when the indexer's softmax equals p, unchanged by a constant shift of
the scores) and to a closed form for one head against uniform scores.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, F32

rng = np.random.default_rng(99)


def _case(n_rows=6, Lk=40, H=3, D=16, dtype=torch.float32, seed=0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(n_rows, H, D, generator=g, dtype=torch.float64).to(dtype)
    kv = torch.randn(Lk, D, generator=g, dtype=torch.float64).to(dtype)
    t_pos = np.sort(rng.choice(Lk, n_rows, replace=False)).astype(np.int64)
    I = torch.randn(n_rows, Lk, generator=g, dtype=torch.float64) * 2
    return q, kv, t_pos, I


def _torch_kl(q, kv, t_pos, I, scale):
    """Independent float64 evaluation with torch library routines."""
    qd, kd = q.double(), kv.double()
    out = []
    for r in range(q.shape[0]):
        n = int(t_pos[r]) + 1
        z = scale * (qd[r] @ kd[:n].T)                      # [H, n]
        p = torch.softmax(z, dim=1).mean(dim=0)             # mean over heads
        logpi = torch.log_softmax(I[r, :n].double(), dim=0)
        out.append(torch.nn.functional.kl_div(logpi, p, reduction="sum").item())
    return np.array(out)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_kl_matches_torch_kl_div(dtype):
    q, kv, t_pos, I = _case(dtype=dtype)
    dt = F32 if dtype == torch.float32 else BF16
    ours = oracle.indexer_kl(q, kv, I.numpy(), t_pos, 0.3, dt)
    np.testing.assert_allclose(ours, _torch_kl(q, kv, t_pos, I, 0.3), rtol=1e-10, atol=1e-12)


def test_kl_is_nonnegative_and_zero_when_scores_are_log_p():
    q, kv, t_pos, I = _case(n_rows=8, Lk=50, H=4, seed=3)
    kl = oracle.indexer_kl(q, kv, I.numpy(), t_pos, 0.25, F32)
    assert np.all(kl >= 0) and np.all(kl > 1e-6)
    # scores equal to log p (+ any constant) make the indexer's softmax equal p
    I2 = torch.full_like(I, -1e30)
    for r in range(q.shape[0]):
        n = int(t_pos[r]) + 1
        z = 0.25 * (q[r].double() @ kv[:n].double().T)
        I2[r, :n] = torch.log(torch.softmax(z, dim=1).mean(dim=0)) + 7.5
    kl0 = oracle.indexer_kl(q, kv, I2.numpy(), t_pos, 0.25, F32)
    np.testing.assert_allclose(kl0, 0.0, atol=1e-12)


def test_kl_shift_invariance_and_single_key():
    q, kv, t_pos, I = _case(n_rows=5, seed=4)
    a = oracle.indexer_kl(q, kv, I.numpy(), t_pos, 0.5, F32)
    b = oracle.indexer_kl(q, kv, (I + 123.0).numpy(), t_pos, 0.5, F32)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    one = oracle.indexer_kl(q[:1], kv, I[:1].numpy(), np.array([0]), 0.5, F32)
    assert one[0] == 0.0                                 # one key: both distributions are [1]


def test_kl_one_head_against_uniform_scores_is_log_n_minus_entropy():
    q, kv, t_pos, _ = _case(n_rows=4, H=1, seed=5)
    I = torch.zeros(4, kv.shape[0], dtype=torch.float64)
    kl = oracle.indexer_kl(q, kv, I.numpy(), t_pos, 0.4, F32)
    for r in range(4):
        n = int(t_pos[r]) + 1
        p = torch.softmax(0.4 * (q[r, 0].double() @ kv[:n].double().T), dim=0)
        ent = -(p * torch.log(p)).sum().item()
        assert kl[r] == pytest.approx(math.log(n) - ent, rel=1e-10, abs=1e-12)
