"""Pins of the oracle's sparse-attention backward (the sparse training stage
of "DeepseekV3.2 拆解", section 预训练策略: the main model is trained through
the selected sets).

Pinned to torch autograd in float64 on the dense formulation (gather the
selected rows, softmax, weighted sum; duplicates and -1 entries included), and
to central finite differences of the oracle's own forward, so a dropped term,
a wrong sign or a transposed operand in either gradient fails.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, F32

rng = np.random.default_rng(2024)


def _case(n_rows=5, Lk=30, H=3, dqk=24, dv=16, k=9, seed=0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(n_rows, H, dqk, generator=g)
    kv = torch.randn(Lk, dqk, generator=g)
    dout = torch.randn(n_rows, H, dv, generator=g)
    idx = torch.randint(0, Lk, (n_rows, k), generator=g, dtype=torch.int32)
    idx[0, 3:] = -1                       # short set
    idx[1, :] = -1                        # empty set
    idx[2, 4] = idx[2, 2]                 # a duplicate
    return q, kv, dout, idx


def _autograd(q, kv, dout, idx, dv, scale):
    qd = q.double().requires_grad_(True)
    kd = kv.double().requires_grad_(True)
    outs = []
    for r in range(q.shape[0]):
        sel = idx[r][idx[r] >= 0].long()
        if sel.numel() == 0:
            outs.append(torch.zeros(q.shape[1], dv, dtype=torch.float64))
            continue
        rows = kd[sel]                                   # [n, dqk]
        p = torch.softmax(scale * qd[r] @ rows.T, dim=1)  # [H, n]
        outs.append(p @ rows[:, :dv])
    loss = (torch.stack(outs) * dout.double()).sum()
    loss.backward()
    return qd.grad.numpy(), kd.grad.numpy()


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_backward_matches_autograd(dtype):
    q, kv, dout, idx = _case()
    if dtype == BF16:
        q, kv, dout = q.to(torch.bfloat16), kv.to(torch.bfloat16), dout.to(torch.bfloat16)
    dq, dkv = oracle.sparse_attn_bwd(q, kv, dout, idx.numpy(), 16, 0.3, dtype)
    rq, rkv = _autograd(q.float(), kv.float(), dout.float(), idx, 16, 0.3)
    np.testing.assert_allclose(dq, rq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dkv, rkv, rtol=1e-10, atol=1e-12)
    assert np.all(dq[1] == 0)                            # empty set: no gradient


def test_backward_matches_finite_differences_of_the_forward():
    """Inputs on a 2^-8 grid and steps of 2^-10, so every perturbed input is
    exact in fp32 and the oracle's forward sees exactly what it should."""
    q, kv, dout, idx = _case(n_rows=4, Lk=12, H=2, dqk=8, dv=6, k=5, seed=1)
    q = torch.round(q * 256) / 256
    kv = torch.round(kv * 256) / 256
    scale, eps = 0.5, 2.0 ** -10

    def loss(qq, kk):
        o, _ = oracle.sparse_attn(qq, kk, idx.numpy(), 6, scale, F32)
        return float((o * dout.double().numpy()).sum())

    dq, dkv = oracle.sparse_attn_bwd(q, kv, dout, idx.numpy(), 6, scale, F32)
    for _ in range(6):
        u = torch.from_numpy(rng.integers(-1, 2, q.shape).astype(np.float32))
        fd = (loss(q + eps * u, kv) - loss(q - eps * u, kv)) / (2 * eps)
        assert fd == pytest.approx(float((dq * u.double().numpy()).sum()), rel=1e-5, abs=1e-7)
        w = torch.from_numpy(rng.integers(-1, 2, kv.shape).astype(np.float32))
        fd = (loss(q, kv + eps * w) - loss(q, kv - eps * w)) / (2 * eps)
        assert fd == pytest.approx(float((dkv * w.double().numpy()).sum()), rel=1e-5, abs=1e-7)
