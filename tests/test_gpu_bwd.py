"""GPU parity of the sparse-attention backward (the sparse training stage of
"DeepseekV3.2 拆解", section 预训练策略) through the C ABI.

Tolerance, per gradient tensor: |g - g_oracle| <= 2^-6 max|g_oracle| element
by element, and ||g - g_oracle||_2 <= 2^-7 ||g_oracle||_2.  The kernels feed P
and dZ to the matrix cores in bf16 (relative rounding 2^-9 each) and take
D = dout . out from the bf16 forward output; summed over up to 2048 selected
rows whose terms largely cancel, these roundings stay within a few 2^-9 of the
largest terms, i.e. of max|g|.  Everything else is fp32.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def dsa(gpu):
    import sparse_attention_04_amd as m
    return m


def _compare(name, g, ref):
    err = np.abs(g.astype(np.float64) - ref)
    amax = np.abs(ref).max()
    rel2 = np.linalg.norm(g.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)
    assert err.max() <= 2.0 ** -6 * amax, f"{name}: max err {err.max():.3g} vs max|ref| {amax:.3g}"
    assert rel2 <= 2.0 ** -7, f"{name}: relative L2 error {rel2:.3g}"
    return float(err.max() / max(amax, 1e-300)), float(rel2)


def _case(dsa, B, Lq, Lk, H, k, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn(B, Lq, H, 576, device=DEV, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, Lk, 576, device=DEV, generator=g).to(torch.bfloat16)
    dout = torch.randn(B, Lq, H, 512, device=DEV, generator=g).to(torch.bfloat16)
    idx = torch.randint(0, Lk, (B, Lq, k), device=DEV, generator=g, dtype=torch.int32)
    idx[0, 0, k // 3:] = -1                          # short set (chunks past it not visited)
    if Lq > 1:
        idx[0, 1, :] = -1                            # empty set: zero dq
    if Lq > 2:
        idx[0, 2, 5] = idx[0, 2, 3]                  # a duplicate counts twice
    scale = 192 ** -0.5
    out, lse = dsa.dsa_sparse_attn(q, kv, idx, 512, scale, q_pos0=Lk - Lq, split=False)
    dq, dkv = dsa.dsa_sparse_attn_bwd(q, kv, idx, out, lse, dout, scale, q_pos0=Lk - Lq)
    torch.cuda.synchronize()
    return q, kv, dout, idx, scale, dq, dkv


@pytest.mark.parametrize("B,Lq,Lk,H,k", [(1, 40, 300, 16, 64), (2, 12, 2000, 128, 2048), (1, 33, 900, 32, 256),
                                         (2, 9, 700, 64, 100)])
def test_backward_matches_oracle(dsa, B, Lq, Lk, H, k):
    q, kv, dout, idx, scale, dq, dkv = _case(dsa, B, Lq, Lk, H, k, seed=B * 7 + H)
    assert torch.all(dq[0, 1] == 0)
    for b in range(B):
        rq, rkv = oracle.sparse_attn_bwd(q[b].cpu(), kv[b].cpu(), dout[b].cpu(), idx[b].cpu().numpy(), 512, scale,
                                         oracle.BF16)
        eq = _compare("dq", dq[b].cpu().numpy(), rq)
        ekv = _compare("dkv", dkv[b].cpu().numpy(), rkv)
        print(f"  [bwd B={B} Lq={Lq} H={H} k={k} b={b}] dq max/amax {eq[0]:.2e} L2 {eq[1]:.2e}; "
              f"dkv max/amax {ekv[0]:.2e} L2 {ekv[1]:.2e}", flush=True)


def test_backward_rows_not_selected_get_zero_and_dq_is_deterministic(dsa):
    q, kv, dout, idx, scale, dq, dkv = _case(dsa, 1, 6, 500, 32, 40, seed=3)
    sel = set(idx[0][idx[0] >= 0].cpu().numpy().tolist())
    unsel = [s for s in range(500) if s not in sel]
    assert torch.all(dkv[0, unsel] == 0)
    out, lse = dsa.dsa_sparse_attn(q, kv, idx, 512, scale, q_pos0=494, split=False)
    dq2, _ = dsa.dsa_sparse_attn_bwd(q, kv, idx, out, lse, dout, scale, q_pos0=494)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2)
