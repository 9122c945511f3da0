"""GPU parity of the 576/512 attention kernel's second pass.

The kernel scores a query's selected rows against a per-head reference
maximum fixed at the first chunk (32 rows) of its list that holds a valid
row, so that the output accumulators are never rescaled.  When a later
logit exceeds that reference by more than 64 (log2 units) it recomputes the
query with the true maximum.  These cases plant such logits ("DeepseekV3.2
拆解", section 核心组件: u_t is the softmax-weighted sum over the selected
latent rows, whatever their logits): for every query row a few selected
latent rows are scaled copies of the row's query direction, placed at list
positions past the first chunk, at the start of a split's range and inside
it, so that both the unsplit kernel and every split of the few-row kernel
see the first chunk's maximum overtaken by more than 2^64.  The output and
log-sum-exp are compared with the fp64 oracle element by element, for bf16
rows and for FP8 latent rows, split and unsplit, at 32, 64 and 128 heads.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.parity import check_attention

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SCALE = 1.0 / math.sqrt(192.0)
LOG2E = 1.0 / math.log(2.0)
# (list position, factor) of the planted rows: chunk 1 (past the first
# chunk), chunk 21 (inside the third of 8 splits) and chunk 57 (the second
# chunk of the last split), with factors that put their logits 60-90
# natural-log units above the other rows'
PLANTS = ((40, 1.5), (700, 2.0), (1830, 1.3))


@pytest.fixture(scope="module")
def dsa(gpu):
    import sparse_attention_04_amd as m
    return m


def _case(B, Lq, Lk, H, k, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    u = torch.randn(B, Lq, 1, 576, generator=g)
    q = u + 0.5 * torch.randn(B, Lq, H, 576, generator=g)
    q[:, :, ::5] = -u + 0.5 * torch.randn(B, Lq, (H + 4) // 5, 576, generator=g)   # heads that never overflow
    kv = torch.randn(B, Lk, 576, generator=g)
    idx = torch.empty(B, Lq, k, dtype=torch.int32)
    for b in range(B):
        perm = torch.randperm(Lk, generator=g)
        used = 0
        for t in range(Lq):
            rows = perm[used:used + k]
            used = (used + k) % (Lk - k)
            idx[b, t] = rows.to(torch.int32)
            for pos, beta in PLANTS:
                kv[b, rows[pos]] = beta * u[b, t, 0]
        idx[b, 0, 3:9] = -1                            # holes in the reference chunk
    idx[0, Lq - 1, :45] = -1                           # first valid chunk is chunk 1 (plant 40 masked)
    q, kv = q.to(torch.bfloat16), kv.to(torch.bfloat16)
    return q, kv, idx


def _check_overflow_planted(q, kv_vals, idx, H):
    """Precondition: for every query row some head's later logit exceeds the
    first valid chunk's maximum by more than 64 in log2 units."""
    B, Lq = idx.shape[:2]
    for b in range(B):
        for t in range(Lq):
            ix = idx[b, t].numpy()
            valid = ix >= 0
            first = int(np.argmax(valid)) // 32
            z = (q[b, t].double().numpy() @ kv_vals[b, np.where(valid, ix, 0)].T) * SCALE * LOG2E
            z[:, ~valid] = -np.inf
            ref = z[:, first * 32:(first + 1) * 32].max(axis=1)
            later = z[:, (first + 1) * 32:].max(axis=1)
            assert (later - ref).max() > 64.0 + 8.0, (b, t, (later - ref).max())


@pytest.mark.parametrize("H", [32, 64, 128])
def test_second_pass_bf16_rows(dsa, H):
    B, Lq, Lk, k = 2, 3, 9000, 2048
    q, kv, idx = _case(B, Lq, Lk, H, k, seed=H)
    _check_overflow_planted(q, kv.double().numpy(), idx, H)
    qd, kvd, ixd = q.to(DEV), kv.to(DEV), idx.to(DEV)
    assert dsa.dsa_sparse_attn_workspace_size(B, Lq, H, 576, 512, k) > 0      # few rows: the split runs
    out_s, lse_s = dsa.dsa_sparse_attn(qd, kvd, ixd, 512, SCALE, q_pos0=Lk - Lq)
    out_u, lse_u = dsa.dsa_sparse_attn(qd, kvd, ixd, 512, SCALE, q_pos0=Lk - Lq, split=False)
    # the same rows among many query rows (one workgroup per row, no split)
    rep = 130
    out_m, lse_m = dsa.dsa_sparse_attn(qd.repeat(1, rep, 1, 1), kvd, ixd.repeat(1, rep, 1), 512, SCALE,
                                       q_pos0=Lk - Lq * rep)
    torch.cuda.synchronize()
    for b in range(B):
        o_ref, l_ref = oracle.sparse_attn(q[b], kv[b], idx[b].numpy(), 512, SCALE, oracle.BF16)
        assert np.abs(o_ref).max() > 2.0                  # the planted rows dominate the output
        for o, l in ((out_s, lse_s), (out_u, lse_u)):
            check_attention(o[b].float().cpu().numpy(), o_ref, l[b].cpu().numpy(), l_ref, True)
        for r in range(rep):
            check_attention(out_m[b, r * Lq:(r + 1) * Lq].float().cpu().numpy(), o_ref,
                            lse_m[b, r * Lq:(r + 1) * Lq].cpu().numpy(), l_ref, True)


@pytest.mark.parametrize("H", [32, 128])
def test_second_pass_fp8_rows(dsa, H):
    B, Lq, Lk, k = 2, 3, 9000, 2048
    q, kv, idx = _case(B, Lq, Lk, H, k, seed=100 + H)
    packed = dsa.dsa_kv_pack_fp8(kv.to(DEV))
    torch.cuda.synchronize()
    kv_vals = oracle.kv_unpack_fp8(packed.cpu())
    _check_overflow_planted(q, kv_vals, idx, H)
    qd, ixd = q.to(DEV), idx.to(DEV)
    out_s, lse_s = dsa.dsa_sparse_attn_fp8kv(qd, packed, ixd, SCALE, q_pos0=Lk - Lq)
    out_u, lse_u = dsa.dsa_sparse_attn_fp8kv(qd, packed, ixd, SCALE, q_pos0=Lk - Lq, split=False)
    torch.cuda.synchronize()
    for b in range(B):
        o_ref, l_ref = oracle.sparse_attn_fp8kv(q[b], packed[b].cpu(), idx[b].numpy(), 512, SCALE)
        for o, l in ((out_s, lse_s), (out_u, lse_u)):
            check_attention(o[b].float().cpu().numpy(), o_ref, l[b].cpu().numpy(), l_ref, True)
