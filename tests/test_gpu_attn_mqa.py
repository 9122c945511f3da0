"""GPU parity of the attention over rows of D = d_qk = d_v in {64, 128} (the
MQA shapes, "DeepseekV3.2 拆解", section 核心组件: every head of query t
attends to the same selected rows c_s, u_t their softmax-weighted sum).

Head counts whose waves (16 heads each) divide the D / 16 copy instructions
of a chunk run the two-slot kernel of attn_mqa.hip; the others (48 heads at
D = 128, 128 heads at D = 64) the older kernel of sparse_attn.hip.  Every
case is compared with the fp64 oracle element by element:
  - index lists with -1 holes, -1 padding at the end (short rows, so the
    chunk loop stops early), rows with no valid entry at all, and repeated
    rows;
  - k = 2048 (64 chunks) and a ragged k = 333 (the last chunk part-filled);
  - planted rows, past the first chunk, whose logits exceed the first valid
    chunk's maximum by more than 2^64, so the kernel's second pass (with the
    true maximum as reference) runs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.parity import check_attention

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def dsa(gpu):
    import sparse_attention_04_amd as m
    return m


def _lists(g, B, Lq, Lk, k):
    idx = torch.empty(B, Lq, k, dtype=torch.int32)
    for b in range(B):
        for t in range(Lq):
            idx[b, t] = torch.randperm(Lk, generator=g)[:k].sort().values.to(torch.int32)
    idx[0, 1, 5:40] = -1                               # holes across the first two chunks
    idx[0, 2, k // 3:] = -1                            # a short row: padding from a third on
    idx[0, 3, :] = -1                                  # no valid entry
    idx[1, 0, 1::2] = idx[1, 0, 0::2][: k // 2]        # every row twice (a repeated row counts twice)
    idx[1, 1, : k - 1] = -1                            # one valid entry, in the last chunk
    return idx


def _run(dsa, q, kv, idx, scale):
    D = q.shape[-1]
    out, lse = dsa.dsa_sparse_attn(q.to(DEV), kv.to(DEV), idx.to(DEV), D, scale)
    torch.cuda.synchronize()
    for b in range(q.shape[0]):
        o_ref, l_ref = oracle.sparse_attn(q[b], kv[b], idx[b].numpy(), D, scale, oracle.BF16)
        check_attention(out[b].float().cpu().numpy(), o_ref, lse[b].cpu().numpy(), l_ref, True)


@pytest.mark.parametrize("D,H", [(128, 16), (128, 32), (128, 64), (128, 128), (64, 16), (64, 32), (64, 64),
                                 (128, 48), (64, 128)])
@pytest.mark.parametrize("k", [2048, 333])
def test_mqa_attention(dsa, D, H, k):
    B, Lq, Lk = 2, 6, 3000
    g = torch.Generator(device="cpu").manual_seed(1000 * D + 10 * H + k)
    q = torch.randn(B, Lq, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, Lk, D, generator=g).to(torch.bfloat16)
    idx = _lists(g, B, Lq, Lk, k)
    _run(dsa, q, kv, idx, 1.0 / math.sqrt(D))


@pytest.mark.parametrize("D,H", [(128, 16), (128, 64), (64, 32)])
def test_mqa_second_pass(dsa, D, H):
    """Rows at list positions 40, 700 and 1830 are scaled copies of the
    query's shared direction u; their logits sit 60-100 natural-log units
    above the others', more than 2^64 past the first chunk's maximum."""
    B, Lq, Lk, k = 2, 3, 9000, 2048
    scale = 1.0 / math.sqrt(D)
    g = torch.Generator(device="cpu").manual_seed(77 + D + H)
    u = torch.randn(B, Lq, 1, D, generator=g)
    q = u + 0.5 * torch.randn(B, Lq, H, D, generator=g)
    q[:, :, ::5] = -u + 0.5 * torch.randn(B, Lq, (H + 4) // 5, D, generator=g)   # heads that never overflow
    kv = torch.randn(B, Lk, D, generator=g)
    beta = 7.0 * math.sqrt(128.0 / D)
    idx = torch.empty(B, Lq, k, dtype=torch.int32)
    for b in range(B):
        perm = torch.randperm(Lk, generator=g)
        for t in range(Lq):
            rows = perm[t * k:(t + 1) * k] if (t + 1) * k <= Lk else perm[:k]
            idx[b, t] = rows.to(torch.int32)
            for pos, f in ((40, 1.0), (700, 1.3), (1830, 0.8)):
                kv[b, rows[pos]] = f * beta * u[b, t, 0]
    idx[0, 0, 3:9] = -1                                # holes in the reference chunk
    q, kv = q.to(torch.bfloat16), kv.to(torch.bfloat16)
    # precondition: some head of every row overtakes its first chunk's maximum by > 64 (log2)
    kvd = kv.double().numpy()
    for b in range(B):
        for t in range(Lq):
            ix = idx[b, t].numpy()
            valid = ix >= 0
            z = (q[b, t].double().numpy() @ kvd[b, np.where(valid, ix, 0)].T) * scale / math.log(2.0)
            z[:, ~valid] = -np.inf
            assert (z[:, 32:].max(axis=1) - z[:, :32].max(axis=1)).max() > 72.0, (b, t)
    _run(dsa, q, kv, idx, scale)
