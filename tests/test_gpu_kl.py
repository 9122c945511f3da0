"""GPU parity of the indexer distillation loss ("DeepseekV3.2 拆解", section
预训练策略, dense warm-up: L^I = sum_t KL(p_t || Softmax(I_t)), p_t the mean
over heads of the dense attention distributions) through the C ABI.

Tolerance: |KL_gpu - KL_oracle| <= 2e-3 + 1e-3 |KL_oracle|.  The kernel's
logits come from fp32-accumulated bf16 products (error well below 1e-3 for
576-long dot products of unit-variance bf16 values at scale 1/sqrt(192));
a logit error e moves log p and log Softmax(I) by at most 2e and the KL by at
most about 2e; the fp32 sums over up to a few thousand keys add ~1e-5 relative.
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def dsa(gpu):
    import sparse_attention_04_amd as m
    return m


def _check(kl_gpu, q, kv, scores, t_pos, scale):
    ref = oracle.indexer_kl(q, kv, scores.astype(np.float64), t_pos, scale, oracle.BF16)
    err = np.abs(kl_gpu.astype(np.float64) - ref)
    tol = 2e-3 + 1e-3 * np.abs(ref)
    assert np.all(err <= tol), f"worst err {err.max():.3g} at row {int(err.argmax())} (ref {ref[err.argmax()]:.4g})"
    assert np.all(ref >= 0)
    return float(err.max())


@pytest.mark.parametrize("H,L,B", [(128, 300, 1), (32, 200, 2), (64, 130, 1)])
def test_kl_prefill_with_indexer_scores(dsa, H, L, B):
    """Scores from the FP8 indexer kernel, every query row."""
    cfg = CONFIGS["mla_prefill_L32768"].with_(name="kl", B=B, Lq=L, Lk=L, n_heads=H)
    inp = make_inputs(cfg, seed=H + L, device=DEV)
    scores = dsa.dsa_indexer_scores(inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["w"])
    kl = dsa.dsa_indexer_kl(inp["q"], inp["kv"], scores, cfg.softmax_scale)
    torch.cuda.synchronize()
    for b in range(B):
        e = _check(kl[b].cpu().numpy(), inp["q"][b].cpu(), inp["kv"][b].cpu(), scores[b].cpu().numpy(),
                   np.arange(L), cfg.softmax_scale)
        print(f"  [kl H={H} L={L} b={b}] max err {e:.3g}", flush=True)


def test_kl_decode_rows_and_planted_zero(dsa):
    """Rows at the end of a long cache (q_pos0 > 0), and scores planted as
    log p + const, for which the loss must vanish."""
    g = torch.Generator(device=DEV).manual_seed(3)
    B, Lq, Lk, H = 2, 3, 1500, 128
    q = torch.randn(B, Lq, H, 576, device=DEV, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, Lk, 576, device=DEV, generator=g).to(torch.bfloat16)
    scores = torch.randn(B, Lq, Lk, device=DEV, generator=g) * 3
    scale = 192 ** -0.5
    kl = dsa.dsa_indexer_kl(q, kv, scores, scale, q_pos0=Lk - Lq)
    torch.cuda.synchronize()
    t_pos = Lk - Lq + np.arange(Lq)
    for b in range(B):
        _check(kl[b].cpu().numpy(), q[b].cpu(), kv[b].cpu(), scores[b].cpu().numpy(), t_pos, scale)
    # planted: I = log p + 5 (p from torch in float64 on the host)
    planted = torch.full((B, Lq, Lk), -1e30)
    for b in range(B):
        for r in range(Lq):
            n = int(t_pos[r]) + 1
            z = scale * (q[b, r].double().cpu() @ kv[b, :n].double().cpu().T)
            planted[b, r, :n] = (torch.log(torch.softmax(z, dim=1).mean(dim=0)) + 5).float()
    kl0 = dsa.dsa_indexer_kl(q, kv, planted.to(DEV).contiguous(), scale, q_pos0=Lk - Lq)
    torch.cuda.synchronize()
    assert float(kl0.abs().max()) <= 2e-3


def test_kl_long_rows_sampled(dsa):
    """L = 4096, sampled rows of the full launch."""
    cfg = CONFIGS["mla_prefill_L32768"].with_(name="kl4k", Lq=4096, Lk=4096)
    inp = make_inputs(cfg, seed=7, device=DEV)
    scores = dsa.dsa_indexer_scores(inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["w"])
    kl = dsa.dsa_indexer_kl(inp["q"], inp["kv"], scores, cfg.softmax_scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, 33, 2047, 2048, 4000, 4095])
    rt = torch.as_tensor(rows, device=DEV)
    _check(kl[0].index_select(0, rt).cpu().numpy(), inp["q"][0].index_select(0, rt).cpu(), inp["kv"][0].cpu(),
           scores[0].index_select(0, rt).cpu().numpy(), rows, cfg.softmax_scale)
