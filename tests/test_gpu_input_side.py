"""GPU parity of the input-side kernels through the C ABI: per-token FP8 e4m3
quantisation ("DeepseekV3.2 拆解", section 核心组件; "DeepSeek模型架构创新解析"
section 4.3 for the scale margin) and the latent / query row assembly with the
rotary part (same page, section 1.1).

Codes and scales are byte work and must match the oracle bit for bit (both
sides decide the codes in fp32).  The rotary rows are floating point: the
compressed part is a copy (bit-exact); the rotated part is within half a bf16
step of the fp64 oracle plus 2^-20 of the pair's magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import quantize_e4m3_per_token

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa(gpu):
    import sparse_attention_04_amd as m
    return m


DEV = torch.device("cuda:0")


def _check_quant(dsa, x: torch.Tensor, token_dims: int, repeat: int = 1, margin: float = 1.0, rows=None):
    codes, scales = dsa.dsa_quantize_e4m3(x, token_dims=token_dims, scale_repeat=repeat, margin=margin)
    torch.cuda.synchronize()
    lead = x.shape[:x.dim() - token_dims]
    xt = x.reshape(int(np.prod(lead)), -1)
    gc = codes.reshape(xt.shape[0], -1)
    gs = scales.reshape(xt.shape[0], repeat)
    if rows is not None:
        rt = torch.as_tensor(rows, device=x.device)
        xt, gc, gs = xt.index_select(0, rt), gc.index_select(0, rt), gs.index_select(0, rt)
    rc, rs = oracle.quantize_e4m3(xt.cpu(), token_dims=1, repeat=repeat, margin=margin)
    assert np.array_equal(gs.cpu().numpy(), rs), "scales differ from the oracle"
    g = gc.cpu().numpy()
    bad = np.argwhere(g != rc)
    assert bad.size == 0, f"{len(bad)} codes differ; first at {bad[0].tolist()}: gpu {g[tuple(bad[0])]:#x} " \
                          f"oracle {rc[tuple(bad[0])]:#x}"
    return codes, scales


def test_quantize_key_and_query_shapes(dsa):
    g = torch.Generator(device=DEV).manual_seed(1)
    k = torch.randn(2, 333, 128, device=DEV, generator=g) * torch.randn(2, 333, 1, device=DEV, generator=g).exp()
    _check_quant(dsa, k, 1)
    q = torch.randn(2, 77, 64, 128, device=DEV, generator=g)
    codes, scales = _check_quant(dsa, q, 2, repeat=64)
    assert scales.shape == (2, 77, 64)
    # the torch-arithmetic quantiser of the input recipe, run on the host
    # (IEEE fp32 division, as here), gives the same bytes
    ref_c, ref_s = quantize_e4m3_per_token(q.cpu(), 2)
    assert torch.equal(codes.cpu(), ref_c) and torch.equal(scales[..., 0].cpu(), ref_s)
    _check_quant(dsa, q, 1)                                   # one scale per head


@pytest.mark.parametrize("tok_len", [8, 24, 136, 2048, 8192, 8200, 16384])
def test_quantize_token_lengths(dsa, tok_len):
    """Every thread-group width: one thread per token up to whole workgroups
    holding 8 chunks per thread; odd token counts leave a ragged last block."""
    g = torch.Generator(device=DEV).manual_seed(tok_len)
    n = max(3, min(1001, 2_000_000 // tok_len))
    x = torch.randn(n, tok_len, device=DEV, generator=g)
    _check_quant(dsa, x, 1)
    _check_quant(dsa, x.to(torch.bfloat16), 1, repeat=3)


def test_quantize_ties_subnormals_zeros_and_margin(dsa):
    """Tokens whose amax is 448 (scale exactly 1), so the values reach the
    conversion unchanged: every midpoint between adjacent e4m3 magnitudes
    (round-to-even decides), one fp32 step either side, and the subnormal
    range; plus all-zero tokens and the pages' 1.2x margin."""
    mags = np.array(sorted({abs(oracle.e4m3_value(c)) for c in range(0x7F)}), dtype=np.float64)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
                           mags.astype(np.float32), np.float32(2.0 ** -10) * np.arange(1, 40, dtype=np.float32)])
    vals = np.concatenate([vals, -vals])
    n_per = 127                                            # + one 448 per token, tok_len 128
    pad = (-len(vals)) % n_per
    vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(-1, n_per)
    x = np.concatenate([np.full((vals.shape[0], 1), 448.0, np.float32), vals], axis=1)
    x = np.concatenate([x, np.zeros((3, 128), np.float32)])
    xt = torch.from_numpy(x).to(DEV)
    codes, scales = _check_quant(dsa, xt, 1)
    assert torch.all(scales[:-3] == 1.0) and torch.all(scales[-3:] == 1.0)
    assert torch.all(codes[-3:] == 0)
    _check_quant(dsa, xt, 1, margin=1.2)
    g = torch.Generator(device=DEV).manual_seed(9)
    _check_quant(dsa, torch.randn(500, 128, device=DEV, generator=g), 1, margin=1.2)


def test_quantize_full_size_indexer_inputs(dsa):
    """The L = 32768 indexer inputs (q_I 32768 x 64 x 128, k_I 32768 x 128) in
    one call each; sampled tokens against the oracle."""
    g = torch.Generator(device=DEV).manual_seed(3)
    rows = np.unique(np.concatenate([[0, 1, 32767], np.random.default_rng(3).integers(0, 32768, 60)]))
    k = torch.randn(1, 32768, 128, device=DEV, generator=g)
    _check_quant(dsa, k, 1, rows=rows)
    q = torch.randn(1, 32768, 64, 128, device=DEV, generator=g)
    _check_quant(dsa, q, 2, repeat=64, rows=rows)


def _check_rope(dsa, B, L, heads, d_nope, d_rope, pos0, base=10000.0, seed=0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    nope = torch.randn(B, L, heads, d_nope, device=DEV, generator=g).to(torch.bfloat16) if d_nope else None
    rope = (torch.randn(B, L, heads, d_rope, device=DEV, generator=g) * 3).to(torch.bfloat16)
    out = dsa.dsa_rope_assemble(nope, rope, pos0=pos0, rope_base=base)
    torch.cuda.synchronize()
    pos = np.tile(pos0 + np.arange(L, dtype=np.int64), B)
    nn = (nope if nope is not None else torch.empty(B, L, heads, 0, dtype=torch.bfloat16, device=DEV))
    ref = oracle.rope_rows(nn.reshape(B * L, heads, d_nope).cpu(), rope.reshape(B * L, heads, d_rope).cpu(),
                           pos, base).reshape(B, L, heads, d_nope + d_rope)
    o = out.float().cpu().numpy().astype(np.float64)
    if d_nope:
        assert np.array_equal(out[..., :d_nope].view(torch.int16).cpu(), nope.view(torch.int16).cpu())
    r = rope.float().cpu().numpy().astype(np.float64).reshape(B, L, heads, d_rope // 2, 2)
    pair_mag = np.repeat(np.abs(r).sum(-1), 2, axis=-1)
    err = np.abs(o[..., d_nope:] - ref[..., d_nope:])
    tol = 2.0 ** -8 * np.abs(ref[..., d_nope:]) + 2.0 ** -20 * pair_mag
    assert np.all(err <= tol), f"rotary part: worst err/tol {float((err / np.maximum(tol, 1e-300)).max()):.3g}"


@pytest.mark.parametrize("B,L,heads,d_nope,d_rope,pos0", [
    (2, 37, 1, 512, 64, 0),            # cached latent rows [c ; RoPE(k_R)], 576 wide
    (2, 37, 128, 512, 64, 65500),      # attention queries of a late decode position
    (1, 5, 4, 0, 128, 7),              # rotary part only, widest supported
    (3, 9, 16, 64, 8, 131000),         # narrow rotary part, far positions
])
def test_rope_assemble_matches_oracle(dsa, B, L, heads, d_nope, d_rope, pos0):
    _check_rope(dsa, B, L, heads, d_nope, d_rope, pos0, seed=B * 1000 + heads)


def test_assembled_rows_feed_the_attention(dsa):
    """Rows assembled on the GPU are the rows the attention consumes: the
    attention over them equals the oracle's attention over the same bytes."""
    g = torch.Generator(device=DEV).manual_seed(21)
    B, L, H = 1, 300, 16
    c = torch.randn(B, L, 1, 512, device=DEV, generator=g).to(torch.bfloat16)
    kr = torch.randn(B, L, 1, 64, device=DEV, generator=g).to(torch.bfloat16)
    qc = torch.randn(B, L, H, 512, device=DEV, generator=g).to(torch.bfloat16)
    qr = torch.randn(B, L, H, 64, device=DEV, generator=g).to(torch.bfloat16)
    kv = dsa.dsa_rope_assemble(c, kr).reshape(B, L, 576)
    q = dsa.dsa_rope_assemble(qc, qr)
    idx = torch.randint(0, L, (B, L, 64), device=DEV, generator=g, dtype=torch.int32)
    idx = torch.minimum(idx, torch.arange(L, device=DEV, dtype=torch.int32)[None, :, None])
    out, lse = dsa.dsa_sparse_attn(q, kv, idx, 512, 192 ** -0.5)
    torch.cuda.synchronize()
    from tests.parity import check_attention
    o_ref, l_ref = oracle.sparse_attn(q[0].cpu(), kv[0].cpu(), idx[0].cpu().numpy(), 512, 192 ** -0.5, oracle.BF16)
    check_attention(out[0].float().cpu().numpy(), o_ref, lse[0].cpu().numpy(), l_ref, True)


# ---------------------------------------------------------------- FP8 latent rows

def test_kv_pack_fp8_matches_oracle(dsa):
    """Packed rows byte for byte: codes, power-of-two block scales, the bf16
    rotary part; wide value ranges, an all-zero block, odd row counts."""
    g = torch.Generator(device=DEV).manual_seed(31)
    kv = (torch.randn(3, 1001, 576, device=DEV, generator=g) *
          torch.randn(3, 1001, 1, device=DEV, generator=g).mul(3).exp()).to(torch.bfloat16)
    kv[0, 5, 128:256] = 0
    packed = dsa.dsa_kv_pack_fp8(kv)
    torch.cuda.synchronize()
    ref = oracle.kv_pack_fp8(kv.cpu())
    got = packed.cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} bytes differ; first at {bad[0].tolist()}"


def _fp8kv_case(dsa, B, Lq, Lk, H, k, seed, short=True):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn(B, Lq, H, 576, device=DEV, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, Lk, 576, device=DEV, generator=g).to(torch.bfloat16)
    packed = dsa.dsa_kv_pack_fp8(kv)
    idx = torch.randint(0, Lk, (B, Lq, k), device=DEV, generator=g, dtype=torch.int32)
    if short:
        idx[0, 0, k // 3:] = -1                   # short set
        if Lq > 1:
            idx[0, 1, :] = -1                     # empty set
    return q, packed, idx


@pytest.mark.parametrize("B,Lq,Lk,H,k", [(2, 3, 3000, 128, 2048), (1, 40, 700, 64, 300), (2, 200, 5000, 32, 512)])
def test_fp8kv_attention_matches_oracle(dsa, B, Lq, Lk, H, k):
    """Attention over the packed rows, split (few rows) and unsplit, against
    the oracle on the same rows' exact values."""
    from tests.parity import check_attention
    q, packed, idx = _fp8kv_case(dsa, B, Lq, Lk, H, k, seed=B * 100 + Lq)
    scale = 192 ** -0.5
    out, lse = dsa.dsa_sparse_attn_fp8kv(q, packed, idx, scale, q_pos0=Lk - Lq)
    out_u, lse_u = dsa.dsa_sparse_attn_fp8kv(q, packed, idx, scale, q_pos0=Lk - Lq, split=False)
    torch.cuda.synchronize()
    for b in range(B):
        o_ref, l_ref = oracle.sparse_attn_fp8kv(q[b].cpu(), packed[b].cpu(), idx[b].cpu().numpy(), 512, scale)
        check_attention(out[b].float().cpu().numpy(), o_ref, lse[b].cpu().numpy(), l_ref, True)
        check_attention(out_u[b].float().cpu().numpy(), o_ref, lse_u[b].cpu().numpy(), l_ref, True)


def test_fp8kv_attention_equals_bf16_attention_on_the_same_values(dsa):
    """The FP8 path widens code * scale to bf16 exactly, so over the unpacked
    rows (as bf16) the bf16 attention computes the same softmax-weighted sums;
    the two kernels differ only in the order of their fp32 additions.  Their
    outputs agree to within one bf16 step (the final rounding may fall either
    side) and their log-sum-exps to fp32 rounding."""
    q, packed, idx = _fp8kv_case(dsa, 2, 300, 4000, 128, 2048, seed=5, short=False)
    kv_vals = torch.from_numpy(oracle.kv_unpack_fp8(packed.cpu())).to(torch.bfloat16).to(DEV)
    out8, lse8 = dsa.dsa_sparse_attn_fp8kv(q, packed, idx, 192 ** -0.5, q_pos0=4000 - 300)
    out16, lse16 = dsa.dsa_sparse_attn(q, kv_vals, idx, 512, 192 ** -0.5, q_pos0=4000 - 300)
    torch.cuda.synchronize()
    a, b = out8.float(), out16.float()
    step = torch.maximum(a.abs(), b.abs()) * 2.0 ** -7 + 2.0 ** -133
    assert bool(((a - b).abs() <= step).all()), float(((a - b).abs() / step).max())
    assert float((lse8 - lse16).abs().max()) <= 1e-5


def test_fp8kv_decode_batch_full_size(dsa):
    """The decode shape (B = 64, cache of 65536, k = 2048) on packed rows, with
    the split; sampled sequences against the oracle."""
    from tests.parity import check_attention
    g = torch.Generator(device=DEV).manual_seed(8)
    B, Lk, H, k = 64, 65536, 128, 2048
    kv = torch.randn(B, Lk, 576, device=DEV, generator=g).to(torch.bfloat16)
    packed = dsa.dsa_kv_pack_fp8(kv)
    del kv
    q = torch.randn(B, 1, H, 576, device=DEV, generator=g).to(torch.bfloat16)
    idx = torch.sort(torch.randint(0, Lk, (B, 1, k), device=DEV, generator=g, dtype=torch.int32), dim=2).values
    out, lse = dsa.dsa_sparse_attn_fp8kv(q, packed, idx, 192 ** -0.5, q_pos0=Lk - 1)
    torch.cuda.synchronize()
    for b in (0, 17, 63):
        o_ref, l_ref = oracle.sparse_attn_fp8kv(q[b].cpu(), packed[b].cpu(), idx[b].cpu().numpy(), 512, 192 ** -0.5)
        check_attention(out[b].float().cpu().numpy(), o_ref, lse[b].cpu().numpy(), l_ref, True)
