"""Pins of the oracle's input-side functions: FP8 e4m3 encoding and per-token
quantisation ("DeepseekV3.2 拆解", section 核心组件: the indexer runs in FP8;
"DeepSeek模型架构创新解析" section 4.3: a 1.2x scale margin against FP8
overflow), and the latent-row assembly with the decoupled rotary part (same
page, section 1.1).

The encoder is pinned to torch's float8_e4m3fn cast on every tie and its
neighbours; the quantiser to torch arithmetic and closed forms; the rotary
assembly to a hand-worked example and to the properties that define a rotary
embedding (norm kept per pair, scores depend on relative position only,
angles add).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import quantize_e4m3_per_token

rng = np.random.default_rng(77)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def _torch_e4m3(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _encode_all(y: np.ndarray) -> np.ndarray:
    return np.array([oracle.e4m3_encode(float(v)) for v in y.ravel()], dtype=np.uint8).reshape(y.shape)


# ---------------------------------------------------------------- e4m3 encode

def test_encode_inverts_decode_on_every_finite_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c, hex(c)


def test_encode_matches_torch_cast_on_ties_and_neighbours():
    """Every midpoint between adjacent finite magnitudes (where round-to-even
    decides), one fp32 ulp either side, and random values, both signs."""
    mags = np.array(sorted({abs(oracle.e4m3_value(c)) for c in range(0x7F)}), dtype=np.float64)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
                          mags.astype(np.float32),
                          rng.uniform(0, 448, 3000).astype(np.float32),
                          (2.0 ** rng.uniform(-14, -5, 1000)).astype(np.float32)])
    pts = np.concatenate([pts, -pts])
    assert np.array_equal(_encode_all(pts), _torch_e4m3(pts))


def test_encode_signed_zero_and_saturation():
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-9) == 0x80                 # rounds to zero, keeps the sign
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00            # half the smallest subnormal: tie to even (0)
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02        # 1.5 subnormal steps: tie to even (2)
    assert oracle.e4m3_encode(460.0) == 0x7E                 # saturates at 448
    assert oracle.e4m3_encode(-1e6) == 0xFE


# ---------------------------------------------------------------- per-token quantisation

def test_quantise_matches_torch_arithmetic_per_token():
    """k^I-shaped tokens (128 values) and q^I-shaped tokens (64 heads x 128,
    one scale per token broadcast to the heads), against the torch-arithmetic
    quantiser of the input recipe (an independent implementation)."""
    k = torch.from_numpy(rng.standard_normal((300, 128)).astype(np.float32) * np.exp(rng.standard_normal((300, 1))).astype(np.float32))
    codes, scales = oracle.quantize_e4m3(k.numpy(), token_dims=1)
    ref_c, ref_s = quantize_e4m3_per_token(k, 1)
    assert np.array_equal(codes, ref_c.numpy()) and np.array_equal(scales[:, 0], ref_s.numpy())
    q = torch.from_numpy(rng.standard_normal((7, 64, 128)).astype(np.float32))
    codes, scales = oracle.quantize_e4m3(q.numpy(), token_dims=2, repeat=64)
    ref_c, ref_s = quantize_e4m3_per_token(q, 2)
    assert np.array_equal(codes, ref_c.numpy())
    assert np.array_equal(scales, np.repeat(ref_s.numpy()[:, None], 64, axis=1))


def test_quantise_closed_forms():
    x = np.zeros((4, 16), np.float32)
    x[0, 3] = -5.0                      # amax element maps to -448 exactly
    x[0, 5] = 2.5
    x[2, :] = np.linspace(-1, 1, 16)
    codes, scales = oracle.quantize_e4m3(x)
    assert scales[0, 0] == np.float32(5.0) / np.float32(448.0)
    assert codes[0, 3] == 0xFE and codes[0, 5] == oracle.e4m3_encode(224.0)
    assert scales[1, 0] == 1.0 and np.all(codes[1] == 0)      # all-zero token: scale 1, zero codes
    assert codes[2, 0] == 0xFE and codes[2, 15] == 0x7E
    # dequantised values are within half an e4m3 step of x (relative 2^-4 for normals)
    deq = oracle.e4m3_table()[codes[2]] * scales[2, 0]
    assert np.all(np.abs(deq - x[2]) <= np.abs(x[2]) * 2.0 ** -4 + scales[2, 0] * 2.0 ** -10)


def test_quantise_margin_from_the_pages():
    margin = json.load(open(GOLDEN))["constants"]["fp8_scale_margin"]["value"]
    x = rng.standard_normal((50, 128)).astype(np.float32)
    codes, scales = oracle.quantize_e4m3(x, margin=margin)
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(scales[:, 0], (amax * np.float32(margin)) / np.float32(448.0))
    # the largest magnitude now encodes to the code nearest 448 / 1.2 = 373.3, i.e. 384
    top = codes[np.arange(50), np.abs(x).argmax(axis=1)] & 0x7F
    assert np.all(top == oracle.e4m3_encode(384.0))
    assert np.all((codes & 0x7F) <= oracle.e4m3_encode(384.0))


def test_quantise_bf16_input_equals_fp32_of_same_values():
    xb = torch.from_numpy(rng.standard_normal((20, 128)).astype(np.float32)).to(torch.bfloat16)
    c1, s1 = oracle.quantize_e4m3(xb)
    c2, s2 = oracle.quantize_e4m3(xb.float().numpy())
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


# ---------------------------------------------------------------- latent row with the rotary part

def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def test_rope_rows_hand_example():
    """d_rope = 4, base 10^4: pair 0 turns by pos rad, pair 1 by pos/100 rad."""
    nope = _bf16(np.array([[[1.5, -2.0]]]))
    rope = _bf16(np.array([[[1.0, 0.0, 0.0, 1.0]]]))
    out = oracle.rope_rows(nope, rope, np.array([1]), base=10000.0)[0, 0]
    assert np.array_equal(out[:2], [1.5, -2.0])
    np.testing.assert_allclose(out[2:], [math.cos(1), math.sin(1), -math.sin(0.01), math.cos(0.01)],
                               rtol=0, atol=1e-15)
    out3 = oracle.rope_rows(nope, rope, np.array([3]), base=10000.0)[0, 0]
    np.testing.assert_allclose(out3[2:], [math.cos(3), math.sin(3), -math.sin(0.03), math.cos(0.03)],
                               rtol=0, atol=1e-15)


def test_rope_rows_position_zero_is_a_copy_and_norms_are_kept():
    nope = _bf16(rng.standard_normal((5, 3, 16)))
    rope = _bf16(rng.standard_normal((5, 3, 64)))
    out0 = oracle.rope_rows(nope, rope, np.zeros(5, np.int64))
    assert np.array_equal(out0, torch.cat([nope, rope], dim=2).double().numpy())
    pos = rng.integers(0, 131072, 5)
    out = oracle.rope_rows(nope, rope, pos)
    r = rope.double().numpy().reshape(5, 3, 32, 2)
    o = out[..., 16:].reshape(5, 3, 32, 2)
    np.testing.assert_allclose((o ** 2).sum(-1), (r ** 2).sum(-1), rtol=1e-12)
    assert np.array_equal(out[..., :16], nope.double().numpy())


def test_rope_rows_scores_depend_on_relative_position_only():
    """<R(p) q, R(s) k> = <R(p + d) q, R(s + d) k>: the property the rotary
    part exists for (the decoupled key is shared by all heads)."""
    q = _bf16(rng.standard_normal((1, 4, 64)))
    k = _bf16(rng.standard_normal((1, 1, 64)))
    z = _bf16(np.zeros((1, 4, 0)))
    z1 = _bf16(np.zeros((1, 1, 0)))
    for p, s, d in [(10, 3, 1000), (70000, 65000, 777), (5, 5, 123456)]:
        a = oracle.rope_rows(z, q, [p])[0] @ oracle.rope_rows(z1, k, [s])[0, 0]
        b = oracle.rope_rows(z, q, [p + d])[0] @ oracle.rope_rows(z1, k, [s + d])[0, 0]
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-9)


def test_rope_rows_angles_add():
    """Rotating by p then by s equals rotating by p + s (re-rotation of the
    fp64 result, so the second step is done here with the same formula's
    closed form: multiplication by a complex phase)."""
    rope = _bf16(rng.standard_normal((3, 2, 8)))
    z = _bf16(np.zeros((3, 2, 0)))
    p, s = np.array([7, 100, 4000]), np.array([5, 31, 90000])
    both = oracle.rope_rows(z, rope, p + s)
    first = oracle.rope_rows(z, rope, p).reshape(3, 2, 4, 2)
    theta = 10000.0 ** (-2.0 * np.arange(4) / 8)
    ph = np.exp(1j * s[:, None] * theta[None, :])[:, None, :]
    c = (first[..., 0] + 1j * first[..., 1]) * ph
    np.testing.assert_allclose(np.stack([c.real, c.imag], -1).reshape(3, 2, 8), both, rtol=0, atol=1e-10)


# ---------------------------------------------------------------- FP8 latent rows (656-byte packed form)

def _blocks(packed):
    codes = packed[..., :512].reshape(*packed.shape[:-1], 4, 128)
    scales = np.ascontiguousarray(packed[..., 512:528]).view(np.float32)
    return codes, scales


def test_kv_pack_scales_are_powers_of_two_covering_amax():
    kv = torch.from_numpy((rng.standard_normal((40, 576)) * np.exp(rng.standard_normal((40, 1)) * 3))
                          .astype(np.float32)).to(torch.bfloat16)
    packed = oracle.kv_pack_fp8(kv)
    codes, scales = _blocks(packed)
    amax = kv.float().numpy()[:, :512].reshape(40, 4, 128).__abs__().max(axis=2)
    mant, _ = np.frexp(scales)
    assert np.all(mant == 0.5), "block scales must be powers of two"
    t = (amax.astype(np.float32) / np.float32(448.0))
    assert np.all(scales >= t) and np.all(scales < 2 * t)
    # codes are torch's e4m3 cast of x / scale, block by block
    x = kv.float().numpy()[:, :512].reshape(40, 4, 128)
    ref = _torch_e4m3(np.clip(x / scales[:, :, None], -448, 448))
    assert np.array_equal(codes, ref)
    # the rotary part is the original bf16, bit for bit
    assert np.array_equal(packed[:, 528:].view(np.uint16), kv.view(torch.int16).numpy()[:, 512:].view(np.uint16))


def test_kv_pack_round_trip_bounds_and_exact_cases():
    kv = torch.from_numpy(rng.standard_normal((30, 576)).astype(np.float32)).to(torch.bfloat16)
    kv[3, 128:256] = 0                                     # an all-zero block
    packed = oracle.kv_pack_fp8(kv)
    codes, scales = _blocks(packed)
    assert scales[3, 1] == 1.0 and np.all(codes[3, 1] == 0)
    u = oracle.kv_unpack_fp8(packed)
    x = kv.float().numpy()
    step = np.repeat(scales, 128, axis=1)
    err = np.abs(u[:, :512] - x[:, :512])
    assert np.all(err <= np.abs(x[:, :512]) * 2.0 ** -4 + step * 2.0 ** -10)
    assert np.array_equal(u[:, 512:], x[:, 512:])
    # rows that are already e4m3 codes times a power of two (with the block
    # maximum 448 present) come back exactly
    c = rng.integers(0, 0x7F, (5, 512)).astype(np.uint8)
    c[:, ::128] = 0x7E
    vals = oracle.e4m3_table()[c] * np.float32(2.0 ** -3)
    tail = _bf16(rng.standard_normal((5, 64))).float().numpy()
    row = np.concatenate([vals, tail], axis=1)
    rb = torch.from_numpy(row).to(torch.bfloat16)
    assert np.array_equal(rb.float().numpy(), row)          # exact in bf16
    pk = oracle.kv_pack_fp8(rb)
    assert np.all(_blocks(pk)[1] == 0.125)
    assert np.array_equal(oracle.kv_unpack_fp8(pk), row)


def test_fp8kv_attention_equals_bf16_attention_on_representable_rows():
    c = rng.integers(0, 0xFF, (60, 512)).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x10
    c[:, ::128] = 0x7E
    vals = oracle.e4m3_table()[c] * np.float32(2.0 ** -6)
    rows = np.concatenate([vals, rng.standard_normal((60, 64)).astype(np.float32)], axis=1)
    kv = torch.from_numpy(rows).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((4, 8, 576)).astype(np.float32)).to(torch.bfloat16)
    idx = rng.integers(-1, 60, (4, 20)).astype(np.int32)
    o1, l1 = oracle.sparse_attn_fp8kv(q, oracle.kv_pack_fp8(kv), idx, 512, 192 ** -0.5)
    o2, l2 = oracle.sparse_attn(q, kv, idx, 512, 192 ** -0.5, oracle.BF16)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
