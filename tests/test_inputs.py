"""The seeded generator: determinism, shapes, and the per-token FP8 quantiser."""
import hashlib
import json
import math
import os

import numpy as np
import torch

from dsa_inputs import CONFIGS, DsaConfig, make_inputs, quantize_e4m3_per_token

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _digest(inp):
    h = hashlib.sha256()
    for k in sorted(inp):
        t = inp[k]
        if t.dtype == torch.bfloat16:
            t = t.view(torch.uint16)
        h.update(k.encode())
        h.update(t.contiguous().numpy().tobytes())
    return h.hexdigest()


def _small_fp8_cfg():
    return CONFIGS["prefill_L4096"].with_(name="small", Lq=100, Lk=100, k=64)


def test_same_seed_same_bytes_and_different_seed_differs():
    cfg = _small_fp8_cfg()
    a = _digest(make_inputs(cfg, seed=0))
    b = _digest(make_inputs(cfg, seed=0))
    c = _digest(make_inputs(cfg, seed=1))
    assert a == b and a != c


def test_shapes_and_dtypes():
    cfg = _small_fp8_cfg()
    inp = make_inputs(cfg, seed=0)
    assert inp["q_idx"].shape == (1, 100, 64, 128) and inp["q_idx"].dtype == torch.uint8
    assert inp["q_scale"].shape == (1, 100, 64) and inp["q_scale"].dtype == torch.float32
    assert inp["k_idx"].shape == (1, 100, 128) and inp["k_scale"].shape == (1, 100)
    assert inp["w"].shape == (1, 100, 64)
    assert inp["q"].shape == (1, 100, 16, 128) and inp["q"].dtype == torch.bfloat16
    assert inp["kv"].shape == (1, 100, 128)
    for key in ("q_idx", "k_idx"):
        codes = inp[key]
        assert not torch.any((codes & 0x7F) == 0x7F), "no NaN codes"
    # per-token scale is broadcast over indexer heads
    qs = inp["q_scale"]
    assert torch.all(qs == qs[..., :1])


def test_quantiser_reaches_full_range_and_bounds_error():
    x = torch.randn(50, 4, 128) * torch.exp(torch.randn(50, 1, 1))
    codes, scale = quantize_e4m3_per_token(x, token_dims=2)
    deq = codes.view(torch.float8_e4m3fn).float() * scale[:, None, None]
    # the largest |x| of each token maps to the code 448
    amax_code = codes.view(torch.float8_e4m3fn).float().abs().amax(dim=(1, 2))
    assert torch.all(amax_code == 448.0)
    # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 for normals, and the
    # absolute error of subnormals is at most half their spacing 2^-9
    err = (deq - x).abs()
    bound = torch.maximum(x.abs() * 2.0 ** -4, scale[:, None, None] * 2.0 ** -10)
    assert torch.all(err <= bound * 1.0001)


def test_decode_config_has_heavy_tailed_key_scales():
    cfg = CONFIGS["decode_B64_ctx65536"].with_(B=2, Lk=4096, q_pos0=4095)
    inp = make_inputs(cfg, seed=0, with_attention=False)
    ks = inp["k_scale"].log()
    # log-normal factor with sigma = 1 on top of N(0,1) amax: spread of log-scales ~ 1
    assert 0.8 < float(ks.std()) < 1.3


def test_configs_follow_the_pages_constants():
    """Constants fixed by the pages (see tests/golden/page_constants.json)."""
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        pc = json.load(f)
    c = {k: v["value"] for k, v in pc["constants"].items()}
    d_h = c["d_h"]
    assert c["d_c_over_d_h"] * d_h == 512 and d_h // c["d_h_over_d_R"] == 64
    for name in ("prefill_L4096", "mla_prefill_L32768", "decode_B64_ctx65536", "prefill_L131072"):
        assert CONFIGS[name].k == c["top_k"]
    for name in ("mla_prefill_L32768", "decode_B64_ctx65536", "prefill_L131072"):
        cfg = CONFIGS[name]
        assert cfg.d_v == c["d_c_over_d_h"] * d_h
        assert cfg.d_qk == cfg.d_v + d_h // c["d_h_over_d_R"]
        assert math.isclose(cfg.softmax_scale, 1.0 / math.sqrt(d_h + d_h // c["d_h_over_d_R"]))
