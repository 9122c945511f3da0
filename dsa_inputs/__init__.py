"""Seeded synthetic inputs for the DSA forward path.

This module only draws random tensors and casts them to the storage formats the
path consumes (FP8 e4m3 with per-token fp32 scales, bf16, fp32).  It holds none
of the method's arithmetic: no indexer scores, no selection, no attention.  Both
the CPU oracle's tests and the GPU path's tests/benchmark draw their inputs from
here, so that the two sides see identical bytes.

Workload shapes follow the pages' statement of the problem ("DeepseekV3.2 拆解",
section 核心组件: indexer heads H^I, k = 2048 from the table under 创新点) and
the MLA row layout of "DeepSeek模型架构创新解析" section 1.1 (latent 4·d_h = 512
plus decoupled-RoPE d_h/2 = 64 = 576 per token; temperature sqrt(d_h + d^R_h) =
sqrt(192), section 4.3).

Draw order (fixed): indexer queries, indexer keys, [per-token log-normal key
factor], head weights w, attention queries, latent KV rows.  Every tensor is
drawn from one ``torch.Generator`` seeded once, in row chunks of a fixed size,
so the stream is reproducible on a given device type.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import torch

E4M3_MAX = 448.0  # largest finite OCP e4m3fn magnitude


@dataclass(frozen=True)
class DsaConfig:
    name: str
    B: int
    Lq: int
    Lk: int
    q_pos0: int
    n_idx_heads: int          # H^I
    idx_dim: int              # d^I
    idx_dtype: str            # "fp8" | "f32"
    n_heads: int              # attention query heads (all share one KV row set)
    d_qk: int                 # key width of a latent row
    d_v: int                  # value width (leading columns of the same row)
    k: int                    # top-k
    softmax_scale: float
    io_dtype: str             # "bf16" | "f32"
    q_idx_std: float = 1.0
    k_idx_std: float = 1.0
    w_std: float = 1.0
    key_lognormal_sigma: float = 0.0   # > 0: per-token factor exp(sigma*z) on indexer keys
    q_tile_rows: int = 0               # query-row tile used by the fused forward (0 = auto)
    note: str = ""

    def with_(self, **kw) -> "DsaConfig":
        return replace(self, **kw)

    @property
    def rows(self) -> int:
        return self.B * self.Lq


# The five workloads.  Sizes, distributions and k are the ones the hot path is
# specified on; the seeds are fixed at 0.
CONFIGS: Dict[str, DsaConfig] = {
    "tiny_fp32_L256": DsaConfig(
        name="tiny_fp32_L256", B=1, Lq=256, Lk=256, q_pos0=0,
        n_idx_heads=4, idx_dim=32, idx_dtype="f32",
        n_heads=4, d_qk=64, d_v=64, k=32, softmax_scale=1.0 / 8.0, io_dtype="f32",
        q_idx_std=math.sqrt(1.0 / 32.0), k_idx_std=math.sqrt(1.0 / 32.0), w_std=0.5,
        note="fp32 throughout; parity config"),
    "prefill_L4096": DsaConfig(
        name="prefill_L4096", B=1, Lq=4096, Lk=4096, q_pos0=0,
        n_idx_heads=64, idx_dim=128, idx_dtype="fp8",
        n_heads=16, d_qk=128, d_v=128, k=2048, softmax_scale=1.0 / math.sqrt(128.0),
        io_dtype="bf16", w_std=0.125, note="MQA, 16 heads x 128"),
    "mla_prefill_L32768": DsaConfig(
        name="mla_prefill_L32768", B=1, Lq=32768, Lk=32768, q_pos0=0,
        n_idx_heads=64, idx_dim=128, idx_dtype="fp8",
        n_heads=128, d_qk=576, d_v=512, k=2048, softmax_scale=1.0 / math.sqrt(192.0),
        io_dtype="bf16", note="MLA latent rows 512+64, value = first 512 columns"),
    "decode_B64_ctx65536": DsaConfig(
        name="decode_B64_ctx65536", B=64, Lq=1, Lk=65536, q_pos0=65535,
        n_idx_heads=64, idx_dim=128, idx_dtype="fp8",
        n_heads=128, d_qk=576, d_v=512, k=2048, softmax_scale=1.0 / math.sqrt(192.0),
        io_dtype="bf16", key_lognormal_sigma=1.0,
        note="one new token per sequence; cache includes it (t_pos = 65535)"),
    "prefill_L131072": DsaConfig(
        name="prefill_L131072", B=1, Lq=131072, Lk=131072, q_pos0=0,
        n_idx_heads=64, idx_dim=128, idx_dtype="fp8",
        n_heads=128, d_qk=576, d_v=512, k=2048, softmax_scale=1.0 / math.sqrt(192.0),
        io_dtype="bf16", q_tile_rows=4096, note="query-row tiles of 4096"),
}


def _randn(shape, gen, device, chunk_rows: int = 1024) -> torch.Tensor:
    """N(0,1) fp32 of ``shape``, drawn in chunks along dim 1 (the row dim)."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    if out.numel() == 0:
        return out
    if len(shape) < 2:
        out.normal_(generator=gen)
        return out
    rows = shape[1]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[:, r0:r1].normal_(generator=gen)
    return out


def quantize_e4m3_per_token(x: torch.Tensor, token_dims: int):
    """Per-token symmetric FP8 e4m3fn quantisation.

    ``token_dims`` trailing dims form one token.  scale = amax/448 (1 if the
    token is all zero); code = e4m3(clamp(x/scale, ±448)) with round to nearest
    even (torch's cast).  Returns (codes as uint8, fp32 scale per token).
    """
    red = tuple(range(x.dim() - token_dims, x.dim()))
    amax = x.abs().amax(dim=red)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    shp = scale.shape + (1,) * token_dims
    y = (x / scale.reshape(shp)).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32)


def make_inputs(cfg: DsaConfig, seed: int = 0, device="cpu",
                with_attention: bool = True) -> Dict[str, torch.Tensor]:
    """Draw one batch of inputs for ``cfg`` on ``device``.

    Returned tensors (all contiguous):
      q_idx   [B,Lq,H^I,d^I]  uint8 e4m3 codes (or fp32 for idx_dtype "f32")
      q_scale [B,Lq,H^I]      fp32 (absent for "f32")
      k_idx   [B,Lk,d^I]      uint8 e4m3 codes (or fp32)
      k_scale [B,Lk]          fp32 (absent for "f32")
      w       [B,Lq,H^I]      fp32
      q       [B,Lq,H,d_qk]   bf16 (or fp32)
      kv      [B,Lk,d_qk]     bf16 (or fp32); value = kv[..., :d_v]
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    B, Lq, Lk = cfg.B, cfg.Lq, cfg.Lk
    HI, DI = cfg.n_idx_heads, cfg.idx_dim
    out: Dict[str, torch.Tensor] = {}

    qi = _randn((B, Lq, HI, DI), gen, dev)
    qi.mul_(cfg.q_idx_std)
    ki = _randn((B, Lk, DI), gen, dev)
    ki.mul_(cfg.k_idx_std)
    if cfg.key_lognormal_sigma > 0:
        z = _randn((B, Lk), gen, dev)
        ki.mul_(torch.exp(cfg.key_lognormal_sigma * z).unsqueeze(-1))
        del z
    if cfg.idx_dtype == "fp8":
        out["q_idx"], qs_tok = quantize_e4m3_per_token(qi, token_dims=2)
        out["q_scale"] = qs_tok.unsqueeze(-1).expand(B, Lq, HI).contiguous()
        out["k_idx"], out["k_scale"] = quantize_e4m3_per_token(ki, token_dims=1)
    elif cfg.idx_dtype == "f32":
        out["q_idx"], out["k_idx"] = qi, ki
    else:
        raise ValueError(f"unknown idx_dtype {cfg.idx_dtype}")
    del qi, ki
    w = _randn((B, Lq, HI), gen, dev)
    w.mul_(cfg.w_std)
    out["w"] = w

    if with_attention:
        io = torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32
        # q is the largest tensor: draw and cast it chunk by chunk.
        q = torch.empty((B, Lq, cfg.n_heads, cfg.d_qk), dtype=io, device=dev)
        step = 1024
        for r0 in range(0, Lq, step):
            r1 = min(Lq, r0 + step)
            blk = torch.empty((B, r1 - r0, cfg.n_heads, cfg.d_qk), dtype=torch.float32, device=dev)
            blk.normal_(generator=gen)
            q[:, r0:r1] = blk.to(io)
            del blk
        out["q"] = q
        out["kv"] = _randn((B, Lk, cfg.d_qk), gen, dev).to(io)
    return out


def t_pos_of_rows(cfg: DsaConfig, rows) -> torch.Tensor:
    """Absolute position t_pos = q_pos0 + t for flattened row ids r = b*Lq + t."""
    r = torch.as_tensor(rows, dtype=torch.int64)
    return cfg.q_pos0 + (r % cfg.Lq)
