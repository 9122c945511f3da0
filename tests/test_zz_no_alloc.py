"""dsa_forward_noalloc: the forward with the library's own device array as
its workspace, for callers that cannot allocate device memory.  Its output
must equal dsa_forward's with a caller workspace, bit for bit, call after
call (the array keeps the previous call's contents; nothing in it is read
before it is written), and problems too large for the array are refused
before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from dsa_inputs import CONFIGS, make_inputs

UNSUP = 4
A = 0x10000


def test_noalloc_refuses_problems_beyond_the_array():
    """Runs without a GPU: the size check comes before any device call."""
    from sparse_attention_04_amd import lib
    # one row of scores alone (B * Lk * 4 bytes) exceeds the 128 MiB array
    st = lib.dsa_forward_noalloc(A, A, A, A, A, 64, 128, 2, A, A, 128, 576, 512, 1, 0.1,
                                 1, 8, 1 << 26, (1 << 26) - 8, 2048, None, A, None, None)
    assert st == UNSUP and b"scratch" in lib.dsa_last_error()
    # the selected sets of every row do not fit without idx_out
    st = lib.dsa_forward_noalloc(A, A, A, A, A, 64, 128, 2, A, A, 128, 576, 512, 1, 0.1,
                                 1, 32768, 32768, 0, 2048, None, A, None, None)
    assert st == UNSUP


def _compare(dsa, cfg, with_idx: bool, seed: int):
    dev = torch.device("cuda:0")
    inp = make_inputs(cfg, seed=seed, device=dev)
    args = (inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["w"], inp["q"], inp["kv"])
    ref_idx = torch.empty((cfg.B, cfg.Lq, cfg.k), dtype=torch.int32, device=dev)
    ref_lse = torch.empty((cfg.B, cfg.Lq, cfg.n_heads), dtype=torch.float32, device=dev)
    ref_out, _, _ = dsa.dsa_forward(*args, k=cfg.k, softmax_scale=cfg.softmax_scale, q_pos0=cfg.q_pos0,
                                    idx=ref_idx, lse=ref_lse, d_v=cfg.d_v)
    idx = torch.full_like(ref_idx, -7) if with_idx else None
    lse = torch.full_like(ref_lse, float("nan"))
    out = torch.full_like(ref_out, float("nan"))
    dsa.dsa_forward_noalloc(*args, k=cfg.k, softmax_scale=cfg.softmax_scale, q_pos0=cfg.q_pos0, out=out,
                            idx=idx, lse=lse, d_v=cfg.d_v)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"{cfg.name}: out differs"
    assert torch.equal(lse, ref_lse), f"{cfg.name}: lse differs"
    if with_idx:
        assert torch.equal(idx, ref_idx), f"{cfg.name}: idx differs"


@pytest.mark.gpu
def test_noalloc_matches_forward_twice(gpu):
    import sparse_attention_04_amd as dsa
    # 1) the L = 32768 MLA prefill: the scores of 1024 query rows fill the
    #    array, so the forward runs in 32 query tiles
    big = CONFIGS["mla_prefill_L32768"]
    print(f"[no-alloc] call 1: {big.name} (selected sets returned)", flush=True)
    _compare(dsa, big, with_idx=True, seed=0)
    # 2) a smaller problem right after it, its selected sets kept in the array
    small = CONFIGS["prefill_L4096"].with_(name="prefill_L1000", Lq=1000, Lk=1000, k=256)
    print(f"[no-alloc] call 2: {small.name} (selected sets in the array)", flush=True)
    _compare(dsa, small, with_idx=False, seed=1)
    # 3) a decode batch (the attention's split partials in the array too)
    dec = CONFIGS["decode_B64_ctx65536"].with_(name="decode_B8_ctx20000", B=8, Lk=20000, q_pos0=19999)
    print(f"[no-alloc] call 3: {dec.name}", flush=True)
    _compare(dsa, dec, with_idx=False, seed=2)
