"""The forward's candidate route (sampled thresholds and per-row candidate
lists) against the score-tile route and the three stage calls, bit for bit
over every row, through the C ABI.

The two routes must select the same sets whatever the sample says: the sample
only decides how long each row's list is, and rows whose list is shorter than
k or longer than 2k go back to their full scores.  The cases below cover rows
whose lists fit, rows that fall back for too short and too long lists (crafted
by scaling the sampled keys), heavy ties at the threshold, chunked prefill
(q_pos0 > 0), several sequences, ragged fallback tiles, and that no full score
row is written when no row falls back.
"""
import pytest
import torch

from dsa_inputs import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

BASE = CONFIGS["prefill_L4096"]      # 64 x 128 FP8 indexer, 16 heads x 128 bf16 attention


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_04_amd as m
    return m


def _sample_shift(k):
    r = 0
    while (128 << (r + 1)) <= k:
        r += 1
    return r


def _forward(dsa, cfg, inp, route, q_tile_rows=0, fill=None):
    fwd = dsa.Forward(cfg.B, cfg.Lq, cfg.Lk, cfg.k, cfg.n_heads, cfg.d_v, inp["q"].dtype,
                      inp["q"].device, q_tile_rows=q_tile_rows, d_qk=cfg.d_qk, select=route)
    if fill is not None:
        fwd.workspace.fill_(fill)
    fwd(inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["w"], inp["q"], inp["kv"],
        cfg.softmax_scale, q_pos0=cfg.q_pos0)
    torch.cuda.synchronize()
    return fwd


def _stage_calls(dsa, cfg, inp):
    scores = dsa.dsa_indexer_scores(inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["w"],
                                    q_pos0=cfg.q_pos0)
    idx = dsa.dsa_topk(scores, cfg.k, q_pos0=cfg.q_pos0)
    out, lse = dsa.dsa_sparse_attn(inp["q"], inp["kv"], idx, cfg.d_v, cfg.softmax_scale, q_pos0=cfg.q_pos0)
    torch.cuda.synchronize()
    del scores
    return idx, out, lse


def _assert_same(a, b, what):
    ia, oa, la = a
    ib, ob, lb = b
    assert torch.equal(ia, ib), f"{what}: selected sets differ in {(ia != ib).any(-1).sum().item()} rows"
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), f"{what}: outputs differ"
    assert torch.equal(la, lb), f"{what}: lse differs"


def _tile_rows_written(fwd, cfg, T):
    """Rows of the workspace's score tile (its first B*T*Lk*4 bytes) that no
    longer hold the 0xFF fill."""
    n = cfg.B * T * cfg.Lk * 4
    tile = fwd.workspace[:n].view(cfg.B * T, cfg.Lk * 4)
    return int((tile != 255).any(dim=1).sum().item())


def _check_routes(dsa, cfg, inp, q_tile_rows=0):
    ref = _stage_calls(dsa, cfg, inp)
    tiles = _forward(dsa, cfg, inp, dsa.SELECT_SCORE_TILES, q_tile_rows)
    _assert_same((tiles.idx, tiles.out, tiles.lse), ref, "score tiles vs stage calls")
    del tiles
    cand = _forward(dsa, cfg, inp, dsa.SELECT_CANDIDATES, q_tile_rows, fill=255)
    _assert_same((cand.idx, cand.out, cand.lse), ref, "candidates vs stage calls")
    if q_tile_rows > 0:
        T = min(q_tile_rows, cfg.Lq)
    else:                                          # the automatic tile: at most 4 GiB of scores
        T = max(1, min(cfg.Lq, (4 << 30) // (cfg.B * cfg.Lk * 4)))
    written = _tile_rows_written(cand, cfg, T)
    return written, T


@pytest.mark.parametrize("Lq,Lk,q_pos0,k,B", [
    (3000, 3000, 0, 256, 1),       # sample every 2nd key, lists of at most 512
    (1500, 2000, 500, 300, 2),     # chunked prefill, two sequences
    (5000, 5000, 0, 1024, 1),      # every 8th key
    (8192, 8192, 0, 2048, 1),      # every 16th key, the bench's k
])
def test_candidates_equal_score_tiles(dsa, Lq, Lk, q_pos0, k, B):
    cfg = BASE.with_(name=f"cand_L{Lq}_k{k}", B=B, Lq=Lq, Lk=Lk, q_pos0=q_pos0, k=k)
    inp = make_inputs(cfg, seed=3, device=torch.device("cuda:0"))
    written, T = _check_routes(dsa, cfg, inp)
    # lists of about 1.5k entries fit: (almost) no row goes back to its scores
    print(f"  [{cfg.name}] score-tile rows written by the candidate route: {written} of {cfg.B * T}", flush=True)
    assert written <= max(16, cfg.B * cfg.Lq // 100)


@pytest.mark.parametrize("q_tile_rows", [0, 700])
def test_candidates_fallback_rows(dsa, q_tile_rows):
    """Sampled keys (s % R == 0) scaled by 64 mislead the thresholds: rows with
    positive head weights get lists far shorter than k, rows with negative
    ones lists far longer than 2k; keys past s = 3000 are left alone, so the
    rows differ in how badly their sample misleads them."""
    cfg = BASE.with_(name="cand_fallback", Lq=6000, Lk=6000, k=1024)
    dev = torch.device("cuda:0")
    inp = make_inputs(cfg, seed=5, device=dev)
    R = 1 << _sample_shift(cfg.k)
    s = torch.arange(cfg.Lk, device=dev)
    scale = torch.where((s % R == 0) & (s < 3000), 64.0, 1.0)
    inp["k_scale"] = (inp["k_scale"] * scale).contiguous()
    t = torch.arange(cfg.Lq, device=dev).view(1, -1, 1)
    w = inp["w"]
    inp["w"] = torch.where(t % 3 == 0, w.abs(), torch.where(t % 3 == 1, -w.abs(), w)).contiguous()
    written, T = _check_routes(dsa, cfg, inp, q_tile_rows)
    print(f"  [{cfg.name}] score-tile rows written (fallback): {written}", flush=True)
    assert written > 0, "the crafted rows were expected to fall back"


def test_candidates_ties(dsa):
    """Few distinct scores per row: every key code from a set of three rows and
    key scales from 12 levels, so many keys tie at each row's k-th largest
    score; the lowest s must win among them."""
    cfg = BASE.with_(name="cand_ties", Lq=4000, Lk=4000, k=512)
    dev = torch.device("cuda:0")
    inp = make_inputs(cfg, seed=7, device=dev)
    g = torch.Generator(device="cpu").manual_seed(11)
    pick = torch.randint(0, 3, (cfg.Lk,), generator=g).to(dev)
    inp["k_idx"] = inp["k_idx"][:, :3][:, pick].contiguous()
    levels = torch.randint(1, 13, (cfg.B, cfg.Lk), generator=g).float().to(dev) / 8
    inp["k_scale"] = levels.contiguous()
    _check_routes(dsa, cfg, inp)


def test_candidates_constant_rows(dsa):
    """Every score of a row equal: rows up to 2k keep every key in their list
    and take the lowest k positions; longer rows overflow and fall back."""
    cfg = BASE.with_(name="cand_const", Lq=2500, Lk=2500, k=256)
    dev = torch.device("cuda:0")
    inp = make_inputs(cfg, seed=9, device=dev)
    inp["k_idx"] = inp["k_idx"][:, :1].expand(-1, cfg.Lk, -1).contiguous()
    inp["k_scale"] = torch.ones_like(inp["k_scale"])
    written, _ = _check_routes(dsa, cfg, inp)
    assert written > 0


def test_candidates_route_errors(dsa):
    """The candidate route refuses problems it does not take, before any launch."""
    cfg = BASE.with_(name="cand_decode", B=2, Lq=4, Lk=3000, q_pos0=2996, k=256)
    inp = make_inputs(cfg, seed=1, device=torch.device("cuda:0"))
    assert dsa.dsa_forward_workspace_size(cfg.B, cfg.Lq, cfg.Lk, cfg.k, cfg.n_heads, cfg.d_qk, cfg.d_v,
                                          inp["q"].dtype, 0, dsa.SELECT_CANDIDATES) == 0
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_forward(inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["w"], inp["q"],
                        inp["kv"], k=cfg.k, softmax_scale=cfg.softmax_scale, q_pos0=cfg.q_pos0, d_v=cfg.d_v,
                        select=dsa.SELECT_CANDIDATES,
                        workspace=torch.empty(1 << 20, dtype=torch.uint8, device=inp["q"].device))
    assert e.value.status == 4
