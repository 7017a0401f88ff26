"""Bounded graph set on the GPU: descending capture into one workspace panel, replays with
changed queries, lengths, zero rows and padded slots equal independent single-request runs
bitwise, an oversized peer takes the eager route with the same bits, and graphs captured before
the bank grows still replay correctly ("DFlash2 concurrent long-context attention, 2026-09-27",
sections "Why the single-request optimization was missing from concurrent decode" and
"Operator validation")."""
import pytest
import torch

from _gpu import note
from verify_attention_e4m3_amd import attention as A
from verify_attention_e4m3_amd import workloads as wl
from verify_attention_e4m3_amd.graphs import LayerCache, VerifyGraphs

pytestmark = pytest.mark.gpu

GEOM = dict(q_len=8, num_q_heads=12, num_kv_heads=2, head_dim=256, page_size=1648)
BOUND = 8192


def _setup(lens, seed, width_tokens=BOUND, layers=2):
    c = wl.make_case(batch=len(lens), seq_lens=lens, seed=seed, device="cuda", max_seq_len=width_tokens, **GEOM)
    caches = [LayerCache(c["k_cache"], c["v_cache"], c["k_scale"], c["v_scale"])]
    qs = [c["q"]]
    for i in range(1, layers):
        k = wl.random_cache(c["k_cache"].shape[0], GEOM["page_size"], GEOM["num_kv_heads"], GEOM["head_dim"],
                            kv_format="e4m3", std=1.0, seed=seed * 31 + i, device="cuda")
        v = wl.random_cache(c["v_cache"].shape[0], GEOM["page_size"], GEOM["num_kv_heads"], GEOM["head_dim"],
                            kv_format="e4m3", std=1.0, seed=seed * 37 + i, device="cuda")
        caches.append(LayerCache(k, v, c["k_scale"], c["v_scale"]))
        g = torch.Generator(device="cuda")
        g.manual_seed(seed * 41 + i)
        qs.append(torch.randn(c["q"].shape, generator=g, device="cuda").to(torch.float16))
    return c, caches, qs


def _plan(width, capacity, bound=BOUND):
    return A.Plan(max_seq_len=bound, max_pages_per_seq=width, batch_capacity=capacity, device="cuda:0", **GEOM)


def _singles(c, caches, qs, rows):
    """Each request alone (B1, eager) through its own plan."""
    p1 = _plan(c["block_table"].shape[1], 1, bound=min(262144, c["block_table"].shape[1] * GEOM["page_size"]))
    outs = []
    for q, L in zip(qs, caches):
        per = [p1.run(q[b:b + 1], L.k_cache, L.v_cache, c["block_table"][b:b + 1], c["seq_lens"][b:b + 1],
                      L.k_scale, L.v_scale) for b in rows]
        outs.append(torch.cat(per))
    torch.cuda.synchronize()
    return outs


def _same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


def test_descending_capture_shares_one_panel_and_replays_match_singles():
    lens = [5000, 8, 0, 8192, 1, 3297, 7000, 64]
    c, caches, qs = _setup(lens, seed=61)
    bank = A.WorkspaceBank()
    gs = VerifyGraphs(_plan(c["block_table"].shape[1], 8), caches, batch_sizes=(1, 2, 4, 8), bank=bank)
    note("graph set capture B8..B1, 2 layers")
    assert gs.capture() == [1, 2, 4, 8]
    assert len(bank.buffers()) == 1                       # the B8 panel, reused by B4/B2/B1
    for n, want in ((8, "graph:8"), (3, "graph:4"), (1, "graph:1"), (5, "graph:8"), (2, "graph:2")):
        rows = list(range(8 - n, 8))                       # a different slice each time
        note(f"graph set replay, live batch {n}")
        outs, route = gs.run([q[rows] for q in qs], c["block_table"][rows], c["seq_lens"][rows],
                             [lens[r] for r in rows])
        assert route == want
        ref = _singles(c, caches, qs, rows)
        for o, r in zip(outs, ref):
            assert _same_bits(o, r), (n, route)


def test_all_zero_batch_replays_to_zero():
    lens = [0, 0, 0]
    c, caches, qs = _setup(lens, seed=62, layers=1)
    gs = VerifyGraphs(_plan(c["block_table"].shape[1], 4), caches, batch_sizes=(4,), bank=A.WorkspaceBank())
    note("graph set, all-zero batch")
    gs.capture()
    outs, route = gs.run(qs, c["block_table"], c["seq_lens"], lens)
    assert route == "graph:4"
    assert (outs[0].view(torch.int16) == 0).all()        # exactly +0


def test_oversized_peer_takes_the_eager_route_with_the_same_bits():
    lens = [3000, 9000, 17]                                # 9000 > the graphs' 8192-token window
    c, caches, qs = _setup(lens, seed=63, width_tokens=9000)
    gs = VerifyGraphs(_plan(-(-BOUND // GEOM["page_size"]), 4), caches, batch_sizes=(4, 2), bank=A.WorkspaceBank())
    note("graph set, oversized peer")
    gs.capture()
    outs, route = gs.run(qs, c["block_table"], c["seq_lens"], lens)
    assert route == "eager"
    ref = _singles(c, caches, qs, [0, 1, 2])
    for o, r in zip(outs, ref):
        assert _same_bits(o, r)
    # without the long peer the same requests fit the window and replay a graph
    outs, route = gs.run([q[[0, 2]] for q in qs], c["block_table"][[0, 2]][:, :5].contiguous(),
                         c["seq_lens"][[0, 2]], [3000, 17])
    assert route == "graph:2"
    ref = _singles(c, caches, qs, [0, 2])
    for o, r in zip(outs, ref):
        assert _same_bits(o, r)


def test_graphs_captured_before_the_bank_grows_still_replay():
    lens = [4000, 100, 7000, 0, 2500, 8000, 33, 6000]
    c, caches, qs = _setup(lens, seed=64)
    bank = A.WorkspaceBank()
    gs = VerifyGraphs(_plan(c["block_table"].shape[1], 8), caches, batch_sizes=(4, 2), bank=bank)
    note("graph set, bank growth")
    gs.capture()
    assert len(bank.buffers()) == 1
    outs, route = gs.run(qs, c["block_table"], c["seq_lens"], lens)      # 8 > largest capture
    assert route == "eager"
    assert len(bank.buffers()) == 2                       # grown; the B4 panel stays alive
    rows = [1, 4, 6]
    outs, route = gs.run([q[rows] for q in qs], c["block_table"][rows], c["seq_lens"][rows],
                         [lens[r] for r in rows])
    assert route == "graph:4"
    ref = _singles(c, caches, qs, rows)
    for o, r in zip(outs, ref):
        assert _same_bits(o, r)


def test_hint_past_the_live_table_width_is_rejected_like_the_eager_route():
    # The live block table is 2 pages wide (3296 tokens), the graphs' window is 8192 tokens: a
    # hint of 4000 fits the window but not the table, so the graph route must not take it (the
    # graph's own wider table would hold -1 past the live width); the eager route rejects it.
    lens = [3000, 17]
    c, caches, qs = _setup(lens, seed=65, layers=1)
    gs = VerifyGraphs(_plan(c["block_table"].shape[1], 2), caches, batch_sizes=(2,), bank=A.WorkspaceBank())
    note("graph set, hint past the live table width")
    gs.capture()
    narrow = c["block_table"][:, :2].contiguous()
    with pytest.raises(ValueError):
        gs.run(qs, narrow, c["seq_lens"], [4000, 17])
    outs, route = gs.run(qs, narrow, c["seq_lens"], [3000, 17])      # within the width: the graph
    assert route == "graph:2"
    ref = _singles(c, caches, qs, [0, 1])
    assert _same_bits(outs[0], ref[0])
