"""GPU parity at the full sizes of the long-context workloads, in the launch configuration the
benchmark times: every benchmarked B8 x 131072 workload (E4M3, E5M2 and FP16 at D256, E4M3 at
D128, Hq4/Hkv1; every output row of layer 0 against the oracle) and B16 mixed lengths up to
262144 with page 3296, captured once in a graph and replayed with fresh queries, lengths and
zero rows (every live row of every replay against the oracle)."""
import numpy as np
import pytest
import torch

from _gpu import compare, note, oracle_pairs, plan_for
from verify_attention_e4m3_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["verify_b8_ctx128k_gqa6_16layers", "verify_b8_ctx128k_gqa6_e5m2_16layers",
                                  "verify_b8_ctx128k_gqa6_fp16_d256_4layers",
                                  "verify_b8_ctx128k_gqa6_e4m3_d128_16layers", "verify_b8_ctx128k_hq4_hkv1_16layers"])
def test_b8_ctx128k_full_layer(name):
    # Every benchmarked B8 x 131072 workload, in the launch configuration the benchmark times
    # (its plan, the full batch, paired / grouped KV heads where the grid allows): every
    # (slot, KV head) pair of layer 0, i.e. every output row, against the oracle.
    w = wl.WORKLOADS[name]
    note(f"{w.name} layer 0, every (slot, KV head) pair")
    c = wl.workload_case(w, device="cuda", layer=0)
    plan = plan_for(c)
    out = plan.run(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"], c["v_scale"])
    torch.cuda.synchronize()
    pairs = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    stats = compare(out, oracle_pairs(c, pairs))
    assert stats["rows"] == w.batch * w.q_len * w.num_q_heads


def test_b16_mixed_graph_replays():
    w = wl.WORKLOADS["verify_b16_mixed_ctx256k_page3296"]
    note(f"{w.name} graph capture at B16/262144, replays with seeds 40..42")
    B = w.batch
    padded = list(range(B - 3, B))
    alloc = [w.max_seq_len] * (B - 3) + [0] * 3
    c = wl.make_case(batch=B, seq_lens=wl.mixed_lengths(B, w.seed), q_len=w.q_len, num_q_heads=w.num_q_heads,
                     num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size, seed=w.seed,
                     device="cuda", max_seq_len=w.max_seq_len, alloc_lens=alloc, padded_slots=padded)
    plan = plan_for(c)
    out = torch.empty_like(c["q"])
    ws = torch.empty(plan.workspace_bytes(B) // 4, dtype=torch.float32, device="cuda")
    args = plan.make_args(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"],
                          c["v_scale"], out, ws)
    plan.split(args)
    plan.combine(args)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.split(args)
        plan.combine(args)
    for seed in (40, 41, 42):
        lens = wl.mixed_lengths(B, seed)
        note(f"replay seed {seed} lengths {lens}")
        c["seq_lens"].copy_(torch.tensor(lens, dtype=torch.int32))
        q = torch.randn(c["q"].shape, generator=torch.Generator("cuda").manual_seed(seed), device="cuda").half()
        q[padded] = float("nan")
        c["q"].copy_(q)
        for rep in range(2):
            g.replay()
            torch.cuda.synchronize()
            if rep == 0:
                first = out.clone()
        assert torch.equal(first.view(torch.int16), out.view(torch.int16))
        live = [b for b in range(B) if lens[b] > 0]
        pairs = [(b, g) for b in live for g in range(w.num_kv_heads)]     # every live row
        stats = compare(out, oracle_pairs(c, pairs))
        assert stats["rows"] == len(live) * w.q_len * w.num_q_heads
        for b in range(B):
            if lens[b] == 0:
                assert (out[b].view(torch.int16) == 0).all(), b
        # eager execution of the same inputs gives the replayed bits
        eager = torch.empty_like(out)
        args_e = plan.make_args(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"],
                                c["v_scale"], eager, ws)
        plan.split(args_e)
        plan.combine(args_e)
        torch.cuda.synchronize()
        assert torch.equal(eager.view(torch.int16), out.view(torch.int16))


# The pages' GPU coverage matrix (batch sizes, contexts 3297 .. 262144, page sizes 1024 / 1536 /
# 1648 / 3296), each checked on sampled (slot, KV head) pairs against the oracle; plus the smallest page
# size at the longest row (16384 block-table entries, 513 of them staged per split).
MATRIX = [(2, 3297, 1024), (4, 8192, 1536), (8, 32768, 1648), (16, 131072, 3296), (2, 262144, 1024),
          (1, 262144, 16)]


@pytest.mark.parametrize("batch,length,page", MATRIX, ids=[f"B{b}-L{l}-p{p}" for b, l, p in MATRIX])
def test_coverage_matrix_sampled(batch, length, page):
    note(f"coverage matrix B{batch} L{length} page {page}")
    lens = [length - (i % 3) * 97 for i in range(batch)]
    c = wl.make_case(batch=batch, seq_lens=lens, q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256,
                     page_size=page, seed=batch * 7 + page, device="cuda", max_seq_len=length)
    plan = plan_for(c)
    out = plan.run(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"], c["v_scale"])
    torch.cuda.synchronize()
    pairs = [(0, 0), (batch - 1, 3)]
    compare(out, oracle_pairs(c, pairs))


def test_library_batch_capacity_sampled():
    # The largest batch the library admits (its reported capacity, 256 slots), short mixed
    # lengths with zero-length slots among them and 16-token pages: sampled pairs against the
    # oracle, every zero-length slot exactly +0.
    from verify_attention_e4m3_amd import attention as A
    B = A.capabilities()["max_batch"]
    note(f"library batch capacity B{B}, lengths <= 2048, page 16")
    rng = np.random.default_rng(83)
    lens = [int(x) for x in rng.integers(0, 2049, size=B)]
    for i in range(0, B, 37):
        lens[i] = 0
    c = wl.make_case(batch=B, seq_lens=lens, q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=16,
                     seed=84, device="cuda", max_seq_len=2048)
    plan = plan_for(c)
    out = plan.run(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"], c["v_scale"])
    torch.cuda.synchronize()
    zero = [b for b in range(B) if lens[b] == 0]
    assert zero and (out[zero].view(torch.int16) == 0).all()
    live = [b for b in range(B) if lens[b] > 0]
    pairs = [(live[0], 0), (live[len(live) // 2], 2), (live[-1], 3), (B - 1 if lens[B - 1] else live[-2], 1)]
    compare(out, oracle_pairs(c, pairs))
