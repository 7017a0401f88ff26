"""attn_run_static (the allocation-free entry point) against attn_run + attn_combine on the GPU.

Both run the same kernels; attn_run_static keeps the split workspace in the library's static
device array instead of a caller buffer, so its output must carry the same bits. Two calls in a
row (the second smaller, on another plan) show that what the first left in the array does not
reach the second; oracle checks keep both within the tolerance of the FP64 definition."""
import ctypes

import pytest
import torch

from _gpu import compare, note, oracle_pairs, plan_for, run_oracle, to_gpu
from verify_attention_e4m3_amd import attention as A
from verify_attention_e4m3_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16)


def _both(plan, c):
    ref = plan.run(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"], c["v_scale"])
    out = torch.full_like(c["q"], float("nan"))
    plan.run_static(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"],
                    c["v_scale"], out=out)
    torch.cuda.synchronize()
    return out, ref


def test_two_calls_in_a_row_match_the_workspace_path():
    w = wl.WORKLOADS["verify_b8_ctx128k_gqa6_16layers"]
    note("attn_run_static call 1: B8 x 131072 Hq24/Hkv4 E4M3 D256")
    c = wl.workload_case(w, device="cuda", layer=0)
    plan = plan_for(c)
    out, ref = _both(plan, c)
    assert torch.equal(_bits(out), _bits(ref))
    compare(out, oracle_pairs(c, [(0, 0), (7, 3), (3, 1)]))
    del c
    torch.cuda.empty_cache()

    note("attn_run_static call 2: B2 [3297, 61] Hq12/Hkv2 E4M3 D256 (smaller, another plan)")
    c2 = to_gpu(wl.make_case(batch=2, seq_lens=[3297, 61], q_len=8, num_q_heads=12, num_kv_heads=2, head_dim=256,
                             page_size=1648, seed=1))
    plan2 = plan_for(c2)
    out2, ref2 = _both(plan2, c2)
    assert torch.equal(_bits(out2), _bits(ref2))
    compare(out2, run_oracle(c2))


def test_other_formats_and_zero_rows_match_the_workspace_path():
    # FP16 D128 q1 (4 packed rows) and E4M3 D128 with zero-length and padded slots.
    note("attn_run_static: FP16 D128 q1 B3 and E4M3 D128 B4 with empty slots")
    c = to_gpu(wl.make_case(batch=3, seq_lens=[40, 1649, 7], q_len=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
                            page_size=1648, kv_format="fp16", seed=77))
    out, ref = _both(plan_for(c), c)
    assert torch.equal(_bits(out), _bits(ref))
    compare(out, run_oracle(c))
    c = to_gpu(wl.make_case(batch=4, seq_lens=[3000, 0, 129, 0], q_len=8, num_q_heads=24, num_kv_heads=4,
                            head_dim=128, page_size=32, seed=78, padded_slots=[3]))
    out, ref = _both(plan_for(c), c)
    assert torch.equal(_bits(out), _bits(ref))
    assert (_bits(out[1]) == 0).all() and (_bits(out[3]) == 0).all()
    compare(out, run_oracle(c))


def test_graph_replays_with_changed_inputs_match_eager():
    note("attn_run_static captured in a graph, replays with new Q and lengths")
    B = 4
    c = to_gpu(wl.make_case(batch=B, seq_lens=[6000] * B, q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256,
                            page_size=1648, seed=79, max_seq_len=6000))
    plan = plan_for(c)
    out = torch.empty_like(c["q"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plan.run_static(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"],
                        c["v_scale"], out=out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run_static(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"],
                        c["v_scale"], out=out)
    for rep, lens in enumerate([[6000, 3297, 0, 1], [17, 5999, 4000, 0], [6000] * 4]):
        c["q"].copy_(torch.randn(c["q"].shape, generator=torch.Generator("cuda").manual_seed(500 + rep),
                                 device="cuda").half())
        c["seq_lens"].copy_(torch.tensor(lens, dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        ref = plan.run(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"],
                       c["v_scale"])
        torch.cuda.synchronize()
        assert torch.equal(_bits(replayed), _bits(ref)), rep
    compare(replayed, run_oracle(c))


def test_batches_beyond_the_static_array_are_refused_before_launch():
    # 16 rows of up to 262144 tokens at Hkv 4 need 101.7 MB of split panels: refused with
    # ATTN_E_STATIC_WORKSPACE, and the output buffer is left as it was.
    note("attn_run_static refuses a batch beyond its static array")
    c = to_gpu(wl.make_case(batch=2, seq_lens=[100, 50], q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256,
                            page_size=3296, seed=80, max_seq_len=262144))
    plan = A.Plan(q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=3296, max_seq_len=262144,
                  max_pages_per_seq=c["block_table"].shape[1], batch_capacity=16, device="cuda:0")
    assert plan.workspace_bytes(16) > A.ATTN_STATIC_WORKSPACE_BYTES >= plan.workspace_bytes(2)
    q = torch.zeros((16,) + tuple(c["q"].shape[1:]), dtype=torch.float16, device="cuda")
    q[:2] = c["q"]
    bt = torch.full((16, c["block_table"].shape[1]), -1, dtype=torch.int32, device="cuda")
    bt[:2] = c["block_table"]
    lens = torch.zeros(16, dtype=torch.int32, device="cuda")
    lens[:2] = c["seq_lens"]
    out = torch.full_like(q, 7.0)
    with pytest.raises(A.AttnError) as e:
        plan.run_static(q, c["k_cache"], c["v_cache"], bt, lens, c["k_scale"], c["v_scale"], out=out)
    assert e.value.status == A.ATTN_E_STATIC_WORKSPACE
    torch.cuda.synchronize()
    assert (out == 7.0).all()
    # the two live rows alone fit
    out2 = plan.run_static(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"],
                           c["v_scale"])
    torch.cuda.synchronize()
    compare(out2, run_oracle(c))
