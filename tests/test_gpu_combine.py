"""attn_combine alone, fed split panels that the oracle computed, against the oracle's merge.

The log-sum-exp combine of split partials is the one named in "perf(fa2): port decode GQA
group-swap into d128 varlen launcher" (PR #48, PR description). Here the split kernel is not run:
each (slot, KV head, split) panel of the workspace is filled from ``oracle.partial_states`` over
that split's token range (the ranges come from ``attn_plan_splits``), so a mistake in the merge
cannot hide behind a matching mistake in the split kernel.

Workspace panel layout (FP32, one panel of ``split_bytes`` per split, ``grid_splits`` panels per
(slot, KV head), slot-major): un-normalised O at ``r*D + d``, the row reference ``m`` in the
log2 domain at ``rows_alloc*D + r``, the row sum ``l`` at ``rows_alloc*D + rows_alloc + r``.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from verify_attention_e4m3_amd import workloads as wl

from _gpu import compare, note, plan_for, to_gpu

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)


def oracle_panels(case, plan):
    """FP32 workspace filled with the oracle's partial states (unused panels hold NaN)."""
    c = wl.to_numpy(case)
    info = plan.info
    B, Hkv, D = c["q"].shape[0], c["num_kv_heads"], c["head_dim"]
    rows = info["rows"]
    rows_alloc = -(-rows // 16) * 16
    split_floats = info["split_bytes"] // 4
    gs = info["grid_splits"]
    ws = np.full((B, Hkv, gs, split_floats), np.nan, dtype=np.float32)
    for b in range(B):
        L = int(c["seq_lens"][b])
        S, P = plan.splits(L)
        for g in range(Hkv):
            for s in range(S):
                m, l, o = oracle.partial_states(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"],
                                                float(c["k_scale"][0]), b=b, kv_head=g, begin=s * P,
                                                end=min((s + 1) * P, L), page_size=c["page_size"],
                                                kv_format=c["kv_format"])
                panel = ws[b, g, s]
                panel[:rows_alloc * D] = 0.0
                panel[:rows * D] = o.reshape(-1)
                panel[rows_alloc * D:rows_alloc * D + rows] = m * LOG2E
                panel[rows_alloc * D + rows_alloc:rows_alloc * D + rows_alloc + rows] = l
    return torch.from_numpy(ws.reshape(-1))


COMBINE_CASES = [
    # (name, kwargs of make_case)
    ("b3_tails", dict(batch=3, seq_lens=[3297, 8195, 5], q_len=8, num_q_heads=12, num_kv_heads=2, head_dim=256,
                      page_size=1648, seed=71)),
    ("b2_fp16_d128_q1", dict(batch=2, seq_lens=[9000, 0], q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                             page_size=16, kv_format="fp16", seed=72)),
    ("b2_q8_short", dict(batch=2, seq_lens=[7, 520], q_len=8, num_q_heads=6, num_kv_heads=1, head_dim=256,
                         page_size=32, seed=73, kv_scale=0.37)),
]


@pytest.mark.parametrize("name,kw", COMBINE_CASES, ids=[c[0] for c in COMBINE_CASES])
def test_combine_of_oracle_panels(name, kw):
    case = wl.make_case(**kw)
    case["v_scale"] = case["v_scale"] * 1.7            # distinct K and V scales
    plan = plan_for(case)
    ws = oracle_panels(case, plan)
    ref = oracle.verify_attention(*[wl.to_numpy(case)[k] for k in ("q", "k_cache", "v_cache", "block_table",
                                                                   "seq_lens")],
                                  float(case["k_scale"][0]), float(case["v_scale"][0]), page_size=case["page_size"],
                                  kv_format=case["kv_format"])
    note(f"combine of oracle panels: {name} splits={[plan.splits(int(L)) for L in case['seq_lens']]}")
    d = to_gpu(case)
    ws_d = ws.cuda()
    out = torch.full_like(d["q"], float("nan"))
    args = plan.make_args(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"], d["k_scale"],
                          d["v_scale"], out, ws_d)
    plan.combine(args)
    torch.cuda.synchronize()
    print(compare(out, ref))
    assert torch.equal(ws_d.cpu().view(torch.int32), ws.view(torch.int32))      # the combine only reads it
