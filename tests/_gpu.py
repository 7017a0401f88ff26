"""Helpers for the GPU tests: run the HIP path through the C ABI, run the oracle, compare."""
import math
import sys

import numpy as np
import torch

import oracle
from verify_attention_e4m3_amd import attention as A
from verify_attention_e4m3_amd import workloads as wl

MAX_ABS = 4e-3       # element-wise bound against the FP64 oracle
REL_L2 = 3e-3        # per-row (one (b, t, h) D-vector) relative L2 bound


def note(msg: str):
    """Say which case is about to run, before it touches the GPU."""
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()


def to_gpu(case: dict) -> dict:
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in case.items()}


def plan_for(case: dict, *, batch_capacity=None, causal=True, sm_scale=0.0, k_strides=None, v_strides=None,
             max_seq_len=None, page_size=None) -> A.Plan:
    return A.Plan(q_len=case["q_len"], num_q_heads=case["num_q_heads"], num_kv_heads=case["num_kv_heads"],
                  head_dim=case["head_dim"], page_size=page_size or case["page_size"],
                  max_seq_len=max_seq_len or case["max_seq_len"],
                  max_pages_per_seq=case["block_table"].shape[1],
                  batch_capacity=batch_capacity or case["q"].shape[0], kv_dtype=case["kv_format"],
                  k_strides=k_strides, v_strides=v_strides, sm_scale=sm_scale, causal=causal, device="cuda:0")


def run_gpu(case: dict, plan: A.Plan = None, **kw) -> torch.Tensor:
    plan = plan or plan_for(case, **kw)
    out = plan.run(case["q"], case["k_cache"], case["v_cache"], case["block_table"], case["seq_lens"],
                   case["k_scale"], case["v_scale"])
    torch.cuda.synchronize()
    return out


def run_oracle(case: dict, pairs=None, causal=True, sm_scale=None) -> np.ndarray:
    c = wl.to_numpy(case)
    return oracle.verify_attention(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"],
                                   float(c["k_scale"][0]), float(c["v_scale"][0]), page_size=c["page_size"],
                                   kv_format=c["kv_format"], causal=causal, sm_scale=sm_scale, pairs=pairs)


def compare(out: torch.Tensor, ref: np.ndarray, *, max_abs=MAX_ABS, rel_l2=REL_L2) -> dict:
    """Check the FP16 GPU output against the FP64 oracle (rows where ref is NaN are skipped)."""
    got = out.float().cpu().numpy().astype(np.float64)
    D = got.shape[-1]
    g = got.reshape(-1, D)
    r = ref.reshape(-1, D)
    live = ~np.isnan(r).any(axis=1)
    g, r = g[live], r[live]
    assert np.isfinite(g).all(), "non-finite GPU output"
    err = np.abs(g - r)
    rn = np.linalg.norm(r, axis=1)
    en = np.linalg.norm(g - r, axis=1)
    zero = rn == 0
    # rows that see no key must be exactly +0
    assert (g[zero] == 0).all() and not np.signbit(g[zero]).any(), "empty rows are not +0"
    rel = en[~zero] / rn[~zero]
    stats = dict(rows=int(live.sum()), max_abs=float(err.max(initial=0.0)),
                 max_rel_l2=float(rel.max(initial=0.0)), zero_rows=int(zero.sum()))
    assert stats["max_abs"] <= max_abs, stats
    assert stats["max_rel_l2"] <= rel_l2, stats
    return stats


def oracle_pairs(case: dict, pairs, causal=True) -> np.ndarray:
    c = wl.host_subset(case, pairs)
    return oracle.verify_attention(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"],
                                   float(c["k_scale"][0]), float(c["v_scale"][0]), page_size=c["page_size"],
                                   kv_format=c["kv_format"], causal=causal, pairs=pairs)


def e4m3_fp16_exact(byte_vals: np.ndarray) -> np.ndarray:
    return oracle.decode_table()[byte_vals].astype(np.float16)


__all__ = ["note", "to_gpu", "plan_for", "run_gpu", "run_oracle", "compare", "oracle_pairs", "math"]
