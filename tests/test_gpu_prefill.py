"""Long prefill (attn_prefill) on the GPU against the FP64 oracle: the oracle's verify-attention
definition with the whole K/V as one page and q_len = the query chunk ("SM70 attention and
quantized projection coverage across TP sizes", sections "Scope" and "Accumulation audit and
rejected tuning"). Small shapes are checked on every row; the Q8192 x KV262144 shape on
sampled query tokens (each through the oracle as a one-token query against the keys it sees)."""
import numpy as np
import pytest
import torch

import oracle
from _gpu import compare, note
from verify_attention_e4m3_amd import attention as A
from verify_attention_e4m3_amd import workloads as wl

pytestmark = pytest.mark.gpu


def oracle_prefill(q, k, v, *, causal=True, sm_scale=None, tokens=None):
    """FP64 oracle rows [len(tokens)][Hq][D] (all tokens by default)."""
    qn = q.cpu().numpy()
    kn = k.cpu().numpy()[None]
    vn = v.cpu().numpy()[None]
    q_len, kv_len = qn.shape[0], kn.shape[1]
    table = np.zeros((1, 1), dtype=np.int32)
    if tokens is None:
        return oracle.verify_attention(qn[None], kn, vn, table, np.array([kv_len], np.int32), 1.0, 1.0,
                                       page_size=kv_len, kv_format="fp16", causal=causal, sm_scale=sm_scale)[0]
    rows = []
    for t in tokens:
        L = kv_len - (q_len - 1 - t) if causal else kv_len
        if L <= 0:
            rows.append(np.zeros(qn.shape[1:]))
            continue
        r = oracle.verify_attention(qn[t][None, None], kn, vn, table, np.array([L], np.int32), 1.0, 1.0,
                                    page_size=kv_len, kv_format="fp16", causal=causal, sm_scale=sm_scale)
        rows.append(r[0, 0])
    return np.stack(rows)


SMALL = [
    dict(q_len=100, kv_len=300, num_q_heads=12, num_kv_heads=2),
    dict(q_len=64, kv_len=64, num_q_heads=6, num_kv_heads=1),          # the triangle alone
    dict(q_len=33, kv_len=1000, num_q_heads=24, num_kv_heads=4),       # ragged tiles
    dict(q_len=40, kv_len=20, num_q_heads=6, num_kv_heads=1),          # first 20 tokens see nothing
    dict(q_len=70, kv_len=500, num_q_heads=8, num_kv_heads=2),         # G = 4
    dict(q_len=40, kv_len=130, num_q_heads=2, num_kv_heads=2),         # G = 1
    dict(q_len=20, kv_len=100, num_q_heads=12, num_kv_heads=1),        # G = 12
    dict(q_len=45, kv_len=257, num_q_heads=6, num_kv_heads=2),         # G = 3
    dict(q_len=1, kv_len=5000, num_q_heads=6, num_kv_heads=1),
]


@pytest.mark.parametrize("kw", SMALL, ids=lambda kw: f"q{kw['q_len']}-kv{kw['kv_len']}-H{kw['num_q_heads']}/{kw['num_kv_heads']}")
def test_prefill_small(kw):
    note(f"prefill {kw}")
    c = wl.prefill_case(seed=kw["q_len"] + kw["kv_len"], device="cuda", **kw)
    out = A.prefill(c["q"], c["k"], c["v"])
    torch.cuda.synchronize()
    compare(out, oracle_prefill(c["q"], c["k"], c["v"]))


def test_prefill_non_causal_and_custom_scale():
    note("prefill non-causal, sm_scale 0.05")
    c = wl.prefill_case(q_len=50, kv_len=200, num_q_heads=6, num_kv_heads=1, seed=3, device="cuda")
    out = A.prefill(c["q"], c["k"], c["v"], causal=False, sm_scale=0.05)
    torch.cuda.synchronize()
    compare(out, oracle_prefill(c["q"], c["k"], c["v"], causal=False, sm_scale=0.05))


def test_prefill_head_major_strides():
    # [heads][tokens][D] buffers seen through [tokens][heads][D] views
    note("prefill head-major layouts")
    c = wl.prefill_case(q_len=80, kv_len=400, num_q_heads=12, num_kv_heads=2, seed=4, device="cuda")
    qh = c["q"].transpose(0, 1).contiguous().transpose(0, 1)
    kh = c["k"].transpose(0, 1).contiguous().transpose(0, 1)
    vh = c["v"].transpose(0, 1).contiguous().transpose(0, 1)
    out = torch.empty(12, 80, 256, dtype=torch.float16, device="cuda").transpose(0, 1)
    A.prefill(qh, kh, vh, out=out)
    torch.cuda.synchronize()
    compare(out, oracle_prefill(c["q"], c["k"], c["v"]))


def test_prefill_reference_overflow_recompute():
    # Keys past the first block score far higher than any in it, so the first pass's references
    # are exceeded by more than 2^10 and the workgroup recomputes with exact row maxima.
    note("prefill reference overflow")
    c = wl.prefill_case(q_len=96, kv_len=700, num_q_heads=6, num_kv_heads=1, seed=5, device="cuda")
    c["k"][300:] *= 6
    out = A.prefill(c["q"], c["k"], c["v"])
    torch.cuda.synchronize()
    compare(out, oracle_prefill(c["q"], c["k"], c["v"]))


def test_prefill_repeatable_bitwise():
    note("prefill run twice")
    c = wl.prefill_case(q_len=200, kv_len=3000, num_q_heads=12, num_kv_heads=2, seed=6, device="cuda")
    a = A.prefill(c["q"], c["k"], c["v"]).clone()
    b = A.prefill(c["q"], c["k"], c["v"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", ["prefill_q8192_kv262144_hkv1", "prefill_q8192_kv262144_hkv2",
                                  "prefill_q8192_kv262144_hkv4"])
def test_prefill_full_size_sampled_tokens(name):
    w = wl.PREFILL_WORKLOADS[name]
    note(f"{name}: sampled tokens")
    c = wl.prefill_case(q_len=w.q_len, kv_len=w.kv_len, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                        head_dim=w.head_dim, seed=w.seed, device="cuda")
    out = A.prefill(c["q"], c["k"], c["v"])
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    tokens = [0, 1, 4095, w.q_len - 1]
    compare(out[tokens], oracle_prefill(c["q"], c["k"], c["v"], tokens=tokens))
