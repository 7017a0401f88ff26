"""GPU parity of the HIP path (through the C ABI) against the FP64 oracle, plus the exact
GPU-vs-GPU invariants: batched == single request, page size / permutation invariance,
replay == eager, run-to-run determinism. Every test here needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import oracle
from _gpu import compare, note, oracle_pairs, plan_for, run_gpu, run_oracle, to_gpu
from verify_attention_e4m3_amd import attention as A
from verify_attention_e4m3_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _case(**kw):
    return to_gpu(wl.make_case(**kw))


def test_e4m3_bytes_decode_exactly():
    # L == q_len: verify token 0 sees only key 0, whose V row holds all 254 finite E4M3
    # byte values; softmax of one key is 1, so the output is exactly those values in FP16
    # (as values: byte 0x80, -0, may come out as +0 after the FP32 accumulation from +0).
    note("e4m3 all bytes, B1 L8 Hq6 Hkv1 page16")
    c = _case(batch=1, seq_lens=[8], q_len=8, num_q_heads=6, num_kv_heads=1, head_dim=256, page_size=16, seed=101)
    vals = np.arange(256, dtype=np.uint8)
    vals[[0x7F, 0xFF]] = 0
    page = int(c["block_table"][0, 0])
    c["v_cache"][page, 0, 0, :] = torch.from_numpy(vals).cuda()
    out = run_gpu(c)
    want = torch.from_numpy(oracle.decode_table()[vals].astype(np.float16)).cuda()
    for h in range(6):
        assert torch.equal(out[0, 0, h], want), h            # value equality: -0 == +0
        nonzero = want != 0
        assert torch.equal(out[0, 0, h][nonzero].view(torch.int16), want[nonzero].view(torch.int16)), h


def test_e5m2_bytes_decode_exactly():
    # As above for E5M2: the only visible key's V row holds all 248 finite E5M2 bytes (up to
    # +-57344 and down to the subnormal 2^-16), so the output is exactly those FP16 values.
    note("e5m2 all bytes, B1 L8 Hq6 Hkv1 page16")
    c = _case(batch=1, seq_lens=[8], q_len=8, num_q_heads=6, num_kv_heads=1, head_dim=256, page_size=16, seed=102,
              kv_format="e5m2")
    vals = np.arange(256, dtype=np.uint8)
    vals[[0x7C, 0x7D, 0x7E, 0x7F, 0xFC, 0xFD, 0xFE, 0xFF]] = 0
    page = int(c["block_table"][0, 0])
    c["v_cache"][page, 0, 0, :] = torch.from_numpy(vals).cuda()
    out = run_gpu(c)
    want = torch.from_numpy(oracle.decode_e5m2_table()[vals].astype(np.float16)).cuda()
    for h in range(6):
        assert torch.equal(out[0, 0, h], want), h
        nonzero = want != 0
        assert torch.equal(out[0, 0, h][nonzero].view(torch.int16), want[nonzero].view(torch.int16)), h


E5M2_SMALL = [
    dict(batch=2, seq_lens=[5, 700], q_len=8, num_q_heads=6, num_kv_heads=1, page_size=16),
    dict(batch=3, seq_lens=[2000, 33, 0], q_len=8, num_q_heads=24, num_kv_heads=4, page_size=1648, kv_std=0.5,
         kv_scale=2.0),
    dict(batch=2, seq_lens=[9000, 300], q_len=4, num_q_heads=16, num_kv_heads=4, page_size=32),
]


@pytest.mark.parametrize("kw", E5M2_SMALL, ids=lambda kw: f"e5m2-B{kw['batch']}-L{max(kw['seq_lens'])}-q{kw['q_len']}-"
                                                           f"H{kw['num_q_heads']}/{kw['num_kv_heads']}")
def test_parity_e5m2(kw):
    note(f"parity e5m2 {kw}")
    c = _case(head_dim=256, kv_format="e5m2", seed=sum(kw["seq_lens"]) + 5, **kw)
    compare(run_gpu(c), run_oracle(c))


SMALL = [
    dict(batch=1, seq_lens=[1], q_len=8, num_q_heads=6, num_kv_heads=1, page_size=16),
    dict(batch=1, seq_lens=[8], q_len=8, num_q_heads=6, num_kv_heads=1, page_size=16),
    dict(batch=2, seq_lens=[5, 33], q_len=8, num_q_heads=6, num_kv_heads=1, page_size=16),
    dict(batch=3, seq_lens=[100, 17, 64], q_len=8, num_q_heads=12, num_kv_heads=2, page_size=32),
    dict(batch=2, seq_lens=[513, 1025], q_len=8, num_q_heads=24, num_kv_heads=4, page_size=48),
    dict(batch=4, seq_lens=[0, 700, 1, 2000], q_len=8, num_q_heads=24, num_kv_heads=4, page_size=1648),
    dict(batch=2, seq_lens=[1000, 31], q_len=4, num_q_heads=16, num_kv_heads=4, page_size=16),
    dict(batch=2, seq_lens=[40, 600], q_len=1, num_q_heads=6, num_kv_heads=1, page_size=16),
    dict(batch=1, seq_lens=[5000], q_len=8, num_q_heads=32, num_kv_heads=8, page_size=64),
    dict(batch=2, seq_lens=[4097, 9000], q_len=8, num_q_heads=6, num_kv_heads=1, page_size=3296, kv_std=0.25,
         kv_scale=3.0),
]


@pytest.mark.parametrize("kw", SMALL, ids=lambda kw: f"B{kw['batch']}-L{max(kw['seq_lens'])}-q{kw['q_len']}-"
                                                      f"H{kw['num_q_heads']}/{kw['num_kv_heads']}-p{kw['page_size']}")
def test_parity_small(kw):
    note(f"parity small {kw}")
    c = _case(head_dim=256, seed=sum(kw["seq_lens"]) + kw["page_size"], **kw)
    stats = compare(run_gpu(c), run_oracle(c))
    assert stats["rows"] > 0


@pytest.mark.parametrize("q_len", range(1, 9))
def test_parity_every_q_len(q_len):
    # q-generic verify: batched q1..q8 with six query heads per KV head (6..48 packed rows, so
    # one, two and three row tiles), lengths around and below q.
    note(f"parity q_len {q_len}, B4 Hq12/Hkv2")
    c = _case(batch=4, seq_lens=[1500, q_len, max(q_len - 1, 0), 4097], q_len=q_len, num_q_heads=12,
              num_kv_heads=2, head_dim=256, page_size=32, seed=200 + q_len)
    compare(run_gpu(c), run_oracle(c))


@pytest.mark.parametrize("q_len", [1, 3, 8])
def test_parity_four_query_heads_on_one_kv_head(q_len):
    note(f"parity Hq4/Hkv1 q_len {q_len}")
    c = _case(batch=3, seq_lens=[3297, 100, 7], q_len=q_len, num_q_heads=4, num_kv_heads=1, head_dim=256,
              page_size=1648, seed=210 + q_len)
    compare(run_gpu(c), run_oracle(c))


@pytest.mark.parametrize("group,q_len", [(3, 8), (5, 8), (8, 6), (12, 4), (16, 3), (48, 1)])
def test_parity_other_head_groups(group, q_len):
    # Packed rows q_len * G for groups that are not powers of two or exceed the q8 GQA6 shape
    # (24 to 48 rows; one to three row tiles, the last one partly filled), two KV heads.
    note(f"parity G{group} q{q_len}, B2 Hkv2")
    c = _case(batch=2, seq_lens=[1777, q_len + 3], q_len=q_len, num_q_heads=2 * group, num_kv_heads=2,
              head_dim=256, page_size=48, seed=300 + group)
    compare(run_gpu(c), run_oracle(c))


def test_parity_non_causal_and_custom_scale():
    note("parity non-causal, sm_scale 0.05")
    c = _case(batch=2, seq_lens=[77, 1500], q_len=8, num_q_heads=6, num_kv_heads=1, head_dim=256, page_size=16,
              seed=7, kv_scale=0.5)
    out = run_gpu(c, causal=False, sm_scale=0.05)
    compare(out, run_oracle(c, causal=False, sm_scale=0.05))


def test_parity_distinct_k_and_v_scales():
    note("parity k_scale 0.25, v_scale 4")
    c = _case(batch=2, seq_lens=[333, 2048], q_len=8, num_q_heads=12, num_kv_heads=2, head_dim=256, page_size=32,
              seed=8)
    c["k_scale"].fill_(0.25)
    c["v_scale"].fill_(4.0)
    compare(run_gpu(c), run_oracle(c))


@pytest.mark.parametrize("k_scale,v_scale", [(-0.75, 1.5), (-2.0, -0.5), (0.0, 1.0)])
def test_parity_negative_and_zero_scales(k_scale, v_scale):
    # A negative k_scale flips the sign of every score (the kernel moves it into Q); a negative
    # v_scale flips the output; k_scale 0 makes every visible key equally likely.
    note(f"parity k_scale {k_scale}, v_scale {v_scale}")
    c = _case(batch=2, seq_lens=[333, 2048], q_len=8, num_q_heads=12, num_kv_heads=2, head_dim=256, page_size=32,
              seed=18)
    c["k_scale"].fill_(k_scale)
    c["v_scale"].fill_(v_scale)
    compare(run_gpu(c), run_oracle(c))


def test_power_of_two_scales_are_exact():
    # Scaling by powers of two commutes with FP32/FP16 rounding (no overflow at these values):
    # (2Q, k_scale) and (Q, 2 k_scale) give the same bits, and doubling v_scale doubles every
    # output whose FP16 value stays normal (subnormals round on a fixed grid).
    note("power-of-two scale metamorphics, B2 L900/5000 Hq12 Hkv2")
    c = _case(batch=2, seq_lens=[900, 5000], q_len=8, num_q_heads=12, num_kv_heads=2, head_dim=256, page_size=32,
              seed=9)
    base = run_gpu(c).clone()
    c2 = dict(c)
    c2["q"] = c["q"] * 2
    c2["k_scale"] = c["k_scale"] * 0.5
    assert torch.equal(run_gpu(c2).view(torch.int16), base.view(torch.int16))
    c3 = dict(c)
    c3["v_scale"] = c["v_scale"] * 2
    doubled = run_gpu(c3)
    big = base.abs() >= 2.0 ** -13
    assert big.float().mean() > 0.9
    assert torch.equal(doubled[big].view(torch.int16), (base[big] * 2).view(torch.int16))
    assert ((doubled[~big].float() - 2 * base[~big].float()).abs() <= 2.0 ** -24).all()


FP16_D128 = [
    dict(batch=2, seq_lens=[1, 3000], q_len=1, num_q_heads=8, num_kv_heads=2, page_size=16),
    dict(batch=3, seq_lens=[40, 1649, 7], q_len=1, num_q_heads=32, num_kv_heads=8, page_size=1648),
    dict(batch=2, seq_lens=[777, 5000], q_len=8, num_q_heads=16, num_kv_heads=4, page_size=32),   # 32 rows
    dict(batch=2, seq_lens=[100, 2500], q_len=8, num_q_heads=48, num_kv_heads=8, page_size=64),   # 48 rows
]


@pytest.mark.parametrize("kw", FP16_D128, ids=lambda kw: f"fp16-B{kw['batch']}-L{max(kw['seq_lens'])}-q{kw['q_len']}-"
                                                           f"H{kw['num_q_heads']}/{kw['num_kv_heads']}")
def test_parity_fp16_d128(kw):
    note(f"parity fp16 d128 {kw}")
    c = _case(head_dim=128, kv_format="fp16", seed=sum(kw["seq_lens"]) + 3, **kw)
    compare(run_gpu(c), run_oracle(c))


def test_fp16_values_pass_through_exactly():
    # q1, L = 1: the only key's V row comes out exactly (softmax of one key is 1).
    note("fp16 d128 identity row")
    c = _case(batch=1, seq_lens=[1], q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=128, page_size=16,
              kv_format="fp16", seed=5)
    out = run_gpu(c)
    page = int(c["block_table"][0, 0])
    want = c["v_cache"][page, 0, 0, :]
    for h in range(4):
        assert torch.equal(out[0, 0, h], want), h


FP16_D256 = [
    dict(batch=2, seq_lens=[5, 700], q_len=8, num_q_heads=6, num_kv_heads=1, page_size=16),
    dict(batch=3, seq_lens=[3000, 33, 0], q_len=8, num_q_heads=24, num_kv_heads=4, page_size=1648),
    dict(batch=2, seq_lens=[9000, 17], q_len=1, num_q_heads=8, num_kv_heads=2, page_size=32),
    dict(batch=2, seq_lens=[1025, 64], q_len=4, num_q_heads=16, num_kv_heads=4, page_size=48),
]


@pytest.mark.parametrize("kw", FP16_D256, ids=lambda kw: f"fp16d256-B{kw['batch']}-L{max(kw['seq_lens'])}-q{kw['q_len']}-"
                                                           f"H{kw['num_q_heads']}/{kw['num_kv_heads']}")
def test_parity_fp16_d256(kw):
    note(f"parity fp16 d256 {kw}")
    c = _case(head_dim=256, kv_format="fp16", seed=sum(kw["seq_lens"]) + 11, **kw)
    compare(run_gpu(c), run_oracle(c))


def test_fp16_d256_values_pass_through_exactly():
    # L == q_len: verify token 0 sees only key 0, so its output is that V row exactly.
    note("fp16 d256 identity row")
    c = _case(batch=1, seq_lens=[8], q_len=8, num_q_heads=6, num_kv_heads=1, head_dim=256, page_size=16,
              kv_format="fp16", seed=12)
    out = run_gpu(c)
    page = int(c["block_table"][0, 0])
    want = c["v_cache"][page, 0, 0, :]
    for h in range(6):
        assert torch.equal(out[0, 0, h], want), h


E4M3_D128 = [
    dict(batch=2, seq_lens=[5, 700], q_len=8, num_q_heads=6, num_kv_heads=1, page_size=16),
    dict(batch=3, seq_lens=[3000, 33, 0], q_len=8, num_q_heads=24, num_kv_heads=4, page_size=1648),
    dict(batch=2, seq_lens=[9000, 17], q_len=1, num_q_heads=8, num_kv_heads=2, page_size=32),
    dict(batch=2, seq_lens=[1025, 64], q_len=4, num_q_heads=16, num_kv_heads=4, page_size=48),
]


@pytest.mark.parametrize("kw", E4M3_D128, ids=lambda kw: f"e4m3d128-B{kw['batch']}-L{max(kw['seq_lens'])}-q{kw['q_len']}-"
                                                           f"H{kw['num_q_heads']}/{kw['num_kv_heads']}")
def test_parity_e4m3_d128(kw):
    note(f"parity e4m3 d128 {kw}")
    c = _case(head_dim=128, seed=sum(kw["seq_lens"]) + 13, **kw)
    compare(run_gpu(c), run_oracle(c))


@pytest.mark.parametrize("half", [0, 1])
def test_e4m3_d128_bytes_decode_exactly(half):
    # The only visible key's V row (128 dims) holds half of the 254 finite E4M3 values.
    note(f"e4m3 d128 bytes, half {half}")
    c = _case(batch=1, seq_lens=[8], q_len=8, num_q_heads=6, num_kv_heads=1, head_dim=128, page_size=16, seed=103)
    vals = np.arange(128 * half, 128 * half + 128, dtype=np.uint8)
    vals[(vals == 0x7F) | (vals == 0xFF)] = 0
    page = int(c["block_table"][0, 0])
    c["v_cache"][page, 0, 0, :] = torch.from_numpy(vals).cuda()
    out = run_gpu(c)
    want = torch.from_numpy(oracle.decode_table()[vals].astype(np.float16)).cuda()
    for h in range(6):
        assert torch.equal(out[0, 0, h], want), h
        nonzero = want != 0
        assert torch.equal(out[0, 0, h][nonzero].view(torch.int16), want[nonzero].view(torch.int16)), h


@pytest.mark.parametrize("name", ["verify_b1_ctx3297_hq6_hkv1", "verify_b4_ctx32k_gqa6",
                                  "decode_b8_ctx32k_d128_fp16_gqa4", "verify_b4_ctx32k_gqa6_e5m2",
                                  "verify_b4_ctx32k_gqa6_fp16_d256", "verify_b4_ctx32k_gqa6_e4m3_d128"])
def test_parity_workload_full(name):
    note(f"parity full workload {name}")
    w = wl.WORKLOADS[name]
    c = to_gpu(wl.workload_case(w))
    stats = compare(run_gpu(c), run_oracle(c))
    assert stats["rows"] == w.batch * w.q_len * w.num_q_heads


def test_batched_equals_single_bitwise():
    note("batched vs single, B5 mixed lengths")
    c = _case(batch=5, seq_lens=[3297, 0, 40000, 8, 131], q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256,
              page_size=1648, seed=9, max_seq_len=65536)
    batched = run_gpu(c, batch_capacity=16)
    for b in range(5):
        one = {k: (v[b:b + 1] if k in ("q", "block_table", "seq_lens") else v) for k, v in c.items()}
        single = run_gpu(one, batch_capacity=1)
        assert torch.equal(single[0].view(torch.int16), batched[b].view(torch.int16)), b


@pytest.mark.parametrize("hkv", [4, 1])
def test_rows_past_131072_tokens_batched_equals_single(hkv):
    # Rows longer than 131072 tokens keep the 131072-token row's partition and get more splits
    # (32 of 8192 at 262144 tokens and Hkv 4; the 64-split ceiling at Hkv 1): sampled pairs of
    # the longest row against the oracle, and each row alone gives the batched bits.
    lens = [262144, 131073, 200001]
    note(f"rows past 131072 tokens, Hkv{hkv}, lengths {lens}")
    c = _case(batch=3, seq_lens=lens, q_len=8, num_q_heads=6 * hkv, num_kv_heads=hkv, head_dim=256,
              page_size=1648, seed=31 + hkv, max_seq_len=262144)
    plan = plan_for(c)
    assert plan.splits(262144)[0] == (32 if hkv == 4 else 64)
    batched = run_gpu(c, plan)
    compare(batched, oracle_pairs(c, [(0, hkv - 1), (1, 0)]))
    for b in range(3):
        one = {k: (v[b:b + 1] if k in ("q", "block_table", "seq_lens") else v) for k, v in c.items()}
        single = run_gpu(one, batch_capacity=1)
        assert torch.equal(single[0].view(torch.int16), batched[b].view(torch.int16)), b


def test_slot_permutation_permutes_the_output_bitwise():
    # Workgroups take slots in order of decreasing partition length, so a permuted batch is
    # served by different workgroups in a different order; every request's bits must follow it.
    note("slot permutation, B6 mixed lengths")
    lens = [100, 40000, 3297, 0, 70000, 8]
    c = _case(batch=6, seq_lens=lens, q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=1648,
              seed=41, max_seq_len=70000)
    base = run_gpu(c)
    perm = [4, 2, 5, 0, 3, 1]
    pc = dict(c)
    for k in ("q", "block_table", "seq_lens"):
        pc[k] = c[k][perm].contiguous()
    out = run_gpu(pc)
    assert torch.equal(out.view(torch.int16), base[perm].view(torch.int16))
    compare(base, oracle_pairs(c, [(4, 0), (1, 3), (2, 1)]))


_LAYOUT_CASES = [
    # (q_len, Hq, Hkv, format, D): one row tile at q1 (the D128 FP16 decode shape) and q2, two
    # row tiles at q3 (one slot alone: two row groups of one tile each), three at q8 (one slot
    # alone: three row groups sharing one LDS ring per token half; odd tile counts at 131 and
    # 3297 tokens, a single tile at 1 and 8)
    (1, 32, 8, "fp16", 128),
    (2, 24, 4, "e5m2", 256),
    (3, 24, 4, "e4m3", 256),
    (3, 24, 4, "fp16", 256),
    (8, 24, 4, "e4m3", 256),
]


@pytest.mark.parametrize("q_len,hq,hkv,fmt,head_dim", _LAYOUT_CASES,
                         ids=[f"q{q}-H{a}/{b}-{f}-d{d}" for q, a, b, f, d in _LAYOUT_CASES])
def test_workgroup_layouts_equal_single_bitwise(q_len, hq, hkv, fmt, head_dim):
    # B8 of a 65536-token plan fills the chip (head-pair workgroups, one row group); each slot
    # alone runs one-head workgroups (with two row groups where it has two row tiles). Every
    # layout computes a row the same way, so each slot alone gives the batched bits.
    lens = [3297, 0, 40000, 8, 131, 65536, 1, 20000]
    note(f"layouts vs single, q{q_len} Hq{hq}/Hkv{hkv} {fmt} D{head_dim}")
    c = _case(batch=8, seq_lens=lens, q_len=q_len, num_q_heads=hq, num_kv_heads=hkv, head_dim=head_dim,
              page_size=1648, seed=71 + q_len + hkv, kv_format=fmt, max_seq_len=65536)
    plan = plan_for(c)
    gs, cus = plan.info["grid_splits"], plan.info["num_cus"]
    assert 8 * (hkv // 2) * gs >= cus > hkv * gs        # batched pairs heads; one slot is a small grid
    batched = run_gpu(c, plan)
    short = [0, 3, 4, 6]                                 # the oracle on the short rows
    compare(batched[short], run_oracle({**c, **{k: c[k][short] for k in ("q", "block_table", "seq_lens")}}))
    for b in range(8):
        one = {k: (v[b:b + 1] if k in ("q", "block_table", "seq_lens") else v) for k, v in c.items()}
        single = run_gpu(one, batch_capacity=1)
        assert torch.equal(single[0].view(torch.int16), batched[b].view(torch.int16)), b


def test_paired_head_workgroups_equal_single_bitwise():
    # B8 at Hkv4 and 64K fills the chip with workgroups that hold two KV heads each; one slot
    # alone runs one head per workgroup. Both run each head's split the same way.
    note("head-pair workgroups vs single-slot runs, B8 Hkv4 max 65536")
    lens = [3297, 0, 40000, 8, 131, 65536, 1, 20000]
    c = _case(batch=8, seq_lens=lens, q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=1648,
              seed=19, max_seq_len=65536)
    plan = plan_for(c)
    gs = plan.info["grid_splits"]
    assert 8 * 2 * gs >= plan.info["num_cus"] > 2 * gs       # batched pairs heads, single does not
    batched = run_gpu(c, plan)
    for b in range(8):
        one = {k: (v[b:b + 1] if k in ("q", "block_table", "seq_lens") else v) for k, v in c.items()}
        single = run_gpu(one, batch_capacity=1)
        assert torch.equal(single[0].view(torch.int16), batched[b].view(torch.int16)), b


def test_four_head_workgroups_e4m3_d128_equal_single_bitwise():
    # E4M3 at D128 groups four KV heads per workgroup when the grid is large enough (B8 at Hkv4
    # and 64K); one slot alone runs one head per workgroup. Both run each head's split the same way.
    note("four-head workgroups vs single-slot runs, E4M3 D128 B8 Hkv4 max 65536")
    lens = [3297, 0, 40000, 8, 131, 65536, 1, 20000]
    c = _case(batch=8, seq_lens=lens, q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=128, page_size=1648,
              seed=23, max_seq_len=65536)
    plan = plan_for(c)
    gs = plan.info["grid_splits"]
    assert 8 * 1 * gs >= plan.info["num_cus"] > 4 * gs       # batched groups four heads, single does not
    batched = run_gpu(c, plan)
    compare(batched, run_oracle(c))
    for b in range(8):
        one = {k: (v[b:b + 1] if k in ("q", "block_table", "seq_lens") else v) for k, v in c.items()}
        single = run_gpu(one, batch_capacity=1)
        assert torch.equal(single[0].view(torch.int16), batched[b].view(torch.int16)), b


def _repaged(c, page_size, seed):
    """The same logical tokens laid out with another page size and a shuffled page order."""
    ps0 = c["page_size"]
    B = c["q"].shape[0]
    lens = c["seq_lens"].cpu().tolist()
    Lmax = max(lens)
    npg = -(-Lmax // page_size)
    rng = np.random.default_rng(seed)
    pool = B * npg + 5
    perm = torch.from_numpy(rng.permutation(pool)).cuda()
    Hkv, D = c["k_cache"].shape[2], c["k_cache"].shape[3]
    k2 = torch.zeros((pool, page_size, Hkv, D), dtype=c["k_cache"].dtype, device="cuda")
    v2 = torch.zeros_like(k2)
    table = torch.full((B, npg), -1, dtype=torch.int32, device="cuda")
    for b in range(B):
        L = lens[b]
        j = torch.arange(L, device="cuda")
        src_pages = c["block_table"][b].long()[j // ps0]
        tok_k = c["k_cache"][src_pages, j % ps0]
        tok_v = c["v_cache"][src_pages, j % ps0]
        dst_pages = perm[b * npg: b * npg + npg]
        table[b, :] = dst_pages.int()
        k2[dst_pages[j // page_size], j % page_size] = tok_k
        v2[dst_pages[j // page_size], j % page_size] = tok_v
    out = dict(c)
    out.update(k_cache=k2, v_cache=v2, block_table=table, page_size=page_size)
    return out


def test_page_size_and_permutation_invariance_bitwise():
    note("page size / permutation invariance")
    c = _case(batch=3, seq_lens=[9000, 1234, 17], q_len=8, num_q_heads=12, num_kv_heads=2, head_dim=256,
              page_size=1648, seed=10, max_seq_len=9000)
    base = run_gpu(c)
    for ps, seed in [(16, 1), (1648, 2), (3296, 3), (48, 4)]:
        other = run_gpu(_repaged(c, ps, seed), max_seq_len=9000)
        assert torch.equal(other.view(torch.int16), base.view(torch.int16)), ps


def test_zero_length_and_padded_slots():
    note("zero-length rows and padded slots")
    c = _case(batch=6, seq_lens=[0, 300, 0, 1700, 0, 0], q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256,
              page_size=16, seed=11, padded_slots=[4, 5])
    out = run_gpu(c)
    compare(out, run_oracle(c))
    for b in (0, 2, 4, 5):
        assert (out[b].view(torch.int16) == 0).all(), b          # exactly +0
    # all-zero batch
    c["seq_lens"].zero_()
    out = run_gpu(c)
    assert (out.view(torch.int16) == 0).all()


def test_interleaved_eight_byte_aligned_strides():
    note("interleaved K/V, 8-byte-only aligned strides")
    B, L, Hkv, Hq, D, ps = 2, 700, 2, 12, 256, 32
    c = wl.make_case(batch=B, seq_lens=[L, 333], q_len=8, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                     page_size=ps, seed=12)
    pool = c["k_cache"].shape[0]
    rec = 2 * D + 8                 # per (token, head): K bytes, V bytes, 8 pad bytes -> 520, not 16-aligned
    tok = Hkv * rec
    page = ps * tok + 8
    buf = torch.zeros(pool * page + 64, dtype=torch.uint8)
    base = 8                          # base address 8 mod 16
    kview = torch.as_strided(buf, (pool, ps, Hkv, D), (page, tok, rec, 1), base)
    vview = torch.as_strided(buf, (pool, ps, Hkv, D), (page, tok, rec, 1), base + D)
    kview.copy_(c["k_cache"])
    vview.copy_(c["v_cache"])
    g = to_gpu(c)
    gbuf = buf.cuda()
    plan = plan_for(g, k_strides=(page, tok, rec), v_strides=(page, tok, rec))
    out = torch.empty_like(g["q"])
    ws = A.default_bank().get(plan, B)
    args = plan.make_args(g["q"], gbuf.data_ptr() + base, gbuf.data_ptr() + base + D, g["block_table"],
                          g["seq_lens"], g["k_scale"], g["v_scale"], out, ws, num_pages=pool)
    plan.split(args)
    plan.combine(args)
    torch.cuda.synchronize()
    compare(out, run_oracle(c))


def test_repeatable_bitwise():
    note("run-to-run determinism")
    c = _case(batch=2, seq_lens=[20000, 5000], q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256,
              page_size=1648, seed=13)
    a = run_gpu(c)
    b = run_gpu(c)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# One encoding of 1.5 per cache format, for the spiked keys below.
_SPIKE = {"e4m3": 0x3C, "e5m2": 0x3E, "fp16": 1.5}
# (kv_format, head_dim) of the five kernels, and q_len at six query heads per KV head giving one,
# two and three row tiles (12, 24 and 48 packed rows).
_FORMATS = [("e4m3", 256), ("e5m2", 256), ("fp16", 256), ("fp16", 128), ("e4m3", 128)]
_ROW_TILES = {1: 2, 2: 4, 3: 8}


def _spike_keys(c, spikes, value):
    """K = 0 for every token of every slot, except `value` (all dims, all KV heads) at the logical
    tokens `spikes[b]` of slot b."""
    kc = c["k_cache"]
    kc.zero_()
    ps = c["page_size"]
    for b, js in enumerate(spikes):
        if not js:
            continue
        j = torch.tensor(js, dtype=torch.long, device=kc.device)
        pages = c["block_table"][b].long()[j // ps]
        kc[pages, j % ps] = value


@pytest.mark.parametrize("row_tiles", [1, 2, 3])
@pytest.mark.parametrize("fmt,head_dim", _FORMATS, ids=[f"{f}-d{d}" for f, d in _FORMATS])
@pytest.mark.parametrize("batch", [1, 8])
def test_reference_slack_overflow_recompute(batch, fmt, head_dim, row_tiles):
    # Q = 1 everywhere; K is 0 except spikes of 1.5 in every dim, which score 1.5 sqrt(D) (24 or 17,
    # i.e. 35 or 24 log2 units) above the zero keys. The first 64 tokens of every 512-token split
    # are zero, so each wave's first tile sets a reference of 0 and a later spike's P (2^35 or
    # 2^24) overflows FP16: every split is recomputed with its exact row maxima. This runs the
    # recompute in every kernel (format x row tiles); at B8 (lengths under 1024 tokens and a
    # 65536-token plan) the workgroups hold two KV heads (four for E4M3 at D128).
    q_len = _ROW_TILES[row_tiles]
    lens = [900, 700, 1000, 513, 64, 899, 640, 1023][:batch]
    note(f"reference overflow -> exact recompute, {fmt} D{head_dim}, {row_tiles} row tiles, B{batch}")
    c = _case(batch=batch, seq_lens=lens, q_len=q_len, num_q_heads=24, num_kv_heads=4, head_dim=head_dim,
              page_size=16, seed=14 + batch + head_dim + row_tiles, kv_format=fmt,
              max_seq_len=65536 if batch > 1 else None)
    c["q"].fill_(1.0)
    spikes = [[j for j in range(L) if j % 97 == 0 and j % 512 >= 64] for L in lens]
    _spike_keys(c, spikes, _SPIKE[fmt])
    plan = plan_for(c)
    if batch > 1:
        gs, cus = plan.info["grid_splits"], plan.info["num_cus"]
        hp = 4 if (fmt, head_dim) == ("e4m3", 128) else 2
        assert batch * (4 // hp) * gs >= cus          # the launch groups hp KV heads per workgroup
    compare(run_gpu(c, plan), run_oracle(c))


_ROW_GROUP_CASES = [("e4m3", 256, 8, 32), ("e5m2", 256, 8, 32), ("fp16", 256, 8, 32), ("fp16", 128, 8, 32),
                    ("e4m3", 256, 4, 16), ("e4m3", 256, 8, 16), ("e5m2", 256, 8, 0)]


@pytest.mark.parametrize("fmt,head_dim,q_len,hot_tile", _ROW_GROUP_CASES,
                         ids=[f"{f}-d{d}-q{q}-hot{h}" for f, d, q, h in _ROW_GROUP_CASES])
def test_row_group_workgroups_recompute_like_batched_bitwise(fmt, head_dim, q_len, hot_tile):
    # One slot alone gives a grid of at most one workgroup per CU, which the library runs with row
    # groups per KV head: two (a second pair of waves on the last row tiles: tiles 2..3 of 48 rows
    # at q8, tile 1 of 24 rows at q4) or, for the one-byte formats at D256 and 48 rows, three (one
    # row tile per wave pair); B8 of the same 65536-token plan runs one group. Spiked keys past the
    # first 64 tokens of every 512-token split score only the rows of the 16-row tile starting at
    # `hot_tile` (Q = 1) so far above their reference that P overflows FP16; the other rows (Q
    # scaled by 0.05) stay near it, but their bits still depend on whether their wave recomputes.
    # Both layouts must recompute the same rows: each slot alone gives the batched bits, and both
    # match the oracle.
    lens = [900, 700, 1000, 513, 64, 899, 640, 1023]
    note(f"row groups vs one group under a partial recompute, {fmt} D{head_dim} q{q_len}")
    c = _case(batch=8, seq_lens=lens, q_len=q_len, num_q_heads=24, num_kv_heads=4, head_dim=head_dim,
              page_size=16, seed=61 + head_dim + q_len, kv_format=fmt, max_seq_len=65536)
    G = 6
    rows = torch.arange(q_len * G, device="cuda")
    hot = ((rows >= hot_tile) & (rows < hot_tile + 16)).view(q_len, G)   # [t][j]: packed row t*G + j
    q = c["q"].view(8, q_len, 4, G, head_dim)                   # [b][t][g][j][d]
    q.mul_(torch.where(hot, 1.0, 0.05).to(q.dtype)[None, :, None, :, None])
    q.masked_fill_(hot[None, :, None, :, None], 1.0)
    kc = c["k_cache"]
    ps = c["page_size"]
    for b, L in enumerate(lens):
        j = torch.tensor([t for t in range(L) if t % 97 == 0 and t % 512 >= 64], dtype=torch.long, device="cuda")
        if len(j):
            pages = c["block_table"][b].long()[j // ps]
            kc[pages, j % ps] = _SPIKE[fmt]
    plan = plan_for(c)
    gs, cus = plan.info["grid_splits"], plan.info["num_cus"]
    assert 8 * 4 * gs > cus >= 4 * gs          # batched: one group; one slot: row groups
    batched = run_gpu(c, plan)
    compare(batched, run_oracle(c))
    for b in range(8):
        one = {k: (v[b:b + 1] if k in ("q", "block_table", "seq_lens") else v) for k, v in c.items()}
        single = run_gpu(one, batch_capacity=1)
        assert torch.equal(single[0].view(torch.int16), batched[b].view(torch.int16)), b


@pytest.mark.parametrize("spike,rise", [(0x2C, 8.7), (0x31, 13.0), (0x32, 14.4), (0x33, 15.9), (0x34, 17.3)])
def test_reference_rise_around_fp16_overflow(spike, rise):
    # Later keys score 8.7, 13.0, 14.4, 15.9 or 17.3 log2 units above the reference the first
    # tiles set (E4M3 0.375, 0.5625, 0.625, 0.6875, 0.75 in every dim against zero keys: 256 k / 16
    # * log2(e)). Up to 15.9 (P about 60000, just under the FP16 maximum) the split takes one pass
    # with those large weights; at 17.3 P overflows FP16 and the split is recomputed with its
    # exact row maxima. Either way the result must match the oracle.
    note(f"reference rise of {rise} log2 units, single pass")
    c = _case(batch=1, seq_lens=[900], q_len=8, num_q_heads=6, num_kv_heads=1, head_dim=256, page_size=16,
              seed=14)
    c["q"].fill_(1.0)
    _spike_keys(c, [[j for j in range(900) if j % 97 == 0 and j >= 64]], spike)
    compare(run_gpu(c), run_oracle(c))


def _graph(plan, case, out, ws):
    args = plan.make_args(case["q"], case["k_cache"], case["v_cache"], case["block_table"], case["seq_lens"],
                          case["k_scale"], case["v_scale"], out, ws)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plan.split(args, s)           # warm up on the capture stream
        plan.combine(args, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        plan.split(args)
        plan.combine(args)
    return g, args


def test_graph_replay_with_changed_inputs_matches_eager():
    note("graph replay with changed Q, lengths, zero rows, scales")
    B, Lmax = 4, 6000
    c = _case(batch=B, seq_lens=[Lmax] * B, q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=1648,
              seed=15, max_seq_len=Lmax)
    plan = plan_for(c)
    out = torch.empty_like(c["q"])
    ws = torch.empty(plan.workspace_bytes(B) // 4, dtype=torch.float32, device="cuda")
    g, _ = _graph(plan, c, out, ws)
    rng = np.random.default_rng(16)
    for rep, lens in enumerate([[6000, 3297, 0, 1], [0, 0, 0, 0], [17, 5999, 4000, 0], [6000, 6000, 6000, 6000]]):
        c["q"].copy_(torch.randn(c["q"].shape, generator=torch.Generator("cuda").manual_seed(100 + rep),
                                 device="cuda").half())
        c["seq_lens"].copy_(torch.tensor(lens, dtype=torch.int32))
        c["k_scale"].fill_(float(rng.choice([0.5, 1.0, 2.0])))
        c["v_scale"].fill_(float(rng.choice([0.5, 1.0, 3.0])))
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        eager = run_gpu(c)
        assert torch.equal(replayed.view(torch.int16), eager.view(torch.int16)), rep
        compare(replayed, run_oracle(c))


# ---- the tests must be able to fail: planted mistakes in the inputs (all reads stay in bounds) ----

def _mismatch(out, ref):
    try:
        compare(out, ref)
    except AssertionError:
        return True
    return False


def test_mutation_wrong_head_stride_is_caught():
    # KV head 1 read 8 bytes from head 0's row instead of its own: the comparison must fail.
    note("mutation: wrong KV head stride")
    c = _case(batch=2, seq_lens=[700, 300], q_len=8, num_q_heads=12, num_kv_heads=2, head_dim=256, page_size=32,
              seed=31)
    ks = A.contiguous_strides(32, 2, 256, "e4m3")
    good = run_gpu(c)
    assert not _mismatch(good, run_oracle(c))
    bad = run_gpu(c, k_strides=(ks[0], ks[1], 8))
    assert _mismatch(bad, run_oracle(c))


def test_mutation_wrong_page_index_is_caught():
    # Swapping two fully visible pages would only permute the keys (attention does not see the
    # order); swapping the first page with the partly filled last one changes the key set.
    note("mutation: first and last block-table entries swapped")
    c = _case(batch=1, seq_lens=[100], q_len=8, num_q_heads=6, num_kv_heads=1, head_dim=256, page_size=16, seed=32)
    ref = run_oracle(c)
    c["block_table"][0, [0, 6]] = c["block_table"][0, [6, 0]].clone()
    assert _mismatch(run_gpu(c), ref)


def test_canary_zones_around_output_and_workspace_stay_intact():
    note("canary zones around out and workspace")
    c = _case(batch=3, seq_lens=[3000, 0, 129], q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256,
              page_size=1648, seed=33)
    plan = plan_for(c)
    guard = 4096 // 2                                    # FP16 elements per 4 KB guard
    n_out = c["q"].numel()
    out_buf = torch.full((guard + n_out + guard,), 12345, dtype=torch.int16, device="cuda")
    out = out_buf[guard:guard + n_out].view(torch.float16).view(c["q"].shape)
    ws_floats = plan.workspace_bytes(3) // 4
    ws_buf = torch.full((1024 + ws_floats + 1024,), -7.0, dtype=torch.float32, device="cuda")
    ws = ws_buf[1024:1024 + ws_floats]
    plan.run(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"], c["v_scale"],
             out=out, workspace=ws)
    torch.cuda.synchronize()
    assert (out_buf[:guard] == 12345).all() and (out_buf[guard + n_out:] == 12345).all()
    assert (ws_buf[:1024] == -7.0).all() and (ws_buf[1024 + ws_floats:] == -7.0).all()
    compare(out, run_oracle(c))
