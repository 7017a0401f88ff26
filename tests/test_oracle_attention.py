"""Pins of the FP64 attention oracle (CPU only).

Each pin checks the oracle against something other than itself: a separate
brute force, a closed form, or an invariant of the definition. The mutation
tests plant plausible mistakes in the oracle (on the CPU) and show that the
pins catch them.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as oa
from _brute import brute_attention
from verify_attention_e4m3_amd import workloads as wl


def _case(**kw):
    c = wl.make_case(**kw)
    return wl.to_numpy(c)


def _run_oracle(c, **kw):
    return oracle.verify_attention(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"],
                                   float(c["k_scale"][0]), float(c["v_scale"][0]), page_size=c["page_size"],
                                   kv_format=c["kv_format"], **kw)


def _run_brute(c, causal=True, sm_scale=None):
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(c["head_dim"])
    return np.array(brute_attention(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"],
                                    float(c["k_scale"][0]), float(c["v_scale"][0]), page_size=c["page_size"],
                                    sm_scale=sm_scale, kv_format=c["kv_format"], causal=causal))


BRUTE_CASES = [
    dict(batch=2, seq_lens=[37, 5], q_len=3, num_q_heads=4, num_kv_heads=2, head_dim=8, page_size=16, seed=11),
    dict(batch=4, seq_lens=[0, 9, 33, 3], q_len=8, num_q_heads=6, num_kv_heads=1, head_dim=16, page_size=16,
         seed=12, kv_std=0.5, kv_scale=2.0),
    dict(batch=1, seq_lens=[20], q_len=2, num_q_heads=2, num_kv_heads=1, head_dim=256, page_size=16, seed=13),
    dict(batch=2, seq_lens=[17, 30], q_len=1, num_q_heads=4, num_kv_heads=2, head_dim=8, page_size=16,
         kv_format="fp16", seed=14),
    dict(batch=3, seq_lens=[40, 16, 1], q_len=8, num_q_heads=6, num_kv_heads=2, head_dim=8, page_size=32,
         seed=15, kv_scale=0.75),
    dict(batch=2, seq_lens=[29, 8], q_len=8, num_q_heads=6, num_kv_heads=1, head_dim=16, page_size=16,
         kv_format="e5m2", seed=16, kv_scale=1.5),
]


@pytest.mark.parametrize("kw", BRUTE_CASES)
def test_oracle_matches_brute_force(kw):
    c = _case(**kw)
    got = _run_oracle(c)
    want = _run_brute(c)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13), np.abs(got - want).max()


def test_oracle_matches_brute_force_non_causal():
    c = _case(**BRUTE_CASES[0])
    got = _run_oracle(c, causal=False)
    want = _run_brute(c, causal=False)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)
    # and the causal mask does change the answer here
    assert not np.allclose(_run_oracle(c), got)


@pytest.mark.parametrize("case_idx", [0, 1, 5])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("sm_scale", [0.05, 0.3])
def test_oracle_matches_brute_force_explicit_scale(sm_scale, causal, case_idx):
    # An explicit softmax scale replaces 1/sqrt(D); the brute force applies it to the raw dot
    # products of its own loops, so a scale that the oracle ignored, applied twice or squared
    # would show here.
    c = _case(**BRUTE_CASES[case_idx])
    got = _run_oracle(c, causal=causal, sm_scale=sm_scale)
    want = _run_brute(c, causal=causal, sm_scale=sm_scale)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13), np.abs(got - want).max()
    # the scale does change the answer at these inputs
    assert not np.allclose(got, _run_oracle(c, causal=causal), rtol=1e-6, atol=1e-9)


def test_row_that_sees_one_key_is_that_value_exactly():
    # L == q_len: verify token t sits at position t and sees keys 0..t; token 0 sees key 0 only.
    c = _case(batch=1, seq_lens=[8], q_len=8, num_q_heads=6, num_kv_heads=1, head_dim=256, page_size=16,
              seed=21, kv_scale=0.5)
    out = _run_oracle(c)
    page = c["block_table"][0][0]
    v0 = 0.5 * oracle.decode_table()[c["v_cache"][page, 0, 0, :]]
    for h in range(6):
        assert np.array_equal(out[0, 0, h], v0)


def test_short_row_first_tokens_see_nothing():
    # L = 3 < q_len = 8: tokens 0..4 see no key (exact zero), token 5 sees key 0 only.
    c = _case(batch=1, seq_lens=[3], q_len=8, num_q_heads=2, num_kv_heads=1, head_dim=16, page_size=16, seed=22)
    out = _run_oracle(c)
    assert np.array_equal(out[0, :5], np.zeros_like(out[0, :5]))
    page = c["block_table"][0][0]
    v0 = oracle.decode_table()[c["v_cache"][page, 0, 0, :]]
    assert np.array_equal(out[0, 5, 0], v0)
    assert not np.array_equal(out[0, 6, 0], v0)


def test_zero_query_gives_mean_of_visible_values():
    c = _case(batch=1, seq_lens=[50], q_len=4, num_q_heads=2, num_kv_heads=1, head_dim=16, page_size=16, seed=23)
    c["q"][:] = 0
    out = _run_oracle(c)
    tab = oracle.decode_table()
    tokens = [c["v_cache"][c["block_table"][0][j // 16], j % 16, 0, :] for j in range(50)]
    V = np.stack([tab[t] for t in tokens])
    for t in range(4):
        n = 50 - 4 + t + 1
        assert np.allclose(out[0, t, 0], V[:n].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_constant_values_give_that_constant():
    c = _case(batch=2, seq_lens=[29, 7], q_len=3, num_q_heads=4, num_kv_heads=2, head_dim=8, page_size=16,
              seed=24, kv_scale=1.5)
    c["v_cache"][:] = 0x3C        # E4M3 1.5
    out = _run_oracle(c)
    assert np.allclose(out, 1.5 * 1.5, rtol=1e-14, atol=0)


def test_zero_length_and_padded_rows_are_exact_zero():
    c = _case(batch=4, seq_lens=[12, 0, 30, 0], q_len=2, num_q_heads=2, num_kv_heads=1, head_dim=8,
              page_size=16, seed=25, padded_slots=[3])
    assert np.isnan(c["q"][3]).all()
    out = _run_oracle(c)
    for b in (1, 3):
        assert np.array_equal(out[b], np.zeros_like(out[b]))
        assert not np.signbit(out[b]).any()
    assert np.isfinite(out).all()


def _repage(tokens_k, tokens_v, page_size, seed):
    """Lay logical tokens [L][Hkv][D] out in a shuffled paged cache."""
    L = tokens_k.shape[0]
    n = -(-L // page_size)
    rng = np.random.default_rng(seed)
    phys = rng.permutation(n + 3)[:n]
    shape = (n + 3, page_size) + tokens_k.shape[1:]
    kc = np.zeros(shape, tokens_k.dtype)
    vc = np.zeros(shape, tokens_v.dtype)
    for j in range(L):
        kc[phys[j // page_size], j % page_size] = tokens_k[j]
        vc[phys[j // page_size], j % page_size] = tokens_v[j]
    return kc, vc, phys[None, :].astype(np.int32)


def test_page_size_and_page_permutation_invariance_bitwise():
    L, Hkv, D = 70, 2, 16
    rng = np.random.default_rng(5)
    tk = rng.integers(0, 0x7F, size=(L, Hkv, D), dtype=np.uint8) | (rng.integers(0, 2, (L, Hkv, D), dtype=np.uint8) << 7)
    tk[tk == 0xFF] = 0x00
    tv = rng.integers(0, 0x7E, size=(L, Hkv, D), dtype=np.uint8)
    q = rng.standard_normal((1, 8, 6, D)).astype(np.float16)
    outs = []
    for ps, seed in [(16, 0), (16, 1), (32, 2), (48, 3), (80, 4)]:
        kc, vc, table = _repage(tk, tv, ps, seed)
        outs.append(oracle.verify_attention(q, kc, vc, table, np.array([L]), 1.0, 1.0, page_size=ps))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_gqa_equals_mha_with_replicated_kv_heads():
    c = _case(batch=2, seq_lens=[45, 19], q_len=3, num_q_heads=6, num_kv_heads=2, head_dim=16, page_size=16, seed=26)
    gqa = _run_oracle(c)
    rep_k = np.repeat(c["k_cache"], 3, axis=2)     # KV head g -> query heads 3g..3g+2
    rep_v = np.repeat(c["v_cache"], 3, axis=2)
    mha = oracle.verify_attention(c["q"], rep_k, rep_v, c["block_table"], c["seq_lens"], 1.0, 1.0, page_size=16)
    assert np.allclose(gqa, mha, rtol=1e-14, atol=1e-16)


def test_power_of_two_scales_are_exact():
    c = _case(batch=2, seq_lens=[33, 10], q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=16, page_size=16, seed=27)
    base = _run_oracle(c)
    c2 = dict(c)
    c2["v_scale"] = c["v_scale"] * 2
    assert np.array_equal(_run_oracle(c2), 2 * base)
    # (2Q, k_scale) == (Q, 2*k_scale): power-of-two scaling is exact in FP64
    c3 = dict(c)
    c3["q"] = (c["q"].astype(np.float32) * 2).astype(np.float16)
    c4 = dict(c)
    c4["k_scale"] = c["k_scale"] * 2
    assert np.array_equal(_run_oracle(c3), _run_oracle(c4))


@pytest.mark.parametrize("splits", [[0, 17, 40], [0, 1, 39, 40], [0, 35, 40], [0, 20, 21, 40]])
def test_full_result_is_the_merge_of_split_partials(splits):
    c = _case(batch=1, seq_lens=[40], q_len=8, num_q_heads=6, num_kv_heads=2, head_dim=16, page_size=16,
              seed=28, kv_scale=0.5)
    full = _run_oracle(c)
    for g in range(2):
        parts = [oracle.partial_states(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], 0.5,
                                       b=0, kv_head=g, begin=a, end=e, page_size=16)
                 for a, e in zip(splits[:-1], splits[1:])]
        merged = oracle.merge_partials(parts, 0.5)            # rows r = t*3 + j
        want = full[0, :, 3 * g:3 * g + 3, :].reshape(24, 16)
        assert np.allclose(merged, want, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("sm_scale", [0.05, 0.3])
def test_partial_states_merge_at_explicit_scale(sm_scale, causal):
    # partial_states over any token split, merged, equals the full oracle at the same scale and
    # mask (the full oracle is itself pinned to the brute force at these settings above); the
    # rows of the last two verify tokens see keys up to the row end, so the causal and the
    # non-causal partials differ in the final part.
    c = _case(batch=2, seq_lens=[40, 13], q_len=8, num_q_heads=6, num_kv_heads=2, head_dim=16, page_size=16,
              seed=29, kv_scale=0.5)
    full = _run_oracle(c, causal=causal, sm_scale=sm_scale)
    for b, splits in ((0, [0, 9, 33, 40]), (1, [0, 5, 6, 13])):
        for g in range(2):
            parts = [oracle.partial_states(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], 0.5,
                                           b=b, kv_head=g, begin=a, end=e, page_size=16, sm_scale=sm_scale,
                                           causal=causal)
                     for a, e in zip(splits[:-1], splits[1:])]
            merged = oracle.merge_partials(parts, 0.5)
            want = full[b, :, 3 * g:3 * g + 3, :].reshape(24, 16)
            assert np.allclose(merged, want, rtol=1e-13, atol=1e-15), (b, g)
    # the brute force agrees with the full result directly
    assert np.allclose(full, _run_brute(c, causal=causal, sm_scale=sm_scale), rtol=1e-12, atol=1e-13)


def test_partial_states_non_causal_sees_every_key():
    # Non-causal: every row of a part sees all of its keys, so a part holding one key gives that
    # key's score as m, l = 1 and o = its V row, for every verify token alike.
    c = _case(batch=1, seq_lens=[20], q_len=4, num_q_heads=2, num_kv_heads=1, head_dim=8, page_size=16, seed=30)
    m, l, o = oracle.partial_states(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], 1.0,
                                    b=0, kv_head=0, begin=19, end=20, page_size=16, sm_scale=0.3, causal=False)
    page = c["block_table"][0][19 // 16]
    k19 = oracle.decode_table()[c["k_cache"][page, 19 % 16, 0, :]]
    v19 = oracle.decode_table()[c["v_cache"][page, 19 % 16, 0, :]]
    for t in range(4):
        for j in range(2):
            r = t * 2 + j
            s = 0.3 * sum(float(c["q"][0, t, j, d]) * float(k19[d]) for d in range(8))
            assert math.isclose(m[r], s, rel_tol=1e-13, abs_tol=1e-15)
            assert l[r] == 1.0 and np.array_equal(o[r], v19)
    # causal: key 19 is visible only to the last verify token (position 19)
    m2, l2, _ = oracle.partial_states(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], 1.0,
                                      b=0, kv_head=0, begin=19, end=20, page_size=16, sm_scale=0.3, causal=True)
    assert np.isneginf(m2[:6]).all() and (l2[:6] == 0).all() and (l2[6:] == 1.0).all()


def test_merge_of_all_empty_parts_is_zero():
    R, D = 4, 8
    parts = [(np.full(R, -np.inf), np.zeros(R), np.zeros((R, D)))] * 3
    out = oracle.merge_partials(parts, 1.0)
    assert np.array_equal(out, np.zeros((R, D)))


# ---- mutation tests: plausible mistakes planted in the oracle must fail the pins ----

def _brute_mismatch(case_kw):
    c = _case(**case_kw)
    return not np.allclose(_run_oracle(c), _run_brute(c), rtol=1e-12, atol=1e-13)


def test_mutation_causal_off_by_one_is_caught(monkeypatch):
    orig = oa.visible_keys
    monkeypatch.setattr(oa, "visible_keys", lambda L, q, t, causal: orig(L, q, t, causal) - 1 if L > 0 else 0)
    assert _brute_mismatch(BRUTE_CASES[0])


def test_mutation_wrong_exponent_bias_is_caught(monkeypatch):
    bad = np.array([oracle.decode_byte(b) * 0.5 for b in range(256)])     # bias 8 instead of 7
    monkeypatch.setattr(oa, "_E4M3", bad)
    assert _brute_mismatch(BRUTE_CASES[1])


def test_mutation_e5m2_read_as_e4m3_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "_E5M2", oa._E4M3)
    assert _brute_mismatch(BRUTE_CASES[5])


def test_mutation_page_slot_swap_is_caught(monkeypatch):
    def bad_gather(cache, table_row, length, kv_head, page_size):
        n = -(-length // page_size)
        pages = np.asarray(table_row[:n], dtype=np.int64)
        tok = cache[pages, :, kv_head, :].transpose(1, 0, 2)      # slot-major instead of page-major
        return tok.reshape(n * page_size, cache.shape[3])[:length]
    monkeypatch.setattr(oa, "gather_tokens", bad_gather)
    assert _brute_mismatch(BRUTE_CASES[0])


def test_mutation_wrong_head_mapping_is_caught():
    # head h -> KV head h % Hkv instead of h // G: emulate by permuting the query heads
    c = _case(**BRUTE_CASES[4])
    good = _run_oracle(c)
    Hq, Hkv = 6, 2
    perm = [(h % Hkv) * (Hq // Hkv) + h // Hkv for h in range(Hq)]
    c2 = dict(c)
    c2["q"] = c["q"][:, :, perm, :]
    bad = _run_oracle(c2)[:, :, np.argsort(perm), :]
    assert not np.allclose(bad, _run_brute(c), rtol=1e-12, atol=1e-13)
    assert np.allclose(good, _run_brute(c), rtol=1e-12, atol=1e-13)


def _mutant_scale_mismatch(monkeypatch, wrap):
    """Plant a softmax-scale mistake into the oracle's entry point and report whether the
    explicit-scale brute-force pin notices it."""
    orig = oa.verify_attention

    def bad(*args, sm_scale=None, **kw):
        return orig(*args, sm_scale=wrap(sm_scale), **kw)
    monkeypatch.setattr(oa, "verify_attention", bad)
    c = _case(**BRUTE_CASES[0])
    got = oa.verify_attention(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"],
                              float(c["k_scale"][0]), float(c["v_scale"][0]), page_size=c["page_size"],
                              kv_format=c["kv_format"], sm_scale=0.3, causal=False)
    return not np.allclose(got, _run_brute(c, causal=False, sm_scale=0.3), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("mistake", ["ignored", "twice", "squared"])
def test_mutation_explicit_scale_mistakes_are_caught(monkeypatch, mistake):
    wrap = {"ignored": lambda s: None, "twice": lambda s: 2 * s, "squared": lambda s: s * s}[mistake]
    assert _mutant_scale_mismatch(monkeypatch, wrap)


def test_mutation_partial_states_scale_ignored_is_caught(monkeypatch):
    orig = oa.partial_states

    def bad(*args, sm_scale=None, **kw):
        return orig(*args, **kw)                 # drops the explicit scale
    monkeypatch.setattr(oa, "partial_states", bad)
    c = _case(batch=1, seq_lens=[40], q_len=8, num_q_heads=6, num_kv_heads=2, head_dim=16, page_size=16,
              seed=29, kv_scale=0.5)
    full = _run_oracle(c, causal=False, sm_scale=0.3)
    parts = [oa.partial_states(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], 0.5, b=0,
                               kv_head=0, begin=a, end=e, page_size=16, sm_scale=0.3, causal=False)
             for a, e in ((0, 17), (17, 40))]
    merged = oracle.merge_partials(parts, 0.5)
    assert not np.allclose(merged, full[0, :, 0:3, :].reshape(24, 16), rtol=1e-13, atol=1e-15)


def test_mutation_partial_states_mask_ignored_is_caught(monkeypatch):
    orig = oa.partial_states

    def bad(*args, causal=True, **kw):
        return orig(*args, causal=True, **kw)    # always causal
    monkeypatch.setattr(oa, "partial_states", bad)
    c = _case(batch=1, seq_lens=[40], q_len=8, num_q_heads=6, num_kv_heads=2, head_dim=16, page_size=16,
              seed=29, kv_scale=0.5)
    full = _run_oracle(c, causal=False, sm_scale=0.3)
    parts = [oa.partial_states(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], 0.5, b=0,
                               kv_head=0, begin=a, end=e, page_size=16, sm_scale=0.3, causal=False)
             for a, e in ((0, 17), (17, 40))]
    merged = oracle.merge_partials(parts, 0.5)
    assert not np.allclose(merged, full[0, :, 0:3, :].reshape(24, 16), rtol=1e-13, atol=1e-15)
