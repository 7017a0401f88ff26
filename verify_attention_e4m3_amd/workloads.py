"""Seeded synthetic inputs for speculative-verify attention (no attention arithmetic here).

Both the oracle-side tests and the GPU-side tests, the smoke check and the
benchmark draw their inputs from this module; it holds only random generation,
quantisation of the random draws to cache bytes, and the paged layout
(physical page pools, block tables). It imports neither the oracle nor the HIP
binding.

Workloads mirror the shapes the pages measure and test: q8 FP16 verify queries,
E4M3 KV with per-tensor FP32 scales, D = 256, six query heads per KV head,
pages of 1648 and 3296 tokens ("DFlash2 concurrent long-context attention",
sections "Operator validation" and "Attention-only measurements", which use
random per-layer KV working sets), plus a head-dim-128 FP16-KV q1 decode variant
(the GQA group-swap PR #48).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import torch

MAX_SEQ_LEN = 262144


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic workload."""
    name: str
    batch: int
    seq_len: Optional[int]          # None: per-slot lengths drawn by ``mixed_lengths``
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_format: str                  # "e4m3", "e5m2" or "fp16"
    kv_std: float                   # K/V values before quantisation are N(0, kv_std**2)
    kv_scale: float                 # per-tensor k_scale = v_scale
    layers: int                     # independent per-layer caches
    seed: int
    max_seq_len: int
    description: str

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


WORKLOADS = {
    w.name: w for w in [
        Workload("verify_b1_ctx3297_hq6_hkv1", 1, 3297, 8, 6, 1, 256, 1648, "e4m3", 1.0, 1.0, 16, 1, 4096,
                 "B1, seq_len 3297 incl. 8 new tokens, Hq6/Hkv1, page 1648, pages from a 64-page pool, "
                 "16 per-layer caches"),
        Workload("verify_b4_ctx32k_gqa6", 4, 32768, 8, 24, 4, 256, 1648, "e4m3", 0.5, 2.0, 8, 2, 32768,
                 "B4 x 32768, Hq24/Hkv4, E4M3 of 0.5*N(0,1) with k/v scales 2.0, shuffled pages, "
                 "8 per-layer caches (2.1 GB, beyond the memory-side cache)"),
        Workload("verify_b8_ctx128k_gqa6_16layers", 8, 131072, 8, 24, 4, 256, 1648, "e4m3", 1.0, 1.0, 16, 3,
                 131072, "B8 x 131072, Hq24/Hkv4, 16 independent per-layer caches, shuffled pages"),
        Workload("verify_b16_mixed_ctx256k_page3296", 16, None, 8, 24, 4, 256, 3296, "e4m3", 1.0, 1.0, 1, 4,
                 MAX_SEQ_LEN, "B16, lengths U{0..262144}, two zero-length rows, three padded slots, page 3296"),
        Workload("decode_b8_ctx32k_d128_fp16_gqa4", 8, 32768, 1, 32, 8, 128, 1648, "fp16", 1.0, 1.0, 1, 5,
                 32768, "B8 x 32768, q1, Hq32/Hkv8, D128, FP16 K/V"),
        # FP16 KV at D256 (another cache format the pages' backend serves)
        Workload("verify_b4_ctx32k_gqa6_fp16_d256", 4, 32768, 8, 24, 4, 256, 1648, "fp16", 1.0, 1.0, 1, 12, 32768,
                 "B4 x 32768, Hq24/Hkv4, FP16 KV at D256, shuffled pages"),
        Workload("verify_b8_ctx128k_gqa6_fp16_d256_4layers", 8, 131072, 8, 24, 4, 256, 1648, "fp16", 1.0, 1.0, 4,
                 13, 131072, "B8 x 131072, Hq24/Hkv4, FP16 KV at D256 (4.3 GB per layer), 4 per-layer caches"),
        # E4M3 KV at D128 (another head dimension)
        Workload("verify_b4_ctx32k_gqa6_e4m3_d128", 4, 32768, 8, 24, 4, 128, 1648, "e4m3", 1.0, 1.0, 1, 14, 32768,
                 "B4 x 32768, Hq24/Hkv4, E4M3 KV at D128, shuffled pages"),
        Workload("verify_b8_ctx128k_gqa6_e4m3_d128_16layers", 8, 131072, 8, 24, 4, 128, 1648, "e4m3", 1.0, 1.0, 16,
                 15, 131072, "B8 x 131072, Hq24/Hkv4, E4M3 KV at D128 (1.07 GB per layer), 16 per-layer caches"),
        # four local query heads on one KV head (the pages' TP4 geometry of another model), q8
        Workload("verify_b8_ctx128k_hq4_hkv1_16layers", 8, 131072, 8, 4, 1, 256, 1648, "e4m3", 1.0, 1.0, 16, 8,
                 131072, "B8 x 131072, q8, Hq4/Hkv1 (32 packed rows), 16 per-layer caches, shuffled pages"),
        # E5M2 KV at D256 (another cache format the pages' backend serves), same shapes as above
        Workload("verify_b4_ctx32k_gqa6_e5m2", 4, 32768, 8, 24, 4, 256, 1648, "e5m2", 1.0, 1.0, 1, 6, 32768,
                 "B4 x 32768, Hq24/Hkv4, E5M2 of N(0,1), shuffled pages"),
        Workload("verify_b8_ctx128k_gqa6_e5m2_16layers", 8, 131072, 8, 24, 4, 256, 1648, "e5m2", 1.0, 1.0, 16, 7,
                 131072, "B8 x 131072, Hq24/Hkv4, E5M2 KV, 16 independent per-layer caches, shuffled pages"),
    ]
}


def quantize_e4m3(x: torch.Tensor) -> torch.Tensor:
    """float tensor -> uint8 E4M3 (OCP, no infinities) bytes, round-to-nearest-even via torch."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def quantize_e5m2(x: torch.Tensor) -> torch.Tensor:
    """float tensor -> uint8 E5M2 (OCP) bytes, round-to-nearest-even via torch."""
    return x.to(torch.float8_e5m2).view(torch.uint8)


ELEMENT_BYTES = {"e4m3": 1, "e5m2": 1, "fp16": 2}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def mixed_lengths(batch: int, seed: int, *, max_len: int = MAX_SEQ_LEN, zero_rows: int = 2,
                  padded: int = 3) -> list:
    """Per-slot lengths: the last ``padded`` slots and ``zero_rows`` seeded live slots are 0,
    the other live slots are uniform on {0..max_len}."""
    g = _gen(seed, "cpu")
    live = batch - padded
    lens = torch.randint(0, max_len + 1, (batch,), generator=g).tolist()
    zero_pos = torch.randperm(live, generator=g)[:zero_rows].tolist()
    for i in zero_pos:
        lens[i] = 0
    for i in range(live, batch):
        lens[i] = 0
    return [int(v) for v in lens]


def random_cache(num_pages: int, page_size: int, num_kv_heads: int, head_dim: int, *, kv_format: str,
                 std: float, seed: int, device="cpu", chunk_pages: int = 64) -> torch.Tensor:
    """[num_pages][page_size][Hkv][D] cache of N(0, std^2) draws, as E4M3 / E5M2 bytes or FP16."""
    if kv_format not in ELEMENT_BYTES:
        raise ValueError(f"unknown kv_format {kv_format!r}")
    dtype = torch.uint8 if ELEMENT_BYTES[kv_format] == 1 else torch.float16
    quant = {"e4m3": quantize_e4m3, "e5m2": quantize_e5m2, "fp16": lambda t: t.to(torch.float16)}[kv_format]
    out = torch.empty((num_pages, page_size, num_kv_heads, head_dim), dtype=dtype, device=device)
    g = _gen(seed, device)
    for p0 in range(0, num_pages, chunk_pages):
        p1 = min(num_pages, p0 + chunk_pages)
        x = torch.randn((p1 - p0, page_size, num_kv_heads, head_dim), generator=g, device=device,
                        dtype=torch.float32) * std
        out[p0:p1] = quant(x)
    return out


def block_tables(seq_lens: Sequence[int], page_size: int, max_pages_per_seq: int, *, seed: int,
                 pool_pages: Optional[int] = None, alloc_lens: Optional[Sequence[int]] = None):
    """Assign distinct physical pages from a seeded shuffled pool.

    Slot b receives ``ceil(alloc_lens[b] / page_size)`` pages (``alloc_lens``
    defaults to ``seq_lens``); entries past them are -1. Returns
    ``(table int32 [B][max_pages_per_seq], pool_pages)``.
    """
    alloc = list(alloc_lens if alloc_lens is not None else seq_lens)
    need = [-(-int(L) // page_size) for L in alloc]
    if max(need, default=0) > max_pages_per_seq:
        raise ValueError("max_pages_per_seq too small for the lengths")
    total = sum(need)
    pool = max(pool_pages or 0, total, 1)
    perm = torch.randperm(pool, generator=_gen(seed, "cpu"))
    table = torch.full((len(alloc), max_pages_per_seq), -1, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n
    return table, pool


def make_case(*, batch: int, seq_lens: Sequence[int], q_len: int, num_q_heads: int, num_kv_heads: int,
              head_dim: int, page_size: int, kv_format: str = "e4m3", kv_std: float = 1.0,
              kv_scale: float = 1.0, seed: int = 0, device="cpu", max_seq_len: Optional[int] = None,
              pool_pages: Optional[int] = None, alloc_lens: Optional[Sequence[int]] = None,
              padded_slots: Sequence[int] = (), q_std: float = 1.0) -> dict:
    """One seeded synthetic batch.

    Returns a dict of torch tensors on ``device``: ``q`` FP16 [B][q_len][Hq][D],
    ``k_cache``/``v_cache`` [pages][page_size][Hkv][D], ``block_table`` int32,
    ``seq_lens`` int32, ``k_scale``/``v_scale`` float32[1]; plus the geometry.
    Padded slots get NaN queries and a block-table row of -1 so that a leak shows.
    """
    seq_lens = [int(v) for v in seq_lens]
    if len(seq_lens) != batch:
        raise ValueError("len(seq_lens) != batch")
    if max_seq_len is None:
        max_seq_len = max(max(seq_lens + list(alloc_lens or [])), 1)
    max_pages = max(1, -(-max_seq_len // page_size))
    table, pool = block_tables(seq_lens, page_size, max_pages, seed=seed * 7919 + 1, pool_pages=pool_pages,
                               alloc_lens=alloc_lens)
    for b in padded_slots:
        table[b, :] = -1
    g = _gen(seed, device)
    q = (torch.randn((batch, q_len, num_q_heads, head_dim), generator=g, device=device) * q_std).to(torch.float16)
    for b in padded_slots:
        q[b] = float("nan")
    k = random_cache(pool, page_size, num_kv_heads, head_dim, kv_format=kv_format, std=kv_std,
                     seed=seed * 7919 + 2, device=device)
    v = random_cache(pool, page_size, num_kv_heads, head_dim, kv_format=kv_format, std=kv_std,
                     seed=seed * 7919 + 3, device=device)
    return dict(
        q=q, k_cache=k, v_cache=v,
        block_table=table.to(device), seq_lens=torch.tensor(seq_lens, dtype=torch.int32, device=device),
        k_scale=torch.tensor([kv_scale], dtype=torch.float32, device=device),
        v_scale=torch.tensor([kv_scale], dtype=torch.float32, device=device),
        page_size=page_size, kv_format=kv_format, max_seq_len=max_seq_len, max_pages_per_seq=max_pages,
        q_len=q_len, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
    )


def workload_case(w: Workload, *, device="cpu", layer: int = 0, seed: Optional[int] = None) -> dict:
    """Inputs of a named workload (one layer). Per-layer caches use seed ``seed*1000 + layer``."""
    base = w.seed if seed is None else seed
    s = base * 1000 + layer if w.layers > 1 else base
    if w.seq_len is None:
        lens = mixed_lengths(w.batch, s)
        padded = list(range(w.batch - 3, w.batch))
    else:
        lens = [w.seq_len] * w.batch
        padded = []
    pool = 64 if w.batch == 1 and w.seq_len is not None and w.seq_len <= 64 * w.page_size else None
    return make_case(batch=w.batch, seq_lens=lens, q_len=w.q_len, num_q_heads=w.num_q_heads,
                     num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size,
                     kv_format=w.kv_format, kv_std=w.kv_std, kv_scale=w.kv_scale, seed=s, device=device,
                     max_seq_len=w.max_seq_len, pool_pages=pool, padded_slots=padded)


def to_numpy(case: dict) -> dict:
    """Host numpy copies of a case's tensors (bytes stay bytes, FP16 stays FP16)."""
    out = {}
    for k, v in case.items():
        out[k] = v.detach().cpu().numpy() if isinstance(v, torch.Tensor) else v
    return out


def host_subset(case: dict, pairs) -> dict:
    """Host numpy copy of only the cache pages that the (slot, KV head) pairs read, with the
    block table remapped onto them (so a large device case can be checked on the host)."""
    import numpy as np
    bt = case["block_table"].cpu()
    lens = case["seq_lens"].cpu()
    ps = case["page_size"]
    slots = sorted({b for b, _ in pairs})
    need = sorted({int(p) for b in slots for p in bt[b, :-(-int(lens[b]) // ps)].tolist()})
    remap = {p: i for i, p in enumerate(need)}
    idx = torch.tensor(need, dtype=torch.long, device=case["k_cache"].device)
    k = case["k_cache"].index_select(0, idx).cpu().numpy()
    v = case["v_cache"].index_select(0, idx).cpu().numpy()
    table = np.full(tuple(bt.shape), -1, dtype=np.int64)
    for b in slots:
        n = -(-int(lens[b]) // ps)
        table[b, :n] = [remap[int(p)] for p in bt[b, :n].tolist()]
    return dict(q=case["q"].cpu().numpy(), k_cache=k, v_cache=v, block_table=table, seq_lens=lens.numpy(),
                k_scale=case["k_scale"].cpu().numpy(), v_scale=case["v_scale"].cpu().numpy(), page_size=ps,
                kv_format=case["kv_format"])


def kv_bytes(seq_lens: Sequence[int], num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Algorithmic KV bytes of one layer: every visible token's K and V row read once per KV head."""
    return int(sum(max(0, int(L)) for L in seq_lens)) * num_kv_heads * head_dim * 2 * elem_bytes


# ---- long prefill ----

@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    name: str
    q_len: int                      # query chunk: the last q_len positions of the sequence
    kv_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seed: int
    description: str


PREFILL_WORKLOADS = {
    w.name: w for w in [
        # The pages' long-prefill operator shapes: Q8192 against KV262144, six query heads per KV
        # head, at the TP4 / TP2 / TP1 local head counts.
        PrefillWorkload("prefill_q8192_kv262144_hkv1", 8192, 262144, 6, 1, 256, 9,
                        "Q8192 x KV262144, Hq6/Hkv1 (TP4 local), FP16 N(0,1) Q/K/V, causal"),
        PrefillWorkload("prefill_q8192_kv262144_hkv2", 8192, 262144, 12, 2, 256, 10,
                        "Q8192 x KV262144, Hq12/Hkv2 (TP2 local), FP16 N(0,1) Q/K/V, causal"),
        PrefillWorkload("prefill_q8192_kv262144_hkv4", 8192, 262144, 24, 4, 256, 11,
                        "Q8192 x KV262144, Hq24/Hkv4 (TP1 local), FP16 N(0,1) Q/K/V, causal"),
    ]
}


def prefill_case(*, q_len: int, kv_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int = 256,
                 seed: int = 0, device="cpu", std: float = 1.0) -> dict:
    """Seeded FP16 N(0, std^2) q [q_len][Hq][D], k / v [kv_len][Hkv][D]."""
    g = _gen(seed, device)
    q = torch.randn((q_len, num_q_heads, head_dim), generator=g, device=device) * std
    k = torch.randn((kv_len, num_kv_heads, head_dim), generator=g, device=device) * std
    v = torch.randn((kv_len, num_kv_heads, head_dim), generator=g, device=device) * std
    return dict(q=q.to(torch.float16), k=k.to(torch.float16), v=v.to(torch.float16))


def prefill_flops(q_len: int, kv_len: int, num_q_heads: int, head_dim: int, causal: bool = True) -> int:
    """Logical (causal) flops: 4 * D per visible (query, key) pair and query head."""
    if causal:
        pairs = sum(max(0, min(kv_len, kv_len - q_len + t + 1)) for t in range(q_len))
    else:
        pairs = q_len * kv_len
    return 4 * head_dim * num_q_heads * pairs
