"""Bounded verify-attention graphs per batch size, and the selector that picks one.

Host-side policy around the replay path of ``attn_run`` + ``attn_combine`` (argument
marshalling and graph bookkeeping only; every step of the attention runs in the HIP library).
It follows "DFlash2 concurrent long-context attention, 2026-09-27", section "Why the
single-request optimization was missing from concurrent decode":

* graphs are captured for a set of verify batch sizes, all bounded by one served context
  window (at most 262144 tokens);
* a bounded graph is replayed only when the host-side length hint of each live request fits
  that window: a single oversized peer sends the whole batch to the ordinary (eager) route;
* a live batch smaller than the graph is padded with zero-length slots, which the kernels never
  read (their queries and block-table rows may hold anything);
* capture runs from the largest batch size down, so the workspace bank allocates the largest
  request panel once and the smaller graphs reuse it; a bank that later grows keeps the older
  panel alive for the graphs that captured it; panels are never shared across streams;
* the loaded library reports its batch capacity, and batch sizes beyond it are not captured
  (a stale library cannot be handed batched workspaces).

The verifier sizes go up to 32 requests (q8 x 32 = 256 verify tokens), the capture-size cap
named in "SM70 attention and quantized projection coverage across TP sizes", section
"Corrected TP2 r5 long context and concurrency".

A graph set binds static device buffers: per layer a query and an output buffer of the
captured batch size, one block table of ``plan.max_pages_per_seq`` columns and one length
vector. ``run`` copies the live batch into them, replays, and returns views of the output
buffers, valid until the next call. Replay a set's graphs on one stream at a time: they share
one workspace panel.
"""
from typing import List, Optional, Sequence

import torch

from . import attention as A

DEFAULT_BATCH_SIZES = (1, 2, 4, 8, 16, 32)


def select_batch_size(captured: Sequence[int], context_bound: int, hints: Sequence[int]) -> Optional[int]:
    """Smallest captured batch size that holds the live batch, or None for the eager route.

    None when there is no live request, when there are more live requests than the largest
    capture, or when any request's CPU length hint is negative or exceeds ``context_bound``
    (the served window the graphs were captured for): one oversized peer is enough.
    """
    n = len(hints)
    if n == 0:
        return None
    if any(int(h) < 0 or int(h) > context_bound for h in hints):
        return None
    fits = [b for b in captured if b >= n]
    return min(fits) if fits else None


def capturable_batch_sizes(batch_sizes: Sequence[int], library_max_batch: int, plan_capacity: int) -> List[int]:
    """The requested sizes the loaded library and the plan can serve, largest first."""
    ok = {int(b) for b in batch_sizes if 1 <= int(b) <= min(library_max_batch, plan_capacity)}
    return sorted(ok, reverse=True)


class LayerCache:
    """One layer's paged K/V caches and per-tensor scales (device tensors)."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor):
        self.k_cache, self.v_cache, self.k_scale, self.v_scale = k_cache, v_cache, k_scale, v_scale


class VerifyGraphs:
    """Bounded graphs of one attention contract over a list of layers."""

    def __init__(self, plan: A.Plan, layers: Sequence[LayerCache], batch_sizes: Sequence[int] = DEFAULT_BATCH_SIZES,
                 bank: Optional[A.WorkspaceBank] = None, stream: Optional[torch.cuda.Stream] = None):
        if plan.device is None:
            raise ValueError("graphs need a device plan")
        self.plan = plan
        self.layers = list(layers)
        self.bank = bank if bank is not None else A.default_bank()
        self.stream = stream if stream is not None else torch.cuda.Stream(plan.device)
        self.sizes = capturable_batch_sizes(batch_sizes, A.capabilities()["max_batch"], plan.batch_capacity)
        self.context_bound = plan.max_seq_len
        self._graphs = {}
        self._static = {}
        self._eager_plans = {}

    # ---- capture ----

    def _buffers(self, B: int) -> dict:
        p, dev = self.plan, self.plan.device
        shape = (B, p.q_len, p.num_q_heads, p.head_dim)
        return {
            "q": [torch.zeros(shape, dtype=torch.float16, device=dev) for _ in self.layers],
            "out": [torch.zeros(shape, dtype=torch.float16, device=dev) for _ in self.layers],
            "block_table": torch.full((B, p.max_pages_per_seq), -1, dtype=torch.int32, device=dev),
            "seq_lens": torch.zeros((B,), dtype=torch.int32, device=dev),
        }

    def capture(self) -> List[int]:
        """Capture every size, largest first; returns the captured sizes."""
        for B in self.sizes:                                    # descending
            st = self._buffers(B)
            ws = self.bank.get(self.plan, B, self.stream)
            args = [self.plan.make_args(st["q"][i], L.k_cache, L.v_cache, st["block_table"], st["seq_lens"],
                                        L.k_scale, L.v_scale, st["out"][i], ws)
                    for i, L in enumerate(self.layers)]
            self.stream.wait_stream(torch.cuda.current_stream(self.plan.device))
            with torch.cuda.stream(self.stream):
                for a in args:                                   # warm run outside the capture
                    self.plan.split(a, self.stream)
                    self.plan.combine(a, self.stream)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                for a in args:
                    self.plan.split(a, self.stream)
                    self.plan.combine(a, self.stream)
            torch.cuda.current_stream(self.plan.device).wait_stream(self.stream)
            self._graphs[B] = g
            self._static[B] = (st, ws, args)
        return sorted(self._graphs)

    @property
    def captured(self) -> List[int]:
        return sorted(self._graphs)

    # ---- run ----

    def select(self, hints: Sequence[int]) -> Optional[int]:
        return select_batch_size(self.captured, self.context_bound, hints)

    def run(self, qs: Sequence[torch.Tensor], block_table: torch.Tensor, seq_lens: torch.Tensor,
            hints: Sequence[int]):
        """Attention of every layer for the live batch; returns (outputs per layer, route).

        ``qs[i]`` is layer i's FP16 [n][q_len][Hq][D] query batch, ``block_table`` int32 [n][W],
        ``seq_lens`` int32 [n] on the device, ``hints`` the n CPU upper bounds of those lengths.
        Route "graph:<B>" replays the bounded graph of B slots; "eager" runs the ordinary path.
        """
        n = len(hints)
        if len(qs) != len(self.layers) or any(q.shape[0] != n for q in qs) or block_table.shape[0] != n \
                or seq_lens.shape[0] != n:
            raise ValueError("qs, block_table, seq_lens and hints must describe the same live batch")
        B = self.select(hints)
        # A hint longer than the live table can address goes to the eager route, which rejects it
        # as the ordinary path does (the graph's own table is wider, and its columns past the live
        # width would hold -1).
        if B is None or max((int(h) for h in hints), default=0) > block_table.shape[1] * self.plan.page_size:
            return self._run_eager(qs, block_table, seq_lens, hints), "eager"
        st, _, _ = self._static[B]
        W = min(block_table.shape[1], self.plan.max_pages_per_seq)
        cur = torch.cuda.current_stream(self.plan.device)
        for i, q in enumerate(qs):
            st["q"][i][:n].copy_(q)
        st["block_table"].fill_(-1)
        # Every hint is at most W * page_size tokens and at most the captured window, so the
        # kernels never read a column past W (those hold -1).
        st["block_table"][:n, :W].copy_(block_table[:, :W])
        st["seq_lens"].zero_()                                   # padded slots are zero-length
        st["seq_lens"][:n].copy_(seq_lens)
        self.stream.wait_stream(cur)
        with torch.cuda.stream(self.stream):
            self._graphs[B].replay()
        cur.wait_stream(self.stream)
        return [st["out"][i][:n] for i in range(len(self.layers))], f"graph:{B}"

    def _eager_plan(self, width: int, longest: int, n: int) -> A.Plan:
        """The graphs' own plan when the batch fits its table width, window and capacity (so eager
        calls share, and may grow, the graphs' workspace panel); otherwise a plan of the same
        geometry for the live table width."""
        p = self.plan
        if width == p.max_pages_per_seq and longest <= p.max_seq_len and n <= p.batch_capacity:
            return p
        caps = A.capabilities()
        bound = min(caps["max_seq_len"], width * p.page_size)
        if longest > bound:
            raise ValueError(f"a length hint ({longest}) exceeds what the block table or the library can hold")
        if n > caps["max_batch"]:
            raise ValueError(f"{n} requests exceed the library's batch capacity {caps['max_batch']}")
        key = (width, bound)
        if key not in self._eager_plans:
            self._eager_plans[key] = A.Plan(q_len=p.q_len, num_q_heads=p.num_q_heads, num_kv_heads=p.num_kv_heads,
                                            head_dim=p.head_dim, page_size=p.page_size, max_seq_len=bound,
                                            max_pages_per_seq=width, batch_capacity=caps["max_batch"],
                                            kv_dtype=p.kv_dtype, k_strides=self._strides("k"),
                                            v_strides=self._strides("v"), sm_scale=p.desc.sm_scale,
                                            causal=p.causal, device=p.device)
        return self._eager_plans[key]

    def _strides(self, which: str):
        d = self.plan.desc
        return (getattr(d, f"{which}_page_stride"), getattr(d, f"{which}_token_stride"),
                getattr(d, f"{which}_head_stride"))

    def _run_eager(self, qs, block_table, seq_lens, hints):
        """The ordinary route, on the set's stream and bank."""
        n = len(hints)
        if n == 0:
            return [q.new_zeros(q.shape) for q in qs]
        plan = self._eager_plan(block_table.shape[1], max(int(h) for h in hints), n)
        cur = torch.cuda.current_stream(self.plan.device)
        self.stream.wait_stream(cur)
        outs = []
        with torch.cuda.stream(self.stream):
            for q, L in zip(qs, self.layers):
                outs.append(plan.run(q, L.k_cache, L.v_cache, block_table, seq_lens, L.k_scale, L.v_scale,
                                     stream=self.stream, bank=self.bank))
        cur.wait_stream(self.stream)
        for o in outs:
            o.record_stream(cur)
        return outs
