"""Plain FP64 oracle of speculative-verify attention over a paged KV cache.

Test infrastructure only: the product path never imports this module.

The operation (stated in the pages' terms):

* "DFlash2 concurrent long-context attention, 2026-09-27", section "Why the
  single-request optimization was missing from concurrent decode": a batch of
  requests, each with its own sequence length, each bringing q = 8 verify
  query tokens in FP16; K and V are E4M3 bytes in a paged cache; D = 256 and
  six query heads share one KV head. Zero-length rows and padded requests must
  stay safe. Section "Operator validation": batched results equal independent
  single-request results, and an FP64 oracle checks them.
* "perf(fa2): port decode GQA group-swap into d128 varlen launcher" (PR #48),
  PR description: the query heads of one KV group are packed together, so query
  head ``h`` reads KV head ``h // G`` (kv-major, group-minor order). The same PR
  names the log-sum-exp combine of split partials; ``merge_partials`` is that
  merge written from its definition.

Readings taken where the pages are silent:

* the verify tokens are the last ``q_len`` positions of the sequence, so query
  token ``t`` sits at position ``L - q_len + t`` and sees keys ``j <= L - q_len + t``
  (bottom-right causal alignment); with ``L < q_len`` the first rows see no key;
* a row that sees no key (zero length, padded slot, or ``t < q_len - L``) is
  exactly zero;
* dequantisation is ``scale * decode(byte)`` with one FP32 scale per tensor;
* the softmax scale defaults to ``1 / sqrt(D)`` and multiplies ``<q, k_scale*K>``.

Pins (tests/test_oracle_*.py): a separate pure-Python brute force on tiny inputs,
closed forms (uniform weights for Q = 0, constant V, a row that sees exactly one
key), invariance to page size and to permuting physical pages, GQA equal to MHA
with replicated KV heads, exact scaling by a power-of-two v_scale, and the
identity "full result == merge of the partial states of any token split".
"""
import math

import numpy as np

from .e4m3 import decode_table
from .e5m2 import decode_table as decode_e5m2_table

_E4M3 = decode_table()
_E5M2 = decode_e5m2_table()


def _values(raw: np.ndarray, kv_format: str) -> np.ndarray:
    """Raw cache elements -> float64 values (before the per-tensor scale)."""
    if kv_format == "e4m3":
        if raw.dtype != np.uint8:
            raise TypeError("E4M3 caches hold uint8 bytes")
        return _E4M3[raw]
    if kv_format == "e5m2":
        if raw.dtype != np.uint8:
            raise TypeError("E5M2 caches hold uint8 bytes")
        return _E5M2[raw]
    if kv_format == "fp16":
        if raw.dtype != np.float16:
            raise TypeError("FP16 caches hold float16 elements")
        return raw.astype(np.float64)
    raise ValueError(f"unknown kv_format {kv_format!r}")


def gather_tokens(cache: np.ndarray, table_row: np.ndarray, length: int, kv_head: int,
                  page_size: int) -> np.ndarray:
    """Elements of KV head ``kv_head`` for logical tokens ``0..length-1``.

    ``cache`` is indexed ``[page][slot][kv_head][d]``; logical token ``j`` lives in
    physical page ``table_row[j // page_size]`` at slot ``j % page_size``.
    Returns the raw elements, shape ``[length][D]``.
    """
    n_pages = -(-length // page_size)
    pages = np.asarray(table_row[:n_pages], dtype=np.int64)
    if n_pages and (pages.min() < 0 or pages.max() >= cache.shape[0]):
        raise IndexError("block table names a page outside the cache")
    tok = cache[pages, :, kv_head, :]                # [n_pages][page_size][D]
    return tok.reshape(n_pages * page_size, cache.shape[3])[:length]


def visible_keys(length: int, q_len: int, t: int, causal: bool) -> int:
    """Number of keys (a prefix 0..n-1) that query token ``t`` of a length-``length`` row sees."""
    if length <= 0:
        return 0
    if not causal:
        return length
    return max(0, min(length, length - q_len + t + 1))


def verify_attention(q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, *,
                     page_size, sm_scale=None, kv_format="e4m3", causal=True, pairs=None):
    """Exact attention output in float64.

    q           [B][q_len][Hq][D] (any float dtype; FP16 inputs are taken at face value)
    k_cache     [num_pages][page_size][Hkv][D] uint8 (E4M3) or float16
    v_cache     same shape and format as k_cache
    block_table [B][max_pages] int
    seq_lens    [B] int (0 = empty row or padded slot)
    k_scale, v_scale  per-tensor scales (floats)
    pairs       optional iterable of (b, kv_head) to evaluate; other outputs are NaN

    out[b][t][h] = sum_j softmax_j(sm_scale * <Q[b,t,h], k_scale*K_j>) * v_scale*V_j over the
    keys row (b, t) sees; exactly 0 when it sees none.
    """
    q = np.asarray(q)
    B, q_len, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    if k_cache.shape[1] != page_size or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape does not match page_size / each other")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    qf = q.astype(np.float64)
    out = np.zeros((B, q_len, Hq, D), dtype=np.float64)
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    else:
        pairs = list(pairs)
        out[:] = np.nan
    for b, g in pairs:
        out[b, :, g * G:(g + 1) * G, :] = 0.0
        L = int(seq_lens[b])
        if L <= 0:
            continue
        K = float(k_scale) * _values(gather_tokens(k_cache, block_table[b], L, g, page_size), kv_format)
        V = float(v_scale) * _values(gather_tokens(v_cache, block_table[b], L, g, page_size), kv_format)
        for t in range(q_len):
            n = visible_keys(L, q_len, t, causal)
            if n == 0:
                continue
            Qt = qf[b, t, g * G:(g + 1) * G, :]      # [G][D]: the group's query heads
            s = sm_scale * (Qt @ K[:n].T)            # [G][n]
            s -= s.max(axis=1, keepdims=True)
            w = np.exp(s)
            p = w / w.sum(axis=1, keepdims=True)
            out[b, t, g * G:(g + 1) * G, :] = p @ V[:n]
    return out


def partial_states(q, k_cache, v_cache, block_table, seq_lens, k_scale, *, b, kv_head, begin, end,
                   page_size, sm_scale=None, kv_format="e4m3", causal=True):
    """Softmax partial state of one (request, KV head) over keys in ``[begin, end)``.

    Returns ``(m, l, o)`` for the packed rows ``r = t*G + j`` (query head
    ``kv_head*G + j``), natural-log domain, V without its scale:

    * ``m[r]`` = max visible score in the range (``-inf`` if the row sees none of it),
    * ``l[r]`` = sum of ``exp(s - m)`` over those keys (0 if none),
    * ``o[r]`` = sum of ``exp(s - m) * decode(V_j)`` (0 if none).
    """
    q = np.asarray(q)
    _, q_len, Hq, D = q.shape
    G = Hq // k_cache.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    R = q_len * G
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    o = np.zeros((R, D))
    L = int(seq_lens[b])
    if L <= 0:
        return m, l, o
    K = float(k_scale) * _values(gather_tokens(k_cache, block_table[b], L, kv_head, page_size), kv_format)
    V = _values(gather_tokens(v_cache, block_table[b], L, kv_head, page_size), kv_format)
    for t in range(q_len):
        hi = min(end, visible_keys(L, q_len, t, causal))
        lo = max(begin, 0)
        if hi <= lo:
            continue
        for j in range(G):
            r = t * G + j
            s = sm_scale * (K[lo:hi] @ q[b, t, kv_head * G + j].astype(np.float64))
            m[r] = s.max()
            w = np.exp(s - m[r])
            l[r] = w.sum()
            o[r] = w @ V[lo:hi]
    return m, l, o


def merge_partials(parts, v_scale):
    """Log-sum-exp merge of partial states ``[(m, l, o), ...]`` into normalised rows.

    ``out[r] = v_scale * sum_s exp(m_s - M) o_s / sum_s exp(m_s - M) l_s`` with
    ``M = max_s m_s``; rows where every part is empty are exactly 0.
    """
    ms = np.stack([p[0] for p in parts])             # [S][R]
    ls = np.stack([p[1] for p in parts])
    os_ = np.stack([p[2] for p in parts])            # [S][R][D]
    M = ms.max(axis=0)
    out = np.zeros(os_.shape[1:])
    live = np.isfinite(M)
    w = np.where(np.isfinite(ms), np.exp(ms - np.where(live, M, 0.0)), 0.0)
    den = (w * ls).sum(axis=0)
    num = (w[:, :, None] * os_).sum(axis=0)
    out[live] = float(v_scale) * num[live] / den[live, None]
    return out
