"""Brute-force pin for the oracle: explicit loops over Python floats.

Written separately from ``oracle/`` from the plain definition
softmax(sm_scale * Q . (k_scale*K)^T) (v_scale*V) over the keys each verify token sees,
with the query head h reading KV head h // (Hq/Hkv) and logical token j read from
physical page block_table[b][j // page_size], slot j % page_size. E4M3 and E5M2 bytes are
decoded by torch's float8_e4m3fn / float8_e5m2 (library routines), not by the oracle's tables.
Only for tiny inputs.
"""
import math

import torch


def _decoder(kv_format):
    if kv_format == "e4m3":
        vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()
        return lambda x: vals[int(x)]
    if kv_format == "e5m2":
        vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).tolist()
        return lambda x: vals[int(x)]
    return lambda x: float(x)


def brute_attention(q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, *, page_size,
                    sm_scale, kv_format="e4m3", causal=True):
    dec = _decoder(kv_format)
    B, q_len, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    group = Hq // Hkv
    out = [[[[0.0] * D for _ in range(Hq)] for _ in range(q_len)] for _ in range(B)]
    for b in range(B):
        L = int(seq_lens[b])
        for t in range(q_len):
            position = L - q_len + t          # absolute position of this verify token
            keys = [j for j in range(L) if (not causal) or j <= position]
            if not keys:
                continue
            for h in range(Hq):
                g = h // group
                scores = []
                rows = []
                for j in keys:
                    page = int(block_table[b][j // page_size])
                    slot = j % page_size
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[b][t][h][d]) * (float(k_scale) * dec(k_cache[page][slot][g][d]))
                    scores.append(float(sm_scale) * acc)
                    rows.append((page, slot))
                top = max(scores)
                ex = [math.exp(s - top) for s in scores]
                z = sum(ex)
                for d in range(D):
                    acc = 0.0
                    for e, (page, slot) in zip(ex, rows):
                        acc += (e / z) * (float(v_scale) * dec(v_cache[page][slot][g][d]))
                    out[b][t][h][d] = acc
    return out
