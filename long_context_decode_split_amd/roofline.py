"""Roofline arithmetic for one decode-attention step (pure Python, no GPU).

Algorithmic bytes are the KV-cache bytes one step must read: every cached
token of every (request, KV head) once, K and V each (V not at all when it is
a prefix of K), plus the per-slab fp8 scales or per-32-element MXFP4 scales.
This is the numerator of the Helix article's KV-read time (section "The
ceiling, in algebra": t_kv = B * 2 * ceil(K/TPA) * Hsz * (S/KVP) * bytes /
MemBW) with TPA = KVP = 1, i.e. one device reading everything.

Flops are 2 * Hq * L * (Dqk + Dv) per request (one multiply-add per query head
per K element and per V element); for Dqk = Dv = Hsz this is the 4 * B * Hq *
S * Hsz of the inference-parallelism survey's decode-CP estimate.
"""
from __future__ import annotations

import math

# MI355X published peaks (dense, no sparsity).
HBM_BYTES_PER_S = 8.0e12
MFMA_BF16_FLOPS = 2.5e15
MFMA_FP8_FLOPS = 5.0e15
VALU_FP32_FLOPS = 157.3e12


def helix_t_kv(B, K, TPA, Hsz, S, KVP, bytes_param, membw_bytes_per_s):
    """Helix per-layer KV read time in seconds (Helix article, "The ceiling, in algebra")."""
    return B * 2 * math.ceil(K / TPA) * Hsz * (S / KVP) * bytes_param / membw_bytes_per_s


def row_bytes(kv_dtype: str, D: int) -> float:
    """Bytes of one cached row of D elements, including its MXFP4 block scales."""
    if kv_dtype == "f32":
        return 4.0 * D
    if kv_dtype == "bf16":
        return 2.0 * D
    if kv_dtype == "fp8":
        return 1.0 * D
    if kv_dtype == "mxfp4":
        return D / 2 + D / 32
    raise ValueError(kv_dtype)


def kv_bytes(Hkv: int, seq_lens, Dqk: int, Dv: int, kv_dtype: str, v_aliases_k: bool) -> int:
    """Algorithmic KV bytes of one step over all requests (seq_lens: per request)."""
    tokens = int(sum(int(s) for s in seq_lens))
    per_token = row_bytes(kv_dtype, Dqk) + (0 if v_aliases_k else row_bytes(kv_dtype, Dv))
    total = Hkv * tokens * per_token
    if kv_dtype == "fp8":
        total += len(seq_lens) * Hkv * 4 * (1 if v_aliases_k else 2)
    return int(round(total))


def attention_flops(Hq: int, seq_lens, Dqk: int, Dv: int) -> int:
    tokens = int(sum(int(s) for s in seq_lens))
    return 2 * Hq * tokens * (Dqk + Dv)


def attention_flops_tokens(Hq: int, seq_lens, T: int, Dqk: int, Dv: int) -> int:
    """Flops of T query tokens per request with causal visibility among them:
    query t of a request with L cached tokens (the T new ones included) sees
    max(0, L - T + 1 + t) of them."""
    tokens = 0
    for s in seq_lens:
        L = int(s)
        tokens += sum(max(0, min(L, L - T + 1 + t)) for t in range(T))
    return 2 * Hq * tokens * (Dqk + Dv)


def partial_bytes(kvp: int, B: int, Hq: int, Dv: int) -> int:
    """Bytes of the shard partials (o_part fp32 + lse_part fp32)."""
    return kvp * B * Hq * (Dv + 1) * 4
