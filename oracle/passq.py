"""Float64 CPU oracle for T >= 1 new query tokens per request (pass-Q
attention of a multi-token turn over the cached history).

TEST INFRASTRUCTURE ONLY, like oracle.py: only ``tests/``,
``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg may use it.
It shares no code with the GPU library.

What is computed.  In the pass-Q scheme of the Context Parallelism knowledge
note (sections "Pass-Q keeps KV stationary for cache-heavy turns" and "A
runtime heuristic chooses the ring direction"), a turn brings T new tokens to
a request that already holds P cached ones: Q has shape [T, N_H, D_H] while K
and V have shape [T + P, N_KV, D_H], i.e. the keys and values of the new
tokens are in the cache (appended before attention) next to the history.
Readings taken here where the note is silent:

* new token t (0-based) sits at global position P + t, and attention among
  the new tokens is causal: query t sees positions 0 .. P + t;
* with L = T + P = seq_len[b] (the cache length after the append), query t
  therefore sees the first vis(t) = L - T + 1 + t positions; a request whose
  L is below T gives its first T - L queries no key at all (o = 0,
  lse = -inf), like an empty shard;
* T = 1 is the single-token decode of oracle.py.

Shards hold the same tokens as for one query (oracle.split_ranges for the
contiguous and paged caches, oracle.cache's ownership rule for the striped
and staggered ones).  The partial of shard j for query t is attention over
the tokens shard j holds whose position is below vis(t); a shard holding none
of them yields o = 0, lse = -inf.  The merge is unchanged: every (request,
query token, head) is one row, B*T*Hq rows in all.  Since the positions a
shard holds increase with its local row, the visible tokens of a shard are a
prefix of its rows.

Layouts: q [B,T,Hq,Dqk]; o [B,T,Hq,Dv], lse [B,T,Hq]; o_part
[kvp,B,T,Hq,Dv], lse_part [kvp,B,T,Hq]; new rows k_new [B,T,Hkv,Dqk], v_new
[B,T,Hkv,Dv], token t of request b stored at position positions[b] + t.

Parity: pinned by tests/test_oracle_passq.py (brute force with explicit
loops, torch's lower-right causal attention in float64, reduction to the
single-token oracle, closed forms, split invariance over every layout).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import cache as oc
from .oracle import Problem, attend, q_to_f64, slab_kv, split_ranges


def visible(L: int, T: int, t: int) -> int:
    """Number of leading positions query token t of a T-token turn sees in an
    L-token cache (clamped to [0, L])."""
    return max(0, min(L, L - T + 1 + t))


def _q4(p: Problem, T: int, q) -> np.ndarray:
    qf = q_to_f64(q, p.q_dtype)
    return qf.reshape(p.B, T, p.Hq, p.Dqk)


def _todo(p: Problem, pairs):
    return pairs if pairs is not None else [(b, h) for b in range(p.B) for h in range(p.Hkv)]


def decode_tokens(p: Problem, T: int, layout: str, kvp: int, q, cache: dict, seq_lens,
                  pairs: Optional[Sequence] = None):
    """Full-context o [B,T,Hq,Dv], lse [B,T,Hq] (float64): query t of request
    b attends to the first visible(L_b, T, t) positions, whichever shard
    stores them.  pairs: optional (b, kvh) list; other entries are NaN."""
    qf = _q4(p, T, q)
    c = oc.gather_contiguous(p, layout, kvp, cache, seq_lens)
    o = np.full((p.B, T, p.Hq, p.Dv), np.nan)
    lse = np.full((p.B, T, p.Hq), np.nan)
    for b, kvh in _todo(p, pairs):
        L = int(seq_lens[b])
        k, v = slab_kv(p, c["k"], c["k_scale"], c["v"], c["v_scale"], b, kvh, 0, L)
        heads = slice(kvh * p.G, (kvh + 1) * p.G)
        for t in range(T):
            n = visible(L, T, t)
            o[b, t, heads], lse[b, t, heads] = attend(qf[b, t, heads], k[:n], v[:n], p.sm_scale)
    return o, lse


def decode_partials_tokens(p: Problem, T: int, layout: str, kvp: int, q, cache: dict, seq_lens,
                           pairs: Optional[Sequence] = None):
    """Shard partials o_part [kvp,B,T,Hq,Dv], lse_part [kvp,B,T,Hq]: partial
    (j, t) is attention of query t over the tokens shard j holds that query t
    sees."""
    qf = _q4(p, T, q)
    o = np.full((kvp, p.B, T, p.Hq, p.Dv), np.nan)
    lse = np.full((kvp, p.B, T, p.Hq), np.nan)
    contiguous = layout in ("contiguous", oc.PAGED)
    c = oc.gather_contiguous(p, layout, kvp, cache, seq_lens) if contiguous else None
    for b, kvh in _todo(p, pairs):
        L = int(seq_lens[b])
        heads = slice(kvh * p.G, (kvh + 1) * p.G)
        if contiguous:
            k, v = slab_kv(p, c["k"], c["k_scale"], c["v"], c["v_scale"], b, kvh, 0, L)
            for j, (s, e) in enumerate(split_ranges(L, kvp)):
                for t in range(T):
                    e_t = max(s, min(e, visible(L, T, t)))
                    o[j, b, t, heads], lse[j, b, t, heads] = attend(qf[b, t, heads], k[s:e_t], v[s:e_t],
                                                                    p.sm_scale)
            continue
        held = oc.shard_tokens(L, kvp, layout)
        for j in range(kvp):
            sub = {n: (None if cache.get(n) is None else
                       (cache[n] if (n.endswith("scale") and p.kv_dtype != "mxfp4") else cache[n][j]))
                   for n in ("k", "k_scale", "v", "v_scale")}
            k, v = slab_kv(p, sub["k"], sub["k_scale"], sub["v"], sub["v_scale"], b, kvh, 0, len(held[j]))
            for t in range(T):
                n = int(np.count_nonzero(held[j] < visible(L, T, t)))
                o[j, b, t, heads], lse[j, b, t, heads] = attend(qf[b, t, heads], k[:n], v[:n], p.sm_scale)
    return o, lse


def append_tokens(p: Problem, T: int, layout: str, kvp: int, cache: dict, positions: Sequence[int],
                  k_new: np.ndarray, v_new: Optional[np.ndarray]) -> None:
    """Encode and store the T new tokens of every request in place: token t of
    request b (rows k_new[b,t], v_new[b,t], fp32) goes to position
    positions[b] + t; a request with a negative positions[b] is skipped, and
    each token whose row falls outside the cache is skipped (oracle.cache.append
    rules)."""
    k4 = np.asarray(k_new, dtype=np.float32).reshape(p.B, T, p.Hkv, p.Dqk)
    v4 = None if v_new is None else np.asarray(v_new, dtype=np.float32).reshape(p.B, T, p.Hkv, p.Dv)
    for t in range(T):
        pos = [(-1 if int(positions[b]) < 0 else int(positions[b]) + t) for b in range(p.B)]
        oc.append(p, layout, kvp, cache, pos, k4[:, t], None if v4 is None else v4[:, t])
