"""Plain float64 oracle of context-parallel attention, simulated on one host.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU-baseline leg).

Source: the Diffusers context-parallelism page (Spanish, "Paralelismo de
contexto"), cited as [CP page, §section]:

* §"Ring Attention": the K/V blocks travel around a ring of GPUs; each GPU
  attends its own queries to the block it holds, then passes the block on;
  after a full cycle every GPU has seen every token's K/V and none stored the
  whole sequence; the sequence length must divide by ring_degree (variant
  table).
* §"Ulysses Attention": a first all-to-all regroups the data so each GPU holds
  every token of a subset of heads, attention runs per head, a second
  all-to-all regroups the result by token; sequence length and head count
  must divide by ulysses_degree (variant table).

Readings where the page is silent (stated again in the design notes): a
ring step's partial result is the block's softmax-normalised output together
with the log-sum-exp of its scaled scores, and the steps are combined by
weighting each partial with exp(lse_i - lse) -- the unique combination under
which the ring result equals attention over the whole sequence; rank c of
the ring owns token chunk c and sees K/V chunk (c - s) mod R at step s;
Ulysses rank r owns the contiguous head block [r H/u, (r+1) H/u) after the
first all-to-all and token chunk r before it.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

from .tp_block import ShardConfigError, attention_heads

__all__ = ["attention_block", "attention_merge", "ring_attention", "ulysses_seq_to_heads",
           "ulysses_heads_to_seq", "ulysses_attention", "check_ring", "check_ulysses"]


def attention_block(q, k, v, num_heads: int, head_dim: int) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of queries q [Tq, H d] against one K/V block k, v [Tk, H d],
    per head h (column block h of each): s = q_h k_h^T / sqrt(d),
    lse[:, h] = log sum_k exp(s) (natural log, row max subtracted first),
    o[:, h] = exp(s - lse) v_h.  Returns (o [Tq, H d], lse [Tq, H])."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    Tq = q.shape[0]
    o = np.zeros((Tq, num_heads * head_dim))
    lse = np.zeros((Tq, num_heads))
    for h in range(num_heads):
        c = slice(h * head_dim, (h + 1) * head_dim)
        s = (q[:, c] @ k[:, c].T) / math.sqrt(head_dim)
        m = s.max(axis=1, keepdims=True)
        lse_h = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
        o[:, c] = np.exp(s - lse_h[:, None]) @ v[:, c]
        lse[:, h] = lse_h
    return o, lse


def attention_merge(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray],
                    head_dim: int) -> Tuple[np.ndarray, np.ndarray]:
    """Combine partial attention results over disjoint key blocks: per
    (token, head), lse = log sum_i exp(lse_i) and o = sum_i exp(lse_i - lse) o_i
    (the row max of the lse_i subtracted first)."""
    L = np.stack([np.asarray(a, dtype=np.float64) for a in lse_parts])   # [n, T, H]
    m = L.max(axis=0)
    lse = m + np.log(np.exp(L - m).sum(axis=0))
    w = np.exp(L - lse)                                                   # [n, T, H]
    o = np.zeros_like(np.asarray(o_parts[0], dtype=np.float64))
    for i, oi in enumerate(o_parts):
        o += np.repeat(w[i], head_dim, axis=1) * np.asarray(oi, dtype=np.float64)
    return o, lse


def check_ring(tokens: int, ring_degree: int) -> None:
    """[CP page, variant table] the sequence must divide by ring_degree."""
    if ring_degree < 1 or tokens % ring_degree:
        raise ShardConfigError("divisibility", f"ring_degree {ring_degree} does not divide {tokens} tokens")


def check_ulysses(tokens: int, num_heads: int, degree: int) -> None:
    """[CP page, variant table] sequence length and head count must divide by
    ulysses_degree."""
    if degree < 1 or tokens % degree or num_heads % degree:
        raise ShardConfigError("divisibility",
                               f"ulysses_degree {degree} must divide {tokens} tokens and {num_heads} heads")


def ring_attention(q, k, v, num_heads: int, head_dim: int, ring_degree: int) -> List[np.ndarray]:
    """[CP page, §Ring Attention] rank c holds token chunk c of q, k, v; at
    step s it attends its queries to the K/V chunk it holds then, (c - s) mod R,
    and passes the chunk on; its output is the merge of its R partials.
    Returns every rank's output chunk (concatenated: the whole output)."""
    T = np.asarray(q).shape[0]
    check_ring(T, ring_degree)
    n = T // ring_degree
    chunk = lambda a, c: np.asarray(a, dtype=np.float64)[c * n:(c + 1) * n]
    outs = []
    for c in range(ring_degree):
        o_parts, lse_parts = [], []
        for s in range(ring_degree):
            j = (c - s) % ring_degree
            o_p, l_p = attention_block(chunk(q, c), chunk(k, j), chunk(v, j), num_heads, head_dim)
            o_parts.append(o_p)
            lse_parts.append(l_p)
        outs.append(attention_merge(o_parts, lse_parts, head_dim)[0])
    return outs


def ulysses_seq_to_heads(chunks: Sequence[np.ndarray], num_heads: int, head_dim: int) -> List[np.ndarray]:
    """First all-to-all [CP page, §Ulysses Attention]: rank s holds token chunk
    s of a [T, H d] tensor; afterwards rank r holds every token of heads
    [r H/u, (r+1) H/u): out_r = concat_s chunks[s][:, head block r]."""
    u = len(chunks)
    w = num_heads // u * head_dim
    return [np.concatenate([np.asarray(c)[:, r * w:(r + 1) * w] for c in chunks]) for r in range(u)]


def ulysses_heads_to_seq(parts: Sequence[np.ndarray], num_heads: int, head_dim: int) -> List[np.ndarray]:
    """Second all-to-all: rank r holds every token of its head block; afterwards
    rank s holds token chunk s of all heads: out_s = concat_r parts[r][chunk s]."""
    u = len(parts)
    n = np.asarray(parts[0]).shape[0] // u
    return [np.concatenate([np.asarray(p)[s * n:(s + 1) * n] for p in parts], axis=1) for s in range(u)]


def ulysses_attention(q, k, v, num_heads: int, head_dim: int, degree: int) -> List[np.ndarray]:
    """[CP page, §Ulysses Attention] token-sharded q, k, v -> first all-to-all ->
    attention over each rank's heads -> second all-to-all.  Returns every
    rank's token chunk of the output."""
    T = np.asarray(q).shape[0]
    check_ulysses(T, num_heads, degree)
    n = T // degree
    split = lambda a: [np.asarray(a, dtype=np.float64)[s * n:(s + 1) * n] for s in range(degree)]
    qh, kh, vh = (ulysses_seq_to_heads(split(a), num_heads, head_dim) for a in (q, k, v))
    hr = num_heads // degree
    o_heads = [attention_heads(qh[r], kh[r], vh[r], hr, head_dim) for r in range(degree)]
    return ulysses_heads_to_seq(o_heads, num_heads, head_dim)
