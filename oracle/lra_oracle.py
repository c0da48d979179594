"""Plain fp64 CPU oracle for attention over a shared-base + low-rank KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg.
It shares no code with the GPU library; the only module both sides use is the
seeded input generator, which holds no arithmetic of the method.

What it computes (stated in words on the pages; the formula is the plain
reading of those words):

* LRAgent: Efficient KV Cache Sharing for Multi-LoRA LLM Agents, abstract:
  the cache is split into a shared base part computed with the pretrained
  weights and an adapter part computed with the LoRA weights; the adapter
  part is stored in its low-rank form, and shared-A adapters share the
  low-rank cache itself. With a LoRA update ``W + A B`` on the key and value
  projections and ``L = X A`` (the low-rank cache), every cached key and
  value is ``K = K_base + L_k B_k`` and ``V = V_base + L_v B_v``.
* PReCache abstract and Figure 1 caption: the shared base cache is computed
  with the pretrained weights and each agent's compact low-rank cache is
  precomputed from hidden states, ``L = X A``.

Readings taken where the pages are silent (each is listed in the design doc):
* the base key cache is stored after the rotary embedding; the adapter key
  term is rotated at its absolute 0-based position before it is added; the
  value is not rotated;
* rotary pairing is rotate-half, (i, i + d/2), with angle ``n * theta**(-2i/d)``;
* query head j reads KV head ``j // (Hq / Hkv)``;
* ``B`` is [r, Hkv*d] with column ``h*d + i``; one L row serves every KV head;
* a decode query sits at position T-1 and sees keys 0..T-1; prefill query i of
  a chunk of q_len new tokens sits at T - q_len + i and sees keys 0..position;
* softmax scale is an explicit argument (1/sqrt(d) unless stated);
* a projection without an adapter (B = None) keeps its base cache unchanged,
  and a sequence without an agent has neither adapter;
* an activation position a (default 0) leaves tokens n < a without adapter
  terms in both K and V; queries are not affected by it.

Everything is evaluated in float64 with materialised full-dimension K and V
and a plain two-pass softmax: this file is the definition, not a fast path.
"""
from __future__ import annotations

import numpy as np


def rope_angles(positions: np.ndarray, d: int, theta: float) -> np.ndarray:
    """Angles [n, d/2]: position times theta**(-2i/d) for pair i (fp64)."""
    i = np.arange(d // 2, dtype=np.float64)
    omega = np.power(np.float64(theta), -2.0 * i / d)
    return np.asarray(positions, dtype=np.float64)[:, None] * omega[None, :]


def rope_rotate(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding of x [n, ..., d] at the given positions [n].

    Pair (i, i + d/2) at position n turns by angle n * omega_i:
      y[i]       = x[i] cos - x[i + d/2] sin
      y[i + d/2] = x[i + d/2] cos + x[i] sin
    theta == 0 means no rotary embedding (identity).
    """
    x = np.asarray(x, dtype=np.float64)
    if theta == 0:
        return x.copy()
    d = x.shape[-1]
    ang = rope_angles(positions, d, theta)
    shape = (ang.shape[0],) + (1,) * (x.ndim - 2) + (d // 2,)
    c = np.cos(ang).reshape(shape)
    s = np.sin(ang).reshape(shape)
    x1, x2 = x[..., : d // 2], x[..., d // 2 :]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def adapter_term(l_rows: np.ndarray, b: np.ndarray, Hkv: int, d: int) -> np.ndarray:
    """Full-dimension adapter contribution L B, reshaped to [T, Hkv, d]."""
    return (np.asarray(l_rows, np.float64) @ np.asarray(b, np.float64)).reshape(-1, Hkv, d)


def materialise_kv(kb, vb, lk, lv, bk, bv, theta: float, adapter_start: int = 0):
    """Full keys and values of one sequence.

    kb, vb [T, Hkv, d] base rows; lk, lv [T, r] low-rank rows; bk, bv [r, Hkv*d].
    K[n] = kb[n] + rope_n(lk[n] bk),  V[n] = vb[n] + lv[n] bv   for n >= adapter_start,
    K[n] = kb[n],                     V[n] = vb[n]              for n <  adapter_start.
    The activation position follows "Efficient Multi-Adapter LLM Serving via
    Cross-Model KV-Cache Reuse with Activated LoRA" (abstract): an activated
    adapter acts only on the tokens from its invocation point on, so the
    cache before that point is the base model's.

    A projection without an adapter passes None for its B (and L): its cache
    is the base part alone. PReCache, appendix Table 13 caption, compares
    against adapters on the query and value projections only (no key
    adapter), and its Figure 1 caption batches adapter-free paths (no adapter
    at all) with adapted ones.
    """
    T, Hkv, d = kb.shape
    K = np.array(kb, dtype=np.float64)
    V = np.array(vb, dtype=np.float64)
    on = (np.arange(T) >= adapter_start)[:, None, None]
    if bk is not None:
        K = K + np.where(on, rope_rotate(adapter_term(lk, bk, Hkv, d), np.arange(T), theta), 0.0)
    if bv is not None:
        V = V + np.where(on, adapter_term(lv, bv, Hkv, d), 0.0)
    return K, V


def kv_head_of(j: int, Hq: int, Hkv: int) -> int:
    return j // (Hq // Hkv)


def attend(q: np.ndarray, positions: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """Causal softmax attention of query rows q [nq, Hq, d] at ``positions``
    over keys/values [T, Hkv, d]; key n is visible to a query at p iff n <= p."""
    nq, Hq, d = q.shape
    Hkv = K.shape[1]
    out = np.zeros((nq, Hq, d), dtype=np.float64)
    for j in range(Hq):
        h = kv_head_of(j, Hq, Hkv)
        scores = sm_scale * (q[:, j, :] @ K[:, h, :].T)  # [nq, T]
        for i in range(nq):
            p = int(positions[i])
            s = scores[i, : p + 1]
            w = np.exp(s - s.max())
            w = w / w.sum()
            out[i, j] = w @ V[: p + 1, h, :]
    return out


def lora_attention(q, kb, vb, lk, lv, bk, bv, *, sm_scale: float, theta: float, q_positions=None,
                   adapter_start: int = 0):
    """Attention of one sequence's query rows over its shared-base + low-rank cache.

    q [nq, Hq, d]; the cache holds T = kb.shape[0] tokens. Default positions
    are the last nq positions (T - nq .. T - 1): one row is a decode step,
    nq rows are a prefill chunk appended at the end of the context. Tokens
    before adapter_start carry no adapter term.
    """
    T = kb.shape[0]
    nq = q.shape[0]
    if q_positions is None:
        q_positions = np.arange(T - nq, T)
    K, V = materialise_kv(kb, vb, lk, lv, bk, bv, theta, adapter_start)
    return attend(np.asarray(q, np.float64), q_positions, K, V, sm_scale)


def lr_cache_build(X: np.ndarray, A: np.ndarray) -> np.ndarray:
    """Low-rank cache rows L = X A (fp64), X [n, hidden], A [hidden, r]."""
    return np.asarray(X, np.float64) @ np.asarray(A, np.float64)


def lr_cache_build_multi(X: np.ndarray, A: np.ndarray, group_cols) -> list:
    """Low-rank rows of several adapters from one X (PReCache, Figure 1
    caption, A1-A3): group g is X times columns group_cols[g]:group_cols[g+1]
    of A, in fp64."""
    L = lr_cache_build(X, A)
    return [L[:, group_cols[g] : group_cols[g + 1]] for g in range(len(group_cols) - 1)]

