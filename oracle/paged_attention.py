"""CPU reference for attention over a paged KV cache -- TEST INFRASTRUCTURE.

This is the plain, slow, obviously correct oracle that the HIP kernels are
checked against.  Only the test suite, the package's ``smoke()`` check and
the benchmark's CPU-baseline leg may import it; the library path never does,
and this file shares no code with it.  Arithmetic is float64 on bf16 inputs
widened exactly; the result stays unrounded.

What it computes, step by step, with the passage each step follows:

1. ``store_kv`` -- each new token's K and V rows are copied into the pool row
   (slot) named by ``out_loc``.  mini-sglang "Engine Class", Key Methods /
   forward_batch (``out_loc``); miniVLLM "Engine Architecture",
   prepare_prefill / prepare_decode (``slot_mapping``: the physical cache slot
   of each new token); zero-to-sglang Ch.1 section 3.2 (prefill writes the
   initial KV cache, decode appends to it).
2. ``request_slots`` / ``gather`` -- a request's logical position t lives in
   physical page ``page_table[r, t // page_size]`` at row ``t % page_size``;
   the pool is ``[num_blocks, block_size, num_kv_heads, head_dim]``
   (miniVLLM "Engine Architecture", allocate_kv_cache), so its flat slot is
   ``page * page_size + t % page_size``.  The page table maps logical to
   physical locations (mini-sglang "Engine Class", Key Attributes:
   page_table; miniVLLM prepare_* ``block_tables``).
3. ``kv_head_of`` -- grouped-query attention: ``num_kv_heads`` K/V heads
   serve ``num_heads`` query heads (miniVLLM "LLMEngine", Config parameters /
   Model architecture: num_heads, num_kv_heads).  Query head h reads K/V head
   ``h // (num_heads // num_kv_heads)``: consecutive query heads share one
   K/V head.
4. ``visible`` -- causal visibility with a cached prefix.  Prefill feeds only
   the tokens after the cached ones (miniVLLM prepare_prefill,
   ``num_cached_tokens``; zero-to-sglang Ch.1 section 3.3, cached length vs.
   sequence length), so new token i of request r sits at absolute position
   ``prefix_r + i`` and sees keys ``0 .. prefix_r + i``.  A decode step is the
   case of one new token at position ``context_len - 1`` (miniVLLM
   prepare_decode: ``context_lens`` counts all tokens so far).
5. ``attend`` -- textbook scaled dot-product attention on the gathered rows:
   ``softmax(scale * q k^T + mask) v``.  The pages name attention but never
   write out its formula; this is the standard definition.
6. ``decode_multi`` -- a decode step that feeds L tokens per request at once
   (the verification step of speculative decoding, zero-to-sglang Part II
   Ch.1 section 4, roadmap): the L new tokens are the last L of the
   request's ``seq_len`` tokens, and step 4's causal rule applies with a
   cached prefix of ``seq_len - L``.  Reading where the pages are silent: a
   token whose position would be negative (seq_len < L) sees no key and,
   like an empty request, gets an all-zero row.

Every function here is pinned by tests against things other than itself:
a library routine (torch's scaled_dot_product_attention in float64 on
unpaged inputs), closed forms, brute force on tiny inputs, and invariants
(page-permutation, GQA-as-repeated-MHA, chunked prefill, decode as prefill).
"""

from __future__ import annotations

from typing import Iterable, Optional

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 bit patterns (uint16) to float64:
    a bf16 value is the top half of the float32 with the same bits."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def store_kv(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray,
             v_new: np.ndarray, out_loc: np.ndarray):
    """Copy of the pools with row ``out_loc[t]`` of the flat
    ``[num_pages * page_size, Hkv, d]`` view replaced by ``k_new[t]`` /
    ``v_new[t]``.  Works on raw bf16 bits (uint16), so it is a bit copy."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    kf = kc.reshape(-1, *kc.shape[2:])
    vf = vc.reshape(-1, *vc.shape[2:])
    for t in range(len(out_loc)):
        kf[int(out_loc[t])] = k_new[t]
        vf[int(out_loc[t])] = v_new[t]
    return kc, vc


def request_slots(page_table_row: np.ndarray, n: int, page_size: int) -> np.ndarray:
    """Flat pool row of logical positions 0..n-1 of one request."""
    pos = np.arange(n, dtype=np.int64)
    pages = page_table_row[pos // page_size].astype(np.int64)
    return pages * page_size + pos % page_size


def slot_of(page_table_row: np.ndarray, t: int, page_size: int) -> int:
    """Flat slot of logical position t, or -1 when t lies outside the row
    (the same page / row rule as ``request_slots``)."""
    i = t // page_size
    if t < 0 or i >= len(page_table_row):
        return -1
    return int(page_table_row[i]) * page_size + t % page_size


def prefill_metadata(seq_lens, prefix_lens, page_table: np.ndarray, page_size: int):
    """cu_seqlens_q and slot_mapping of a prefill batch (miniVLLM "Engine
    Architecture", prepare_prefill): only the tokens after each sequence's
    cached prefix are fed, ``cu_seqlens_q`` accumulates their counts
    (``len(seq) - num_cached_tokens``), and each new token gets the slot of
    its position."""
    cu, slots = [0], []
    for r, (n, c) in enumerate(zip(seq_lens, prefix_lens)):
        first = max(int(c), 0)
        count = max(int(n) - first, 0)
        cu.append(cu[-1] + count)
        for i in range(count):
            slots.append(slot_of(page_table[r], first + i, page_size))
    return np.array(cu, dtype=np.int32), np.array(slots, dtype=np.int32)


def decode_slots(seq_lens, page_table: np.ndarray, page_size: int) -> np.ndarray:
    """slot_mapping of a decode step (miniVLLM prepare_decode): each sequence
    contributes its most recent token, at position context_len - 1; a padding
    row (length <= 0) gets -1."""
    return np.array([slot_of(page_table[r], int(n) - 1, page_size) if int(n) > 0 else -1
                     for r, n in enumerate(seq_lens)], dtype=np.int32)


def gather(cache: np.ndarray, page_table_row: np.ndarray, n: int) -> np.ndarray:
    """Contiguous ``[n, Hkv, d]`` float64 copy of one request's K or V."""
    ps = cache.shape[1]
    flat = cache.reshape(-1, *cache.shape[2:])
    return bf16_to_f64(flat[request_slots(page_table_row, n, ps)])


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """K/V head read by query head h (consecutive query heads share one)."""
    return h // (num_q_heads // num_kv_heads)


def visible(first_pos: int, num_rows: int, num_keys: int) -> np.ndarray:
    """Bool ``[num_rows, num_keys]``: row i (absolute position first_pos + i)
    sees key j iff j <= first_pos + i."""
    rows = first_pos + np.arange(num_rows)[:, None]
    return np.arange(num_keys)[None, :] <= rows


def attend(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray,
           first_pos: int, scale: float) -> np.ndarray:
    """softmax(scale * q k^T, causal) v for rows at positions first_pos...
    q_rows ``[L, d]``, k/v ``[n, d]``; returns ``[L, d]`` float64."""
    s = (q_rows @ k.T) * scale
    s = np.where(visible(first_pos, q_rows.shape[0], k.shape[0]), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return (e / e.sum(axis=1, keepdims=True)) @ v


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
           page_table: np.ndarray, seq_lens: np.ndarray, scale: float,
           requests: Optional[Iterable[int]] = None,
           heads: Optional[Iterable[int]] = None) -> np.ndarray:
    """One query per request (``q`` ``[B, Hq, d]`` bf16 bits) attending to
    all ``seq_lens[r]`` tokens.  Returns ``[B, Hq, d]`` float64; entries of
    requests/heads not asked for are NaN."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    out = np.full((B, Hq, d), np.nan)
    reqs = range(B) if requests is None else requests
    hs = list(range(Hq)) if heads is None else list(heads)
    for r in reqs:
        n = int(seq_lens[r])
        kr = gather(k_cache, page_table[r], n)
        vr = gather(v_cache, page_table[r], n)
        qr = bf16_to_f64(q[r])
        for h in hs:
            kvh = kv_head_of(h, Hq, Hkv)
            out[r, h] = attend(qr[h][None, :], kr[:, kvh], vr[:, kvh], n - 1, scale)[0]
    return out


def prefill(q: np.ndarray, cu_seqlens_q: np.ndarray, prefix_lens: np.ndarray,
            k_cache: np.ndarray, v_cache: np.ndarray, page_table: np.ndarray,
            scale: float, requests: Optional[Iterable[int]] = None,
            heads: Optional[Iterable[int]] = None,
            rows: Optional[dict] = None) -> np.ndarray:
    """Flat ragged queries ``q`` ``[T, Hq, d]`` (bf16 bits); request r owns
    rows ``cu_seqlens_q[r] .. cu_seqlens_q[r+1]`` at positions
    ``prefix_lens[r] + i`` and attends causally to its pool rows, which must
    already hold the new tokens.  ``rows`` optionally maps a request to the
    subset of its local row indices to compute.  Returns ``[T, Hq, d]``
    float64 with NaN where nothing was asked for."""
    T, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    out = np.full((T, Hq, d), np.nan)
    B = len(prefix_lens)
    reqs = range(B) if requests is None else requests
    hs = list(range(Hq)) if heads is None else list(heads)
    for r in reqs:
        s0, s1 = int(cu_seqlens_q[r]), int(cu_seqlens_q[r + 1])
        L = s1 - s0
        if L <= 0:
            continue
        P = int(prefix_lens[r])
        n = P + L
        kr = gather(k_cache, page_table[r], n)
        vr = gather(v_cache, page_table[r], n)
        qr = bf16_to_f64(q[s0:s1])
        sel = np.arange(L) if rows is None or r not in rows else np.asarray(rows[r])
        for h in hs:
            kvh = kv_head_of(h, Hq, Hkv)
            for i in sel:
                out[s0 + i, h] = attend(qr[i, h][None, :], kr[:, kvh], vr[:, kvh],
                                        P + int(i), scale)[0]
    return out


def prefill_dense(q: np.ndarray, cu_seqlens_q: np.ndarray, prefix_lens: np.ndarray,
                  k_cache: np.ndarray, v_cache: np.ndarray, page_table: np.ndarray,
                  scale: float, heads: Optional[Iterable[int]] = None) -> np.ndarray:
    """Same result as ``prefill`` for all rows of the given heads, computed
    one [L, n] score block per (request, head) instead of row by row."""
    T, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    out = np.full((T, Hq, d), np.nan)
    for r in range(len(prefix_lens)):
        s0, s1 = int(cu_seqlens_q[r]), int(cu_seqlens_q[r + 1])
        L = s1 - s0
        if L <= 0:
            continue
        P = int(prefix_lens[r])
        kr = gather(k_cache, page_table[r], P + L)
        vr = gather(v_cache, page_table[r], P + L)
        qr = bf16_to_f64(q[s0:s1])
        for h in (range(Hq) if heads is None else heads):
            kvh = kv_head_of(h, Hq, Hkv)
            out[s0:s1, h] = attend(qr[:, h], kr[:, kvh], vr[:, kvh], P, scale)
    return out


def decode_multi(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 page_table: np.ndarray, seq_lens: np.ndarray, scale: float) -> np.ndarray:
    """``q`` ``[B, L, Hq, d]`` (bf16 bits): new token t of request r sits at
    position ``seq_lens[r] - L + t`` and attends causally to the pool rows up
    to there (step 6).  Returns ``[B, L, Hq, d]`` float64; rows with no
    visible key, and every row of a request with ``seq_lens[r] <= 0``, are
    zero."""
    B, L, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    out = np.zeros((B, L, Hq, d))
    for r in range(B):
        n = int(seq_lens[r])
        if n <= 0:
            continue
        first = n - L                     # position of new token 0
        t0 = max(0, -first)               # first token with a non-negative position
        kr = gather(k_cache, page_table[r], n)
        vr = gather(v_cache, page_table[r], n)
        qr = bf16_to_f64(q[r, t0:])
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            out[r, t0:, h] = attend(qr[:, h], kr[:, kvh], vr[:, kvh], first + t0, scale)
    return out
