"""Seeded synthetic inputs for paged-KV attention.

This module only builds inputs: request lengths, a shuffled assignment of
physical pages, the page table, the per-token write slots, and bf16 tensors
drawn from N(0, 1).  It holds none of the attention arithmetic, and both the
HIP path's tests and the CPU reference consume what it returns.

Shapes follow the pages' data structures:

* KV pool: one K and one V tensor per layer, each ``[num_pages, page_size,
  num_kv_heads, head_dim]`` (miniVLLM "Engine Architecture",
  section allocate_kv_cache).  A token's *slot* is its row in the flat
  ``[num_pages * page_size, num_kv_heads, head_dim]`` view.
* Page table: ``[num_seqs, width]`` int32, logical page -> physical page
  (mini-sglang "Engine Class", Key Attributes: page_table; miniVLLM
  "Engine Architecture", prepare_prefill / prepare_decode: block_tables).
* ``out_loc`` / slot mapping: the slot each new token's K/V row goes to
  (mini-sglang "Engine Class", forward_batch; miniVLLM prepare_* slot_mapping).
* Prefill: flat ragged queries with ``cu_seqlens_q`` and a cached prefix per
  request (miniVLLM prepare_prefill; zero-to-sglang Ch.1 section 3.3, cached
  length vs. sequence length).

Physical pages are a seeded permutation of a pool 1.25x the total need; one
extra "poison" page (id = pool size) fills the unused table entries.  Pages
nobody owns, the poison page, the unused tail of each request's last page,
and slots that a store is about to write are filled with NaN, so that any
read the method must not make shows up in the output.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# Named workloads.  Seeds are 1000 + the workload's position in the list.
WORKLOADS = {
    "tiny_decode": dict(
        kind="decode", num_seqs=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
        page_size=16, len_range=(64, 64), pool_pages=16, store_new=False,
        seed=1001),
    "llama_decode": dict(
        kind="decode", num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=64,
        page_size=16, len_range=(128, 2048), store_new=True, seed=1002),
    "qwen_decode": dict(
        kind="decode", num_seqs=128, num_q_heads=16, num_kv_heads=8, head_dim=128,
        page_size=256, len_range=(512, 8192), store_new=False, seed=1003),
    "chunked_prefill": dict(
        kind="prefill", num_seqs=16, num_q_heads=32, num_kv_heads=8, head_dim=64,
        page_size=16, prefix_range=(0, 1024), new_range=(64, 2048),
        max_new_total=16384, seed=1004),
    "long_decode": dict(
        kind="decode", num_seqs=16, num_q_heads=16, num_kv_heads=8, head_dim=128,
        page_size=16, len_range=(32768, 131072), store_new=False,
        outlier_frac=0.01, outlier_scale=8.0, seed=1005),
    # Llama-shaped decode whose requests share a 1024-token cached prefix:
    # the first 64 pages of every page table alias the same physical pages
    # (prefix caching), each request then continues with its own pages.
    "shared_prefix_decode": dict(
        kind="decode", num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=64,
        page_size=16, len_range=(1024 + 64, 1024 + 1024), shared_prefix=1024,
        store_new=True, seed=1006),
    # Llama-shaped decode feeding 4 tokens per request at once (speculative
    # decoding's verification step); the 4 tokens are already in the pool.
    "spec_decode": dict(
        kind="decode", num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=64,
        page_size=16, len_range=(128, 2048), q_len=4, store_new=False, seed=1007),
}

POOL_FACTOR = 1.25
_CHUNK = 1 << 26  # elements per randn draw when filling large pools


@dataclasses.dataclass
class Workload:
    """One batch of inputs.  Tensors live on ``device``; index arrays are
    also kept as numpy copies (``*_np``) for host-side use."""

    name: str
    kind: str                      # "decode" or "prefill"
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int                 # pool pages + 1 poison page
    poison_page: int
    scale: float
    seq_lens_np: np.ndarray        # [B] total tokens visible to the last query
    prefix_lens_np: np.ndarray     # [B] cached tokens (prefill); n - q_len (decode)
    q_lens_np: np.ndarray          # [B] new tokens per request
    page_table_np: np.ndarray      # [B, W]
    out_loc_np: Optional[np.ndarray]
    q: torch.Tensor                # [B, Hq, d] or [B, q_len, Hq, d] (decode); [T, Hq, d] (prefill)
    k_cache: torch.Tensor          # [num_pages, ps, Hkv, d] bf16
    v_cache: torch.Tensor
    k_new: Optional[torch.Tensor]  # [T_new, Hkv, d] bf16 rows to store
    v_new: Optional[torch.Tensor]
    out_loc: Optional[torch.Tensor]
    page_table: torch.Tensor
    seq_lens: torch.Tensor
    prefix_lens: torch.Tensor
    cu_seqlens_q: torch.Tensor     # [B+1]

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens_np.max()) if self.num_seqs else 0

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens_np.max()) if self.num_seqs else 0

    @property
    def num_tokens(self) -> int:
        return int(self.q_lens_np.sum())

    @property
    def width(self) -> int:
        return int(self.page_table_np.shape[1])

    def to(self, device) -> "Workload":
        """Copy of this workload with every tensor moved to ``device``."""
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Workload(**kw)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bfloat16 bit patterns of a tensor as a host uint16 array."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _randn_bf16(shape, gen: torch.Generator, device) -> torch.Tensor:
    """N(0,1) drawn in fp32 and rounded to bf16 (round-to-nearest-even),
    chunked so the fp32 staging buffer stays small."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device,
                                dtype=torch.float32).to(torch.bfloat16)
    return out


def _generator(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return g


def _assign_pages(rng: np.random.Generator, pages_needed: np.ndarray,
                  pool_pages: Optional[int], width: int, shared: int = 0):
    """Shuffle physical page ids and hand them to requests in order.  The
    first ``shared`` pages of every request are the same physical pages
    (a cached prefix shared by all of them); the rest are private.
    Returns (page_table [B, W], pool size, poison page id)."""
    if shared and (pages_needed <= shared).any():
        raise ValueError("every request needs a private page after the shared prefix")
    total = int(pages_needed.sum()) - shared * max(len(pages_needed) - 1, 0)
    if pool_pages is None:
        pool_pages = int(math.ceil(POOL_FACTOR * total))
    if pool_pages < total:
        raise ValueError("pool smaller than the pages requested")
    perm = rng.permutation(pool_pages).astype(np.int32)
    poison = pool_pages
    table = np.full((len(pages_needed), width), poison, dtype=np.int32)
    table[:, :shared] = perm[:shared]
    off = shared
    for r, k in enumerate(pages_needed):
        own = int(k) - shared
        table[r, shared:shared + own] = perm[off:off + own]
        off += own
    return table, pool_pages, poison


def _slot_rows(table_row: np.ndarray, positions: np.ndarray, ps: int) -> np.ndarray:
    """Flat pool row holding each logical position of one request: the slot
    a scheduler hands out (layout [num_pages, page_size, ...] flattened)."""
    return table_row[positions // ps].astype(np.int64) * ps + positions % ps


def _poison(cache: torch.Tensor, table: np.ndarray, seq_lens: np.ndarray,
            ps: int, pool_pages: int, extra_rows: Optional[np.ndarray]):
    """Fill with NaN everything no query may read: unowned pages, the poison
    page, tails of partly used pages and rows a store is about to write."""
    dev = cache.device
    owned = np.zeros(pool_pages + 1, dtype=bool)
    for r, n in enumerate(seq_lens):
        owned[table[r, :(int(n) + ps - 1) // ps]] = True
    unowned = np.nonzero(~owned)[0]
    nan = float("nan")
    if len(unowned):
        cache[torch.from_numpy(unowned).to(dev)] = nan
    flat = cache.view(-1, *cache.shape[2:])
    rows = []
    for r, n in enumerate(seq_lens):
        n = int(n)
        tail = (-n) % ps
        if tail:
            rows.append(_slot_rows(table[r], np.arange(n, n + tail), ps))
    if extra_rows is not None and len(extra_rows):
        rows.append(np.asarray(extra_rows, dtype=np.int64))
    if rows:
        idx = torch.from_numpy(np.concatenate(rows)).to(dev)
        flat[idx] = nan


def build_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                 seq_lens, *, seed, device="cpu", pool_pages=None, width=None,
                 store_new=False, outlier_frac=0.0, outlier_scale=8.0,
                 poison=True, name="custom_decode", shared_pages=0, q_len=1) -> Workload:
    """Decode batch: one query per request at position n_r - 1 attending to
    all n_r tokens.  With ``store_new`` the token at n_r - 1 is not yet in the
    pool: its K/V rows come in ``k_new``/``v_new`` with slots ``out_loc``.
    With ``q_len`` > 1, q is ``[B, q_len, Hq, d]``: the last q_len tokens of
    each request, all already in the pool."""
    assert q_len >= 1 and not (store_new and q_len > 1)
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert len(seq_lens) == num_seqs
    ps = page_size
    need = (seq_lens.astype(np.int64) + ps - 1) // ps
    if width is None:
        width = int(need.max()) if num_seqs else 1
    table, pool, poison_id = _assign_pages(rng, need, pool_pages, max(width, 1), shared_pages)
    gen = _generator(seed, device)
    shape = (pool + 1, ps, num_kv_heads, head_dim)
    k_cache = _randn_bf16(shape, gen, device)
    v_cache = _randn_bf16(shape, gen, device)
    q_shape = (num_seqs, num_q_heads, head_dim) if q_len == 1 else \
        (num_seqs, q_len, num_q_heads, head_dim)
    q = _randn_bf16(q_shape, gen, device)
    k_new = v_new = out_loc = out_loc_np = None
    if store_new:
        k_new = _randn_bf16((num_seqs, num_kv_heads, head_dim), gen, device)
        v_new = _randn_bf16((num_seqs, num_kv_heads, head_dim), gen, device)
        out_loc_np = np.array(
            [_slot_rows(table[r], np.array([int(seq_lens[r]) - 1]), ps)[0]
             for r in range(num_seqs)], dtype=np.int32)
    if outlier_frac > 0:
        # a row = one (slot, kv head) K vector; scaled after bf16 rounding,
        # which is exact (an exponent shift)
        mask = torch.rand(shape[0] * ps * num_kv_heads, generator=gen,
                          device=device) < outlier_frac
        kf = k_cache.view(-1, head_dim)
        kf[mask] = kf[mask] * outlier_scale
    if poison:
        _poison(k_cache, table, seq_lens, ps, pool, out_loc_np)
        _poison(v_cache, table, seq_lens, ps, pool, out_loc_np)
    if out_loc_np is not None:
        out_loc = torch.from_numpy(out_loc_np).to(device)
    prefix = np.maximum(seq_lens - q_len, 0).astype(np.int32)
    qlens = np.full(num_seqs, q_len, dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return Workload(
        name=name, kind="decode", seed=seed, num_seqs=num_seqs,
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        page_size=ps, num_pages=pool + 1, poison_page=poison_id,
        scale=1.0 / math.sqrt(head_dim), seq_lens_np=seq_lens,
        prefix_lens_np=prefix, q_lens_np=qlens, page_table_np=table,
        out_loc_np=out_loc_np, q=q, k_cache=k_cache, v_cache=v_cache,
        k_new=k_new, v_new=v_new, out_loc=out_loc,
        page_table=torch.from_numpy(table).to(device),
        seq_lens=torch.from_numpy(seq_lens).to(device),
        prefix_lens=torch.from_numpy(prefix).to(device),
        cu_seqlens_q=torch.from_numpy(cu).to(device))


def build_prefill(num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                  prefix_lens, q_lens, *, seed, device="cpu", pool_pages=None,
                  width=None, poison=True, name="custom_prefill") -> Workload:
    """Prefill batch with a cached prefix: request r has prefix_lens[r]
    tokens already in the pool and q_lens[r] new tokens whose K/V rows
    (``k_new``/``v_new``, flat ``[T, Hkv, d]``) go to slots ``out_loc``."""
    rng = np.random.default_rng(seed)
    prefix = np.asarray(prefix_lens, dtype=np.int32)
    qlens = np.asarray(q_lens, dtype=np.int32)
    seq_lens = (prefix + qlens).astype(np.int32)
    ps = page_size
    need = (seq_lens.astype(np.int64) + ps - 1) // ps
    if width is None:
        width = int(need.max()) if num_seqs else 1
    table, pool, poison_id = _assign_pages(rng, need, pool_pages, max(width, 1))
    gen = _generator(seed, device)
    shape = (pool + 1, ps, num_kv_heads, head_dim)
    T = int(qlens.sum())
    k_cache = _randn_bf16(shape, gen, device)
    v_cache = _randn_bf16(shape, gen, device)
    q = _randn_bf16((T, num_q_heads, head_dim), gen, device)
    k_new = _randn_bf16((T, num_kv_heads, head_dim), gen, device)
    v_new = _randn_bf16((T, num_kv_heads, head_dim), gen, device)
    out_loc_np = np.concatenate(
        [_slot_rows(table[r], np.arange(prefix[r], seq_lens[r]), ps)
         for r in range(num_seqs)] + [np.zeros(0, np.int64)]).astype(np.int32)
    if poison:
        _poison(k_cache, table, seq_lens, ps, pool, out_loc_np)
        _poison(v_cache, table, seq_lens, ps, pool, out_loc_np)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return Workload(
        name=name, kind="prefill", seed=seed, num_seqs=num_seqs,
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        page_size=ps, num_pages=pool + 1, poison_page=poison_id,
        scale=1.0 / math.sqrt(head_dim), seq_lens_np=seq_lens,
        prefix_lens_np=prefix, q_lens_np=qlens, page_table_np=table,
        out_loc_np=out_loc_np, q=q, k_cache=k_cache, v_cache=v_cache,
        k_new=k_new, v_new=v_new,
        out_loc=torch.from_numpy(out_loc_np).to(device),
        page_table=torch.from_numpy(table).to(device),
        seq_lens=torch.from_numpy(seq_lens).to(device),
        prefix_lens=torch.from_numpy(prefix).to(device),
        cu_seqlens_q=torch.from_numpy(cu).to(device))


def draw_lengths(name: str, seed: Optional[int] = None):
    """Request lengths of a named workload (integers, both ends inclusive).
    Decode: seq_lens.  Prefill: (prefix_lens, q_lens), the new-token vector
    redrawn whole until its sum fits ``max_new_total``."""
    cfg = WORKLOADS[name]
    seed = cfg["seed"] if seed is None else seed
    rng = np.random.default_rng(seed + 7919)
    B = cfg["num_seqs"]
    if cfg["kind"] == "decode":
        lo, hi = cfg["len_range"]
        return rng.integers(lo, hi + 1, size=B).astype(np.int32)
    plo, phi = cfg["prefix_range"]
    nlo, nhi = cfg["new_range"]
    prefix = rng.integers(plo, phi + 1, size=B).astype(np.int32)
    while True:
        qlens = rng.integers(nlo, nhi + 1, size=B).astype(np.int32)
        if int(qlens.sum()) <= cfg["max_new_total"]:
            return prefix, qlens


def make_workload(name: str, *, seed: Optional[int] = None, device="cpu",
                  poison: bool = True) -> Workload:
    """Build one of the named workloads."""
    cfg = WORKLOADS[name]
    seed = cfg["seed"] if seed is None else seed
    ps = cfg["page_size"]
    if cfg["kind"] == "decode":
        lens = draw_lengths(name, seed)
        width = -(-cfg["len_range"][1] // ps)
        return build_decode(
            cfg["num_seqs"], cfg["num_q_heads"], cfg["num_kv_heads"],
            cfg["head_dim"], ps, lens, seed=seed, device=device,
            pool_pages=cfg.get("pool_pages"), width=width,
            store_new=cfg["store_new"],
            outlier_frac=cfg.get("outlier_frac", 0.0),
            outlier_scale=cfg.get("outlier_scale", 8.0), poison=poison,
            name=name, shared_pages=cfg.get("shared_prefix", 0) // ps,
            q_len=cfg.get("q_len", 1))
    prefix, qlens = draw_lengths(name, seed)
    width = -(-(cfg["prefix_range"][1] + cfg["new_range"][1]) // ps)
    return build_prefill(
        cfg["num_seqs"], cfg["num_q_heads"], cfg["num_kv_heads"],
        cfg["head_dim"], ps, prefix, qlens, seed=seed, device=device,
        width=width, poison=poison, name=name)
