"""Seeded synthetic inputs for MLA paged decode.

This module only *makes* inputs: random numbers, their bf16 / fp8-e4m3
encodings, a paged pool, a block table and the per-request lengths.  It holds
none of the attention arithmetic, so both the fp64 oracle (``oracle/``) and
the HIP library (``mla_paged_decode_02_amd``) can consume the same workloads
without sharing any code that computes a result.

Layouts follow the problem statement of the AITER MLA backend pages:

* ``q``        [T, H, 576]  -- 512 latent (q_nope absorbed) + 64 rope dims.
* ``kv_cache`` [num_blocks, block_size, 576] -- one latent row per token
  (first 512 dims are also V).
* ``block_table`` int32 [num_reqs, max_blocks], ``seq_lens`` int32 [num_reqs],
  ``qo_indptr`` int32 [num_reqs + 1].

Encodings are returned as raw bits (numpy has no bf16 / fp8 type):
bf16 -> uint16, fp8-e4m3fn -> uint8.  Float-to-code rounding is done by
torch's CPU casts (round to nearest even); fp8 values are clamped to +-448
first so nothing saturates to NaN.

The five named workloads mirror the sizes the pages measure on (bs=52,
qlen=1, 16384 KV tokens per request) plus a tiny and a ragged case.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

HEAD_DIM = 576
KV_LORA_RANK = 512
ROPE_DIM = HEAD_DIM - KV_LORA_RANK
FP8_E4M3_MAX = 448.0

# Poison codes written into pages the kernel must never read.
BF16_NAN_BITS = 0x7FC0
FP8_E4M3_NAN_BYTE = 0x7F


@dataclass
class Workload:
    """One decode batch, fully described by host arrays (encoded bits)."""

    name: str
    num_heads: int
    block_size: int
    q_dtype: str  # "bf16" | "fp8_e4m3"
    kv_dtype: str  # "bf16" | "fp8_e4m3"
    q: np.ndarray  # [T, H, 576] uint16 (bf16 bits) or uint8 (e4m3 bytes)
    kv_cache: np.ndarray  # [num_blocks, block_size, 576] uint16 / uint8
    block_table: np.ndarray  # int32 [num_reqs, max_blocks]
    seq_lens: np.ndarray  # int32 [num_reqs]
    qo_indptr: np.ndarray  # int32 [num_reqs + 1]
    softmax_scale: float
    causal: bool = False
    q_scale: Optional[float] = None  # dequant multiplier (None -> 1.0)
    kv_scale: Optional[float] = None
    sinks: Optional[np.ndarray] = None  # float32 [H]
    bt_indptr: Optional[np.ndarray] = None  # int32 [R+1]: block_table is one flat page list
    tile_size: int = 0  # 0 -> largest pow2 divisor of block, capped at 128
    num_segments: int = 0  # 0 -> library planner decides
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def num_reqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_qlen(self) -> int:
        d = np.diff(self.qo_indptr)
        return int(d.max()) if d.size else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    def kv_bytes_touched(self) -> int:
        """Bytes of cache rows the batch must read once (the pages' 1x unit)."""
        esz = 2 if self.kv_dtype == "bf16" else 1
        return int(self.seq_lens.astype(np.int64).sum()) * HEAD_DIM * esz


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _encode(x: torch.Tensor, dtype: str) -> tuple[np.ndarray, Optional[float]]:
    """fp32 values -> (code array, per-tensor dequant scale or None)."""
    if dtype == "bf16":
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), None
    if dtype == "fp8_e4m3":
        amax = float(x.abs().max()) if x.numel() else 1.0
        scale = amax / FP8_E4M3_MAX if amax > 0 else 1.0
        y = (x / scale).clamp_(-FP8_E4M3_MAX, FP8_E4M3_MAX)
        return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), float(np.float32(scale))
    raise ValueError(f"unknown dtype {dtype}")


def _poison_code(dtype: str):
    return BF16_NAN_BITS if dtype == "bf16" else FP8_E4M3_NAN_BYTE


def make_workload(
    *,
    name: str,
    seq_lens,
    num_heads: int,
    block_size: int,
    dtype: str = "bf16",
    qlens=None,
    causal: bool = False,
    sinks: bool = False,
    softmax_scale: float = 1.0 / math.sqrt(192.0),
    tile_size: int = 0,
    num_segments: int = 0,
    seed: int = 0,
    poison: bool = True,
    shuffle_pool: bool = True,
    extra_bt_cols: int = 0,
    q_scale_override: Optional[float] = None,
) -> Workload:
    """Build a paged decode batch.

    * Every request's pages are drawn from one pool through a random
      permutation (``shuffle_pool``).
    * With ``poison`` one extra block filled with NaN codes is appended; the
      unused tail of each request's last page and every block-table entry past
      the request's last page are pointed at / filled with NaN.  A kernel that
      reads a row it should not read turns the output into NaN.
    * ``qlens`` gives the new query tokens per request (default 1).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    num_reqs = int(seq_lens.shape[0])
    if qlens is None:
        qlens = np.ones(num_reqs, dtype=np.int64)
    qlens = np.asarray(qlens, dtype=np.int64)
    assert qlens.shape == (num_reqs,)
    g = _gen(seed)

    pages_per_req = (seq_lens + block_size - 1) // block_size
    n_pages = int(pages_per_req.sum())
    max_blocks = max(int(pages_per_req.max()) if num_reqs else 0, 1) + extra_bt_cols
    num_blocks = n_pages + (1 if poison else 0)
    poison_block = n_pages  # index of the NaN block when poison=True

    # Values ~N(0,1): KV rows and queries.
    kv = torch.randn(num_blocks * block_size * HEAD_DIM, generator=g, dtype=torch.float32)
    kv = kv.view(num_blocks, block_size, HEAD_DIM)
    T = int(qlens.sum())
    q = torch.randn(T * num_heads * HEAD_DIM, generator=g, dtype=torch.float32)
    q = q.view(T, num_heads, HEAD_DIM)

    kv_codes, kv_scale = _encode(kv, dtype)
    q_codes, q_scale = _encode(q, dtype)
    if q_scale_override is not None:
        q_scale = q_scale_override
    del kv, q

    perm = torch.randperm(n_pages, generator=g).numpy() if shuffle_pool else np.arange(n_pages)
    fill = poison_block if poison else 0
    bt = np.full((num_reqs, max_blocks), fill, dtype=np.int32)
    cursor = 0
    for r in range(num_reqs):
        k = int(pages_per_req[r])
        bt[r, :k] = perm[cursor : cursor + k]
        cursor += k

    if poison:
        code = _poison_code(dtype)
        kv_codes[poison_block] = code
        for r in range(num_reqs):
            k = int(pages_per_req[r])
            tail = int(seq_lens[r]) - (k - 1) * block_size if k else 0
            if k and tail < block_size:
                kv_codes[bt[r, k - 1], tail:] = code

    qo = np.zeros(num_reqs + 1, dtype=np.int32)
    qo[1:] = np.cumsum(qlens)

    sink_arr = None
    if sinks:
        sink_arr = torch.randn(num_heads, generator=g, dtype=torch.float32).numpy()

    return Workload(
        name=name,
        num_heads=num_heads,
        block_size=block_size,
        q_dtype=dtype,
        kv_dtype=dtype,
        q=q_codes,
        kv_cache=kv_codes,
        block_table=bt,
        seq_lens=seq_lens.astype(np.int32),
        qo_indptr=qo,
        softmax_scale=float(softmax_scale),
        causal=causal,
        q_scale=q_scale,
        kv_scale=kv_scale,
        sinks=sink_arr,
        tile_size=tile_size,
        num_segments=num_segments,
        seed=seed,
        meta={"poison_block": poison_block if poison else None},
    )


# ---------------------------------------------------------------------------
# Named workloads.  Full sizes are those the decode measurements are quoted
# on (bs=52, qlen=1, 16384 KV tokens per request); ``scale`` < 1 shrinks the
# batch and context so the fp64 oracle finishes in seconds.
# ---------------------------------------------------------------------------

def as_ragged_pages(w: Workload) -> Workload:
    """The same batch with its page lists as one flat list plus offsets
    (``bt_indptr``): request r keeps exactly its cdiv(len, block) pages, so a
    read past its last page lands on the next request's pages (or, for the
    last one, past the list)."""
    B = w.block_size
    counts = [(int(L) + B - 1) // B for L in w.seq_lens]
    flat = np.concatenate([w.block_table[r, :c] for r, c in enumerate(counts)] +
                          [np.zeros(0, dtype=np.int32)]).astype(np.int32)
    ip = np.zeros(w.num_reqs + 1, dtype=np.int32)
    ip[1:] = np.cumsum(counts)
    return with_(w, block_table=flat, bt_indptr=ip, name=w.name + "-ragged-pages")


def sparse_batch(*, num_tokens: int, topk: int, ctx: int, num_heads: int, dtype: str = "bf16",
                 counts=None, sinks: bool = True, seed: int = 0,
                 name: Optional[str] = None) -> Workload:
    """Index-stream (sparse top-k) decode batch: token t belongs to a request
    with ``ctx`` cached positions and attends to ``counts[t]`` (default
    ``topk``) distinct positions of it, drawn at random.  The cache is a
    [num_tokens * ctx (+1 poison), 1, 576] view (page size 1) and the block
    table is the flat index stream with per-token offsets, as the sparse MLA
    page passes ``paged_kv_indptr`` / ``paged_kv_indices``."""
    g = _gen(seed)
    if counts is None:
        counts = [topk] * num_tokens
    counts = np.asarray(counts, dtype=np.int64)
    assert counts.shape == (num_tokens,) and (counts <= ctx).all()
    rows = num_tokens * ctx
    kv = torch.randn((rows + 1) * HEAD_DIM, generator=g, dtype=torch.float32).view(rows + 1, 1, HEAD_DIM)
    q = torch.randn(num_tokens * num_heads * HEAD_DIM, generator=g, dtype=torch.float32)
    q = q.view(num_tokens, num_heads, HEAD_DIM)
    kv_codes, kv_scale = _encode(kv, dtype)
    q_codes, q_scale = _encode(q, dtype)
    del kv, q
    kv_codes[rows] = _poison_code(dtype)
    lists = [(t * ctx + torch.randperm(ctx, generator=g)[: int(c)].numpy()).astype(np.int32)
             for t, c in enumerate(counts)]
    flat = np.concatenate(lists + [np.zeros(0, dtype=np.int32)]).astype(np.int32)
    ip = np.zeros(num_tokens + 1, dtype=np.int32)
    ip[1:] = np.cumsum(counts)
    sink_arr = torch.randn(num_heads, generator=g, dtype=torch.float32).numpy() if sinks else None
    return Workload(
        name=name or f"sparse_t{num_tokens}_top{topk}_ctx{ctx}_h{num_heads}_{dtype}",
        num_heads=num_heads, block_size=1, q_dtype=dtype, kv_dtype=dtype, q=q_codes,
        kv_cache=kv_codes, block_table=flat, seq_lens=counts.astype(np.int32),
        qo_indptr=np.arange(num_tokens + 1, dtype=np.int32), softmax_scale=1.0 / math.sqrt(192.0),
        q_scale=q_scale, kv_scale=kv_scale, sinks=sink_arr, bt_indptr=ip, seed=seed,
        meta={"poison_block": rows})


def sparse_bs52(num_heads: int = 16, dtype: str = "bf16", topk: int = 2048, ctx: int = 16384,
                bs: int = 52) -> Workload:
    """52 decode tokens, each attending to 2048 of its request's 16384 cached
    positions (a top-k index stream), sinks on."""
    return sparse_batch(num_tokens=bs, topk=topk, ctx=ctx, num_heads=num_heads, dtype=dtype,
                        sinks=True, seed=6 if dtype == "bf16" else 7)


def dcp_shards(w: Workload, num_shards: int) -> list:
    """Key shards of a batch as decode context parallelism lays them out:
    position t of a request lives on shard t % W at local position t // W,
    in local pages of the same block size (a fresh random page permutation
    per shard, NaN-poisoned tails).  Shards carry no sinks (the combine
    applies them once).

    Plain route (qlen 1, or no causal mask): the shard keeps the batch's
    requests, each with its local key count.  Causal blocks of qlen > 1 take
    the segmented route of the backend page's DCP routing note: every query
    token becomes its own one-token request whose length is the number of
    local keys inside its causal window."""
    W = int(num_shards)
    B = w.block_size
    flat = w.kv_cache.reshape(-1, HEAD_DIM)
    qo = np.asarray(w.qo_indptr)
    qlens = np.diff(qo)
    segmented = bool(w.causal) and w.num_reqs > 0 and int(qlens.max()) > 1
    shards = []
    g = _gen(w.seed + 77)
    for s in range(W):
        local = [max(0, -(-(int(L) - s) // W)) for L in w.seq_lens]   # keys t < L with t % W == s
        pages = [(n + B - 1) // B for n in local]
        n_pages = int(sum(pages))
        perm = torch.randperm(n_pages, generator=g).numpy() if n_pages else np.zeros(0, dtype=np.int64)
        cache = np.empty((n_pages + 1, B, HEAD_DIM), dtype=w.kv_cache.dtype)
        cache[:] = _poison_code(w.kv_dtype)
        bt = np.full((w.num_reqs, max(max(pages, default=1), 1)), n_pages, dtype=np.int32)
        cur = 0
        for r in range(w.num_reqs):
            bt[r, :pages[r]] = perm[cur:cur + pages[r]]
            cur += pages[r]
            src_pages = w.block_table[r] if w.bt_indptr is None else \
                w.block_table[int(w.bt_indptr[r]):int(w.bt_indptr[r + 1])]
            j = np.arange(local[r], dtype=np.int64)
            t = j * W + s
            src = np.asarray(src_pages, dtype=np.int64)[t // B] * B + t % B
            cache.reshape(-1, HEAD_DIM)[bt[r, j // B].astype(np.int64) * B + j % B] = flat[src]
        if not segmented:
            sw = replace(w, kv_cache=cache, block_table=bt, bt_indptr=None,
                         seq_lens=np.asarray(local, dtype=np.int32), sinks=None,
                         name=f"{w.name}-dcp{W}.{s}", meta={"poison_block": n_pages})
        else:
            T = w.num_tokens
            row_bt = np.empty((T, bt.shape[1]), dtype=np.int32)
            row_len = np.zeros(T, dtype=np.int32)
            for r in range(w.num_reqs):
                L, ql = int(w.seq_lens[r]), int(qlens[r])
                for i in range(ql):
                    vis = max(0, L - ql + i + 1)              # global causal window of token i
                    row_len[qo[r] + i] = max(0, -(-(vis - s) // W))
                    row_bt[qo[r] + i] = bt[r]
            sw = replace(w, kv_cache=cache, block_table=row_bt, bt_indptr=None, seq_lens=row_len,
                         qo_indptr=np.arange(T + 1, dtype=np.int32), causal=False, sinks=None,
                         name=f"{w.name}-dcp{W}.{s}", meta={"poison_block": n_pages})
        shards.append(sw)
    return shards


def with_bf16_q(w: Workload, *, q_values: Optional[np.ndarray] = None, q_scale: Optional[float] = None,
                seed: int = 0) -> Workload:
    """The batch with its q handed over in bf16 while the cache stays fp8 (the
    q the MLA layer produces before its fp8 quantisation).  Values ~N(0,1) by
    default; the q scale defaults to amax / 448 (a static per-tensor scale)."""
    assert w.kv_dtype == "fp8_e4m3"
    if q_values is None:
        q_values = torch.randn(w.q.shape, generator=_gen(seed + 313), dtype=torch.float32).numpy()
    qt = torch.from_numpy(np.ascontiguousarray(q_values, dtype=np.float32))
    codes = qt.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if q_scale is None:
        amax = float(qt.abs().max()) if qt.numel() else 1.0
        q_scale = float(np.float32(amax / FP8_E4M3_MAX)) if amax > 0 else 1.0
    return replace(w, q=codes, q_dtype="bf16", q_scale=q_scale, name=w.name + "-bf16q")


def tiny() -> Workload:
    """2 requests, lengths {100, 257}, 16 heads, bf16, page = TILE = 16, S = 4."""
    return make_workload(name="tiny", seq_lens=[100, 257], num_heads=16, block_size=16,
                         dtype="bf16", num_segments=4, seed=1, extra_bt_cols=0)


def uniform_batch(*, num_heads: int, dtype: str, block_size: int, bs: int = 52,
                  ctx: int = 16384, seed: int = 2, num_segments: int = 0,
                  poison: bool = False, name: Optional[str] = None) -> Workload:
    """bs requests of identical length ``ctx``, qlen = 1, random page permutation."""
    return make_workload(name=name or f"bs{bs}_ctx{ctx}_h{num_heads}_{dtype}_blk{block_size}",
                         seq_lens=[ctx] * bs, num_heads=num_heads, block_size=block_size,
                         dtype=dtype, seed=seed, num_segments=num_segments, poison=poison)


def bs52_h16_bf16(bs: int = 52, ctx: int = 16384) -> Workload:
    return uniform_batch(num_heads=16, dtype="bf16", block_size=64, bs=bs, ctx=ctx, seed=2)


def bs52_fp8(num_heads: int = 48, bs: int = 52, ctx: int = 16384) -> Workload:
    return uniform_batch(num_heads=num_heads, dtype="fp8_e4m3", block_size=64, bs=bs, ctx=ctx,
                         seed=3)


def bs52_h128_bf16(bs: int = 52, ctx: int = 16384) -> Workload:
    return uniform_batch(num_heads=128, dtype="bf16", block_size=256, bs=bs, ctx=ctx, seed=4)


def ragged_lengths(num_reqs: int, max_len: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Log-uniform lengths in [1, max_len] and qlen ~ U{1..4}; len >= qlen."""
    g = _gen(seed + 1000)
    u = torch.rand(num_reqs, generator=g, dtype=torch.float64).numpy()
    qlens = torch.randint(1, 5, (num_reqs,), generator=g).numpy().astype(np.int64)
    lens = np.rint(np.exp(u * math.log(max_len))).astype(np.int64)
    lens = np.clip(lens, np.maximum(1, qlens), max_len)
    return lens, qlens


def ragged_h96_fp8(num_reqs: int = 128, max_len: int = 32768, num_heads: int = 96,
                   seed: int = 5) -> Workload:
    """Ragged causal batch: log-uniform lengths, qlen 1..4, H=96, fp8, sinks."""
    lens, qlens = ragged_lengths(num_reqs, max_len, seed)
    return make_workload(name=f"ragged{num_reqs}_max{max_len}_h{num_heads}_fp8",
                         seq_lens=lens, qlens=qlens, num_heads=num_heads, block_size=64,
                         dtype="fp8_e4m3", causal=True, sinks=True, seed=seed, poison=True)


def with_(w: Workload, **kw) -> Workload:
    return replace(w, **kw)


def to_torch(w: Workload, device="cuda") -> dict:
    """Upload a workload's codes and metadata as device tensors (codes keep
    their bits: bf16 as torch.bfloat16, fp8 as torch.float8_e4m3fn)."""
    def codes(a: np.ndarray, dtype: str) -> torch.Tensor:
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dtype == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        else:
            t = t.view(torch.uint8).view(torch.float8_e4m3fn)
        return t.to(device)

    d = {
        "q": codes(w.q, w.q_dtype),
        "kv_cache": codes(w.kv_cache, w.kv_dtype),
        "block_table": torch.from_numpy(np.ascontiguousarray(w.block_table)).to(device),
        "bt_indptr": None if w.bt_indptr is None else torch.from_numpy(np.ascontiguousarray(w.bt_indptr)).to(device),
        "seq_lens": torch.from_numpy(np.ascontiguousarray(w.seq_lens)).to(device),
        "qo_indptr": torch.from_numpy(np.ascontiguousarray(w.qo_indptr)).to(device),
        "q_scale": None if w.q_scale is None else torch.tensor([w.q_scale], dtype=torch.float32, device=device),
        "kv_scale": None if w.kv_scale is None else torch.tensor([w.kv_scale], dtype=torch.float32, device=device),
        "sinks": None if w.sinks is None else torch.from_numpy(np.ascontiguousarray(w.sinks)).to(device),
    }
    return d


def call_args(w: Workload, d: dict, *, use_indptr: Optional[bool] = None) -> dict:
    """Keyword arguments for the library's decode entry points."""
    if use_indptr is None:
        use_indptr = w.max_qlen != 1 or w.num_tokens != w.num_reqs
    return dict(q=d["q"], kv_cache=d["kv_cache"], block_table=d["block_table"],
                seq_lens=d["seq_lens"], softmax_scale=w.softmax_scale,
                max_seq_len=w.max_seq_len, qo_indptr=d["qo_indptr"] if use_indptr else None,
                max_qlen=w.max_qlen if use_indptr else None, causal=w.causal,
                q_scale=d["q_scale"], kv_scale=d["kv_scale"], tile_size=w.tile_size,
                bt_indptr=d.get("bt_indptr"),
                sum_seq_lens=int(np.asarray(w.seq_lens, dtype=np.int64).sum()))
