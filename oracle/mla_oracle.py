"""fp64 CPU oracle for MLA paged decode with split-K segments and their merge.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never calls it; it works from the encoded input bits a
workload holds and nothing else.

Pages followed (cited by page title and the section on it):

* [merge page] vLLM API page "vllm.v1.attention.ops.rocm_aiter_mla_merge":
  module description (segment partition ``tiles_per_segment = cdiv(seq_len,
  NUM_SEGMENTS * TILE_SIZE)``; partials are base 2; the merge returns a
  natural-log LSE) and ``merge_mla_segments_triton`` (shapes
  [T, H, S, 512] -> out [T, H, 512] + lse [T, H] fp32, LOGE2 conversion).
* [sparse page] vLLM API page "vllm.v1.attention.backends.mla.rocm_aiter_mla_sparse":
  ``ROCMAiterMLASparseImpl._forward_mla`` tail (sink post-merge: empty rows get
  LSE -inf before ``logaddexp`` with the sink and output 0; otherwise output is
  scaled by ``exp(lse - sink_lse)``), and ``triton_convert_req_index_to_global_index``
  (global row = ``block_table[req, j // B] * B + j % B``).
* [backend page] source page "rocm_aiter_mla.py" (vLLM AITER MLA backend):
  ``_segmented_mla_page_size`` (TILE = min(128, largest power-of-two divisor of
  the block)), ``_fill_dcp_verify_page_table`` (a block is viewed as
  block/TILE subpages: subpage id = block * (block/TILE) + offset),
  ``dcp_local_verify_row_lens`` (row t of a qlen-token block sees positions
  [0, seq_len - qlen + t]), ``_forward_segmented_dcp_verify`` (q = [q_nope ||
  q_pe], kv_lora_rank 512 + rope 64, ``kv_descale`` multiplies the cache) and
  the ``AiterMLAImpl`` class note (segment statistics are base 2, converted
  with LOGE2; the returned LSE is natural log).

Readings where the pages are silent are listed with each function.  Every
float computation runs in float64 on values decoded from the stored codes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

HEAD_DIM = 576
KV_LORA_RANK = 512
LOG2E = 1.0 / math.log(2.0)  # log2(e)
LOGE2 = math.log(2.0)  # ln(2): converts a base-2 LSE to natural log
FP8_E4M3_MAX = 448.0  # largest finite OCP e4m3fn value


# ---------------------------------------------------------------------------
# Code decoding (the cache and q arrive as bf16 bits or fp8-e4m3fn bytes).
# ---------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an IEEE binary32: widen the 16 bits and read
    them as a float32, which is exact in float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    """OCP 8-bit float E4M3 ("fn": finite, no infinities).

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0
    holds subnormals m/8 * 2^-6; S.1111.111 is the only NaN pattern, so
    S.1111.110 = 1.75 * 2^8 = 448 is the largest finite value.
    """
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode(codes: np.ndarray, dtype: str, scale: Optional[float]) -> np.ndarray:
    """Stored code -> real value.  Dequantisation is value x scale, the way the
    backend page passes ``kv_descale`` / q scales (scale None means 1)."""
    if dtype == "bf16":
        v = decode_bf16(codes)
    elif dtype == "fp8_e4m3":
        v = decode_e4m3fn(codes)
    else:
        raise ValueError(dtype)
    if scale is not None:
        v = v * float(scale)
    return v


def quantize_e4m3(values: np.ndarray, scale: Optional[float]) -> np.ndarray:
    """[sparse page] ``forward_mqa``, fp8 branch: the bf16 q (ql_nope || q_pe)
    is quantised with the layer's q scale before the decode, and the scale
    later dequantises it.  The page does not print the quantiser.  Reading:
    divide by the scale in IEEE single precision, saturate at +-448, round to
    the nearest e4m3 code (ties to even), which torch's float8_e4m3fn cast
    does.  The code is an integer decision, so it is taken in the precision the
    library's q load uses (single).  Returns uint8 codes."""
    s = np.float32(1.0 if scale is None else scale)
    y = np.asarray(values, dtype=np.float32) / s
    y = np.where(np.isnan(y), y, np.clip(y, -FP8_E4M3_MAX, FP8_E4M3_MAX)).astype(np.float32)
    return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------------------
# Partitioning (integers, exact).
# ---------------------------------------------------------------------------

def largest_pow2_divisor(n: int) -> int:
    if n <= 0:
        raise ValueError("block size must be positive")
    p = 1
    while n % (2 * p) == 0:
        p *= 2
    return p


def tile_size_for_block(block_size: int) -> int:
    """[backend page] ``_segmented_mla_page_size``: the largest power of two
    that divides the block, capped at 128."""
    return min(128, largest_pow2_divisor(block_size))


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def tiles_per_segment(seq_len: int, num_segments: int, tile_size: int) -> int:
    """[merge page] module description: cdiv(seq_len, NUM_SEGMENTS * TILE_SIZE)."""
    return cdiv(seq_len, num_segments * tile_size)


def segment_bounds(seq_len: int, num_segments: int, tile_size: int) -> list[tuple[int, int]]:
    """Key ranges [start, end) of the segments that hold at least one position.

    Reading (the pages give the tile count per segment only): segment s covers
    tiles [s*tps, (s+1)*tps) of the request, clipped to seq_len; a segment whose
    first position is >= seq_len is not valid and is skipped.  seq_len == 0
    has no valid segment.
    """
    if num_segments < 1 or tile_size < 1:
        raise ValueError("num_segments and tile_size must be >= 1")
    if seq_len <= 0:
        return []
    span = tiles_per_segment(seq_len, num_segments, tile_size) * tile_size
    out = []
    for s in range(num_segments):
        a = s * span
        if a >= seq_len:
            break
        out.append((a, min(a + span, seq_len)))
    return out


def visible_len(seq_len: int, qlen: int, i: int, causal: bool) -> int:
    """[backend page] ``dcp_local_verify_row_lens``: with a causal mask, the
    i-th of a request's qlen new tokens sees positions [0, seq_len - qlen + i],
    its own included (clamped at 0).  Without the mask every row sees all
    seq_len positions."""
    if not causal:
        return seq_len
    return max(0, seq_len - qlen + i + 1)


def cache_row_index(block_table_row: np.ndarray, j: int, block_size: int) -> int:
    """[sparse page] ``triton_convert_req_index_to_global_index``: logical
    position j lives at row block_table[req, j // B] * B + j % B of the flattened
    cache."""
    return int(block_table_row[j // block_size]) * block_size + j % block_size


def subpage_table(block_table: np.ndarray, block_size: int, tile_size: int) -> np.ndarray:
    """[backend page] ``_fill_dcp_verify_page_table``: view each physical block
    as block/TILE subpages of TILE rows; subpage id = block * (block/TILE) + k."""
    ppb = block_size // tile_size
    bt = np.asarray(block_table, dtype=np.int64)
    return (bt[:, :, None] * ppb + np.arange(ppb)[None, None, :]).reshape(bt.shape[0], -1)


def pages_of(block_table: np.ndarray, bt_indptr: Optional[np.ndarray], r: int) -> np.ndarray:
    """Request r's page list: row r of a [R, max_blocks] table, or with
    ``bt_indptr`` the slice [bt_indptr[r], bt_indptr[r+1]) of a flat list.
    With page size 1 the flat form is the per-token index stream of [sparse
    page] ``_forward_mla`` (``paged_kv_indptr`` / ``paged_kv_indices`` over a
    [rows, 1, 576] cache view)."""
    if bt_indptr is None:
        return block_table[r]
    return block_table[int(bt_indptr[r]):int(bt_indptr[r + 1])]


def gather_rows(kv_flat: np.ndarray, block_table_row: np.ndarray, n: int,
                block_size: int) -> np.ndarray:
    """Rows of the first n positions of one request, in logical order."""
    idx = np.array([cache_row_index(block_table_row, j, block_size) for j in range(n)],
                   dtype=np.int64)
    return kv_flat[idx] if n else np.zeros((0, kv_flat.shape[-1]), dtype=kv_flat.dtype)


# ---------------------------------------------------------------------------
# The result itself: plain softmax attention over the gathered rows.
# ---------------------------------------------------------------------------

def attend(q: np.ndarray, rows: np.ndarray, scale: float,
           sink: Optional[np.ndarray] = None) -> tuple[np.ndarray, np.ndarray]:
    """Softmax attention of query rows q [M, 576] over key rows [n, 576].

    score_j = scale * (q . row_j) over all 576 dims, V_j = row_j[:512]
    (the latent part of the same row).  Returns O [M, 512] and the natural-log
    LSE [M] = ln sum_j e^score_j.

    Sinks ([sparse page] ``_forward_mla``): a per-row logit sigma that joins the
    softmax denominator with a zero value vector: LSE = ln(sum e^s + e^sigma),
    O = sum_j e^(s_j - LSE) V_j.  With no key: O = 0 and LSE = -inf, or sigma
    when a sink is present.
    """
    M = q.shape[0]
    n = rows.shape[0]
    out = np.zeros((M, KV_LORA_RANK), dtype=np.float64)
    lse = np.full(M, -np.inf, dtype=np.float64)
    if n:
        s = scale * (q @ rows.T)  # [M, n]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1)
        lse = m[:, 0] + np.log(z)
        out = (e @ rows[:, :KV_LORA_RANK]) / z[:, None]
    if sink is not None:
        sink = np.broadcast_to(np.asarray(sink, dtype=np.float64), (M,))
        new_lse = np.logaddexp(lse, sink)
        factor = np.where(np.isfinite(lse), np.exp(lse - new_lse), 0.0) if n else np.zeros(M)
        out = out * factor[:, None]
        lse = new_lse
    return out, lse


@dataclass
class DecodedBatch:
    """Float64 view of a workload: q [T, H, 576], flattened cache [rows, 576]."""

    q: np.ndarray
    kv_flat: np.ndarray
    block_table: np.ndarray
    bt_indptr: Optional[np.ndarray]
    seq_lens: np.ndarray
    qo_indptr: np.ndarray
    block_size: int
    scale: float
    causal: bool
    sinks: Optional[np.ndarray]


def decode_workload(w, reqs: Optional[Sequence[int]] = None) -> DecodedBatch:
    """Decode a workload's codes to float64.  With ``reqs`` only the cache rows
    those requests reach are decoded (the rest stay 0) to bound memory."""
    kv = np.asarray(w.kv_cache)
    nb, bsz, d = kv.shape
    if reqs is None:
        kv_flat = decode(kv.reshape(-1, d), w.kv_dtype, w.kv_scale)
    else:
        kv_flat = np.zeros((nb * bsz, d), dtype=np.float64)
        flat = kv.reshape(-1, d)
        for r in reqs:
            n = int(w.seq_lens[r])
            if n == 0:
                continue
            pages = pages_of(np.asarray(w.block_table), w.bt_indptr, r)
            idx = np.array([cache_row_index(pages, j, bsz) for j in range(n)])
            kv_flat[idx] = decode(flat[idx], w.kv_dtype, w.kv_scale)
    if w.q_dtype == "bf16" and w.kv_dtype == "fp8_e4m3":
        # bf16 q with an fp8 cache: quantised first (the fused q prologue)
        q = decode(quantize_e4m3(decode_bf16(np.asarray(w.q)), w.q_scale), "fp8_e4m3", w.q_scale)
    else:
        q = decode(np.asarray(w.q), w.q_dtype, w.q_scale)
    return DecodedBatch(q=q, kv_flat=kv_flat, block_table=np.asarray(w.block_table),
                        bt_indptr=None if w.bt_indptr is None else np.asarray(w.bt_indptr),
                        seq_lens=np.asarray(w.seq_lens), qo_indptr=np.asarray(w.qo_indptr),
                        block_size=bsz, scale=float(w.softmax_scale), causal=bool(w.causal),
                        sinks=None if w.sinks is None else np.asarray(w.sinks, np.float64))


def mla_decode(w, reqs: Optional[Sequence[int]] = None,
               db: Optional[DecodedBatch] = None) -> tuple[np.ndarray, np.ndarray]:
    """Direct definition: per query row, softmax attention over its visible
    positions.  Returns O [T, H, 512] and natural-log LSE [T, H] (float64).
    With ``reqs`` only those requests' tokens are filled (others stay NaN)."""
    db = db or decode_workload(w, reqs)
    T, H, _ = db.q.shape
    out = np.full((T, H, KV_LORA_RANK), np.nan)
    lse = np.full((T, H), np.nan)
    R = db.seq_lens.shape[0]
    for r in (range(R) if reqs is None else reqs):
        t0, t1 = int(db.qo_indptr[r]), int(db.qo_indptr[r + 1])
        qlen = t1 - t0
        L = int(db.seq_lens[r])
        rows = gather_rows(db.kv_flat, pages_of(db.block_table, db.bt_indptr, r), L, db.block_size)
        for i in range(qlen):
            n = visible_len(L, qlen, i, db.causal)
            o, l = attend(db.q[t0 + i], rows[:n], db.scale, db.sinks)
            out[t0 + i] = o
            lse[t0 + i] = l
    return out, lse


# ---------------------------------------------------------------------------
# Segment mode: base-2 partials per segment, then the merge.
# ---------------------------------------------------------------------------

def segment_partials(q: np.ndarray, rows: np.ndarray, scale: float, start: int, end: int,
                     n_visible: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Base-2 partials of one segment for query rows q [M, 576].

    Reading of "base-2 segment partials" ([merge page]; LOGE2 converts them):
    x_j = scale * log2(e) * (q . row_j); over the visible positions of
    [start, end): m = max_j x_j, l = sum_j 2^(x_j - m) and an *unnormalised*
    acc = sum_j 2^(x_j - m) * V_j.  A segment with no visible position yields
    (acc 0, m -inf, l 0).
    """
    M = q.shape[0]
    hi = min(end, n_visible)
    if hi <= start:
        return (np.zeros((M, KV_LORA_RANK)), np.full(M, -np.inf), np.zeros(M))
    seg = rows[start:hi]
    x = (scale * LOG2E) * (q @ seg.T)
    m = x.max(axis=1)
    p = np.exp2(x - m[:, None])
    return p @ seg[:, :KV_LORA_RANK], m, p.sum(axis=1)


def mla_decode_segments(w, num_segments: int, tile_size: int,
                        reqs: Optional[Sequence[int]] = None,
                        db: Optional[DecodedBatch] = None):
    """Per-segment partials for every query row.

    The partition of a request is the one its seq_len gives (one set of bounds
    for all of its qlen rows); rows with a causal window see a prefix of it.
    Returns (segm_output [T,H,S,512], segm_max [T,H,S], segm_expsum [T,H,S],
    valid [T,S] bool, part_lens [T] int).  Slots of invalid segments are NaN.
    """
    db = db or decode_workload(w, reqs)
    T, H, _ = db.q.shape
    S = num_segments
    so = np.full((T, H, S, KV_LORA_RANK), np.nan)
    sm = np.full((T, H, S), np.nan)
    se = np.full((T, H, S), np.nan)
    valid = np.zeros((T, S), dtype=bool)
    part_lens = np.zeros(T, dtype=np.int64)
    R = db.seq_lens.shape[0]
    for r in (range(R) if reqs is None else reqs):
        t0, t1 = int(db.qo_indptr[r]), int(db.qo_indptr[r + 1])
        qlen = t1 - t0
        L = int(db.seq_lens[r])
        rows = gather_rows(db.kv_flat, pages_of(db.block_table, db.bt_indptr, r), L, db.block_size)
        bounds = segment_bounds(L, S, tile_size)
        for i in range(qlen):
            t = t0 + i
            part_lens[t] = L
            n = visible_len(L, qlen, i, db.causal)
            for s, (a, b) in enumerate(bounds):
                acc, m, l = segment_partials(db.q[t], rows, db.scale, a, b, n)
                so[t, :, s] = acc
                sm[t, :, s] = m
                se[t, :, s] = l
                valid[t, s] = True
    return so, sm, se, valid, part_lens


def merge_segments(segm_output: np.ndarray, segm_max: np.ndarray, segm_expsum: np.ndarray,
                   part_lens: np.ndarray, tile_size: int,
                   sinks: Optional[np.ndarray] = None) -> tuple[np.ndarray, np.ndarray]:
    """[merge page] ``merge_mla_segments_triton`` + [sparse page] sink tail.

    Per (t, h), over the valid segments of part_lens[t] (the partition the
    decode used): M = max_s m_s, L = sum_s l_s 2^(m_s - M),
    O = sum_s acc_s 2^(m_s - M) / L, LSE = LOGE2 * (M + log2 L).  A row whose
    segments hold no key (M = -inf) gets O = 0, LSE = -inf.  Then the optional
    per-head sink sigma: LSE' = logaddexp(LSE, sigma), O' = O e^(LSE - LSE'),
    and rows without keys keep O' = 0.  Only valid slots are read.
    """
    T, H, S, D = segm_output.shape
    out = np.zeros((T, H, D))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        nv = len(segment_bounds(int(part_lens[t]), S, tile_size))
        if nv == 0:
            continue
        m = segm_max[t, :, :nv]
        M = m.max(axis=1)
        has = np.isfinite(M)
        Msafe = np.where(has, M, 0.0)
        w8 = np.where(np.isfinite(m), np.exp2(m - Msafe[:, None]), 0.0)  # [H, nv]
        Lsum = (segm_expsum[t, :, :nv] * w8).sum(axis=1)
        acc = np.einsum("hs,hsd->hd", w8, segm_output[t, :, :nv])
        with np.errstate(divide="ignore", invalid="ignore"):
            o = np.where(has[:, None], acc / np.where(has, Lsum, 1.0)[:, None], 0.0)
            l = np.where(has, LOGE2 * (Msafe + np.log2(np.where(has, Lsum, 1.0))), -np.inf)
        out[t] = o
        lse[t] = l
    if sinks is not None:
        sg = np.asarray(sinks, dtype=np.float64)[None, :]
        new = np.logaddexp(lse, sg)
        has = np.isfinite(lse)
        factor = np.where(has, np.exp(np.where(has, lse, 0.0) - new), 0.0)
        out = np.where(has[:, :, None], out * factor[:, :, None], 0.0)
        lse = new
    return out, lse


def mla_decode_via_segments(w, num_segments: int, tile_size: int,
                            reqs: Optional[Sequence[int]] = None):
    """Segment mode end to end: partials of every valid segment, then merge."""
    so, sm, se, valid, part_lens = mla_decode_segments(w, num_segments, tile_size, reqs)
    return merge_segments(so, sm, se, part_lens, tile_size,
                          None if w.sinks is None else np.asarray(w.sinks, np.float64))


# ---------------------------------------------------------------------------
# Decode context parallelism: the LSE combine of key shards.
# ---------------------------------------------------------------------------

def combine_lse(shard_out: np.ndarray, shard_lse: np.ndarray,
                sinks: Optional[np.ndarray] = None) -> tuple[np.ndarray, np.ndarray]:
    """[backend page] DCP decode routing note (each rank attends over its
    round-robin shard of the keys; partial outputs are merged across ranks by
    LSE) and [merge page] module description (the natural-log LSE is what that
    cross-rank merge consumes).

    Shard w saw a disjoint subset of a row's keys and returned its softmax
    output O_w and natural LSE_w = ln sum_{j in w} e^{s_j}.  Over the union:
    LSE = ln sum_w e^{LSE_w} and O = sum_w O_w e^{LSE_w - LSE} (each O_w is
    its shard's sum_j e^{s_j - LSE_w} V_j).  Shards with LSE_w = -inf hold no
    key and add nothing.  The sink joins once, after the union, as in
    ``attend``.  shard_out [W, T, H, 512], shard_lse [W, T, H].
    """
    so = np.asarray(shard_out, dtype=np.float64)
    sl = np.asarray(shard_lse, dtype=np.float64)
    W, T, H, D = so.shape
    out = np.zeros((T, H, D))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        for h in range(H):
            ls = sl[:, t, h]
            if np.isnan(ls).any():
                out[t, h] = np.nan
                lse[t, h] = np.nan
                continue
            fin = np.isfinite(ls)
            if not fin.any():
                continue
            M = ls[fin].max()
            total = M + math.log(sum(math.exp(x - M) for x in ls[fin]))
            lse[t, h] = total
            out[t, h] = sum(so[w, t, h] * math.exp(ls[w] - total) for w in range(W) if fin[w])
    if sinks is not None:
        sk = np.asarray(sinks, dtype=np.float64)
        for t in range(T):
            for h in range(H):
                if np.isnan(lse[t, h]):
                    continue
                new = np.logaddexp(lse[t, h], sk[h])
                out[t, h] *= math.exp(lse[t, h] - new) if np.isfinite(lse[t, h]) else 0.0
                lse[t, h] = new
    return out, lse


# ---------------------------------------------------------------------------
# Byte accounting used to express throughput in the pages' unit.
# ---------------------------------------------------------------------------

def kv_reference_bytes(seq_lens: Sequence[int], elem_bytes: int) -> int:
    """[PR page] "Pad the AITER MLA decode head count to a native tile",
    measurement note: the 1x KV reference is every request's rows read once,
    sum(seq_len) * 576 * element size."""
    return int(sum(int(x) for x in seq_lens)) * HEAD_DIM * int(elem_bytes)
