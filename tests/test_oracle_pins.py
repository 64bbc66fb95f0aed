"""Pins for the fp64 oracle: it is checked against things other than itself.

* number formats against torch's own casts and the OCP E4M3 definition,
* a pure-Python brute force on tiny batches (its own page walk, math.fsum),
* torch's scaled_dot_product_attention / logsumexp on an identity page table,
* closed forms (identical keys, one key, q = 0 integer counts, rope shift),
* partition invariance of segments + merge against the direct definition,
* the sink as an extra key with logit sigma and a zero value vector,
* invariances (request order, physical page relabelling, head subset),
* the causal window against shortened qlen = 1 decodes,
* the pages' printed 1x KV byte count.

All CPU-only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import mla_inputs as mi
from oracle import mla_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- formats ----

def test_e4m3_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.decode_e4m3fn(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e4m3_definition_points():
    # OCP 8-bit float spec: E4M3 bias 7, max 448 = S.1111.110, NaN = S.1111.111,
    # smallest subnormal 2^-9, smallest normal 2^-6, 1.0 = 0.0111.000.
    v = orc.decode_e4m3fn(np.array([0x7E, 0xFE, 0x01, 0x08, 0x38, 0x00, 0x80], np.uint8))
    assert list(v) == [448.0, -448.0, 2.0 ** -9, 2.0 ** -6, 1.0, 0.0, 0.0]
    assert math.isnan(orc.decode_e4m3fn(np.array([0x7F], np.uint8))[0])
    assert math.isnan(orc.decode_e4m3fn(np.array([0xFF], np.uint8))[0])


def test_bf16_decode_matches_torch_cast():
    g = torch.Generator().manual_seed(0)
    bits = torch.randint(0, 1 << 16, (4096,), generator=g, dtype=torch.int32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # no inf/nan patterns
    ref = bits.to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.decode_bf16(bits.numpy().astype(np.uint16))
    assert np.array_equal(ref, got)


def test_fp8_workload_dequant_within_half_ulp():
    w = mi.make_workload(name="f", seq_lens=[40], num_heads=2, block_size=8, dtype="fp8_e4m3",
                         seed=11, poison=False)
    kv = orc.decode(w.kv_cache, "fp8_e4m3", w.kv_scale)
    # The codes came from N(0,1) values / scale: the decoded magnitudes stay
    # inside +-448 * scale and are not all equal.
    assert np.abs(kv).max() <= 448 * w.kv_scale * (1 + 1e-12)
    assert np.unique(kv).size > 50


# ------------------------------------------------------------ partitioning ---

def test_tile_rule_closed_form():
    # largest power-of-two divisor, capped at 128
    cases = {1: 1, 2: 2, 16: 16, 48: 16, 64: 64, 96: 32, 128: 128, 256: 128, 544: 32, 1024: 128}
    for b, t in cases.items():
        assert orc.tile_size_for_block(b) == t
        assert b % t == 0 and (t & (t - 1)) == 0 and t <= 128


def test_segment_bounds_worked_examples():
    # len 100, S 4, TILE 16: tps = cdiv(100, 64) = 2 -> spans of 32 positions.
    assert orc.segment_bounds(100, 4, 16) == [(0, 32), (32, 64), (64, 96), (96, 100)]
    # len 257, S 4, TILE 16: tps = cdiv(257, 64) = 5 -> spans of 80.
    assert orc.segment_bounds(257, 4, 16) == [(0, 80), (80, 160), (160, 240), (240, 257)]
    # len 17, S 4, TILE 16: tps = 1 -> only two segments hold a position.
    assert orc.segment_bounds(17, 4, 16) == [(0, 16), (16, 17)]
    # 16384 positions, TILE 64, S 5: tps = cdiv(16384, 320) = 52 -> spans of 3328.
    b = orc.segment_bounds(16384, 5, 64)
    assert b[0] == (0, 3328) and b[-1] == (13312, 16384) and len(b) == 5
    assert orc.segment_bounds(0, 4, 16) == []


@pytest.mark.parametrize("tile", [1, 2, 4, 16, 64, 128])
@pytest.mark.parametrize("S", [1, 2, 3, 5, 8, 19, 64])
def test_segment_bounds_properties(tile, S):
    for L in [1, 2, 15, 16, 17, 63, 100, 257, 1000, 4097, 16384, 32768]:
        b = orc.segment_bounds(L, S, tile)
        assert 1 <= len(b) <= S
        assert b[0][0] == 0 and b[-1][1] == L
        for (a0, a1), (c0, _) in zip(b, b[1:]):
            assert a1 == c0
        span = orc.tiles_per_segment(L, S, tile) * tile
        for a0, a1 in b[:-1]:
            assert a1 - a0 == span and a0 % tile == 0
        # no valid segment is empty; the next (invalid) one would start at >= L
        assert all(a1 > a0 for a0, a1 in b)
        assert len(b) == S or len(b) * span >= L


def test_subpage_table_addresses_same_rows():
    bt = np.array([[5, 2, 7], [0, 3, 1]], np.int32)
    B, T = 256, 128
    sub = orc.subpage_table(bt, B, T)
    for r in range(2):
        for j in range(0, 3 * B, 37):
            direct = orc.cache_row_index(bt[r], j, B)
            via_sub = int(sub[r, j // T]) * T + j % T
            assert direct == via_sub


def test_kv_reference_bytes_matches_pr_page():
    g = json.load(open(os.path.join(GOLDEN, "pr54899_measurements.json")))
    wl = g["workload"]
    nbytes = orc.kv_reference_bytes([wl["kv_tokens_per_request"]] * wl["bs"], wl["kv_elem_bytes"])
    assert round(nbytes / 1e6, 2) == g["kv_reference_MB"]
    for h, rec in g["aiter_v0_1_19_fetch"].items():
        assert round(rec["fetch_MB"] * 1e6 / nbytes, 2) == pytest.approx(rec["x"], abs=0.006)


# ------------------------------------------------------------ brute force ----

def _brute_force(w):
    """Pure Python: expand each request's block table into flat row ids (one
    per position), then softmax with math.exp and math.fsum per query row."""
    kv = w.kv_cache.reshape(-1, w.kv_cache.shape[-1])
    dec = lambda codes, dt, sc: [float(x) for x in orc.decode(codes, dt, sc)]
    B = w.block_size
    out, lse = {}, {}
    for r in range(w.num_reqs):
        L = int(w.seq_lens[r])
        flat = []
        for blk in range((L + B - 1) // B):
            for off in range(B):
                if blk * B + off < L:
                    flat.append(int(w.block_table[r, blk]) * B + off)
        rows = [dec(kv[i], w.kv_dtype, w.kv_scale) for i in flat]
        t0, t1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        for t in range(t0, t1):
            n = L - (t1 - t0) + (t - t0) + 1 if w.causal else L
            n = max(n, 0)
            for h in range(w.num_heads):
                q = dec(w.q[t, h], w.q_dtype, w.q_scale)
                s = [w.softmax_scale * math.fsum(a * b for a, b in zip(q, rows[j])) for j in range(n)]
                terms = [math.exp(x) for x in s]
                if w.sinks is not None:
                    terms_all = terms + [math.exp(float(w.sinks[h]))]
                else:
                    terms_all = terms
                if not terms_all:
                    out[t, h] = [0.0] * 512
                    lse[t, h] = -math.inf
                    continue
                z = math.fsum(terms_all)
                lse[t, h] = math.log(z)
                out[t, h] = [math.fsum(terms[j] * rows[j][d] for j in range(n)) / z
                             for d in range(512)]
    return out, lse


@pytest.mark.parametrize("dtype,causal,sinks", [("bf16", False, False), ("bf16", True, True),
                                                 ("fp8_e4m3", True, False), ("fp8_e4m3", False, True)])
def test_oracle_matches_brute_force(dtype, causal, sinks):
    w = mi.make_workload(name="bf", seq_lens=[1, 5, 13, 0], qlens=[1, 2, 3, 1], num_heads=2,
                         block_size=4, dtype=dtype, causal=causal, sinks=sinks, seed=7,
                         softmax_scale=0.3)
    o, l = orc.mla_decode(w)
    bo, bl = _brute_force(w)
    for (t, h), v in bl.items():
        if math.isinf(v):
            assert l[t, h] == v
        else:
            assert abs(l[t, h] - v) <= 1e-12 * max(1, abs(v))
        assert np.max(np.abs(o[t, h] - np.array(bo[t, h]))) <= 1e-12


# ------------------------------------------------------- library special case

def test_oracle_matches_torch_sdpa_identity_table():
    w = mi.make_workload(name="sdpa", seq_lens=[300, 77], num_heads=8, block_size=16,
                         dtype="bf16", seed=3, poison=False, shuffle_pool=False)
    o, l = orc.mla_decode(w)
    kv = torch.from_numpy(orc.decode(w.kv_cache, "bf16", None)).reshape(-1, 576)
    q = torch.from_numpy(orc.decode(w.q, "bf16", None))
    start = 0
    for r, L in enumerate(w.seq_lens):
        L = int(L)
        # identity table: request r's pages are consecutive in the pool
        k = kv[start:start + L]
        start += ((L + 15) // 16) * 16
        qr = q[r:r + 1].transpose(0, 1)  # [H, 1, 576]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qr, k.expand(8, L, 576), k[:, :512].expand(8, L, 512).contiguous(),
            scale=w.softmax_scale)
        ref_lse = torch.logsumexp(w.softmax_scale * (qr[:, 0] @ k.T), dim=-1)
        assert np.max(np.abs(o[r] - ref[:, 0].numpy())) < 1e-12
        assert np.max(np.abs(l[r] - ref_lse.numpy())) < 1e-12


# -------------------------------------------------------------- closed forms

def _float_workload(rows_fn, L, H=4, scale=0.25, sinks=None, block=8, qlen=1, causal=False):
    """A workload whose cache rows are given as exact bf16 values."""
    w = mi.make_workload(name="cf", seq_lens=[L], qlens=[qlen], num_heads=H, block_size=block,
                         dtype="bf16", seed=5, causal=causal, softmax_scale=scale)
    flat = w.kv_cache.reshape(-1, 576)
    for j in range(L):
        flat[orc.cache_row_index(w.block_table[0], j, block)] = rows_fn(j)
    if sinks is not None:
        w.sinks = np.asarray(sinks, np.float32)
    return w


def _bf16_bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_identical_keys_closed_form():
    g = np.random.default_rng(0)
    row = _bf16_bits(g.standard_normal(576))
    L = 37
    sig = np.array([0.5, -1.0, 2.0, 0.0], np.float32)
    for sinks in (None, sig):
        w = _float_workload(lambda j: row, L, sinks=sinks)
        o, l = orc.mla_decode(w)
        v = orc.decode_bf16(row)
        q = orc.decode_bf16(w.q[0])
        s = w.softmax_scale * (q @ v)  # one score per head
        if sinks is None:
            assert np.allclose(l[0], np.log(L) + s, rtol=0, atol=1e-12)
            assert np.max(np.abs(o[0] - v[:512][None])) < 1e-12
        else:
            sg = sig.astype(np.float64)
            z = L * np.exp(s) + np.exp(sg)
            assert np.allclose(l[0], np.log(z), rtol=0, atol=1e-12)
            assert np.max(np.abs(o[0] - (L * np.exp(s) / z)[:, None] * v[:512][None])) < 1e-12


def test_single_key_closed_form():
    w = mi.make_workload(name="one", seq_lens=[1, 1], num_heads=3, block_size=2, dtype="bf16",
                         seed=9)
    o, l = orc.mla_decode(w)
    kv = orc.decode(w.kv_cache, "bf16", None).reshape(-1, 576)
    for r in range(2):
        row = kv[int(w.block_table[r, 0]) * 2]
        q = orc.decode_bf16(w.q[r])
        assert np.max(np.abs(o[r] - row[:512][None])) == 0.0
        assert np.allclose(l[r], w.softmax_scale * (q @ row), atol=1e-13, rtol=0)


def test_zero_query_integer_partials():
    """q = 0 and V entries in {0, 1} (bits of the logical position): each valid
    segment has m = 0, l = its position count, acc[d] = count of positions with
    bit d set.  Merged O = per-bit mean and LSE = ln n."""
    L, B, S, T = 150, 16, 4, 16
    w = _float_workload(lambda j: _bf16_bits([(j >> (d % 9)) & 1 for d in range(576)]), L,
                        block=B)
    w.q[:] = 0
    so, sm, se, valid, pl = orc.mla_decode_segments(w, S, T)
    for s, (a, b) in enumerate(orc.segment_bounds(L, S, T)):
        assert np.all(sm[0, :, s] == 0.0) and np.all(se[0, :, s] == b - a)
        for d in range(9):
            cnt = sum((j >> d) & 1 for j in range(a, b))
            assert np.all(so[0, :, s, d] == cnt)
    o, l = orc.merge_segments(so, sm, se, pl, T)
    assert np.allclose(l[0], math.log(L), atol=1e-13)
    for d in range(9):
        assert np.allclose(o[0, :, d], sum((j >> d) & 1 for j in range(L)) / L, atol=1e-13)


def test_single_key_segment_is_base2():
    """One position per segment: m = scale * log2(e) * (q . k), l = 1, acc = V."""
    w = mi.make_workload(name="b2", seq_lens=[3], num_heads=2, block_size=1, dtype="bf16", seed=4)
    so, sm, se, valid, pl = orc.mla_decode_segments(w, 3, 1)
    kv = orc.decode(w.kv_cache, "bf16", None).reshape(-1, 576)
    q = orc.decode_bf16(w.q[0])
    for s in range(3):
        k = kv[int(w.block_table[0, s])]
        assert np.allclose(sm[0, :, s], w.softmax_scale * (q @ k) / math.log(2), atol=1e-12, rtol=0)
        assert np.all(se[0, :, s] == 1.0)
        assert np.max(np.abs(so[0, :, s] - k[:512][None])) == 0.0


def test_rope_shift_closed_form():
    g = np.random.default_rng(2)
    u = _bf16_bits(g.standard_normal(64))
    lat = [_bf16_bits(g.standard_normal(512)) for _ in range(40)]
    w = _float_workload(lambda j: np.concatenate([lat[j], u]), 40, H=3)
    old = orc.decode_bf16(w.q[0, :, 512:]).copy()
    o1, l1 = orc.mla_decode(w)
    w.q[0, :, 512:] = _bf16_bits(g.standard_normal((3, 64)))
    new = orc.decode_bf16(w.q[0, :, 512:])
    o2, l2 = orc.mla_decode(w)
    shift = w.softmax_scale * ((new - old) @ orc.decode_bf16(u))
    assert np.max(np.abs(o2 - o1)) < 1e-12
    assert np.allclose(l2[0] - l1[0], shift, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- sinks ------

def test_sink_equals_extra_key_with_zero_value():
    g = np.random.default_rng(3)
    q = g.standard_normal((1, 576))
    rows = g.standard_normal((23, 576))
    scale = 0.2
    for sigma in [-3.0, 0.0, 1.7, 8.0]:
        o, l = orc.attend(q, rows, scale, sink=np.array([sigma]))
        qr = q[0, 512:]
        extra = np.zeros(576)
        extra[512:] = qr * (sigma / (scale * (qr @ qr)))  # logit sigma, V = 0
        o2, l2 = orc.attend(q, np.vstack([rows, extra]), scale)
        assert np.allclose(l, l2, atol=1e-12, rtol=0)
        assert np.max(np.abs(o - o2)) < 1e-12


def test_sink_only_row():
    q = np.ones((2, 576))
    o, l = orc.attend(q, np.zeros((0, 576)), 0.1, sink=np.array([0.25, -1.5]))
    assert np.all(o == 0) and list(l) == [0.25, -1.5]
    o, l = orc.attend(q, np.zeros((0, 576)), 0.1)
    assert np.all(o == 0) and np.all(np.isneginf(l))


# ------------------------------------------------------ partition invariance -

@pytest.mark.parametrize("tile", [1, 2, 4, 8, 16])
def test_partition_invariance(tile):
    w = mi.make_workload(name="pi", seq_lens=[17, 100, 1, 48, 257, 0], qlens=[1, 2, 1, 3, 1, 1],
                         num_heads=3, block_size=16, dtype="bf16", causal=True, sinks=True,
                         seed=12)
    ref_o, ref_l = orc.mla_decode(w)
    for S in [1, 2, 3, 4, 7, 64]:
        o, l = orc.mla_decode_via_segments(w, S, tile)
        fin = np.isfinite(ref_l)
        assert np.array_equal(fin, np.isfinite(l))
        assert np.max(np.abs(o - ref_o)) < 1e-12
        assert np.max(np.abs(l[fin] - ref_l[fin])) < 1e-12


def test_partition_invariance_fp8_subpages():
    w = mi.make_workload(name="pi8", seq_lens=[600, 257, 129], qlens=[2, 1, 4], num_heads=5,
                         block_size=256, dtype="fp8_e4m3", causal=True, seed=13)
    ref_o, ref_l = orc.mla_decode(w)
    tile = orc.tile_size_for_block(256)
    assert tile == 128
    for S in [1, 2, 3, 5]:
        o, l = orc.mla_decode_via_segments(w, S, tile)
        assert np.max(np.abs(o - ref_o)) < 1e-12 and np.max(np.abs(l - ref_l)) < 1e-12


def test_merge_empty_rows():
    so = np.zeros((2, 3, 4, 512))
    sm = np.zeros((2, 3, 4))
    se = np.ones((2, 3, 4))
    o, l = orc.merge_segments(so, sm, se, np.array([0, 0]), 16)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    sinks = np.array([0.1, 0.2, -0.3])
    o, l = orc.merge_segments(so, sm, se, np.array([0, 0]), 16, sinks)
    assert np.all(o == 0) and np.allclose(l, sinks[None])


# ------------------------------------------------------------ invariances ----

def test_request_permutation_and_page_relabel():
    w = mi.make_workload(name="inv", seq_lens=[33, 70, 5], qlens=[1, 2, 1], num_heads=4,
                         block_size=8, dtype="bf16", causal=True, seed=21)
    o, l = orc.mla_decode(w)
    # relabel physical pages: permute the pool and remap the table
    nb = w.kv_cache.shape[0]
    perm = np.random.default_rng(0).permutation(nb)  # new position of old block b is perm[b]
    kv2 = np.empty_like(w.kv_cache)
    kv2[perm] = w.kv_cache
    w2 = mi.with_(w, kv_cache=kv2, block_table=perm[w.block_table].astype(np.int32))
    o2, l2 = orc.mla_decode(w2)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    # reverse the request order
    order = [2, 1, 0]
    tok = [list(range(w.qo_indptr[r], w.qo_indptr[r + 1])) for r in order]
    flat = [t for ts in tok for t in ts]
    qlens = np.diff(w.qo_indptr)[order]
    qo = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    w3 = mi.with_(w, q=w.q[flat], block_table=w.block_table[order], seq_lens=w.seq_lens[order],
                  qo_indptr=qo)
    o3, l3 = orc.mla_decode(w3)
    assert np.array_equal(o3, o[flat]) and np.array_equal(l3, l[flat])


def test_head_subset_independent():
    w = mi.make_workload(name="hs", seq_lens=[90, 41], num_heads=6, block_size=16,
                         dtype="fp8_e4m3", sinks=True, seed=22)
    o, l = orc.mla_decode(w)
    sub = [4, 1]
    w2 = mi.with_(w, q=w.q[:, sub].copy(), num_heads=2, sinks=w.sinks[sub].copy())
    o2, l2 = orc.mla_decode(w2)
    assert np.array_equal(o2, o[:, sub]) and np.array_equal(l2, l[:, sub])


def test_causal_rows_equal_shortened_decodes():
    w = mi.make_workload(name="cz", seq_lens=[40, 9], qlens=[4, 3], num_heads=2, block_size=8,
                         dtype="bf16", causal=True, seed=23)
    o, l = orc.mla_decode(w)
    for r in range(2):
        t0, t1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        for i in range(t1 - t0):
            n = int(w.seq_lens[r]) - (t1 - t0) + i + 1
            wi = mi.with_(w, q=w.q[t0 + i:t0 + i + 1], block_table=w.block_table[r:r + 1],
                          seq_lens=np.array([n], np.int32), qo_indptr=np.array([0, 1], np.int32),
                          causal=False)
            oi, li = orc.mla_decode(wi)
            assert np.array_equal(oi[0], o[t0 + i]) and np.array_equal(li[0], l[t0 + i])


def test_poison_pages_not_read():
    """Workloads carry a NaN block and NaN page tails; the oracle's outputs
    stay finite, so any reader that touches them would show it."""
    w = mi.make_workload(name="pz", seq_lens=[5, 17, 64], num_heads=2, block_size=16,
                         dtype="bf16", seed=24, extra_bt_cols=2)
    flat = w.kv_cache.reshape(-1, 576)
    assert np.any(np.isnan(orc.decode_bf16(flat)))
    o, l = orc.mla_decode(w)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


# ------------------------------------------------- ragged page lists ----

def test_ragged_page_lists_reach_the_same_rows():
    """The flat page list + offsets form of a batch names the same cache rows
    as its 2-D table, position by position (so the oracle's result is the
    same), and the list ends exactly at each request's last page."""
    w = mi.make_workload(name="rp", seq_lens=[5, 17, 64, 0, 33], num_heads=2, block_size=16,
                         dtype="bf16", seed=25, extra_bt_cols=2)
    wr = mi.as_ragged_pages(w)
    assert wr.block_table.ndim == 1 and wr.bt_indptr[-1] == wr.block_table.shape[0]
    for r, L in enumerate(w.seq_lens):
        pages = orc.pages_of(wr.block_table, wr.bt_indptr, r)
        assert len(pages) == (int(L) + 15) // 16
        for j in range(int(L)):
            assert orc.cache_row_index(pages, j, 16) == orc.cache_row_index(w.block_table[r], j, 16)
    o1, l1 = orc.mla_decode(w)
    o2, l2 = orc.mla_decode(wr)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_sparse_index_stream_is_attention_over_the_listed_rows():
    """Page size 1 + flat index lists: token t attends exactly to the rows its
    list names.  Checked against numpy fancy indexing of the decoded cache
    (no page walk) and torch's logsumexp, with the sink as an extra logit."""
    w = mi.sparse_batch(num_tokens=4, topk=9, ctx=20, num_heads=3, dtype="bf16",
                        counts=[9, 0, 1, 5], seed=26)
    o, l = orc.mla_decode(w)
    kv = orc.decode_bf16(w.kv_cache.reshape(-1, 576)).astype(np.float64)
    q = orc.decode_bf16(w.q).astype(np.float64)
    for t in range(4):
        idx = w.block_table[w.bt_indptr[t]:w.bt_indptr[t + 1]]
        assert len(idx) == w.seq_lens[t] and np.all(idx // 20 == t)   # rows of the token's own request
        rows = kv[idx]
        s = w.softmax_scale * (q[t] @ rows.T)                           # [H, n]
        logits = np.concatenate([s, np.asarray(w.sinks, np.float64)[:, None]], axis=1)
        lse = torch.logsumexp(torch.from_numpy(logits), dim=1).numpy()
        p = np.exp(s - lse[:, None])
        assert np.allclose(l[t], lse, atol=1e-12, rtol=0)
        assert np.allclose(o[t], p @ rows[:, :512], atol=1e-12, rtol=0)
    assert np.all(o[1] == 0) and np.allclose(l[1], w.sinks, atol=0)  # empty list: sink only


# ------------------------------------------ decode context parallelism ----

@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_dcp_shards_combine_to_the_direct_decode(W, causal):
    """Round-robin key shards, each decoded without sinks, then the LSE
    combine with the sinks applied once, reproduce the direct decode of the
    whole batch (plain route for qlen 1; the segmented route, one request per
    verify token with its local causal window, for causal qlen > 1)."""
    w = mi.make_workload(name="dcp", seq_lens=[37, 5, 64, 1, 0, 20], num_heads=3, block_size=8,
                         dtype="bf16", qlens=[1, 3, 2, 1, 1, 4] if causal else None, causal=causal,
                         sinks=True, seed=27)
    ref_o, ref_l = orc.mla_decode(w)
    shards = mi.dcp_shards(w, W)
    outs, lses = [], []
    for sw in shards:
        assert sw.sinks is None
        o, l = orc.mla_decode(sw)
        outs.append(o)
        lses.append(l)
    o, l = orc.combine_lse(np.stack(outs), np.stack(lses), w.sinks)
    assert np.allclose(o, ref_o, atol=1e-12, rtol=0)
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(l)) and np.allclose(l[fin], ref_l[fin], atol=1e-12, rtol=0)
    # every key is on exactly one shard
    total = sum(int(sw.seq_lens.sum()) for sw in shards)
    if not causal:
        assert total == int(w.seq_lens.sum())


def test_combine_lse_closed_forms():
    """Two shards with equal LSE average their outputs and add ln 2; a shard
    with LSE -inf is ignored; a NaN LSE poisons only its row; no shard with a
    key gives out 0 and LSE -inf, or the sink."""
    rng = np.random.default_rng(3)
    o = rng.standard_normal((2, 3, 2, 512))
    l = np.array([[[0.5, -np.inf], [1.0, -np.inf], [np.nan, 2.0]],
                  [[0.5, 3.0], [-np.inf, -np.inf], [0.0, 2.0]]])
    out, lse = orc.combine_lse(o, l)
    assert np.allclose(out[0, 0], (o[0, 0, 0] + o[1, 0, 0]) / 2, atol=1e-15)
    assert abs(lse[0, 0] - (0.5 + math.log(2))) < 1e-15
    assert np.array_equal(out[0, 1], o[1, 0, 1]) and lse[0, 1] == 3.0
    assert np.array_equal(out[1, 0], o[0, 1, 0]) and lse[1, 0] == 1.0
    assert np.all(out[1, 1] == 0) and lse[1, 1] == -np.inf
    assert np.all(np.isnan(out[2, 0])) and np.isnan(lse[2, 0])
    assert np.allclose(out[2, 1], (o[0, 2, 1] + o[1, 2, 1]) / 2, atol=1e-15)
    sinks = np.array([0.25, -1.0])
    out2, lse2 = orc.combine_lse(o, l, sinks)
    assert np.all(out2[1, 1] == 0) and lse2[1, 1] == -1.0
    assert abs(lse2[0, 0] - np.logaddexp(0.5 + math.log(2), 0.25)) < 1e-15


# ---------------------------------------------------------- q prologue ----

def test_e4m3_quantiser_is_nearest_code_ties_to_even():
    """The q quantiser (division in single precision, saturation, torch's
    e4m3fn cast) picks the nearest code of the OCP table, ties to the even
    code, on values drawn to hit ties, subnormals and saturation."""
    table = orc._E4M3_TABLE
    finite = [c for c in range(256) if np.isfinite(table[c])]
    rng = np.random.default_rng(5)
    exact = np.array([table[c] for c in finite])
    mids = (np.sort(np.unique(exact))[1:] + np.sort(np.unique(exact))[:-1]) / 2   # exact ties
    vals = np.concatenate([exact, mids, rng.standard_normal(2000) * 40, [600.0, -1e4, 2.0 ** -11]])
    vals = vals.astype(np.float32).astype(np.float64)
    codes = orc.quantize_e4m3(vals, 1.0)
    for v, c in zip(vals, codes):
        y = min(max(v, -448.0), 448.0)
        d = np.abs(exact - y)
        best = np.flatnonzero(d == d.min())
        cands = [finite[i] for i in best]
        if len(set(table[c2] for c2 in cands)) > 1:        # a tie between two values: even mantissa
            cands = [c2 for c2 in cands if (c2 & 1) == 0]
        assert table[c] in [table[c2] for c2 in cands], (v, c)
    # the scale divides first: 3.0 / 2.0 = 1.5 is a code
    assert table[orc.quantize_e4m3(np.array([3.0]), 2.0)[0]] == 1.5


def test_bf16_q_with_fp8_cache_uses_the_quantised_q():
    """A bf16 q with an fp8 cache decodes as the batch whose fp8 q holds the
    quantised codes (same q scale)."""
    w = mi.make_workload(name="qp", seq_lens=[40, 7], num_heads=2, block_size=16, dtype="fp8_e4m3", seed=28)
    wb = mi.with_bf16_q(w, seed=1)
    codes = orc.quantize_e4m3(orc.decode_bf16(wb.q), wb.q_scale)
    w8 = mi.with_(w, q=codes, q_scale=wb.q_scale)
    o1, l1 = orc.mla_decode(wb)
    o2, l2 = orc.mla_decode(w8)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
