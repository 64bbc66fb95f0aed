"""GPU numerics and call-contract tests (run with -m gpu).

* fp8 P precision: the P.V product takes P rounded to e4m3, which flushes
  weights below 2^-10 (relative to the running max) to zero.  The output must
  be normalised by the rounded weights the product used (else it shrinks
  towards zero) while the LSE keeps the exact exp-sum (else it drops by the
  flushed weight).  The sharpest case is a value vector with a large common
  offset and a piece whose first tile holds its largest logit; rows that see
  only 2-5 keys carry the largest relative rounding of a single weight.
* Graph capture: mla_decode (both launches) recorded once in a HIP graph
  through torch and replayed with new q and cache contents equals the eager
  call bit for bit.
* Malformed query ranges: a request whose qo_indptr range is longer than
  max_qlen gets NaN rows from every route, and the other requests are exact.
* Query ranges and the merge's token records: a batch with empty query
  ranges (qlen 0) still tiles the tokens, so the merge reads the split
  kernel's per-token records; a token that no range covers gets NaN rows
  (the merge falls back to searching the ranges and finds none).
* Rising logits: keys whose logits climb steadily drive the lazy running
  max through many moves and, in the 32-row fp8 body, past the range of one
  reference into the second pass.

Every call goes through the C ABI (ctypes binding).
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
from oracle import mla_oracle as orc

from gpu_helpers import assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import mla_paged_decode_02_amd as m
    m.lib()


def _print_case(name):
    print(f"[case] {name}", flush=True)


def _reencode_fp8(w, values):
    """fp8 workload with new cache values (fp32 [blocks, page, 576]); the
    poison rows stay NaN codes."""
    nan_rows = np.isnan(orc.decode(w.kv_cache.reshape(-1, 576), "fp8_e4m3", 1.0)).any(axis=1)
    codes, scale = mi._encode(torch.from_numpy(values.reshape(-1, 576).astype(np.float32)), "fp8_e4m3")
    codes = codes.reshape(-1, 576)
    codes[nan_rows] = mi.FP8_E4M3_NAN_BYTE
    return mi.with_(w, kv_cache=codes.reshape(w.kv_cache.shape), kv_scale=scale)


def _offset_v_first_tile_max(H, lens, offset, seed, lift=12.0):
    """fp8 batch with V = offset + N(0,1) on the 512 latent dims, and key 0 of
    every request lifted ~`lift` base-2 units above the others' logits for
    every head (all heads of a token share their 64 rope dims u, and key 0's
    rope dims are a multiple of u): each row's largest logit sits in the first
    tile of its first piece, so the running max is final from the first tile
    on and e4m3 flushes the most weight."""
    w = mi.make_workload(name="offset-v", seq_lens=lens, num_heads=H, block_size=64, dtype="fp8_e4m3",
                         sinks=True, seed=seed)
    vals = orc.decode(w.kv_cache.reshape(-1, 576), "fp8_e4m3", w.kv_scale).reshape(w.kv_cache.shape)
    vals = np.where(np.isnan(vals), 0.0, vals)
    vals[..., :512] += offset
    q = orc.decode(w.q, "fp8_e4m3", w.q_scale).copy()     # [T, H, 576]
    rng = np.random.default_rng(seed)
    base2 = w.softmax_scale / orc.LOGE2                      # score -> base-2 units
    for r in range(w.num_reqs):
        t = int(w.qo_indptr[r])
        u = rng.standard_normal(64)
        q[t, :, 512:] = u
        row0 = orc.cache_row_index(w.block_table[r], 0, w.block_size)
        vals.reshape(-1, 576)[row0, 512:] = lift / (base2 * float(u @ u)) * u
    w = _reencode_fp8(w, vals)
    qc, qs = mi._encode(torch.from_numpy(q.astype(np.float32)), "fp8_e4m3")
    return mi.with_(w, q=qc, q_scale=qs)


@pytest.mark.parametrize("schedule", ["balanced", "segments"])
@pytest.mark.parametrize("H", [16, 64])
def test_fp8_offset_values_with_first_tile_max(H, schedule):
    import mla_paged_decode_02_amd as m
    _print_case(f"fp8 V = 20 + N(0,1), first-tile max, H={H} {schedule}")
    w = _offset_v_first_tile_max(H, [3000, 700, 5000], 20.0, seed=500 + H)
    ref_o, ref_l = orc.mla_decode(w)
    # the construction puts each row's largest logit on key 0, well above the rest
    d = mi.to_torch(w, "cuda")
    out, lse = m.decode(**mi.call_args(w, d), sinks=d["sinks"], schedule=schedule, out_dtype=torch.float32)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert_close(w, out, lse, ref_o, ref_l)
    # no one-sided shrink: the mean output stays at the mean of the reference
    # (the offset would pull a numerator/denominator mismatch visibly low)
    assert abs(out[..., :512].mean() / ref_o[..., :512].mean() - 1) < 5e-3


@pytest.mark.parametrize("schedule", ["balanced", "segments"])
@pytest.mark.parametrize("H", [16, 96])
def test_fp8_rows_with_two_to_five_keys(H, schedule):
    """Rows that see 2-5 keys: causal verify blocks over short requests."""
    import mla_paged_decode_02_amd as m
    rng = np.random.default_rng(H)
    lens = rng.integers(2, 6, size=40).tolist() + [5, 4, 3, 2]
    qlens = [1 + (i % 2) * (min(l, 4) - 1) for i, l in enumerate(lens)]   # 1 or up to 4 (<= len)
    _print_case(f"fp8 short rows H={H} {schedule}")
    w = mi.make_workload(name="short", seq_lens=lens, num_heads=H, block_size=64, dtype="fp8_e4m3",
                         qlens=qlens, causal=True, sinks=True, seed=600 + H)
    vals = orc.decode(w.kv_cache.reshape(-1, 576), "fp8_e4m3", w.kv_scale).reshape(w.kv_cache.shape)
    vals = np.where(np.isnan(vals), 0.0, vals)
    vals[..., :512] += 3.0
    w = _reencode_fp8(w, vals)
    ref_o, ref_l = orc.mla_decode(w)
    d = mi.to_torch(w, "cuda")
    out, lse = m.decode(**mi.call_args(w, d), sinks=d["sinks"], schedule=schedule, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l)


def _rising_logits(H, lens, dtype, rise_per_32, seed):
    """A batch whose logits climb steadily along each request's keys: all
    heads of a request's token share rope dims u, and key j's rope dims are
    c_j u with c_j set so that its base-2 logit grows by `rise_per_32` every
    32 keys (plus the latent part, q's latent dims scaled to 1/4).  One piece
    over L keys then sees its running max climb by rise_per_32 * L / 32
    units: the lazy reference moves many times, and past 64 units (32 in
    bf16) the wide bodies must take their second pass from the exact
    maximum."""
    w = mi.make_workload(name="rising", seq_lens=lens, num_heads=H, block_size=64, dtype=dtype,
                         sinks=True, seed=seed)
    scale = w.kv_scale if dtype != "bf16" else None
    vals = orc.decode(w.kv_cache.reshape(-1, 576), dtype, scale).reshape(w.kv_cache.shape)
    poison = np.isnan(vals).any(axis=-1)
    vals = np.where(np.isnan(vals), 0.0, vals)
    q = orc.decode(w.q, dtype, w.q_scale if dtype != "bf16" else None).copy()
    q[..., :512] *= 0.25
    rng = np.random.default_rng(seed)
    base2 = w.softmax_scale / orc.LOGE2
    flat = vals.reshape(-1, 576)
    for r in range(w.num_reqs):
        t = int(w.qo_indptr[r])
        u = rng.standard_normal(64)
        q[t, :, 512:] = u
        for j in range(int(w.seq_lens[r])):
            row = orc.cache_row_index(w.block_table[r], j, w.block_size)
            flat[row, 512:] = (rise_per_32 * j / 32.0) / (base2 * float(u @ u)) * u
    codes, kscale = mi._encode(torch.from_numpy(vals.reshape(-1, 576).astype(np.float32)), dtype)
    codes = codes.reshape(-1, 576)
    codes[poison.reshape(-1)] = mi.BF16_NAN_BITS if dtype == "bf16" else mi.FP8_E4M3_NAN_BYTE
    qc, qs = mi._encode(torch.from_numpy(q.astype(np.float32)), dtype)
    return mi.with_(w, kv_cache=codes.reshape(w.kv_cache.shape), kv_scale=kscale, q=qc, q_scale=qs)


@pytest.mark.parametrize("dtype,H,schedule,S", [
    ("fp8_e4m3", 64, "segments", 1),   # 32-row waves, one piece per request: second pass
    ("fp8_e4m3", 64, "balanced", 0),
    ("fp8_e4m3", 48, "segments", 1),   # 16-row waves: repeated lazy rescales
    ("fp8_e4m3", 16, "balanced", 0),   # k-split waves
    ("bf16", 16, "segments", 1),
    ("bf16", 128, "segments", 2),      # 32-row bf16 waves: second pass past 32 units
    ("bf16", 128, "balanced", 0),
])
def test_rising_logits(dtype, H, schedule, S):
    import mla_paged_decode_02_amd as m
    _print_case(f"rising logits {dtype} H={H} {schedule} S={S}")
    w = _rising_logits(H, [8192, 3000, 700], dtype, 0.6, seed=1100 + H)
    ref_o, ref_l = orc.mla_decode(w)
    d = mi.to_torch(w, "cuda")
    kw = {"num_segments": S} if schedule == "segments" else {}
    out, lse = m.decode(**mi.call_args(w, d), sinks=d["sinks"], schedule=schedule, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    assert_close(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l)
    # the construction does what it says: the largest logit sits at the end
    # of each request, 0.6 * len / 32 base-2 units above the first key's
    assert np.all(np.isfinite(ref_l))


def _fresh_codes(w, seed):
    """The batch with new N(0,1) q and cache codes (new scales for fp8) and
    the same table, lengths and NaN poison rows."""
    g = torch.Generator().manual_seed(seed)
    kvc, kvs = mi._encode(torch.randn(w.kv_cache.shape, generator=g), w.kv_dtype)
    qc, qs = mi._encode(torch.randn(w.q.shape, generator=g), w.q_dtype)
    poison = np.isnan(orc.decode(w.kv_cache.reshape(-1, 576), w.kv_dtype, w.kv_scale)).any(axis=1)
    kvc.reshape(-1, 576)[poison] = mi.BF16_NAN_BITS if w.kv_dtype == "bf16" else mi.FP8_E4M3_NAN_BYTE
    return mi.with_(w, q=qc, kv_cache=kvc, q_scale=qs, kv_scale=kvs)


@pytest.mark.parametrize("schedule", ["balanced", "segments"])
@pytest.mark.parametrize("dtype,H", [("bf16", 16), ("fp8_e4m3", 64)])
def test_graph_capture_replays_match_eager(dtype, H, schedule):
    """mla_decode captured in a graph, replayed three times with new q and
    cache contents (and, for fp8, new device scales), with eager work and
    synchronisations in between: every replay equals the eager call on the
    same contents bit for bit, and the last matches the oracle."""
    import mla_paged_decode_02_amd as m
    _print_case(f"graph capture {dtype} H={H} {schedule}")
    w = mi.make_workload(name="graph", seq_lens=[1500, 64, 3000, 1], num_heads=H, block_size=64, dtype=dtype,
                         sinks=True, seed=700 + H)
    d = mi.to_torch(w, "cuda")
    dec = m.Decoder(**mi.call_args(w, d), sinks=d["sinks"], schedule=schedule, out_dtype=torch.bfloat16)
    dec.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec.run()
    torch.cuda.synchronize()
    prev = None
    for rep in range(3):
        w2 = _fresh_codes(w, 800 + 10 * H + rep)
        d2 = mi.to_torch(w2, "cuda")
        for k in ("q", "kv_cache", "q_scale", "kv_scale"):
            if d[k] is not None:
                d[k].copy_(d2[k])
        g.replay()
        torch.cuda.synchronize()
        go, gl = dec.out.clone(), dec.lse.clone()
        dec.out.zero_()
        dec.lse.zero_()
        torch.cuda.synchronize()
        eo, el = dec.run()
        torch.cuda.synchronize()
        assert torch.equal(go, eo) and torch.equal(gl, el), f"replay {rep} differs from eager"
        if prev is not None:
            assert not torch.equal(prev, go), "replay did not see the new contents"
        prev = go
    ref_o, ref_l = orc.mla_decode(w2)
    assert_close(w2, eo.float().cpu().numpy().astype(np.float64), el.cpu().numpy().astype(np.float64),
                 ref_o, ref_l)


@pytest.mark.parametrize("route", ["balanced", "segments", "two-call"])
def test_malformed_query_range_gives_nan_rows(route):
    """Request 0 claims three query tokens while max_qlen is 2: its rows are
    NaN on every route; request 1 is unaffected.  (The kernels check the
    range themselves; every access stays inside the buffers.)"""
    import mla_paged_decode_02_amd as m
    _print_case(f"malformed qo_indptr {route}")
    w = mi.make_workload(name="bad-qo", seq_lens=[300, 200], qlens=[3, 1], num_heads=16, block_size=64,
                         dtype="bf16", causal=True, seed=901)
    ref_o, ref_l = orc.mla_decode(w)
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d)
    args["max_qlen"] = 2            # request 0's 3 tokens exceed it
    if route == "two-call":
        so, sm, se = m.decode_segments(**args, num_segments=3)
        part = torch.tensor([300, 300, 300, 200], dtype=torch.int32, device="cuda")
        out, lse = m.merge_segments(so, sm, se, part, 64, out_dtype=torch.float32)
    else:
        out, lse = m.decode(**args, schedule=route, out_dtype=torch.float32)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert np.isnan(out[:3]).all() and np.isnan(lse[:3]).all()
    assert_close(w, out, lse, ref_o, ref_l, reqs=[1], tok=np.array([3]))


@pytest.mark.parametrize("route", ["balanced", "segments"])
def test_empty_query_ranges(route):
    """Requests 1 and 4 have no query tokens (qo_indptr repeats a value); the
    other requests' rows match the oracle on both routes."""
    import mla_paged_decode_02_amd as m
    _print_case(f"empty query ranges {route}")
    w = mi.make_workload(name="qlen0", seq_lens=[900, 300, 2500, 64, 700, 1], qlens=[2, 0, 3, 1, 0, 2],
                         num_heads=32, block_size=64, dtype="fp8_e4m3", causal=True, sinks=True, seed=911)
    ref_o, ref_l = orc.mla_decode(w)
    d = mi.to_torch(w, "cuda")
    out, lse = m.decode(**mi.call_args(w, d), sinks=d["sinks"], schedule=route, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l)


@pytest.mark.parametrize("route", ["balanced", "segments"])
def test_token_outside_every_range_gives_nan_rows(route):
    """qo_indptr ends at 3 for a batch of 4 query tokens: token 3 belongs to no
    request and gets NaN rows; tokens 0-2 are exact (non-causal, so token 2,
    now request 1's only token, sees the same keys as before)."""
    import mla_paged_decode_02_amd as m
    _print_case(f"uncovered token {route}")
    w = mi.make_workload(name="gap", seq_lens=[500, 1300], qlens=[2, 2], num_heads=16, block_size=64,
                         dtype="bf16", causal=False, seed=913)
    ref_o, ref_l = orc.mla_decode(w)
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d)
    args["qo_indptr"] = torch.tensor([0, 2, 3], dtype=torch.int32, device="cuda")
    out, lse = m.decode(**args, schedule=route, out_dtype=torch.float32)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert np.isnan(out[3]).all() and np.isnan(lse[3]).all()
    assert_close(w, out, lse, ref_o, ref_l, tok=np.arange(3))
