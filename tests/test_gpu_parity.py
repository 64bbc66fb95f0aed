"""GPU parity of the HIP path against the fp64 oracle (run with -m gpu).

Every call goes through the C ABI (ctypes binding); nothing here computes a
result on the host except the oracle.
"""
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
from oracle import mla_oracle as orc

from gpu_helpers import LSE_TOL, assert_close, out_tol, run_decode, run_segments, vmax

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import mla_paged_decode_02_amd as m
    m.lib()  # the HIP library must load; no fallback exists


def _print_case(name):
    print(f"[case] {name}", flush=True)


# ------------------------------------------------------------ tiny (page C1) --

def test_tiny_fused_and_segmented():
    w = mi.tiny()
    _print_case(w.name)
    ref_o, ref_l = orc.mla_decode(w)
    out, lse = run_decode(w, num_segments=4)
    assert_close(w, out, lse, ref_o, ref_l)
    # bf16 output rounding on top
    out_b, lse_b = run_decode(w, num_segments=4, out_dtype=torch.bfloat16)
    assert_close(w, out_b, lse_b, ref_o, ref_l)
    # two-call path: partials then merge
    import mla_paged_decode_02_amd as m
    so, sm, se, d = run_segments(w, 4, 16)
    o2, l2 = m.merge_segments(torch.from_numpy(so).cuda(), torch.from_numpy(sm).cuda(),
                              torch.from_numpy(se).cuda(), d["seq_lens"], 16,
                              out_dtype=torch.float32)
    assert_close(w, o2.cpu().numpy().astype(np.float64), l2.cpu().numpy().astype(np.float64),
                 ref_o, ref_l)


def test_tiny_partials_match_oracle_segments():
    w = mi.tiny()
    S, T = 4, 16
    so, sm, se, _ = run_segments(w, S, T)
    rso, rsm, rse, valid, _ = orc.mla_decode_segments(w, S, T)
    vm = vmax(w)
    for t in range(w.num_tokens):
        for s in range(S):
            if not valid[t, s]:
                continue
            # base-2 max: fp32 dot products of exact bf16 products
            assert np.max(np.abs(sm[t, :, s] - rsm[t, :, s])) < 1e-4
            assert np.max(np.abs(se[t, :, s] / rse[t, :, s] - 1)) < 1e-3
            norm = so[t, :, s] / se[t, :, s][:, None]
            rnorm = rso[t, :, s] / rse[t, :, s][:, None]
            assert np.max(np.abs(norm - rnorm)) <= 1e-2 * vm


# ------------------------------------------------ bit-exact partition check --

def _bits_workload(seq_lens, block, dtype, H=16, qlens=None, causal=False, seed=0):
    """q = 0 and V[d] = bit (d % 16) of (logical position + 1000 * request):
    every visible position has p = 1, so a segment's partials are integers."""
    w = mi.make_workload(name="bits", seq_lens=seq_lens, num_heads=H, block_size=block,
                         dtype=dtype, qlens=qlens, causal=causal, seed=seed)
    one = 0x3F80 if dtype == "bf16" else 0x38
    flat = w.kv_cache.reshape(-1, 576)
    for r, n in enumerate(w.seq_lens):
        for j in range(int(n)):
            code = (j + 1000 * r)
            bits = [(code >> (d % 16)) & 1 for d in range(576)]
            flat[orc.cache_row_index(w.block_table[r], j, block)] = np.array(bits) * one
    w.q[:] = 0
    w.kv_scale = None
    w.q_scale = None
    return w


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("lens,block,tile,S", [
    ([17, 100, 257, 1], 16, 16, 4),
    ([17, 100, 257, 1], 16, 4, 7),
    ([1000, 63, 64, 65], 64, 64, 3),
    ([4097, 31, 2048], 256, 128, 5),
    ([333, 700], 96, 32, 9),
    ([50, 129], 1, 1, 64),
])
def test_partition_bit_exact(dtype, lens, block, tile, S):
    _print_case(f"bits {dtype} lens={lens} block={block} tile={tile} S={S}")
    w = _bits_workload(lens, block, dtype)
    so, sm, se, _ = run_segments(w, S, tile)
    for r, n in enumerate(lens):
        bounds = orc.segment_bounds(n, S, tile)
        for s, (a, b) in enumerate(bounds):
            assert np.all(sm[r, :, s] == 0.0), (r, s)
            assert np.all(se[r, :, s] == b - a), (r, s, se[r, 0, s], b - a)
            for d in range(16):
                cnt = sum(((j + 1000 * r) >> d) & 1 for j in range(a, b))
                assert np.all(so[r, :, s, d] == cnt), (r, s, d)
            # dims repeat with period 16
            assert np.array_equal(so[r, :, s, 16:32], so[r, :, s, 0:16])


def test_partition_bit_exact_causal():
    lens, qlens = [40, 200, 5], [4, 3, 2]
    w = _bits_workload(lens, 16, "bf16", H=5, qlens=qlens, causal=True)
    S, tile = 3, 16
    so, sm, se, _ = run_segments(w, S, tile)
    for r, n in enumerate(lens):
        t0 = int(w.qo_indptr[r])
        for i in range(qlens[r]):
            vis = orc.visible_len(n, qlens[r], i, True)
            for s, (a, b) in enumerate(orc.segment_bounds(n, S, tile)):
                cnt = max(0, min(b, vis) - a)
                if cnt == 0:
                    assert np.all(np.isneginf(sm[t0 + i, :, s])) and np.all(se[t0 + i, :, s] == 0)
                    assert np.all(so[t0 + i, :, s] == 0)
                else:
                    assert np.all(sm[t0 + i, :, s] == 0) and np.all(se[t0 + i, :, s] == cnt)


# ---------------------------------------------------------- parity sweep -----

SWEEP = [
    # (dtype, H, block, lens, qlens, causal, sinks, S)
    ("bf16", 16, 64, [3000, 1, 64, 700], None, False, False, 5),
    ("bf16", 1, 16, [300, 17], None, False, True, 3),
    ("bf16", 3, 256, [1500, 129], None, False, True, 2),
    ("bf16", 20, 64, [999, 64], None, False, False, 4),
    ("bf16", 48, 64, [1200, 31], None, False, True, 3),
    ("bf16", 64, 32, [777, 2048], None, False, False, 2),
    ("bf16", 96, 64, [600, 65], None, False, True, 2),
    ("bf16", 128, 256, [1300, 200], None, False, False, 3),
    ("bf16", 16, 64, [500, 2000, 7, 64], [1, 2, 3, 4], True, True, 3),
    ("fp8_e4m3", 16, 64, [3000, 2, 640], None, False, False, 5),
    ("fp8_e4m3", 48, 64, [1600, 100], None, False, True, 3),
    ("fp8_e4m3", 64, 64, [1111, 4096], None, False, False, 2),
    ("fp8_e4m3", 96, 64, [900, 44, 3000], [1, 4, 2], True, True, 3),
    ("fp8_e4m3", 128, 128, [1024, 3], None, False, False, 2),
    ("fp8_e4m3", 7, 8, [170, 33], [3, 1], True, True, 4),
    # pages that are not a power of two: a k-split wave's next tile lies one or
    # more pages on (48 < 4 waves x 16 keys, 96 < 4 waves x 32 keys)
    ("bf16", 16, 48, [777, 100, 48], None, False, False, 3),
    ("fp8_e4m3", 16, 96, [1000, 300, 97], None, False, True, 3),
    # four-wave chunks with waves that hold no rows (40 heads; qlen 2 leaves a
    # 16-row chunk): a row-less wave issues the whole tile's loads
    ("fp8_e4m3", 40, 64, [900, 130], [2, 1], True, True, 3),
    # 49-64 rows per chunk run the 32-row fp8 waves: causal verify blocks whose
    # wave holds rows of two tokens with different causal limits (16 heads x
    # qlen 4, 28 heads x qlen 2), and 52 heads with 12 empty rows in the second
    # wave over 32-key pages
    ("fp8_e4m3", 16, 64, [700, 2500, 40], [4, 3, 4], True, True, 3),
    ("fp8_e4m3", 28, 64, [1300, 61], [2, 2], True, True, 2),
    ("fp8_e4m3", 52, 32, [900, 333], None, False, True, 3),
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"{c[0]}-H{c[1]}-blk{c[2]}-q{c[4] is not None}-S{c[7]}")
def test_parity_sweep(case):
    dtype, H, block, lens, qlens, causal, sinks, S = case
    _print_case(str(case))
    w = mi.make_workload(name="sweep", seq_lens=lens, num_heads=H, block_size=block, dtype=dtype,
                         qlens=qlens, causal=causal, sinks=sinks,
                         seed=1000 * H + block + (7 if dtype == "bf16" else 0))
    ref_o, ref_l = orc.mla_decode(w)
    out, lse = run_decode(w, num_segments=S)
    assert_close(w, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("schedule", ["segments", "balanced"])
def test_fp8_one_wave_tiles_every_tail_length(schedule):
    """fp8 at 16 heads over 64-key pages: the one-wave ring loads whole cache
    lines of 32-row tiles and exchanges 64 chunks per tile.  One request per
    count of valid rows in its last tile (1..32), at one to three tiles in
    front of it, so rows past a tile's end (zeros) never reach a result."""
    lens = [32 * (1 + r % 3) + r for r in range(1, 33)]
    _print_case(f"fp8 one-wave tail lengths {schedule}")
    w = mi.make_workload(name="tails", seq_lens=lens, num_heads=16, block_size=64, dtype="fp8_e4m3",
                         sinks=True, seed=4242)
    ref_o, ref_l = orc.mla_decode(w)
    for S in ((0, 2) if schedule == "segments" else (0,)):
        out, lse = run_decode(w, num_segments=S, schedule=schedule)
        assert_close(w, out, lse, ref_o, ref_l)
    out_b, lse_b = run_decode(w, num_segments=0, schedule=schedule, out_dtype=torch.bfloat16)
    assert_close(w, out_b, lse_b, ref_o, ref_l)


@pytest.mark.parametrize("schedule", ["segments", "balanced"])
def test_planner_choice_and_empty_requests(schedule):
    """num_segments = 0 (the planner's S, or the balanced split) and requests
    of length 0, with sinks."""
    w = mi.make_workload(name="empty", seq_lens=[0, 500, 0, 64], num_heads=16, block_size=64,
                         dtype="bf16", sinks=True, seed=31)
    ref_o, ref_l = orc.mla_decode(w)
    out, lse = run_decode(w, num_segments=0, schedule=schedule)
    assert_close(w, out, lse, ref_o, ref_l)
    assert np.all(out[0] == 0) and np.allclose(lse[0], w.sinks, atol=0, rtol=0)
    out2, lse2 = run_decode(w, num_segments=0, sinks=False, schedule=schedule)
    assert np.all(out2[0] == 0) and np.all(np.isneginf(lse2[0]))


@pytest.mark.parametrize("dtype,H,Hs,same_shape", [
    ("fp8_e4m3", 64, 56, True),    # both 32-row waves
    ("fp8_e4m3", 48, 16, True),    # both 16-row waves
    ("fp8_e4m3", 128, 80, True),   # both eight 16-row waves
    ("fp8_e4m3", 64, 48, False),   # 32-row waves against 16-row waves
    ("bf16", 64, 48, True),
    ("bf16", 48, 16, False),
    ("bf16", 128, 80, True),       # both four 32-row waves
    ("bf16", 128, 64, False),      # 32-row waves against 16-row waves
])
def test_head_count_independent(dtype, H, Hs, same_shape):
    """Heads are independent (no head folding): the first Hs heads of an
    H-head batch give the same results as an Hs-head batch of those heads,
    bit for bit when both head counts run the same kernel body (the per-row
    arithmetic does not depend on the number of rows beside it), within the
    decode tolerance where the head counts pick different bodies."""
    w = mi.make_workload(name="heads", seq_lens=[2000, 300], num_heads=H, block_size=64, dtype=dtype, seed=41)
    ws = mi.with_(w, q=np.ascontiguousarray(w.q[:, :Hs]), num_heads=Hs)
    o, l = run_decode(w, num_segments=3)
    os_, ls = run_decode(ws, num_segments=3)
    if same_shape:
        assert np.array_equal(o[:, :Hs], os_) and np.array_equal(l[:, :Hs], ls)
    else:
        ref_o, ref_l = orc.mla_decode(ws)
        assert_close(ws, o[:, :Hs], l[:, :Hs], ref_o, ref_l)
        assert_close(ws, os_, ls, ref_o, ref_l)


def test_strided_views():
    """q as a head-strided view, block table read through a column stride."""
    import mla_paged_decode_02_amd as m
    w = mi.make_workload(name="strided", seq_lens=[900, 130], num_heads=8, block_size=32,
                         dtype="bf16", seed=51)
    ref_o, ref_l = orc.mla_decode(w)
    d = mi.to_torch(w, "cuda")
    big = torch.zeros((w.num_tokens, w.num_heads, 640), dtype=torch.bfloat16, device="cuda")
    big[:, :, :576] = d["q"]
    qv = big[:, :, :576]
    btT = d["block_table"].t().contiguous().t()  # column stride != 1
    assert btT.stride(1) != 1
    out, lse = m.decode(qv, d["kv_cache"], btT, d["seq_lens"], softmax_scale=w.softmax_scale,
                        max_seq_len=w.max_seq_len, num_segments=3, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                 ref_o, ref_l)


@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float16, torch.float32])
def test_output_dtypes(odt):
    w = mi.make_workload(name="odt", seq_lens=[700, 40], num_heads=16, block_size=64, dtype="bf16",
                         seed=61)
    ref_o, ref_l = orc.mla_decode(w)
    out, lse = run_decode(w, num_segments=2, out_dtype=odt)
    assert_close(w, out, lse, ref_o, ref_l)


def test_poison_never_read():
    """Pages past a request's end and page tails hold NaN: outputs stay finite."""
    w = mi.make_workload(name="poison", seq_lens=[65, 1, 127, 64], num_heads=16, block_size=64,
                         dtype="bf16", seed=71, extra_bt_cols=3)
    out, lse = run_decode(w, num_segments=2)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_prepared_decoder_matches_decode():
    """The prepared call gives the bits of the one-shot call, run after run."""
    import mla_paged_decode_02_amd as m
    w = mi.make_workload(name="prep", seq_lens=[1500, 64, 333], num_heads=16, block_size=64,
                         dtype="bf16", sinks=True, seed=81)
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d)
    o1, l1 = m.decode(**args, sinks=d["sinks"], num_segments=3)
    dec = m.Decoder(**args, sinks=d["sinks"], num_segments=3)
    for _ in range(3):
        o2, l2 = dec.run()
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------- balanced split ----
# mla_decode with schedule "balanced" cuts the batch's units (request, row chunk,
# tile) into equal workgroup ranges.  max_workgroups forces few workgroups so
# that ranges hold several whole requests, start or end inside one, or lie
# inside one; the default uses every slot of the device.

@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"{c[0]}-H{c[1]}-blk{c[2]}-q{c[4] is not None}")
@pytest.mark.parametrize("wgs", [0, 1, 3, 7])
def test_split_parity_sweep(case, wgs):
    import mla_paged_decode_02_amd as m
    dtype, H, block, lens, qlens, causal, sinks, _ = case
    _print_case(f"split wgs={wgs} {case}")
    w = mi.make_workload(name="split", seq_lens=lens, num_heads=H, block_size=block, dtype=dtype,
                         qlens=qlens, causal=causal, sinks=sinks,
                         seed=1000 * H + block + (7 if dtype == "bf16" else 0))
    ref_o, ref_l = orc.mla_decode(w)
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d)
    out, lse = m.decode(**args, sinks=d["sinks"], schedule="balanced", max_workgroups=wgs,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                 ref_o, ref_l)


@pytest.mark.parametrize("R,wgs", [(64, 0), (65, 0), (70, 7), (70, 37), (130, 0), (130, 11)])
def test_split_many_requests(R, wgs):
    """Batches of more than 64 requests: the split kernel keeps the first 64
    requests' fields in registers and loads later ones, so workgroup ranges
    that start past request 63, or that run from one side of it to the
    other, must still find their pieces (ragged lengths, mixed query counts,
    causal, sinks)."""
    import mla_paged_decode_02_amd as m
    _print_case(f"split many requests R={R} wgs={wgs}")
    rng = np.random.default_rng(4000 + R)
    lens = [int(x) for x in rng.integers(1, 400, R)]
    qlens = [int(x) for x in rng.integers(1, 3, R)]
    w = mi.make_workload(name="manyreq", seq_lens=lens, qlens=qlens, num_heads=16, block_size=16, dtype="bf16",
                         causal=True, sinks=True, seed=4100 + R)
    ref_o, ref_l = orc.mla_decode(w)
    d = mi.to_torch(w, "cuda")
    out, lse = m.decode(**mi.call_args(w, d), sinks=d["sinks"], schedule="balanced", max_workgroups=wgs,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l)


PER_JOB = [
    # (dtype, H, block, lens, qlens, workgroups, sum_seq_lens hint or None for the exact sum)
    # k workgroups per job (request row chunk) of U units:
    ("bf16", 16, 64, [1000] * 6, None, 30, None),             # 63 units per job, 5 per job
    ("fp8_e4m3", 48, 64, [1500] * 5, None, 45, None),         # producer wave: 47 units, 9 per job
    ("bf16", 16, 64, [700] * 4, [2] * 4, 24, None),           # 2 row chunks per request, records
    ("fp8_e4m3", 64, 64, [900] * 3, None, 12, None),          # wide fp8 waves: 29 units, 4 per job
    ("bf16", 128, 128, [800] * 3, None, 18, None),            # wide bf16 waves: 25 units, 6 per job
    ("bf16", 16, 64, [1000] * 6, None, 6, None),              # one workgroup per job: finished in place
    ("bf16", 16, 64, [20] * 6, None, 30, None),               # 2 units over 5 workgroups: empty pieces
    ("bf16", 16, 64, [1000, 900] + [1000] * 4, None, 30, 6000),  # a hint that claims equal lengths
]


@pytest.mark.parametrize("case", PER_JOB, ids=lambda c: f"{c[0]}-H{c[1]}-L{c[3][0]}-wg{c[5]}-hint{c[6]}")
def test_split_per_job_ranges(case):
    """Equal jobs (one request's row chunk each) on k workgroups per job, also
    when k does not divide a job's units: the shares of the whole unit
    sequence then still end on job boundaries (floor((k j + i) U / k) =
    j U + floor(i U / k)).  Also one workgroup per job (rows finished in
    place), jobs of fewer units than workgroups (empty ranges), and a length
    hint that claims equal lengths when they are not."""
    import mla_paged_decode_02_amd as m
    dtype, H, block, lens, qlens, wgs, hint = case
    _print_case(f"split per-job ranges {case}")
    w = mi.make_workload(name="perjob", seq_lens=lens, qlens=qlens, num_heads=H, block_size=block, dtype=dtype,
                         causal=qlens is not None, sinks=True, seed=4700 + H + wgs)
    ref_o, ref_l = orc.mla_decode(w)
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d)
    if hint is not None:
        args["sum_seq_lens"] = hint
    for out_dtype in (torch.float32, torch.bfloat16):
        out, lse = m.decode(**args, sinks=d["sinks"], schedule="balanced", max_workgroups=wgs, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert_close(w, out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                     ref_o, ref_l)


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_split_long_row_among_short_ones(dtype):
    """One long request among many short ones: the merge's step size follows
    the usual piece count per row (small here), while the long request's rows
    gather far more than 64 pieces (the merge's long-row path)."""
    import mla_paged_decode_02_amd as m
    lens = [16] * 60 + [40000]
    _print_case(f"long row among short ones {dtype} lens=60x16+40000")
    w = mi.make_workload(name="longrow", seq_lens=lens, num_heads=16, block_size=64, dtype=dtype,
                         sinks=True, seed=77 if dtype == "bf16" else 78)
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d)
    out, lse = m.decode(**args, sinks=d["sinks"], schedule="balanced", out_dtype=torch.float32)
    torch.cuda.synchronize()
    g, rows_wg, tt = m.split_plan(m.make_problem(**args, schedule="balanced"))
    assert (40000 // tt) * g // (sum(-(-n // tt) for n in lens)) > 64  # the long row's pieces
    ref_o, ref_l = orc.mla_decode(w, reqs=[0, 59, 60])
    sel = [0, 59, 60]
    o = out.cpu().numpy().astype(np.float64)[sel]
    l = lse.cpu().numpy().astype(np.float64)[sel]
    vm = vmax(w, sel)
    assert np.abs(o - ref_o[sel]).max() <= out_tol(w) * vm
    assert np.abs(l - ref_l[sel]).max() <= LSE_TOL


@pytest.mark.parametrize("wgs", [0, 2, 5, 13])
@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_split_counts_every_key_once(dtype, wgs):
    """q = 0 and V = bits of (position, request): every key weighs 1, so the
    output is the exact per-bit mean and LSE = ln(len); a key dropped or seen
    twice by the split moves them by >= 1/len."""
    import mla_paged_decode_02_amd as m
    lens = [1, 15, 16, 17, 100, 333, 1024, 1500]
    w = mi.make_workload(name="split-bits", seq_lens=lens, num_heads=4, block_size=16,
                         dtype=dtype, seed=91, qlens=[1, 2, 1, 3, 1, 1, 2, 1], causal=True)
    w.q[:] = 0
    flat = w.kv_cache.reshape(-1, 576)
    one = 0x3F80 if dtype == "bf16" else 0x38  # 1.0 in bf16 / e4m3
    for r, L in enumerate(lens):
        for j in range(L):
            row = orc.cache_row_index(w.block_table[r], j, w.block_size)
            bits = [(j >> b) & 1 for b in range(11)] + [(r >> b) & 1 for b in range(3)]
            flat[row, :] = 0
            flat[row, :14] = [one * x for x in bits]
    w = mi.with_(w, kv_scale=None if dtype == "bf16" else 1.0, q_scale=None if dtype == "bf16" else 1.0)
    d = mi.to_torch(w, "cuda")
    out, lse = m.decode(**mi.call_args(w, d), schedule="balanced", max_workgroups=wgs,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qo = w.qo_indptr
    for r, L in enumerate(lens):
        ql = qo[r + 1] - qo[r]
        for i in range(ql):
            n = L - ql + i + 1
            t = qo[r] + i
            exp_o = [np.mean([(j >> b) & 1 for j in range(n)]) for b in range(11)] + \
                    [float((r >> b) & 1) for b in range(3)]
            assert np.allclose(out[t, :, :14], np.array(exp_o)[None], atol=2e-6, rtol=0), (r, i)
            assert np.all(out[t, :, 14:] == 0)
            assert np.allclose(lse[t], math.log(n), atol=2e-6, rtol=0), (r, i)


def test_split_stages_and_decoder():
    """The two stages run separately equal one mla_decode call, and a
    prepared split decoder repeats the same bits."""
    import mla_paged_decode_02_amd as m
    w = mi.make_workload(name="stages", seq_lens=[3000, 64, 700, 1], num_heads=32, block_size=64,
                         dtype="fp8_e4m3", sinks=True, seed=101)
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d)
    o1, l1 = m.decode(**args, sinks=d["sinks"], schedule="balanced")
    dec = m.Decoder(**args, sinks=d["sinks"], schedule="balanced")
    assert dec.split_workgroups > 0 and dec.num_segments == 0
    for _ in range(3):
        dec.run_stage(1)
        o2, l2 = dec.run_stage(2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref_o, ref_l = orc.mla_decode(w)
    assert_close(w, o1.float().cpu().numpy().astype(np.float64), l1.cpu().numpy().astype(np.float64),
                 ref_o, ref_l)
