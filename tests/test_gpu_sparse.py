"""Ragged page lists and the index-stream (sparse top-k) decode on the GPU.

The block table given as one flat page list with per-request offsets
(``bt_indptr``) must give what the 2-D table gives, and with page size 1 the
same kernels run the sparse MLA page's decode: one request per query token,
its list the cache rows it attends to.  Both are compared with the fp64
oracle at the decode tolerances, for the balanced split and for a fixed
segment count.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mla_inputs as mi
from gpu_helpers import assert_close
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu


def _print_case(name):
    print(f"[case] {name}", flush=True)

PAGED = [
    # (dtype, H, block, lens, qlens, causal, sinks)
    ("bf16", 16, 64, [3000, 1, 64, 700, 0], None, False, True),
    ("bf16", 48, 16, [1200, 31, 257], None, False, False),
    ("bf16", 16, 64, [500, 2000, 7, 64], [1, 2, 3, 4], True, True),
    ("fp8_e4m3", 64, 64, [1111, 4096], None, False, True),
    ("fp8_e4m3", 96, 8, [900, 44, 3000], [1, 4, 2], True, True),
    ("bf16", 128, 256, [1300, 200], None, False, False),
]


def _run(w, S, wgs=0):
    """S None: the balanced split (at most wgs workgroups, 0 = all slots);
    else the segment partition (0 = the planner's S)."""
    import mla_paged_decode_02_amd as m
    d = mi.to_torch(w, "cuda")
    sched = dict(schedule="balanced", max_workgroups=wgs) if S is None else dict(num_segments=S)
    out, lse = m.decode(**mi.call_args(w, d), sinks=d["sinks"], **sched, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", PAGED, ids=lambda c: f"{c[0]}-H{c[1]}-blk{c[2]}-q{c[4] is not None}")
@pytest.mark.parametrize("S,wgs", [(None, 0), (None, 3), (0, 0), (3, 0)])
def test_ragged_page_lists_match_table(case, S, wgs):
    dtype, H, block, lens, qlens, causal, sinks = case
    _print_case(f"ragged-pages S={S} wgs={wgs} {case}")
    w = mi.make_workload(name="rp", seq_lens=lens, num_heads=H, block_size=block, dtype=dtype,
                         qlens=qlens, causal=causal, sinks=sinks, seed=7000 + H + block)
    wr = mi.as_ragged_pages(w)
    ref_o, ref_l = orc.mla_decode(wr)
    out, lse = _run(wr, S, wgs)
    assert_close(wr, out, lse, ref_o, ref_l)
    # the 2-D table form of the same batch gives the same bits
    out2, lse2 = _run(w, S, wgs)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


SPARSE = [
    # (dtype, H, counts, ctx)
    ("bf16", 16, [300, 0, 17, 300, 1, 299], 1000),
    ("bf16", 128, [256, 31, 0, 256], 600),
    ("fp8_e4m3", 16, [512, 5, 512, 0, 100], 2000),
    ("fp8_e4m3", 48, [200, 200, 1], 500),
    ("fp8_e4m3", 128, [333, 64, 2], 700),
    ("bf16", 1, [64, 65, 3], 100),
]


@pytest.mark.parametrize("case", SPARSE, ids=lambda c: f"{c[0]}-H{c[1]}-n{len(c[2])}")
@pytest.mark.parametrize("S,wgs", [(None, 0), (None, 2), (0, 0), (2, 0)])
def test_sparse_index_stream_parity(case, S, wgs):
    dtype, H, counts, ctx = case
    _print_case(f"sparse S={S} wgs={wgs} {case}")
    w = mi.sparse_batch(num_tokens=len(counts), topk=max(counts), ctx=ctx, num_heads=H, dtype=dtype,
                        counts=counts, seed=8000 + H)
    ref_o, ref_l = orc.mla_decode(w)
    out, lse = _run(w, S, wgs)
    assert_close(w, out, lse, ref_o, ref_l)
    empty = [t for t, c in enumerate(counts) if c == 0]
    for t in empty:  # sink mass only
        assert np.all(out[t] == 0) and np.allclose(lse[t], w.sinks, atol=0, rtol=0)
