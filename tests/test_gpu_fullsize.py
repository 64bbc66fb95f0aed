"""Parity at full size, in the launch configuration the benchmark times.

Each workload is built at its real shape (52 requests x 16384 tokens, the
128-request ragged causal batch, or 52 index-stream tokens of 2048 rows) and
decoded on the GPU with the balanced split through one prepared
``mla_decode`` call, bf16 output (the call ``bench.py`` times for its
headline).  The fp64 oracle then computes a sample of the requests one by
one, and the outputs of every token row of those requests are compared at
the decode tolerances.  The fused call on the planner's segment partition
(merged output) and the segment partials of the same sample are checked
too.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mla_inputs as mi
from gpu_helpers import LSE_TOL, assert_close, out_tol, vmax
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu

FULL = {
    "bs52_ctx16k_h16_bf16_blk64": lambda: mi.bs52_h16_bf16(),
    "bs52_ctx16k_h16_fp8_blk64": lambda: mi.bs52_fp8(16),
    "bs52_ctx16k_h48_fp8_blk64": lambda: mi.bs52_fp8(48),
    "bs52_ctx16k_h64_fp8_blk64": lambda: mi.bs52_fp8(64),
    "bs52_ctx16k_h128_bf16_blk256": lambda: mi.bs52_h128_bf16(),
    "ragged128_max32k_h96_fp8_causal_sinks": lambda: mi.ragged_h96_fp8(),
    "sparse_bs52_top2048_ctx16k_h16_bf16": lambda: mi.sparse_bs52(16, "bf16"),
    "sparse_bs52_top2048_ctx16k_h128_fp8": lambda: mi.sparse_bs52(128, "fp8_e4m3"),
}


def _sample(w, k=4, seed=0):
    """First, last and a few random requests; for a ragged batch also the
    longest, the shortest and one with the largest qlen."""
    R = w.num_reqs
    pick = {0, R - 1}
    lens = np.asarray(w.seq_lens)
    qlens = np.diff(np.asarray(w.qo_indptr))
    pick.add(int(np.argmax(lens)))
    pick.add(int(np.argmin(lens)))
    pick.add(int(np.argmax(qlens)))
    g = np.random.default_rng(seed)
    pick.update(int(x) for x in g.choice(R, size=min(k, R), replace=False))
    return sorted(pick)


def _tokens(w, reqs):
    qo = np.asarray(w.qo_indptr)
    return np.concatenate([np.arange(qo[r], qo[r + 1]) for r in reqs])


@pytest.mark.parametrize("name", sorted(FULL))
def test_fullsize_sampled_parity(name):
    import mla_paged_decode_02_amd as m

    w = FULL[name]()
    print(f"[fullsize] {name}: T={w.num_tokens} H={w.num_heads} {w.kv_dtype}", flush=True)
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d)
    dec = m.Decoder(**args, sinks=d["sinks"], schedule="balanced", out_dtype=torch.bfloat16)
    out, lse = dec.run()
    torch.cuda.synchronize()
    # The segment partition the planner picks for the same batch.
    S = m.resolve_num_segments(m.make_problem(**args))
    out = out.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(out).all()

    reqs = _sample(w)
    db = orc.decode_workload(w, reqs)
    ref_o, ref_l = orc.mla_decode(w, reqs, db)
    tok = _tokens(w, reqs)
    err_o, err_l = assert_close(w, out, lse, ref_o, ref_l, reqs=reqs, tok=tok)
    print(f"[fullsize] {name}: split={dec.split} S={S} reqs={reqs} max|dO|={err_o:.3e} "
          f"max|dLSE|={err_l:.3e}", flush=True)
    del out, lse

    # The fused call on the planner's segment partition: merged output of the
    # same sample.
    dseg = m.Decoder(**args, sinks=d["sinks"], num_segments=0, out_dtype=torch.bfloat16)
    assert dseg.split is None and dseg.num_segments == S
    out_s, lse_s = dseg.run()
    torch.cuda.synchronize()
    out_s = out_s.float().cpu().numpy().astype(np.float64)
    lse_s = lse_s.cpu().numpy().astype(np.float64)
    assert np.isfinite(out_s).all()
    err_o, err_l = assert_close(w, out_s, lse_s, ref_o, ref_l, reqs=reqs, tok=tok)
    print(f"[fullsize] {name}: segments S={S} max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    del out_s, lse_s, dseg

    # Segment partials of the same sample, same segment count and tile.
    tile = w.tile_size or m.tile_size_for_block(w.block_size)
    so, sm, se = m.decode_segments(**args, num_segments=S)
    torch.cuda.synchronize()
    so_ref, sm_ref, se_ref, valid, _ = orc.mla_decode_segments(w, S, tile, reqs, db)
    tol_o = out_tol(w) * vmax(w, reqs)
    sel = torch.from_numpy(tok).to(so.device)
    so_s, sm_s, se_s = (x.index_select(0, sel).cpu().numpy() for x in (so, sm, se))
    for i, t in enumerate(tok):
        v = valid[t]
        gm, gs, go = sm_s[i][:, v], se_s[i][:, v], so_s[i][:, v]
        rm, rs, ro = sm_ref[t][:, v], se_ref[t][:, v], so_ref[t][:, v]
        fin = np.isfinite(rm)
        assert np.array_equal(fin, np.isfinite(gm)), f"token {t}: masked-segment pattern differs"
        assert np.all(gs[~fin] == 0) and np.all(go[~fin] == 0)
        # base-2 max: the LSE tolerance in base-2 units
        assert np.abs(gm[fin] - rm[fin]).max(initial=0) <= LSE_TOL / orc.LOGE2
        assert np.abs(gs[fin] / rs[fin] - 1).max(initial=0) <= 1e-3
        # normalised per-segment output
        no = go[fin] / gs[fin][:, None]
        nr = ro[fin] / rs[fin][:, None]
        assert np.abs(no - nr).max(initial=0) <= tol_o
    del so, sm, se, dec, d
    torch.cuda.empty_cache()
