"""Shared helpers of the GPU parity tests: run the HIP library on a workload
and compare with the fp64 oracle at the tolerances of the decode contract
(output max-abs <= 1e-2 * max|V| for bf16, 3e-2 * max|V| for fp8; LSE
max-abs <= 1e-3; partition indexing bit-exact)."""
from __future__ import annotations

import numpy as np
import torch

import mla_inputs as mi
from oracle import mla_oracle as orc

LSE_TOL = 1e-3


def out_tol(w) -> float:
    return 3e-2 if w.kv_dtype == "fp8_e4m3" else 1e-2


def vmax(w, reqs=None) -> float:
    """max |V| over the dequantised rows the batch (or `reqs`) reads."""
    bsz = w.block_size
    flat = w.kv_cache.reshape(-1, 576)
    best = 0.0
    for r in (range(w.num_reqs) if reqs is None else reqs):
        n = int(w.seq_lens[r])
        if n == 0:
            continue
        pages = orc.pages_of(np.asarray(w.block_table), w.bt_indptr, r)
        idx = np.array([orc.cache_row_index(pages, j, bsz) for j in range(n)])
        v = orc.decode(flat[idx][:, :512], w.kv_dtype, w.kv_scale)
        best = max(best, float(np.abs(v).max()))
    return best


def run_decode(w, *, num_segments=None, out_dtype=torch.float32, use_indptr=None, sinks=True,
               schedule="segments"):
    import mla_paged_decode_02_amd as m
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d, use_indptr=use_indptr)
    S = w.num_segments if num_segments is None else num_segments
    out, lse = m.decode(**args, sinks=d["sinks"] if sinks else None, num_segments=S,
                        out_dtype=out_dtype, schedule=schedule)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_segments(w, num_segments, tile):
    import mla_paged_decode_02_amd as m
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d)
    args["tile_size"] = tile
    so, sm, se = m.decode_segments(**args, num_segments=num_segments)
    torch.cuda.synchronize()
    return so.cpu().numpy(), sm.cpu().numpy(), se.cpu().numpy(), d


def assert_close(w, out, lse, ref_o, ref_l, reqs=None, tok=None):
    """Compare rows `tok` (default all) of out/lse with the oracle."""
    tol_o = out_tol(w) * max(vmax(w, reqs), 1e-30)
    sel = slice(None) if tok is None else tok
    o, l, ro, rl = out[sel], lse[sel], ref_o[sel], ref_l[sel]
    assert np.isfinite(o).all(), "non-finite output"
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(l)), "finite/-inf pattern of LSE differs"
    assert np.array_equal(rl[~fin], l[~fin])
    err_o = float(np.abs(o - ro).max()) if o.size else 0.0
    err_l = float(np.abs(l[fin] - rl[fin]).max()) if fin.any() else 0.0
    assert err_o <= tol_o, f"output max-abs {err_o:.3e} > {tol_o:.3e}"
    assert err_l <= LSE_TOL, f"LSE max-abs {err_l:.3e} > {LSE_TOL}"
    return err_o, err_l
