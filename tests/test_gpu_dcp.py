"""Decode context parallelism emulated on one GPU: key shards and their LSE
combine (``mla_combine_lse``).

Each shard of a batch (token t of a request on shard t % W) is decoded by the
library without sinks; ``mla_combine_lse`` merges the shard outputs by their
natural-log LSE and applies the sinks once.  The result must match the fp64
oracle's direct decode of the whole batch at the decode tolerances, and the
combine kernel alone must match the oracle's combine on arbitrary inputs.
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


@pytest.mark.parametrize("W", [1, 3, 8])
@pytest.mark.parametrize("H", [1, 16, 128])
@pytest.mark.parametrize("in_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("sinks", [False, True])
def test_combine_kernel_matches_oracle(W, H, in_dtype, sinks):
    import mla_paged_decode_02_amd as m
    _print_case(f"combine W={W} H={H} {in_dtype} sinks={sinks}")
    g = torch.Generator().manual_seed(100 * W + H)
    T = 5
    so = torch.randn((W, T, H, 512), generator=g).to(in_dtype)
    sl = torch.randn((W, T, H), generator=g) * 3
    sl[0, 1] = -np.inf               # shard 0 saw no key of token 1
    sl[:, 2, 0] = -np.inf            # no shard saw token 2, head 0
    if W > 1:
        sl[W - 1, 3, H - 1] = float("nan")
    sk = torch.randn(H, generator=g) if sinks else None
    out, lse = m.combine_lse(so.cuda(), sl.cuda(), sinks=None if sk is None else sk.cuda(),
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_o, ref_l = orc.combine_lse(so.float().numpy(), sl.numpy(), None if sk is None else sk.numpy())
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    nan = np.isnan(ref_l)
    assert np.array_equal(nan, np.isnan(lse)) and np.all(np.isnan(out[nan]))
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.array_equal(ref_l[~fin & ~nan], lse[~fin & ~nan])
    assert np.abs(lse[fin] - ref_l[fin]).max(initial=0) <= 1e-5
    assert np.abs(out[~nan] - ref_o[~nan]).max(initial=0) <= 1e-5 * max(1.0, np.abs(ref_o[~nan]).max())


DCP = [
    # (dtype, H, block, lens, qlens, causal)
    ("bf16", 16, 64, [3000, 1, 64, 700, 0], None, False),
    ("fp8_e4m3", 48, 64, [900, 44, 3000], [1, 4, 2], True),
    ("bf16", 128, 16, [1300, 200], None, False),
    ("bf16", 16, 16, [500, 2000, 7, 64], [1, 2, 3, 4], True),
]


@pytest.mark.parametrize("case", DCP, ids=lambda c: f"{c[0]}-H{c[1]}-blk{c[2]}-causal{c[5]}")
@pytest.mark.parametrize("W", [2, 4])
@pytest.mark.parametrize("shard_dtype", [torch.float32, torch.bfloat16])
def test_dcp_emulation_parity(case, W, shard_dtype):
    import mla_paged_decode_02_amd as m
    dtype, H, block, lens, qlens, causal = case
    _print_case(f"dcp W={W} {shard_dtype} {case}")
    w = mi.make_workload(name="dcp", seq_lens=lens, num_heads=H, block_size=block, dtype=dtype,
                         qlens=qlens, causal=causal, sinks=True, seed=9000 + H + block)
    ref_o, ref_l = orc.mla_decode(w)
    outs, lses = [], []
    for sw in mi.dcp_shards(w, W):
        d = mi.to_torch(sw, "cuda")
        o, l = m.decode(**mi.call_args(sw, d), sinks=None, schedule="balanced", out_dtype=shard_dtype)
        outs.append(o)
        lses.append(l)
    d = mi.to_torch(w, "cuda")
    out, lse = m.combine_lse(torch.stack(outs), torch.stack(lses), sinks=d["sinks"],
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                 ref_o, ref_l)
