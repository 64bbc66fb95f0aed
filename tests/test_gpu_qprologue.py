"""The fused q prologue on the GPU: q handed over as (q_nope, q_pe), and a
bf16 q quantised to e4m3 in the q load when the cache is fp8.

* Split q (views of one tensor or two separate tensors) gives the bits of
  the concatenated q.
* bf16 q with an fp8 cache matches the fp64 oracle, which quantises q first.
* The quantised codes themselves are recovered exactly: single-key requests
  whose key is one-hot in one dim make the LSE equal to
  softmax_scale * q_scale * value(code), so each code is read back and
  compared with the oracle's quantiser.
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


CASES = [
    # (dtype, H, block, lens, qlens, causal)
    ("bf16", 16, 64, [3000, 1, 700], None, False),
    ("bf16", 128, 256, [1300, 200], None, False),
    ("fp8_e4m3", 48, 64, [900, 44, 3000], [1, 4, 2], True),
    ("fp8_e4m3", 16, 16, [500, 33], None, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-H{c[1]}")
@pytest.mark.parametrize("S", [0, 3])
@pytest.mark.parametrize("views", [True, False])
def test_split_q_gives_the_concatenated_bits(case, S, views):
    import mla_paged_decode_02_amd as m
    dtype, H, block, lens, qlens, causal = case
    _print_case(f"split-q S={S} views={views} {case}")
    w = mi.make_workload(name="sq", seq_lens=lens, num_heads=H, block_size=block, dtype=dtype,
                         qlens=qlens, causal=causal, sinks=True, seed=9500 + H)
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d)
    o1, l1 = m.decode(**args, sinks=d["sinks"], num_segments=S, out_dtype=torch.float32)
    q = args.pop("q")
    qn, qp = (q[..., :512], q[..., 512:]) if views else (q[..., :512].contiguous(), q[..., 512:].contiguous())
    o2, l2 = m.decode(q=qn, q_pe=qp, **args, sinks=d["sinks"], num_segments=S, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("H", [16, 64, 128])
@pytest.mark.parametrize("S", [0, 2])
@pytest.mark.parametrize("split_q", [False, True])
def test_bf16_q_with_fp8_cache_parity(H, S, split_q):
    import mla_paged_decode_02_amd as m
    _print_case(f"bf16-q fp8-cache H={H} S={S} split_q={split_q}")
    w = mi.make_workload(name="bq", seq_lens=[2000, 64, 1, 777], num_heads=H, block_size=64,
                         dtype="fp8_e4m3", qlens=[1, 3, 1, 2], causal=True, sinks=True, seed=9600 + H)
    w = mi.with_bf16_q(w, seed=H)
    ref_o, ref_l = orc.mla_decode(w)
    d = mi.to_torch(w, "cuda")
    args = mi.call_args(w, d)
    assert args["q"].dtype == torch.bfloat16 and args["kv_cache"].dtype == torch.float8_e4m3fn
    if split_q:
        q = args.pop("q")
        args.update(q=q[..., :512].contiguous(), q_pe=q[..., 512:].contiguous())
    out, lse = m.decode(**args, sinks=d["sinks"], num_segments=S, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l)


@pytest.mark.parametrize("S", [0, 1])
def test_quantised_q_codes_are_exact(S):
    import mla_paged_decode_02_amd as m
    _print_case(f"q codes S={S}")
    T, H, q_scale = 96, 8, 0.5
    w = mi.make_workload(name="qc", seq_lens=[1] * T, num_heads=H, block_size=16, dtype="fp8_e4m3",
                         seed=77, poison=False)
    dims = np.array([(9 * t + 5) % 576 for t in range(T)])
    flat = w.kv_cache.reshape(-1, 576)
    for t in range(T):  # request t's only key: 1.0 in dim dims[t], 0 elsewhere
        row = orc.cache_row_index(w.block_table[t], 0, w.block_size)
        flat[row] = 0
        flat[row, dims[t]] = 0x38  # e4m3 code of 1.0
    # q values: ties between codes (after the division), subnormal range,
    # saturation, and N(0,1) draws
    table = orc._E4M3_TABLE
    vals = np.unique(np.array([table[c] for c in range(256) if np.isfinite(table[c])]))
    ties = (vals[1:] + vals[:-1]) / 2
    g = np.random.default_rng(8)
    qv = (g.standard_normal((T, H, 576)) * 2).astype(np.float32)
    special = np.concatenate([ties[::7], [600.0, -700.0, 2.0 ** -10, -(2.0 ** -8) * 3]])
    for t in range(T):
        for h in range(H):
            qv[t, h, dims[t]] = special[(t * H + h) % len(special)] * q_scale
    w = mi.with_bf16_q(mi.with_(w, kv_scale=1.0), q_values=qv, q_scale=q_scale)
    d = mi.to_torch(w, "cuda")
    _, lse = m.decode(**mi.call_args(w, d), num_segments=S, out_dtype=torch.float32)
    torch.cuda.synchronize()
    lse = lse.cpu().numpy().astype(np.float64)
    codes = orc.quantize_e4m3(orc.decode_bf16(w.q), q_scale)
    got = lse / (w.softmax_scale * q_scale)
    for t in range(T):
        exp = table[codes[t, :, dims[t]]]
        nearest = vals[np.abs(vals[None, :] - got[t][:, None]).argmin(axis=1)]
        assert np.array_equal(nearest, exp), (t, got[t], exp)
        assert np.abs(got[t] - exp).max() <= 1e-5 * max(1.0, np.abs(exp).max())
