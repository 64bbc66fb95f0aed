"""mla_decode_no_alloc (static device scratch) against mla_decode (caller
workspace), through the C ABI, on two calls in a row with the second batch
smaller than the first, for both schedules.  The two entry points run the
same kernels on the same partition, so the results are equal bit for bit;
they are also held to the oracle's tolerances."""
import ctypes

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


def _no_alloc(m, w, d, schedule):
    args = mi.call_args(w, d)
    p = m.make_problem(**args, schedule=schedule)
    out = torch.full((w.num_tokens, w.num_heads, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.num_tokens, w.num_heads), float("nan"), dtype=torch.float32, device="cuda")
    st = m.lib().mla_decode_no_alloc(ctypes.byref(p), m._ptr(d["sinks"]), out.data_ptr(), m.MLA_DTYPE_FP32,
                                     lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == m.MLA_OK, m.lib().mla_last_error().decode()
    return out, lse


@pytest.mark.parametrize("schedule", ["segments", "balanced"])
@pytest.mark.parametrize("dtype,H,block", [("bf16", 16, 64), ("fp8_e4m3", 64, 64), ("bf16", 128, 256)])
def test_no_alloc_matches_workspace_call(dtype, H, block, schedule):
    import mla_paged_decode_02_amd as m
    batches = [
        dict(seq_lens=[3000, 17, 5000, 640], qlens=[1, 2, 1, 3], seed=11),   # first call
        dict(seq_lens=[700, 1], qlens=[2, 1], seed=12),                    # second, smaller
    ]
    for i, b in enumerate(batches):
        print(f"[case] no-alloc {dtype} H={H} {schedule} call {i}", flush=True)
        w = mi.make_workload(name="noalloc", seq_lens=b["seq_lens"], qlens=b["qlens"], num_heads=H,
                             block_size=block, dtype=dtype, causal=True, sinks=True, seed=b["seed"] + H)
        d = mi.to_torch(w, "cuda")
        need = m.workspace_bytes(m.make_problem(**mi.call_args(w, d), schedule=schedule))
        assert need <= m.NO_ALLOC_SCRATCH_BYTES
        o1, l1 = _no_alloc(m, w, d, schedule)
        o2, l2 = m.decode(**mi.call_args(w, d), sinks=d["sinks"], schedule=schedule, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"call {i}: differs from mla_decode"
        ref_o, ref_l = orc.mla_decode(w)
        assert_close(w, o1.cpu().numpy().astype(np.float64), l1.cpu().numpy().astype(np.float64), ref_o, ref_l)
