"""Seeded random launch shapes against the fp64 oracle (run with -m gpu).

Each case draws a dtype, a head count (1-128, including counts that leave
row groups or waves empty), a page size (1-256), up to six requests of
random length (0 and 1 included), optional query ranges with or without the
causal mask, optional sinks, the schedule, the segment count and the output
dtype, from a generator seeded by the case number, and compares the fused
decode through the C ABI with the oracle at the usual tolerances.  The
shapes stay small, so the oracle takes milliseconds per case.
"""
import random

import pytest
import torch

import mla_inputs as mi
from oracle import mla_oracle as orc

from gpu_helpers import assert_close, run_decode

pytestmark = pytest.mark.gpu

HEADS = [1, 3, 7, 16, 16, 20, 28, 33, 40, 48, 52, 64, 64, 80, 96, 100, 128, 128]
BLOCKS = [1, 8, 16, 32, 48, 64, 64, 96, 128, 256]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import mla_paged_decode_02_amd as m
    m.lib()  # the HIP library must load; no fallback exists


def draw(case: int) -> dict:
    rng = random.Random(7919 * case + 17)
    dtype = rng.choice(["bf16", "fp8_e4m3"])
    H = rng.choice(HEADS)
    block = rng.choice(BLOCKS)
    R = rng.randint(1, 6)
    maxlen = 2500 if H <= 64 else 1200
    lens = [rng.choice([0, 1, rng.randint(1, 40), rng.randint(1, maxlen), rng.randint(1, maxlen)])
            for _ in range(R)]
    qlens = [rng.randint(1, 4) for _ in range(R)] if rng.random() < 0.5 else None
    causal = qlens is not None and rng.random() < 0.7
    if causal:
        lens = [max(n, q) for n, q in zip(lens, qlens)]
    schedule = rng.choice(["segments", "balanced"])
    return dict(dtype=dtype, H=H, block=block, lens=lens, qlens=qlens, causal=causal,
                sinks=rng.random() < 0.5, schedule=schedule,
                S=rng.choice([0, 0, 1, 2, 3, 5, 8]) if schedule == "segments" else 0,
                out_dtype=rng.choice([torch.float32, torch.bfloat16]))


@pytest.mark.parametrize("case", range(64))
def test_random_shape(case):
    c = draw(case)
    print(f"[case] random shape {case}: {c}", flush=True)
    w = mi.make_workload(name=f"random{case}", seq_lens=c["lens"], num_heads=c["H"], block_size=c["block"],
                         dtype=c["dtype"], qlens=c["qlens"], causal=c["causal"], sinks=c["sinks"],
                         seed=50000 + case)
    ref_o, ref_l = orc.mla_decode(w)
    out, lse = run_decode(w, num_segments=c["S"], schedule=c["schedule"], out_dtype=c["out_dtype"])
    assert_close(w, out, lse, ref_o, ref_l)
