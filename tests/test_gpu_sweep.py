"""GPU parity over a seeded sweep of option combinations.

The named cases in test_gpu_parity.py pin the workloads and the known edge
shapes; this sweep draws further small problems from the whole space the C ABI
accepts (dtype, head dim, causal, P-quant format or none, per-token Q/K/V
codes, fp8 V, K smoothing, ragged lengths, the workspace or the static-scratch
backward), so that combinations no named case happens to pair are compared
with the oracle too.  The draw is fixed (seeded): every run tests the same
cases, and a failing id names the options to reproduce it.
"""
from __future__ import annotations

import random

import numpy as np
import pytest

from quantization_aware_attention_amd import workloads as W
from tests._harness import assert_within, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

BASE = W.WORKLOADS["dit_image"].with_(k_offset_var=0.0)


def _draw(n: int, seed: int = 20261202):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n:
        D = rng.choice([64, 128])
        dtype = rng.choice(["bf16", "fp16"])
        causal = rng.random() < 0.35
        Nq = rng.randint(1, 260)
        Nkv = Nq if causal else rng.randint(1, 260)
        p_quant = rng.random() < 0.85
        p_fmt = rng.choice(["e4m3", "e5m2"])
        qkv = rng.random() < 0.35
        vfp8 = dtype == "bf16" and not qkv and rng.random() < 0.3
        smooth = rng.random() < 0.25
        entry = rng.choice(["workspace", "noalloc"])
        w = BASE.with_(B=rng.choice([1, 2]), H=rng.choice([1, 2, 3]), Nq=Nq, Nkv=Nkv, D=D, dtype=dtype,
                       causal=causal, p_fmt=p_fmt, qkv_quant=qkv, v_fp8=vfp8, smooth_k=smooth,
                       k_offset_var=1.0 if smooth else 0.0, seed=3000 + len(cases))
        name = (f"{dtype}_d{D}_{'causal_' if causal else ''}{Nq}x{Nkv}_B{w.B}H{w.H}_"
                f"{p_fmt if p_quant else 'nopq'}{'_qkv' if qkv else ''}{'_fp8v' if vfp8 else ''}"
                f"{'_smoothk' if smooth else ''}_{entry}")
        cases.append((name, w, p_quant, entry))
    return cases


CASES = _draw(80)


@pytest.mark.parametrize("name,w,p_quant,entry", CASES, ids=[c[0] for c in CASES])
def test_sweep_matches_oracle(name, w, p_quant, entry):
    print(f"case {name}: {w}", flush=True)
    inp = W.make_inputs(w)
    gpu = run_gpu(w, inp, p_quant=p_quant, bwd_entry=entry)
    ref = run_oracle(w, inp, p_quant=p_quant)
    if w.v_fp8:
        assert np.array_equal(gpu["v_codes"], ref["v_codes"])
        assert np.array_equal(gpu["v_scale"], ref["v_scale"])
    assert_within(compare(gpu, ref), name)
