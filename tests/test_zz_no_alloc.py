"""qat_attn_bwd_noalloc (the backward on the library's static device scratch,
for callers that cannot allocate) against qat_attn_bwd on a caller workspace,
through the C ABI: two calls in a row, the second on a smaller problem (the
scratch then holds the first call's data).  dQ must be bitwise equal (same
kernels, same order); dK and dV may differ only by the fp32 summation order of
key blocks that qat_attn_bwd splits over query ranges, which can flip the
bf16 rounding of single elements there (bar: rel-L2 <= 1e-3, against 1e-2
for parity with the oracle, and most elements bitwise equal)."""
import numpy as np
import pytest
import torch

from quantization_aware_attention_amd import ops
from quantization_aware_attention_amd import workloads as W
from tests._harness import flags_of, rel_l2, to_dev, to_np

pytestmark = pytest.mark.gpu

BASE = W.WORKLOADS["dit_image"].with_(k_offset_var=0.0)
CASES = [
    # 24 heads x 36 key blocks of 128: 864 blocks, so qat_attn_bwd splits the
    # last ones over query ranges and the static path runs them whole
    BASE.with_(B=1, H=24, Nq=4608, Nkv=4608, seed=71),
    BASE.with_(B=1, H=2, Nq=200, Nkv=200, D=64, dtype="fp16", causal=True, p_fmt="e5m2", seed=72),
]


def _run(w):
    inp = W.make_inputs(w)
    q, k, v, do = (to_dev(inp[n + "_bits"], w.dtype) for n in ("q", "k", "v", "do"))
    flags = flags_of(w, True)
    o, o_hp, lse = ops.attn_fwd(q, k, v, w.sm_scale, w.causal, flags)
    ref = ops.attn_bwd(q, k, v, o_hp, lse, do, w.sm_scale, w.causal, flags)
    got = ops.attn_bwd_noalloc(q, k, v, o_hp, lse, do, w.sm_scale, w.causal, flags)
    torch.cuda.synchronize()
    return [to_np(t) for t in ref], [to_np(t) for t in got]


def test_noalloc_matches_workspace_backward_twice():
    for i, w in enumerate(CASES):
        print(f"no-alloc call {i}: {w}", flush=True)
        (dq, dk, dv), (dq2, dk2, dv2) = _run(w)
        assert np.array_equal(dq, dq2), "dq"
        for name, a, b in (("dk", dk, dk2), ("dv", dv, dv2)):
            e = rel_l2(b, a)
            print(f"  {name}: rel-L2 {e:.2e}", flush=True)
            assert e <= 1e-3, (name, e)
            assert np.mean(a != b) < 0.2, (name, np.mean(a != b))
        assert np.isfinite(dk2).all() and np.isfinite(dv2).all()


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    w = W.WORKLOADS["long_video"]
    q = torch.zeros((1, w.H, w.Nq, w.D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ops.QatError) as e:
        ops.attn_bwd_noalloc(q, q, q, q, torch.zeros(q.shape[:3], device="cuda"), q, w.sm_scale,
                             quant_flags=ops.QAT_P_QUANT | ops.QAT_QKV_QUANT)
    assert e.value.status == ops.QAT_ESCRATCH
