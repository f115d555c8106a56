"""GPU chunked-KV mode: forward per KV chunk + qat_attn_merge, backward per
chunk with the merged lse and O_hp + qat_attn_sum of the dQ parts, against
the float64 oracle (unchunked) and the unchunked GPU run.  Bars as in the
parity contract (O_hp 5e-3, O / dQ / dK / dV 1e-2 rel-L2, lse 1e-3)."""
import numpy as np
import pytest
import torch

from oracle import qat_attention as oracle
from quantization_aware_attention_amd import ops
from quantization_aware_attention_amd import workloads as W
from tests._harness import TOL, rel_l2, run_gpu, run_oracle, to_dev, to_np

pytestmark = pytest.mark.gpu

BASE = W.WORKLOADS["dit_image"].with_(k_offset_var=0.0)


def test_merge_kernel_matches_oracle():
    rng = np.random.default_rng(41)
    B, H, N, D, C = 1, 3, 70, 128, 3
    o = [rng.standard_normal((B, H, N, D)) for _ in range(C)]
    oh = [rng.standard_normal((B, H, N, D)) for _ in range(C)]
    lse = [rng.standard_normal((B, H, N)) * 3 for _ in range(C)]
    lse[0][0, 0, 5] = -np.inf                       # masked in one chunk
    for c in range(C):
        lse[c][0, 1, 7] = -np.inf                   # masked in every chunk
    ob = [W.round_to_dtype(x, "bf16") for x in o]
    ohb = [W.round_to_dtype(x, "bf16") for x in oh]
    print("merge case: bf16 B1 H3 N70 D128, 3 chunks", flush=True)
    mo, moh, ml = ops.attn_merge([to_dev(b, "bf16") for _, b in ob], [to_dev(b, "bf16") for _, b in ohb],
                                 [torch.from_numpy(x.astype(np.float32)).cuda() for x in lse])
    torch.cuda.synchronize()
    Ro, Roh, Rl = oracle.merge_chunks([v for v, _ in ob], [v for v, _ in ohb], lse)
    mo, moh, ml = to_np(mo), to_np(moh), to_np(ml)
    assert ml[0, 1, 7] == -np.inf and not mo[0, 1, 7].any() and not moh[0, 1, 7].any()
    fin = np.isfinite(Rl)
    assert np.max(np.abs(ml[fin] - Rl[fin])) < 1e-5
    assert rel_l2(mo, Ro) < 5e-3 and rel_l2(moh, Roh) < 5e-3


def test_sum_kernel():
    rng = np.random.default_rng(42)
    parts = [W.round_to_dtype(rng.standard_normal((2, 2, 33, 64)), "fp16") for _ in range(4)]
    print("sum case: fp16 B2 H2 N33 D64, 4 parts", flush=True)
    out = to_np(ops.attn_sum([to_dev(b, "fp16") for _, b in parts]))
    ref = sum(v.astype(np.float64) for v, _ in parts)
    assert rel_l2(out, ref) < 1e-3


def test_merge_rejects_too_many_chunks():
    t = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    l = torch.zeros(1, 1, 8, dtype=torch.float32, device="cuda")
    with pytest.raises(ops.QatError):
        ops.attn_merge([t] * (ops.QAT_MERGE_MAX_CHUNKS + 1), [t] * (ops.QAT_MERGE_MAX_CHUNKS + 1),
                       [l] * (ops.QAT_MERGE_MAX_CHUNKS + 1))


@pytest.mark.parametrize("bounds", [[(0, 128), (128, 320)], [(0, 64), (64, 192), (192, 256), (256, 320)]])
def test_chunked_forward_backward(bounds):
    w = BASE.with_(B=1, H=2, Nq=200, Nkv=320, seed=43)
    print(f"chunked case: {w} chunks {bounds}", flush=True)
    inp = W.make_inputs(w)
    q, k, v, do = (to_dev(inp[n + "_bits"], w.dtype) for n in ("q", "k", "v", "do"))
    parts = [ops.attn_fwd(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), w.sm_scale) for a, b in bounds]
    o, o_hp, lse = ops.attn_merge([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
    dq_parts, dk, dv = [], [], []
    for a, b in bounds:
        dqc, dkc, dvc = ops.attn_bwd(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), o_hp, lse, do,
                                     w.sm_scale)
        dq_parts.append(dqc)
        dk.append(dkc)
        dv.append(dvc)
    dq = ops.attn_sum(dq_parts)
    torch.cuda.synchronize()
    got = {"o": to_np(o), "o_hp": to_np(o_hp), "lse": to_np(lse), "dq": to_np(dq),
           "dk": np.concatenate([to_np(t) for t in dk], axis=2), "dv": np.concatenate([to_np(t) for t in dv], axis=2)}
    ref = run_oracle(w, inp)
    whole = run_gpu(w, inp)
    for n in ("o", "o_hp", "dq", "dk", "dv"):
        assert rel_l2(got[n], ref[n]) <= TOL[n], (n, rel_l2(got[n], ref[n]))
        assert rel_l2(got[n], whole[n]) <= TOL[n], (n, "vs unchunked", rel_l2(got[n], whole[n]))
    assert np.max(np.abs(got["lse"] - ref["lse"])) <= TOL["lse"]
