"""Helpers shared by the GPU parity tests: run one workload through the HIP
library (via the ctypes binding) and through the float64 oracle on the same
seeded inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

from oracle import qat_attention as oracle
from quantization_aware_attention_amd import workloads as W

# Tolerances of the parity contract (rel-L2 over the compared tensor; LSE
# absolute).  O may flip single fp8 bins where accumulation order differs, so
# it gets the looser bound.
TOL = {"o": 1e-2, "o_hp": 5e-3, "lse": 1e-3, "dq": 1e-2, "dk": 1e-2, "dv": 1e-2}

TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def flags_of(w: W.Workload, p_quant=True) -> int:
    from quantization_aware_attention_amd import ops
    f = 0
    if p_quant:
        f |= ops.QAT_P_QUANT
        if w.p_fmt == "e5m2":
            f |= ops.QAT_P_E5M2
    if w.qkv_quant:
        f |= ops.QAT_QKV_QUANT
    if w.v_fp8:
        f |= ops.QAT_V_FP8_E5M2
    if w.smooth_k:
        f |= ops.QAT_SMOOTH_K
    return f


def to_dev(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DT[dtype]).cuda()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(x, y) -> float:
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / den) if den > 0 else float(np.linalg.norm(x - y))


def run_gpu(w: W.Workload, inp: dict, p_quant=True, backward=True, bwd_entry="workspace"):
    """Forward (+ backward) on the GPU; returns dict of numpy float64 arrays
    plus the fp8 V codes / scales when V is fp8.  bwd_entry "noalloc" runs
    the backward through qat_attn_bwd_noalloc (static scratch, P-quant
    absmax formed inside the dK/dV kernel)."""
    from quantization_aware_attention_amd import ops
    q = to_dev(inp["q_bits"], w.dtype)
    k = to_dev(inp["k_bits"], w.dtype)
    v = to_dev(inp["v_bits"], w.dtype)
    do = to_dev(inp["do_bits"], w.dtype)
    flags = flags_of(w, p_quant)
    v_scale = None
    out = {}
    if w.v_fp8:
        v, v_scale = ops.quant_v_fp8(v)
        out["v_codes"] = v.cpu().numpy()
        out["v_scale"] = v_scale.cpu().numpy()
    o, o_hp, lse = ops.attn_fwd(q, k, v, w.sm_scale, w.causal, flags, v_scale=v_scale)
    res = {"o": o, "o_hp": o_hp, "lse": lse}
    if backward:
        bwd = ops.attn_bwd_noalloc if bwd_entry == "noalloc" else ops.attn_bwd
        dq, dk, dv = bwd(q, k, v, o_hp, lse, do, w.sm_scale, w.causal, flags, v_scale=v_scale)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    out.update({n: to_np(t) for n, t in res.items()})
    return out


def run_oracle(w: W.Workload, inp: dict, p_quant=True, backward=True, heads=None,
               q_rows=None, k_rows=None):
    """Oracle forward (+ backward) for the (b, h) pairs ``heads`` and the
    sampled query / key rows.  Returns arrays restricted the same way."""
    v_codes = v_scale = None
    if w.v_fp8:
        v_codes, v_scale = oracle.quantize_v_channels(inp["v"], "e5m2")
    kw = dict(causal=w.causal, p_quant=p_quant, p_fmt=w.p_fmt, qkv_quant=w.qkv_quant,
              v_codes=v_codes, v_scale=v_scale, heads=heads, smooth_k=w.smooth_k, dtype=w.dtype)
    O, O_hp, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], w.sm_scale, rows=q_rows, **kw)
    res = {"o": O, "o_hp": O_hp, "lse": lse, "v_codes": v_codes, "v_scale": v_scale}
    if backward:
        dq, dk, dv = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], w.sm_scale,
                                               q_rows=q_rows, k_rows=k_rows, **kw)
        res.update(dq=dq, dk=dk, dv=dv)
    return res


def compare(gpu: dict, ref: dict, heads=None, q_rows=None, k_rows=None, names=None):
    """Per-output error over the compared subset: rel-L2 pooled over every
    compared head (``name``) and the largest rel-L2 of a single (b, h) head
    (``name@head``), so that one wrong head among many is not diluted; LSE is
    max-abs (pooled and per head alike)."""
    errs = {}
    names = names or [n for n in ("o", "o_hp", "lse", "dq", "dk", "dv") if n in ref]
    for n in names:
        g = gpu[n]
        r = ref[n]
        rows = k_rows if n in ("dk", "dv") else q_rows
        if heads is not None:
            g = np.stack([g[b, h] for b, h in heads])
            r = np.stack([r[b, h] for b, h in heads])
        else:
            g = g.reshape((-1,) + g.shape[2:])
            r = r.reshape((-1,) + r.shape[2:])
        if rows is not None:   # the oracle's arrays are already restricted to the rows
            g = g[:, rows]
        if n == "lse":
            errs[n] = float(np.max(np.abs(g - r))) if g.size else 0.0
        else:
            errs[n] = rel_l2(g, r)
            if g.shape[0] > 1:
                errs[n + "@head"] = max(rel_l2(g[i], r[i]) for i in range(g.shape[0]))
    return errs


def assert_within(errs: dict, what: str):
    """Every error within its bar; a per-head maximum takes the bar of its
    tensor."""
    bad = {n: e for n, e in errs.items() if not (e <= TOL[n.split("@")[0]])}
    msg = f"{what}: " + ", ".join(f"{n}={e:.3e}" for n, e in errs.items())
    print(msg, flush=True)
    assert not bad, msg
