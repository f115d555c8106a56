"""GPU parity of the HIP forward and backward against the float64 oracle.

Small cases compare every element at sizes that span several tiles and a
ragged tail; the five workloads run at their full sizes in the launch
configuration the benchmark uses, and are compared on sampled heads and rows
that the oracle computes one by one (heads are independent, rows of the
forward and dQ are independent; dK/dV of a sampled key needs every query, so
the oracle forms all rows of those heads).

Bars (written here, from the parity contract): O_hp rel-L2 <= 5e-3,
O <= 1e-2, dQ/dK/dV <= 1e-2, LSE max abs <= 1e-3.
"""
import numpy as np
import pytest
import torch

from quantization_aware_attention_amd import workloads as W
from tests._harness import assert_within, compare, rel_l2, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

BASE = W.WORKLOADS["dit_image"].with_(k_offset_var=0.0)

SMALL = {
    "tiny_probe_shape": W.WORKLOADS["tiny"],
    "bf16_d128_ragged": BASE.with_(B=1, H=2, Nq=300, Nkv=300, seed=11),
    "bf16_d128_causal_ragged": BASE.with_(B=2, H=1, Nq=333, Nkv=333, causal=True, seed=12),
    "fp16_d64_cross_ragged": BASE.with_(B=1, H=2, Nq=200, Nkv=130, D=64, dtype="fp16", seed=13),
    "bf16_d64_e5m2": BASE.with_(B=1, H=2, Nq=257, Nkv=257, D=64, p_fmt="e5m2", seed=14),
    "bf16_qkv_quant": BASE.with_(B=1, H=2, Nq=190, Nkv=190, qkv_quant=True, seed=15),
    "bf16_fp8v_nkv500": W.WORKLOADS["cross_fp8v"].with_(B=1, H=2, Nq=150, Nkv=500, seed=16),
    "bf16_fp8v_d64_ragged": W.WORKLOADS["cross_fp8v"].with_(B=1, H=2, Nq=300, Nkv=200, D=64, seed=29),
    "bf16_k_offset": W.WORKLOADS["dit_image"].with_(H=2, Nq=256, Nkv=256, seed=17),
    "fp16_causal_d128": BASE.with_(B=1, H=2, Nq=129, Nkv=129, dtype="fp16", causal=True, seed=18),
    "one_key": BASE.with_(B=1, H=1, Nq=70, Nkv=1, seed=19),
    "one_query": BASE.with_(B=1, H=2, Nq=1, Nkv=200, seed=20),
    "causal_one": BASE.with_(B=1, H=1, Nq=1, Nkv=1, causal=True, seed=21),
    "tile_aligned": BASE.with_(B=1, H=1, Nq=256, Nkv=128, seed=22),
    # per-token codes over many key tiles (the forward's key-scale buffers are
    # reused), in both kernels' other variants
    "bf16_qkv_quant_long_cross": BASE.with_(B=1, H=2, Nq=150, Nkv=900, qkv_quant=True, seed=31),
    "fp16_qkv_quant_causal_d64": BASE.with_(B=1, H=2, Nq=400, Nkv=400, D=64, dtype="fp16", causal=True,
                                            qkv_quant=True, seed=32),
    # 300 key blocks of 128: on 256 compute units, 256 run whole and the last
    # 44 are split over four query ranges whose partials are merged
    "many_heads_tail_split": BASE.with_(B=1, H=300, Nq=128, Nkv=128, seed=24),
    # K smoothing: plain, before the Q/K/V quantization, fp16 causal D64, fp8 V
    "smoothk_bf16": BASE.with_(B=1, H=3, Nq=200, Nkv=200, k_offset_var=2.0, smooth_k=True, seed=25),
    "smoothk_qkv_quant": BASE.with_(B=1, H=2, Nq=190, Nkv=190, qkv_quant=True, k_offset_var=2.0,
                                    smooth_k=True, seed=26),
    "smoothk_fp16_causal_d64": BASE.with_(B=2, H=1, Nq=130, Nkv=130, D=64, dtype="fp16", causal=True,
                                          k_offset_var=1.0, smooth_k=True, seed=27),
    "smoothk_fp8v": W.WORKLOADS["cross_fp8v"].with_(B=1, H=2, Nq=150, Nkv=500, k_offset_var=1.0,
                                                     smooth_k=True, seed=28),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_compare(name):
    w = SMALL[name]
    print(f"case {name}: {w}", flush=True)
    inp = W.make_inputs(w)
    gpu = run_gpu(w, inp)
    ref = run_oracle(w, inp)
    if w.v_fp8:
        assert np.array_equal(gpu["v_codes"], ref["v_codes"])
        assert np.array_equal(gpu["v_scale"], ref["v_scale"])
    assert_within(compare(gpu, ref), name)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_compare_in_kernel_absmax(name):
    # the same cases through the static-scratch backward, whose dK/dV kernel
    # forms the P-quant absmax of each (query, 64-key group) itself (as the
    # backward does for problems whose absmax record would exceed its bound)
    w = SMALL[name]
    print(f"case {name} (in-kernel absmax): {w}", flush=True)
    inp = W.make_inputs(w)
    gpu = run_gpu(w, inp, bwd_entry="noalloc")
    ref = run_oracle(w, inp)
    assert_within(compare(gpu, ref), name + " in-kernel absmax")


def test_p_quant_off_gives_identical_outputs():
    w = BASE.with_(B=1, H=2, Nq=200, Nkv=150, seed=23)
    inp = W.make_inputs(w)
    gpu = run_gpu(w, inp, p_quant=False)
    assert np.array_equal(gpu["o"], gpu["o_hp"])
    ref = run_oracle(w, inp, p_quant=False)
    assert_within(compare(gpu, ref), "p_quant_off")


def test_deterministic_bitwise():
    w = BASE.with_(B=1, H=2, Nq=300, Nkv=300, causal=True, seed=24)
    inp = W.make_inputs(w)
    a = run_gpu(w, inp)
    b = run_gpu(w, inp)
    for n in ("o", "o_hp", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("w", [BASE.with_(B=1, H=2, Nq=300, Nkv=260, seed=33),
                               BASE.with_(B=1, H=2, Nq=150, Nkv=200, D=64, dtype="fp16", causal=False, seed=34),
                               BASE.with_(B=2, H=1, Nq=200, Nkv=200, causal=True, qkv_quant=True, seed=35),
                               W.WORKLOADS["cross_fp8v"].with_(B=1, H=2, Nq=150, Nkv=300, seed=36)],
                         ids=["bf16_d128", "fp16_d64", "causal_qkv_quant", "fp8v"])
def test_backward_stages_match_the_whole_backward_bitwise(w):
    # With Delta and dQ in one call the dQ kernel forms Delta itself; run as
    # separate stages, the Delta pass does.  dK/dV read that Delta, so equal
    # bits everywhere show that both form it identically.
    from quantization_aware_attention_amd import ops
    from tests._harness import flags_of, to_dev, to_np
    print(f"stage split case: {w}", flush=True)
    inp = W.make_inputs(w)
    q, k, v, do = (to_dev(inp[n + "_bits"], w.dtype) for n in ("q", "k", "v", "do"))
    flags = flags_of(w, True)
    v_scale = None
    if w.v_fp8:
        v, v_scale = ops.quant_v_fp8(v)
    o, o_hp, lse = ops.attn_fwd(q, k, v, w.sm_scale, w.causal, flags, v_scale=v_scale)
    whole = ops.attn_bwd(q, k, v, o_hp, lse, do, w.sm_scale, w.causal, flags, v_scale=v_scale)
    dims = ops.dims_of(q, k)
    ws = torch.zeros(max(ops.workspace_bytes(dims, flags, 1), 256), device="cuda", dtype=torch.uint8)
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty(k.shape, device="cuda", dtype=q.dtype))
    for st in (ops.QAT_BWD_PREPARE | ops.QAT_BWD_DELTA, ops.QAT_BWD_DQ, ops.QAT_BWD_DKDV):
        ops.attn_bwd(q, k, v, o_hp, lse, do, w.sm_scale, w.causal, flags, v_scale=v_scale, out=out, workspace=ws,
                     stages=st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), whole, out):
        assert np.array_equal(to_np(a), to_np(b)), name


def test_empty_batch_is_a_no_op():
    from quantization_aware_attention_amd import ops
    q = torch.zeros((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    o, o_hp, lse = ops.attn_fwd(q, q, q, 0.125)
    assert o.numel() == 0
    q2 = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    k2 = torch.zeros((1, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    ops.attn_fwd(q2, k2, k2, 0.125)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- full sizes
def _sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    pick = rng.choice(n, size=min(k, n), replace=False)
    return np.unique(np.concatenate([pick, [0, n - 1]]))


def _sample_key_groups(n, groups, seed, G=64):
    """Every key of a few whole 64-key P groups (first, last, random ones):
    the oracle then quantizes only those groups."""
    ng = -(-n // G)
    rng = np.random.default_rng(seed)
    pick = np.unique(np.concatenate([[0, ng - 1], rng.choice(ng, size=min(groups, ng), replace=False)]))
    return np.concatenate([np.arange(g * G, min(n, (g + 1) * G)) for g in pick])


FULL = {
    "tiny": (W.WORKLOADS["tiny"], None),
    "dit_image": (W.WORKLOADS["dit_image"], [(0, 0), (0, 23)]),
    "long_video": (W.WORKLOADS["long_video"], [(0, 17)]),
    "causal_lm": (W.WORKLOADS["causal_lm"], [(0, 0), (3, 31)]),
    "cross_fp8v": (W.WORKLOADS["cross_fp8v"], [(0, 5), (1, 23)]),
    "dit_image_smoothk": (W.WORKLOADS["dit_image_smoothk"], [(0, 0), (0, 23)]),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled(name):
    w, heads = FULL[name]
    print(f"case {name} full size: {w}", flush=True)
    inp = W.make_inputs(w)
    gpu = run_gpu(w, inp)
    q_rows = k_rows = None
    if heads is not None:
        q_rows = _sample_rows(w.Nq, 384, 1)
        k_rows = _sample_key_groups(w.Nkv, 3, 2)
    ref = run_oracle(w, inp, heads=heads, q_rows=q_rows, k_rows=k_rows)
    if w.v_fp8:
        assert np.array_equal(gpu["v_codes"], ref["v_codes"])
    errs = compare(gpu, ref, heads=heads, q_rows=q_rows, k_rows=k_rows)
    assert_within(errs, name)
    # properties that hold at any size, over every head: finite outputs and
    # sum_j dK_j = 0 per head (up to bf16 rounding of dK)
    for n in ("o", "o_hp", "lse", "dq", "dk", "dv"):
        assert np.isfinite(gpu[n]).all(), n
    dk = gpu["dk"]
    colsum = np.abs(dk.sum(axis=2)) / (np.abs(dk).sum(axis=2) + 1e-30)
    assert colsum.max() < 2e-2


def _run_on_device(w, inp):
    """Forward + backward as run_gpu does, outputs left on the device."""
    from quantization_aware_attention_amd import ops
    from tests._harness import flags_of, to_dev
    q, k, v, do = (to_dev(inp[n + "_bits"], w.dtype) for n in ("q", "k", "v", "do"))
    flags = flags_of(w, True)
    v_scale = None
    if w.v_fp8:
        v, v_scale = ops.quant_v_fp8(v)
    o, o_hp, lse = ops.attn_fwd(q, k, v, w.sm_scale, w.causal, flags, v_scale=v_scale)
    dq, dk, dv = ops.attn_bwd(q, k, v, o_hp, lse, do, w.sm_scale, w.causal, flags, v_scale=v_scale)
    torch.cuda.synchronize()
    return {"o": o, "o_hp": o_hp, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


@pytest.mark.parametrize("name", ["dit_image", "long_video", "causal_lm", "cross_fp8v", "dit_image_smoothk"])
def test_full_size_reruns_bitwise(name):
    # The kernels' barriers follow hazard arguments (the forward syncs after
    # every other phase, dK/dV after every third query block); at full size,
    # with every compute unit busy and waves drifting apart, a missing
    # ordering would show as differences between identical runs.
    w, _ = FULL[name]
    print(f"rerun case {name} full size: {w}", flush=True)
    inp = W.make_inputs(w)
    first = _run_on_device(w, inp)
    for _ in range(2):
        again = _run_on_device(w, inp)
        for n, t in first.items():
            assert torch.equal(t, again[n]), n
        del again


def test_smoothing_equals_plain_on_shifted_keys():
    """K = K0 + c with every channel of K0 made of +/- pairs on a 1/8 grid and
    c on a 1/4 grid: the mean over batch, heads and tokens is exactly c in any
    summation order, and K - c = K0 exactly.  The smoothed run must then be the
    plain run on K0 bit for bit (O, O_hp, lse, dK, dV).  dQ differs by
    sm_scale rowsum(dS) c: zero in exact arithmetic, but the kernels take Delta
    from the dtype-rounded O_hp, which leaves rowsum(dS) at about 1e-3 of its
    terms; the difference stays inside the dQ parity bar."""
    w = BASE.with_(B=1, H=2, Nq=160, Nkv=160, k_offset_var=0.0, seed=29)
    inp = W.make_inputs(w)
    rng = np.random.default_rng(29)
    half = rng.integers(-24, 25, size=(w.B, w.H, w.Nkv // 2, w.D)) / 8.0
    k0 = np.concatenate([half, -half], axis=2)
    c = rng.integers(-6, 7, size=w.D) / 4.0
    sh = dict(inp)
    sh["k"], sh["k_bits"] = W.round_to_dtype(k0 + c, w.dtype)
    base = dict(inp)
    base["k"], base["k_bits"] = W.round_to_dtype(k0, w.dtype)
    smooth = run_gpu(w.with_(smooth_k=True), sh)
    plain = run_gpu(w, base)
    for n in ("o", "o_hp", "lse", "dk", "dv"):
        assert np.array_equal(smooth[n], plain[n]), n
    assert rel_l2(smooth["dq"], plain["dq"]) < 1e-2
