"""The Python binding checks every tensor before the library sees a pointer
(no GPU needed: every call here fails validation before any library call).

The C ABI receives raw device pointers and sizes taken from q and k, so a
tensor of the wrong shape, dtype or device handed to the binding would turn
into an out-of-bounds device access; the binding raises ValueError instead.
"""
import pytest
import torch

from quantization_aware_attention_amd import ops

B, H, NQ, NKV, D = 1, 2, 16, 24, 64
bf = torch.bfloat16


def t(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def fwd_args(**over):
    a = dict(q=t(B, H, NQ, D), k=t(B, H, NKV, D), v=t(B, H, NKV, D), sm_scale=0.125)
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(k=t(B, H, NKV, 128)), "k must have shape"),
    (dict(k=t(B, 3, NKV, D)), "k must have shape"),
    (dict(v=t(B, H, NKV + 1, D)), "v must have shape"),
    (dict(k=t(B, H, NKV, D, dtype=torch.float16)), "k must be torch.bfloat16"),
    (dict(q=t(B, H, NQ, D, dtype=torch.float32)), "q must be a 4-D bf16 or fp16"),
    (dict(q=t(H, NQ, D)), "q must be a 4-D"),
])
def test_forward_rejects_mismatched_inputs(over, msg):
    with pytest.raises(ValueError, match=msg):
        ops.attn_fwd(**fwd_args(**over))


def test_forward_fp8_v_needs_codes_and_scale():
    flags = ops.QAT_P_QUANT | ops.QAT_V_FP8_E5M2
    with pytest.raises(ValueError, match="v must be torch.uint8"):
        ops.attn_fwd(**fwd_args(), quant_flags=flags, v_scale=t(B, H, D, dtype=torch.float32))
    codes = t(B, H, NKV, D, dtype=torch.uint8)
    with pytest.raises(ValueError, match="v_scale is required"):
        ops.attn_fwd(**fwd_args(v=codes), quant_flags=flags)
    with pytest.raises(ValueError, match="v_scale must have shape"):
        ops.attn_fwd(**fwd_args(v=codes), quant_flags=flags, v_scale=t(B, H, NKV, dtype=torch.float32))
    with pytest.raises(ValueError, match="only used with"):
        ops.attn_fwd(**fwd_args(), v_scale=t(B, H, D, dtype=torch.float32))


@pytest.mark.parametrize("out,msg", [
    ((t(B, H, NQ + 1, D), t(B, H, NQ, D), t(B, H, NQ, dtype=torch.float32)), r"out\[0\] \(o\) must have shape"),
    ((t(B, H, NQ, D), t(B, H, NQ, D, dtype=torch.float16), t(B, H, NQ, dtype=torch.float32)), r"out\[1\]"),
    ((t(B, H, NQ, D), t(B, H, NQ, D), t(B, H, NQ)), r"out\[2\] \(lse\) must be torch.float32"),
])
def test_forward_rejects_mismatched_outputs(out, msg):
    with pytest.raises(ValueError, match=msg):
        ops.attn_fwd(**fwd_args(), out=out)


def test_forward_rejects_bad_workspace():
    with pytest.raises(ValueError, match="workspace must be torch.uint8"):
        ops.attn_fwd(**fwd_args(), workspace=t(256, dtype=torch.float32))


def test_backward_rejects_mismatched_tensors():
    a = fwd_args()
    good = dict(o_hp=t(B, H, NQ, D), lse=t(B, H, NQ, dtype=torch.float32), dout=t(B, H, NQ, D))
    for name, bad, msg in [("o_hp", t(B, H, NKV, D), "o_hp must have shape"),
                           ("lse", t(B, H, NQ, D, dtype=torch.float32), "lse must have shape"),
                           ("dout", t(B, H, NQ, D, dtype=torch.float16), "dout must be torch.bfloat16")]:
        kw = dict(good)
        kw[name] = bad
        with pytest.raises(ValueError, match=msg):
            ops.attn_bwd(a["q"], a["k"], a["v"], kw["o_hp"], kw["lse"], kw["dout"], 0.125)
    outs = (t(B, H, NQ, D), t(B, H, NQ, D), t(B, H, NKV, D))   # dk with q's shape
    with pytest.raises(ValueError, match=r"out\[1\] \(dk\) must have shape"):
        ops.attn_bwd(a["q"], a["k"], a["v"], good["o_hp"], good["lse"], good["dout"], 0.125, out=outs)


def test_merge_and_sum_reject_mismatched_parts():
    o = [t(B, H, NQ, D), t(B, H, NQ, D)]
    lse = [t(B, H, NQ, dtype=torch.float32), t(B, H, NQ + 1, dtype=torch.float32)]
    with pytest.raises(ValueError, match=r"lse_parts\[1\] must have shape"):
        ops.attn_merge(o, o, lse)
    with pytest.raises(ValueError, match="equal length"):
        ops.attn_merge(o, o[:1], lse)
    with pytest.raises(ValueError, match=r"parts\[1\] must have shape"):
        ops.attn_sum([t(B, H, NQ, D), t(B, H, NQ, 2 * D)])
    with pytest.raises(ValueError, match="out must have shape"):
        ops.attn_sum(o, out=t(B, H, NQ + 1, D))


def test_well_formed_host_tensors_are_still_refused():
    # every shape and dtype right, but in host memory: refused before any
    # library call (the library only takes device pointers)
    with pytest.raises(ValueError, match="must be a contiguous CUDA tensor"):
        ops.attn_fwd(**fwd_args())
