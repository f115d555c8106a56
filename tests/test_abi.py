"""Host-side checks of the C ABI (no GPU work is launched).

* the library loads and exports every function include/qat_attn.h declares;
* validation errors come back before any launch: every call here is invalid
  in at least one argument, so nothing is enqueued;
* workspace sizing follows the documented layout.
"""
import ctypes
import os

import pytest

from quantization_aware_attention_amd import ops


@pytest.fixture(scope="module")
def L():
    # a fresh checkout has no library yet: build it (hipcc cross-compiles for
    # gfx950 without a GPU) rather than skipping the boundary checks
    if not os.path.exists(ops.LIB_PATH):
        from quantization_aware_attention_amd import build
        build.build()
    return ops.lib()


def test_exports_every_declared_symbol(L):
    names = ops.header_functions()
    assert {"qat_attn_fwd", "qat_attn_bwd", "qat_attn_workspace_bytes", "qat_quant_v_fp8",
            "qat_fake_quant_rows", "qat_attn_p_group", "qat_attn_strerror"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_binding_constants_match_the_header():
    import re
    vals = {}
    for line in open(ops.HEADER):
        m = re.match(r"#define (QAT_\w+)\s+(.+?)\s*(/\*.*)?$", line)
        if m and m.group(1) != "QAT_ATTN_H":
            expr = re.sub(r"\(size_t\)|(?<=\d)u\b", "", m.group(2))
            vals[m.group(1)] = eval(expr, {}, dict(vals))
    for name, v in vals.items():
        if hasattr(ops, name):
            assert getattr(ops, name) == v, name
    for name in ("QAT_P_QUANT", "QAT_ESCRATCH", "QAT_NOALLOC_SCRATCH_BYTES", "QAT_P_ABSMAX_MAX_BYTES"):
        assert name in vals and hasattr(ops, name), name


def test_constants(L):
    assert L.qat_attn_p_group() == 64
    assert L.qat_attn_strerror(ops.QAT_EINVAL) == b"invalid argument"
    assert L.qat_attn_strerror(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x100000)       # aligned, never dereferenced: every call below fails validation
MISALIGNED = ctypes.c_void_p(0x100008)


def _fwd(L, dims, flags=ops.QAT_P_QUANT, causal=0, sm=0.125, v_scale=None, ws=None, ws_bytes=0, q=FAKE):
    return L.qat_attn_fwd(ctypes.byref(dims) if dims is not None else None, q, FAKE, FAKE, v_scale, sm,
                          causal, flags, FAKE, FAKE, FAKE, ws, ws_bytes, None)


def test_fwd_validation(L):
    D = ops.Dims
    assert _fwd(L, None) == ops.QAT_EINVAL
    assert _fwd(L, D(1, 1, 16, 16, 96, 0)) == ops.QAT_EUNSUPPORTED          # head dim
    assert _fwd(L, D(1, 1, 16, 16, 64, 7)) == ops.QAT_EINVAL                # dtype
    assert _fwd(L, D(1, 1, 16, 16, 64, 0), flags=1 << 9) == ops.QAT_EINVAL  # unknown flag
    assert _fwd(L, D(1, 1, 16, 16, 64, 0), flags=ops.QAT_P_E5M2) == ops.QAT_EINVAL
    assert _fwd(L, D(1, 1, 16, 32, 64, 0), causal=1) == ops.QAT_EUNSUPPORTED  # causal Nq != Nkv
    assert _fwd(L, D(1, 1, 16, 16, 64, 0), sm=0.0) == ops.QAT_EINVAL
    assert _fwd(L, D(1, 1, 16, 16, 64, 0), sm=float("nan")) == ops.QAT_EINVAL
    assert _fwd(L, D(1, 1, 16, 16, 64, 0), v_scale=FAKE) == ops.QAT_EINVAL   # scale without fp8 V
    assert _fwd(L, D(1, 1, 16, 16, 64, 0), flags=ops.QAT_P_QUANT | ops.QAT_V_FP8_E5M2) == ops.QAT_EINVAL
    assert _fwd(L, D(1, 1, 16, 16, 64, 1), flags=ops.QAT_P_QUANT | ops.QAT_V_FP8_E5M2,
                v_scale=FAKE) == ops.QAT_EUNSUPPORTED                          # fp8 V needs bf16
    assert _fwd(L, D(1, 1, 16, 0, 64, 0)) == ops.QAT_EINVAL                  # no keys
    assert _fwd(L, D(-1, 1, 16, 16, 64, 0)) == ops.QAT_EINVAL
    assert _fwd(L, D(1, 1, 16, 16, 64, 0), q=None) == ops.QAT_EINVAL         # null input
    assert _fwd(L, D(1, 1, 16, 16, 64, 0), q=MISALIGNED) == ops.QAT_EINVAL
    assert _fwd(L, D(300, 300, 16, 16, 64, 0)) == ops.QAT_EUNSUPPORTED       # B*H beyond the grid
    # Q/K/V quantization needs a workspace
    assert _fwd(L, D(1, 1, 16, 16, 64, 0), flags=ops.QAT_P_QUANT | ops.QAT_QKV_QUANT) == ops.QAT_EWORKSPACE
    # empty problems succeed without touching the device
    assert _fwd(L, D(0, 1, 16, 16, 64, 0)) == ops.QAT_OK
    assert _fwd(L, D(1, 1, 0, 16, 64, 0)) == ops.QAT_OK


def test_bwd_validation(L):
    D = ops.Dims

    def bwd(dims, ws=None, ws_bytes=0, flags=ops.QAT_P_QUANT):
        return L.qat_attn_bwd(ctypes.byref(dims), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 0.125, 0, flags,
                              FAKE, FAKE, FAKE, ws, ws_bytes, None)
    assert bwd(D(1, 1, 16, 16, 64, 0)) == ops.QAT_EWORKSPACE                # Delta needs space
    need = ops.workspace_bytes(D(1, 1, 16, 16, 64, 0), ops.QAT_P_QUANT, 1)
    assert bwd(D(1, 1, 16, 16, 64, 0), FAKE, need - 1) == ops.QAT_EWORKSPACE
    assert bwd(D(1, 1, 16, 16, 80, 0), FAKE, need) == ops.QAT_EUNSUPPORTED
    # staged backward: an empty or unknown stage mask is rejected
    for mask in (0, 1 << 6):
        assert L.qat_attn_bwd_stages(ctypes.byref(D(1, 1, 16, 16, 64, 0)), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                     0.125, 0, ops.QAT_P_QUANT, FAKE, FAKE, FAKE, FAKE, need, mask,
                                     None) == ops.QAT_EINVAL


def test_workspace_layout():
    D = ops.Dims
    d = D(2, 3, 100, 130, 128, 0)
    assert ops.workspace_bytes(d, ops.QAT_P_QUANT, 0) == 0
    up = lambda x: -(-x // 256) * 256
    delta = up(2 * 3 * 100 * 4)
    # fp32 dK/dV partials: up to 4 query ranges per 128-key block, at most 768 in all
    part = up(min(6 * 2 * 4, 768) * 2 * 128 * 128 * 4)
    amax = up(2 * 3 * 3 * 100 * 4)            # P-quant absmax record: ceil(130 / 64) = 3 groups
    assert ops.workspace_bytes(d, 0, 1) == delta + part
    assert ops.workspace_bytes(d, ops.QAT_P_QUANT, 1) == delta + amax + part
    # Q, K code values and V^ (dtype), per-token scales, e4m3 code bytes of Q and K
    qkv = (up(6 * 100 * 128 * 2) + 2 * up(6 * 130 * 128 * 2) + up(6 * 100 * 4) + up(6 * 130 * 4)
           + up(6 * 100 * 128) + up(6 * 130 * 128))
    assert ops.workspace_bytes(d, ops.QAT_P_QUANT | ops.QAT_QKV_QUANT, 0) == qkv
    assert ops.workspace_bytes(d, ops.QAT_P_QUANT | ops.QAT_QKV_QUANT, 1) == delta + amax + part + qkv
    # K smoothing (both passes): mean partial sums [256, D] and the mean [D] fp32, and
    # K - mean (dtype) unless Q/K/V quantization subtracts it on the way
    sk = up(256 * 128 * 4) + up(128 * 4)
    ksm = up(6 * 130 * 128 * 2)
    assert ops.workspace_bytes(d, ops.QAT_SMOOTH_K, 0) == sk + ksm
    assert ops.workspace_bytes(d, ops.QAT_P_QUANT | ops.QAT_SMOOTH_K, 1) == delta + amax + part + sk + ksm
    assert ops.workspace_bytes(d, ops.QAT_QKV_QUANT | ops.QAT_SMOOTH_K, 0) == sk + qkv
    big = D(1, 24, 4608, 4608, 128, 0)        # 864 key blocks: capped at 768 partial blocks
    assert ops.workspace_bytes(big, 0, 1) == up(24 * 4608 * 4) + up(768 * 2 * 128 * 128 * 4)
    # the absmax record is bounded: at 40 heads of 32768 it would take 2.7 GB,
    # so it is left out and the workspace stays linear in the sequence length
    lv = D(1, 40, 32768, 32768, 128, 0)
    rec = 40 * 512 * 32768 * 4
    assert rec > ops.QAT_P_ABSMAX_MAX_BYTES
    assert ops.workspace_bytes(lv, ops.QAT_P_QUANT, 1) == ops.workspace_bytes(lv, 0, 1)
    assert ops.workspace_bytes(big, ops.QAT_P_QUANT, 1) == (ops.workspace_bytes(big, 0, 1)
                                                            + up(24 * 72 * 4608 * 4))
    assert ops.workspace_bytes(d, 0, 2) == 0


def test_other_entry_points_validate(L):
    D = ops.Dims
    assert L.qat_fake_quant_rows(None, 4, 4, 4, 0, None, None, None, None) == ops.QAT_EINVAL
    assert L.qat_fake_quant_rows(FAKE, 4, 4, 0, 0, None, None, None, None) == ops.QAT_EINVAL
    assert L.qat_fake_quant_rows(FAKE, 4, 4, 4, 2, None, None, None, None) == ops.QAT_EINVAL
    assert L.qat_quant_v_fp8(ctypes.byref(D(1, 1, 0, 16, 96, 0)), FAKE, FAKE, FAKE, None) == ops.QAT_EUNSUPPORTED
    assert L.qat_quant_v_fp8(ctypes.byref(D(1, 1, 0, 16, 64, 0)), None, FAKE, FAKE, None) == ops.QAT_EINVAL
    assert L.qat_quant_v_fp8(ctypes.byref(D(1, 1, 0, 0, 64, 0)), None, None, None, None) == ops.QAT_OK
    assert L.qat_selftest_exp2_monotone(0.0, 1.0, None, None) == ops.QAT_EINVAL
    assert L.qat_selftest_exp2_monotone(2.0, 1.0, FAKE, None) == ops.QAT_EINVAL
    assert L.qat_selftest_exp2_monotone(float("nan"), 1.0, FAKE, None) == ops.QAT_EINVAL
    assert L.qat_selftest_fq_scale(0, None, None) == ops.QAT_EINVAL
    assert L.qat_selftest_fq_scale(2, FAKE, None) == ops.QAT_EINVAL
    assert L.qat_selftest_fq_scale(-1, FAKE, None) == ops.QAT_EINVAL


def test_noalloc_rejects_oversized_problem_before_any_device_call(L):
    # long-video size with per-token Q/K/V quantization needs far more than
    # the static scratch: refused before the library looks at the device
    d = ops.Dims(1, 40, 32768, 32768, 128, ops.QAT_DTYPE_BF16)
    flags = ops.QAT_P_QUANT | ops.QAT_QKV_QUANT
    assert L.qat_attn_workspace_bytes(ctypes.byref(d), flags, 1) > ops.QAT_NOALLOC_SCRATCH_BYTES
    st = L.qat_attn_bwd_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 0.088, 0, flags,
                                FAKE, FAKE, FAKE, None)
    assert st == ops.QAT_ESCRATCH
    assert L.qat_attn_strerror(ops.QAT_ESCRATCH).startswith(b"problem needs more")
