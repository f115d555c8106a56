"""GPU parity on inputs that drive the forward's lazy rescale and the
zero-scale paths of the quantizers.

The forward keeps a stale running maximum per row and rescales both
accumulators and the row sum by alpha = exp2(m_old - m_new) only when a key
tile raises the row maximum (in scaled log2 units) by more than 8 (the source
rescales on every tile: _attn_fwd_inner, alpha applied to acc and l_i).  With
N(0, 1) inputs and sm_scale = 1/sqrt(D) no row ever gets there after its first
tile, so these cases grow the key norms tile by tile: the row maxima then jump
by about 10 per tile.  Each case first replays the kernels' rescale rule on
the CPU over its own inputs (64-key tiles in key order, the masks, the 8-unit
slack) and requires that a sizeable share of rows rescale after their first
tile, so that a change of inputs cannot silently stop covering the branch.

The zero-scale cases put all-zero token rows into Q, K and V under per-token
quantization (scale 0, codes 0) and an all-zero V channel under fp8 V
(v_scale 0).
"""
import numpy as np
import pytest

from oracle import qat_attention as oracle
from quantization_aware_attention_amd import workloads as W
from tests._harness import assert_within, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

BASE = W.WORKLOADS["dit_image"].with_(k_offset_var=0.0)
CROSS = W.WORKLOADS["cross_fp8v"]
TILE = 64          # key tile of the forward kernels
SLACK = 8.0        # rescale threshold of the forward kernels (scaled log2 units)
GROWTH = 3.0       # key tile t is scaled by 1 + GROWTH * t


def grow_keys(w, inp):
    """Scale the keys of tile t by 1 + GROWTH t (then round to the dtype)."""
    out = dict(inp)
    f = 1.0 + GROWTH * (np.arange(w.Nkv) // TILE)
    out["k"], out["k_bits"] = W.round_to_dtype(inp["k"].astype(np.float64) * f[None, None, :, None], w.dtype)
    return out


def rescale_share(w, inp):
    """Share of query rows whose running maximum, replayed with the kernels'
    rule, is raised by more than SLACK on some tile after the row's first."""
    v_codes = v_scale = None
    if w.v_fp8:
        v_codes, v_scale = oracle.quantize_v_channels(inp["v"], "e5m2")
    qh, kh, _ = oracle.prepare_inputs(inp["q"], inp["k"], inp["v"], qkv_quant=w.qkv_quant,
                                      v_codes=v_codes, v_scale=v_scale)
    c = w.sm_scale * np.log2(np.e)
    hit = total = 0
    for b in range(w.B):
        for h in range(w.H):
            S = (qh[b, h] @ kh[b, h].T) * c
            if w.causal:
                S = np.where(np.arange(w.Nkv)[None, :] > np.arange(w.Nq)[:, None], -np.inf, S)
            m = np.full(w.Nq, -np.inf)
            rows_hit = np.zeros(w.Nq, dtype=bool)
            for t0 in range(0, w.Nkv, TILE):
                tmax = S[:, t0:t0 + TILE].max(axis=1)
                resc = tmax > m + SLACK
                rows_hit |= resc & np.isfinite(m)
                m = np.where(resc, tmax, m)
            hit += int(rows_hit.sum())
            total += w.Nq
    return hit / total


RESCALE = {
    "bf16_d128_ragged": BASE.with_(B=1, H=2, Nq=200, Nkv=300, seed=41),
    "fp16_d64_causal": BASE.with_(B=2, H=1, Nq=333, Nkv=333, D=64, dtype="fp16", causal=True, seed=42),
    "bf16_d128_causal_e5m2": BASE.with_(B=1, H=2, Nq=257, Nkv=257, causal=True, p_fmt="e5m2", seed=43),
    "qkv_quant_bf16_ragged": BASE.with_(B=1, H=2, Nq=150, Nkv=330, qkv_quant=True, seed=44),
    "qkv_quant_fp16_d64_causal": BASE.with_(B=1, H=2, Nq=260, Nkv=260, D=64, dtype="fp16", causal=True,
                                            qkv_quant=True, seed=45),
    "fp8v_ragged": CROSS.with_(B=1, H=2, Nq=150, Nkv=500, seed=46),
    "fp8v_causal": CROSS.with_(B=1, H=2, Nq=300, Nkv=300, causal=True, seed=47),
}


@pytest.mark.parametrize("name", list(RESCALE))
def test_lazy_rescale_parity(name):
    w = RESCALE[name]
    inp = grow_keys(w, W.make_inputs(w))
    share = rescale_share(w, inp)
    print(f"case rescale {name}: {w}; rows rescaled after their first tile: {share:.2f}", flush=True)
    assert share >= 0.3, f"inputs no longer drive the rescale branch ({share:.2f} of rows)"
    gpu = run_gpu(w, inp)
    ref = run_oracle(w, inp)
    if w.v_fp8:
        assert np.array_equal(gpu["v_codes"], ref["v_codes"])
    assert_within(compare(gpu, ref), f"rescale {name}")


def _zero_rows(w, inp, q_rows, k_rows, v_rows):
    out = dict(inp)
    for n, rows in (("q", q_rows), ("k", k_rows), ("v", v_rows)):
        x = inp[n].copy()
        x[:, :, rows] = 0.0
        out[n], out[n + "_bits"] = W.round_to_dtype(x, w.dtype)
    return out


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_zero_token_rows_under_qkv_quant(causal):
    # an all-zero token row has scale 0 and codes 0: its scores are 0 (a zero
    # query row attends uniformly), and the kernels must keep masked scores
    # at -inf after the scale product
    w = BASE.with_(B=1, H=2, Nq=190, Nkv=190, qkv_quant=True, causal=causal, seed=48)
    inp = _zero_rows(w, W.make_inputs(w), q_rows=[0, 3, 77, 189], k_rows=[0, 5, 130], v_rows=[9, 64])
    print(f"case zero rows qkv quant: {w}", flush=True)
    gpu = run_gpu(w, inp)
    ref = run_oracle(w, inp)
    for n in ("o", "o_hp", "lse", "dq", "dk", "dv"):
        assert np.isfinite(gpu[n]).all(), n
    assert_within(compare(gpu, ref), f"zero rows qkv quant causal={causal}")


def test_zero_v_channel_under_fp8_v():
    w = CROSS.with_(B=1, H=2, Nq=150, Nkv=300, seed=49)
    inp = W.make_inputs(w)
    v = inp["v"].copy()
    v[0, 1, :, 7] = 0.0
    v[0, 0, :, 100] = 0.0
    inp["v"], inp["v_bits"] = W.round_to_dtype(v, w.dtype)
    print(f"case zero V channel fp8 V: {w}", flush=True)
    gpu = run_gpu(w, inp)
    ref = run_oracle(w, inp)
    assert np.array_equal(gpu["v_codes"], ref["v_codes"])
    assert np.array_equal(gpu["v_scale"], ref["v_scale"])
    assert ref["v_scale"][0, 1, 7] == 0.0 and ref["v_scale"][0, 0, 100] == 0.0
    for n in ("o", "o_hp", "lse", "dq", "dk", "dv"):
        assert np.isfinite(gpu[n]).all(), n
    assert np.all(gpu["o"][0, 1, :, 7] == 0.0) and np.all(gpu["o_hp"][0, 0, :, 100] == 0.0)
    assert_within(compare(gpu, ref), "zero V channel fp8 V")
