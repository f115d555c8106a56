"""Seeded synthetic workloads for quantization-aware attention.

This module only draws random inputs and rounds them to the storage dtype; it
holds none of the attention or quantizer arithmetic.  Tests feed the same
arrays to the HIP path and to the float64 oracle, and ``bench.py`` uses it to
build its timed batch.

Shapes and distributions follow the workloads the pages describe: the
``requires_grad`` probe of "support for pytorch autograd" (batch 2, 4 heads,
sequence 8, head dim 64, fp16), DiT image joint attention (4096 image + 512
text tokens, 24 heads of 128), long-video DiT self attention (32768 tokens,
40 heads, per-token Q/K/V fake quant), causal LM-shaped attention and
cross attention with an fp8 V.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nkv: int
    D: int
    dtype: str            # "bf16" or "fp16": storage and MFMA operand type
    causal: bool
    p_fmt: str            # P fake-quant grid: "e4m3" or "e5m2"
    qkv_quant: bool       # per-token e4m3 fake quant of Q, K, V
    v_fp8: bool           # V handed over as e5m2 codes + per-channel scale
    k_offset_var: float   # variance of a per-(head, channel) K offset (0: none)
    seed: int
    smooth_k: bool = False   # subtract the mean of K over batch, heads, tokens first

    @property
    def sm_scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.D)))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 2, 4, 8, 8, 64, "fp16", False, "e4m3", False, False, 0.0, 1001),
    "dit_image": Workload("dit_image", 1, 24, 4608, 4608, 128, "bf16", False, "e4m3", False, False, 2.0, 1002),
    "long_video": Workload("long_video", 1, 40, 32768, 32768, 128, "bf16", False, "e4m3", True, False, 0.0, 1003),
    "causal_lm": Workload("causal_lm", 4, 32, 2048, 2048, 128, "bf16", True, "e4m3", False, False, 0.0, 1004),
    "cross_fp8v": Workload("cross_fp8v", 2, 24, 8192, 512, 128, "bf16", False, "e5m2", False, True, 0.0, 1005),
    # the DiT image shape with per-token Q/K/V quantization of the smoothed K
    # (its per-channel offsets are what the smoothing takes out before K is quantized)
    "dit_image_smoothk": Workload("dit_image_smoothk", 1, 24, 4608, 4608, 128, "bf16", False, "e4m3", True, False,
                                  2.0, 1006, smooth_k=True),
}


def round_to_dtype(x: np.ndarray, dtype: str):
    """Round float64 samples to bf16 or fp16 storage.

    Returns ``(values, bits)``: ``values`` as float32 holding exactly the
    rounded numbers, ``bits`` as uint16 storage words.  bf16 keeps the top
    16 bits of the fp32 value after round-to-nearest-even on the dropped 16.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "fp16":
        h = x32.astype(np.float16)
        return h.astype(np.float32), h.view(np.uint16)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    bits = u.astype(np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    return vals, bits


def make_inputs(w: Workload, heads=None):
    """Draw q, k, v, dO for a workload.

    Returns a dict of float32 value arrays ``q, k, v, do`` (exactly the
    dtype-rounded numbers) and uint16 storage arrays ``q_bits`` ... .  With
    ``heads`` (an int ``n``) only the first ``n`` (b, h) heads in batch-major
    order are drawn, as a [1, n, N, D] tensor, with the same per-head streams
    as the full tensor.

    Every (b, h) head has its own PCG64 stream derived from the workload seed,
    so a head's data does not depend on how many heads are drawn.
    """
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    if heads is not None:
        pairs = pairs[:heads]
    B = w.B if heads is None else 1
    H = w.H if heads is None else len(pairs)
    shapes = {"q": (w.Nq, w.D), "k": (w.Nkv, w.D), "v": (w.Nkv, w.D), "do": (w.Nq, w.D)}
    out = {}
    for n, s in shapes.items():
        out[n] = np.empty((B, H) + s, dtype=np.float32)
        out[n + "_bits"] = np.empty((B, H) + s, dtype=np.uint16)
    offset_rng = np.random.Generator(np.random.PCG64([w.seed, 7]))
    k_off = offset_rng.standard_normal((w.H, w.D)) * np.sqrt(w.k_offset_var)
    for i, (b, h) in enumerate(pairs):
        rng = np.random.Generator(np.random.PCG64([w.seed, b, h]))
        bb, hh = (b, h) if heads is None else (0, i)
        for n in ("q", "k", "v", "do"):
            x = rng.standard_normal(shapes[n])
            if n == "k" and w.k_offset_var:
                x += k_off[h][None, :]
            out[n][bb, hh], out[n + "_bits"][bb, hh] = round_to_dtype(x, w.dtype)
    return out
