"""Plain float64 CPU oracle of quantization-aware (fake-quant) attention.

TEST INFRASTRUCTURE ONLY.  This module is the yardstick the HIP kernels are
checked against.  It shares no code with the HIP path and imports nothing from
the product package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It is slow on purpose:
every step is the textbook definition, written so that it can be checked
against the sources by eye.

Sources (web pages):
* "support for pytorch autograd" (SageAttention issue 60): the training use
  case and the rematerialisation idea for the backward.
* FastVideo ``attn_qat_train.py`` (the Triton QAT attention source):
  ``_attn_fwd_inner`` / ``_attn_fwd`` (forward with a fake-quantized P tile,
  two accumulators and the base-2 log-sum-exp), ``_attn_bwd_preprocess``
  (Delta), ``_attn_bwd_dkdv`` / ``_attn_bwd_dkdv_cross`` and
  ``_attn_bwd_dq`` / ``_attn_bwd_dq_cross`` (backward), and
  ``_attention.forward`` / ``_attention.backward`` (the Q/K/V fake-quant
  pre-pass and the straight-through return of the gradients).

What the oracle computes (one (batch, head) pair at a time; ``^`` marks a
fake-quantized value):

  inputs     Q^, K^, V^ = FQ(Q), FQ(K), FQ(V) per token row over D when Q/K/V
             quantization is on, V^ = decode(code) * v_scale for fp8 V, else
             the inputs themselves
  scores     S = sm_scale * Q^ K^T, entries with key index > query index set to
             -inf under the causal mask (top-left aligned, diagonal kept)
  softmax    lse_i = log sum_j exp(S_ij),  P = exp(S - lse)
  P quant    P^ = FQ_P(P), one scale per row and per group of G_P absolute
             key columns [g*G_P, (g+1)*G_P)
  outputs    O_hp = P V^,  O = P^ V^
  backward   Delta_i = sum_d dO_id O_hp_id,  dP = dO V^T,  dS = P o (dP - Delta)
             dV = P^T dO (with P^),  dQ = sm_scale dS K^,  dK = sm_scale dS^T Q^
             returned as gradients of the un-quantized Q, K, V (straight
             through every quantizer).

Readings taken where the pages are silent (the quantizer module itself is not
on the pages):
* FQ: per group a = max|x|; s = fp32(a / FMAX), r = fp32(FMAX / a) (one
  correctly rounded division each); v = fp32(x * r); the code is v rounded to
  the fp8 grid (nearest, ties to even, saturating); x^ = fp32(code * s).  A
  group with a == 0, or whose r overflows fp32, quantizes to zeros.  FMAX is
  448 (e4m3) or 57344 (e5m2).
* P-quant groups are G_P = 64 absolute key columns, used identically by the
  forward and the backward; masked entries are zeros inside their group.
* The forward of the source quantizes the running, un-normalised tile
  exp2(S*c - m_running) rather than the final P.  Per-row absmax scaling is
  invariant to a positive row factor (x/s does not change), so in real
  arithmetic both give the same O; the oracle uses the plain normalised form.
* Delta uses O_hp (the straight-through output), which makes
  Delta_i = sum_j P_ij dP_ij hold exactly.
* The log-sum-exp is returned in natural-log units (the source keeps base 2).
* fp8 V (cross-attention case): one scale per (batch, head, channel d) over
  the key axis, e5m2 grid.
* K smoothing (``_attention.forward``, "smoothing k", and the SMOOTH_K term of
  ``_attn_bwd_dq``): k_mean[d] is the mean of K over every batch, head and
  token, rounded to the storage dtype (the source keeps it in K's dtype);
  K_s = K - k_mean rounded to the dtype replaces K before anything else,
  Q/K/V quantization included; dQ = sm_scale (dS K^_s + rowsum(dS) k_mean),
  the gradient for the original K.  dK is the one of the smoothed K.
  Rounding to the dtype goes through float32 (round to nearest even), then
  to bf16 (nearest even on the upper 16 bits) or fp16.
"""
from __future__ import annotations

import numpy as np

from . import fp8

P_GROUP = 64  # G_P: key columns sharing one P-quant scale per row


# --------------------------------------------------------------------------
# Quantizer FQ (fp32 arithmetic, emulated exactly in float64)
# --------------------------------------------------------------------------
def _to_f32(x) -> np.ndarray:
    """Round float64 values to fp32 (RNE) and return them as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def fake_quant_groups(x, fmt: str, group: int):
    """FQ of a 2-D array, one scale per row per group of ``group`` columns.

    Groups are the absolute column ranges [g*group, min((g+1)*group, cols)).
    Returns ``(codes uint8 [rows, cols], scales fp32 [rows, n_groups],
    xhat fp32 [rows, cols])``.

    A product or quotient of two fp32 numbers formed in float64 and rounded to
    fp32 equals the correctly rounded fp32 operation (the product is exact in
    float64; for the quotient 53 >= 2*24 + 2 makes the double rounding
    harmless), so this is exactly the fp32 recipe.
    """
    x = _to_f32(x)                      # step 1: the group's values in fp32
    if x.ndim != 2:
        raise ValueError("fake_quant_groups expects a 2-D array")
    rows, cols = x.shape
    FMAX = fp8.fmax(fmt)
    n_groups = max(1, -(-cols // group))
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros((rows, n_groups), dtype=np.float32)
    xhat = np.zeros((rows, cols), dtype=np.float32)
    for g in range(n_groups):
        c0, c1 = g * group, min((g + 1) * group, cols)
        if c0 >= c1:
            continue
        blk = x[:, c0:c1]
        a = np.max(np.abs(blk), axis=1)                 # absmax, exact
        s = _to_f32(a / FMAX)                           # scale
        with np.errstate(divide="ignore", over="ignore"):
            r = np.where(a > 0, FMAX / np.where(a > 0, a, 1.0), np.inf)
            r = _to_f32(r)                              # reciprocal scale
        ok = (a > 0) & np.isfinite(r)
        r_use = np.where(ok, r, 0.0)
        v = _to_f32(blk * r_use[:, None])               # v = fp32(x * r)
        vals, c = fp8.round_rne_sat(v, fmt)             # onto the fp8 grid
        xh = _to_f32(vals * s[:, None])                 # dequantized value
        c[~ok] = 0
        xh[~ok] = 0.0
        codes[:, c0:c1] = c
        scales[:, g] = np.where(ok, s, 0.0).astype(np.float32)
        xhat[:, c0:c1] = xh.astype(np.float32)
    return codes, scales, xhat


def quantize_token_rows(x, fmt: str = "e4m3"):
    """Per-token FQ of a [..., N, D] tensor: one scale per row over D.

    This is the Q/K/V fake-quant pre-pass (``fake_quantize_q`` /
    ``fake_quantize_kv`` launched in ``_attention.forward``) under the
    per-token reading.  Returns (codes, scales [..., N], xhat).
    """
    x = np.asarray(x)
    lead = x.shape[:-1]
    D = x.shape[-1]
    codes, scales, xhat = fake_quant_groups(x.reshape(-1, D), fmt, D)
    return (codes.reshape(x.shape), scales.reshape(lead), xhat.reshape(x.shape))


def quantize_v_channels(v, fmt: str = "e5m2"):
    """FQ of V [B, H, N, D] with one scale per (b, h, d) over the N tokens.

    The cross-attention case stores V as fp8 codes with a per-channel absmax
    scale.  Returns (codes uint8 [B, H, N, D], v_scale fp32 [B, H, D]).
    """
    v = np.asarray(v)
    B, H, N, D = v.shape
    vt = np.swapaxes(v, 2, 3).reshape(B * H * D, N)     # rows = channels
    codes, scales, _ = fake_quant_groups(vt, fmt, N)
    codes = np.swapaxes(codes.reshape(B, H, D, N), 2, 3).copy()
    return codes, scales.reshape(B, H, D)


def dequant_v_channels(codes, v_scale, fmt: str = "e5m2") -> np.ndarray:
    """V^ = fp32(decode(code) * v_scale[b, h, d]) as float64."""
    vals = fp8.decode(codes, fmt)
    return _to_f32(vals * np.asarray(v_scale, dtype=np.float64)[:, :, None, :])


# --------------------------------------------------------------------------
# Attention, one (b, h) head
# --------------------------------------------------------------------------
# --------------------------------------------------------------------------
# K smoothing
# --------------------------------------------------------------------------
def round_storage(x, dtype: str) -> np.ndarray:
    """float64 values rounded to bf16 or fp16 storage, through float32."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "fp16":
        return x32.astype(np.float16).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x32.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def smooth_key_mean(k, dtype: str) -> np.ndarray:
    """k_mean[d]: the mean of K [B, H, N, D] over batch, heads and tokens,
    rounded to the dtype."""
    return round_storage(np.asarray(k, dtype=np.float64).mean(axis=(0, 1, 2)), dtype)


def smooth_keys(kh, k_mean, dtype: str) -> np.ndarray:
    """K_s = K - k_mean, rounded to the dtype."""
    return round_storage(np.asarray(kh, dtype=np.float64) - k_mean, dtype)


def _scores(qh, kh, sm_scale, causal, rows):
    """S for the query rows ``rows`` (absolute indices), causal mask applied."""
    S = float(sm_scale) * (qh[rows] @ kh.T)
    if causal:
        cols = np.arange(kh.shape[0])
        S = np.where(cols[None, :] > rows[:, None], -np.inf, S)
    return S


def _softmax_rows(S):
    """(P, lse) with lse_i = log sum_j exp(S_ij), evaluated stably."""
    m = np.max(S, axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.sum(np.exp(S - m), axis=1))
    P = np.exp(S - lse[:, None])
    return P, lse


def _p_hat(P, p_quant, p_fmt, group):
    if not p_quant:
        return P
    return fake_quant_groups(P, p_fmt, group)[2].astype(np.float64)


def forward_head(qh, kh, vh, sm_scale, causal=False, p_quant=True, p_fmt="e4m3",
                 group=P_GROUP, rows=None, row_block=2048):
    """Forward of one head from already-prepared Q^, K^, V^ (float64 [N, D]).

    Returns ``(O, O_hp, lse)`` for the query rows ``rows`` (all rows when
    None).  Rows are independent, so they are processed in blocks of
    ``row_block`` only to bound memory.
    """
    Nq = qh.shape[0]
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((rows.size, vh.shape[1]))
    O_hp = np.zeros_like(O)
    lse = np.zeros(rows.size)
    for b0 in range(0, rows.size, row_block):
        r = rows[b0:b0 + row_block]
        S = _scores(qh, kh, sm_scale, causal, r)
        P, l_ = _softmax_rows(S)
        Ph = _p_hat(P, p_quant, p_fmt, group)
        O_hp[b0:b0 + r.size] = P @ vh
        O[b0:b0 + r.size] = Ph @ vh
        lse[b0:b0 + r.size] = l_
    return O, O_hp, lse


def backward_head(qh, kh, vh, do, sm_scale, causal=False, p_quant=True, p_fmt="e4m3",
                  group=P_GROUP, q_rows=None, k_rows=None, row_block=2048, k_mean=None,
                  lse=None, o_hp=None):
    """Straight-through backward of one head.

    ``do`` is dO [Nq, D].  Returns ``(dQ[q_rows], dK[k_rows], dV[k_rows])``
    (all rows when None).  With ``lse`` and ``o_hp`` (the merged forward of a
    KV chunk's full row set, chunked mode) P = exp(S - lse) and Delta come
    from them instead of from this head's own keys.  With ``k_mean`` (K
    smoothing; ``kh`` is then the
    smoothed K) dQ takes the term sm_scale rowsum(dS) k_mean.  The sums over
    query rows that make dK and dV are
    split into row blocks only to bound memory, and only the columns of P
    that the requested keys need are formed (with their whole P-quant group,
    since a group's scale depends on all of its columns); within a block
    every step is the plain definition.
    """
    Nq, D = qh.shape
    Nkv = kh.shape[0]
    q_rows = np.arange(Nq) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
    k_rows = np.arange(Nkv) if k_rows is None else np.asarray(k_rows, dtype=np.int64)
    do = np.asarray(do, dtype=np.float64)
    dK = np.zeros((k_rows.size, D))
    dV = np.zeros((k_rows.size, D))
    dQ = np.zeros((Nq, D))
    need_dq = np.zeros(Nq, dtype=bool)
    need_dq[q_rows] = True
    groups = np.unique(k_rows // group)
    for b0 in range(0, Nq, row_block):
        r = np.arange(b0, min(Nq, b0 + row_block))
        S = _scores(qh, kh, sm_scale, causal, r)
        if lse is None:
            P, _ = _softmax_rows(S)
            O_hp = P @ vh
        else:                                                 # chunk of a longer key set
            P = np.exp(S - np.asarray(lse, dtype=np.float64)[r][:, None])
            O_hp = np.asarray(o_hp, dtype=np.float64)[r]
        Delta = np.sum(do[r] * O_hp, axis=1)                  # rowsum(dO o O_hp)
        Ph = np.zeros_like(P)                                 # P^, needed groups only
        for g in groups:
            c = slice(g * group, min(Nkv, (g + 1) * group))
            Ph[:, c] = _p_hat(P[:, c], p_quant, p_fmt, group)
        dP = do[r] @ vh[k_rows].T                             # dP = dO V^T (needed keys)
        dS = P[:, k_rows] * (dP - Delta[:, None])             # dS = P o (dP - Delta)
        dV += Ph[:, k_rows].T @ do[r]                         # dV = P^T dO
        dK += float(sm_scale) * (dS.T @ qh[r])                # dK = scale dS^T Q
        sel = need_dq[r]
        if sel.any():
            dP_q = do[r[sel]] @ vh.T
            dS_q = P[sel] * (dP_q - Delta[sel, None])
            dQ[r[sel]] = float(sm_scale) * (dS_q @ kh)        # dQ = scale dS K
            if k_mean is not None:                            # + scale rowsum(dS) k_mean
                dQ[r[sel]] += float(sm_scale) * np.sum(dS_q, axis=1)[:, None] * np.asarray(k_mean)[None, :]
    return dQ[q_rows], dK, dV


# --------------------------------------------------------------------------
# Whole tensors [B, H, N, D]
# --------------------------------------------------------------------------
def prepare_inputs(q, k, v, qkv_quant=False, v_codes=None, v_scale=None, heads=None):
    """Q^, K^, V^ as float64 arrays [B, H, N, D] (only the (b, h) pairs in
    ``heads`` are filled when given; the others stay zero).

    ``q``, ``k``, ``v`` hold the exact values the kernels receive (bf16 or
    fp16 values carried in a wider float type).  With ``v_codes`` given, V^ is
    the dequantized e5m2 V and ``v`` is ignored.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    qh = np.zeros((B, H, Nq, D))
    kh = np.zeros((B, H, Nkv, D))
    vh = np.zeros((B, H, Nkv, D))
    for b, h in pairs:
        qh[b, h], kh[b, h], vh[b, h] = _prepare_head(q, k, v, b, h, qkv_quant, v_codes, v_scale)
    return qh, kh, vh


def _prepare_head(q, k, v, b, h, qkv_quant, v_codes, v_scale, k_mean=None, dtype="bf16"):
    qh = np.asarray(q[b, h], dtype=np.float64)
    kh = np.asarray(k[b, h], dtype=np.float64)
    if k_mean is not None:
        kh = smooth_keys(kh, k_mean, dtype)
    if qkv_quant:
        qh = quantize_token_rows(qh, "e4m3")[2].astype(np.float64)
        kh = quantize_token_rows(kh, "e4m3")[2].astype(np.float64)
    if v_codes is not None:
        vh = dequant_v_channels(v_codes[b:b + 1, h:h + 1], v_scale[b:b + 1, h:h + 1], "e5m2")[0, 0]
    else:
        vh = np.asarray(v[b, h], dtype=np.float64)
        if qkv_quant:
            vh = quantize_token_rows(vh, "e4m3")[2].astype(np.float64)
    return qh, kh, vh


def attention_forward(q, k, v, sm_scale, causal=False, p_quant=True, p_fmt="e4m3",
                      qkv_quant=False, v_codes=None, v_scale=None, group=P_GROUP,
                      heads=None, rows=None, smooth_k=False, dtype="bf16"):
    """Forward over [B, H, N, D] inputs.

    Returns ``(O, O_hp, lse)`` with shapes [B, H, Nq, D] and [B, H, Nq] (only
    the (b, h) pairs in ``heads`` and the query ``rows`` are computed when
    given; the others stay zero / the arrays are restricted to ``rows``).
    """
    q = np.asarray(q)
    B, H, Nq, D = q.shape
    nr = Nq if rows is None else len(rows)
    O = np.zeros((B, H, nr, D))
    O_hp = np.zeros_like(O)
    lse = np.zeros((B, H, nr))
    k_mean = smooth_key_mean(k, dtype) if smooth_k else None
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        qh, kh, vh = _prepare_head(q, k, v, b, h, qkv_quant, v_codes, v_scale, k_mean, dtype)
        O[b, h], O_hp[b, h], lse[b, h] = forward_head(
            qh, kh, vh, sm_scale, causal, p_quant, p_fmt, group, rows)
    return O, O_hp, lse


def attention_backward(q, k, v, do, sm_scale, causal=False, p_quant=True, p_fmt="e4m3",
                       qkv_quant=False, v_codes=None, v_scale=None, group=P_GROUP,
                       heads=None, q_rows=None, k_rows=None, smooth_k=False, dtype="bf16",
                       lse=None, o_hp=None):
    """Straight-through backward over [B, H, N, D]: returns (dQ, dK, dV).
    ``lse`` [B, H, Nq] and ``o_hp`` [B, H, Nq, D] (chunked mode: the merged
    forward over all chunks) replace this call's own softmax and O_hp."""
    q = np.asarray(q)
    B, H, Nq, D = q.shape
    Nkv = np.asarray(k).shape[2]
    nq = Nq if q_rows is None else len(q_rows)
    nk = Nkv if k_rows is None else len(k_rows)
    dQ = np.zeros((B, H, nq, D))
    dK = np.zeros((B, H, nk, D))
    dV = np.zeros((B, H, nk, D))
    k_mean = smooth_key_mean(k, dtype) if smooth_k else None
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        qh, kh, vh = _prepare_head(q, k, v, b, h, qkv_quant, v_codes, v_scale, k_mean, dtype)
        dQ[b, h], dK[b, h], dV[b, h] = backward_head(
            qh, kh, vh, np.asarray(do[b, h], dtype=np.float64), sm_scale, causal, p_quant, p_fmt,
            group, q_rows, k_rows, k_mean=k_mean,
            lse=None if lse is None else lse[b, h], o_hp=None if o_hp is None else o_hp[b, h])
    return dQ, dK, dV


def merge_chunks(o_parts, o_hp_parts, lse_parts):
    """Forward results of KV chunks merged by their log-sum-exp:
    lse = log sum_c exp(lse_c), O = sum_c exp(lse_c - lse) O_c (O_hp alike)."""
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])      # [C, ...rows]
    m = np.max(L, axis=0)
    finite = np.isfinite(m)
    ms = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(L), np.exp(L - ms), 0.0)
    tot = np.where(finite, np.sum(w, axis=0), 1.0)                        # >= 1 where finite
    lse = np.where(finite, ms + np.log(tot), -np.inf)
    wn = np.where(finite, w / tot, 0.0)                                      # exp(lse_c - lse)
    O = sum(wn[c][..., None] * np.asarray(o_parts[c], dtype=np.float64) for c in range(len(o_parts)))
    O_hp = sum(wn[c][..., None] * np.asarray(o_hp_parts[c], dtype=np.float64) for c in range(len(o_parts)))
    return O, O_hp, lse
