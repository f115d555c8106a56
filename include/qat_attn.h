/*
 * qat_attn.h -- C ABI of the MI355X (gfx950) quantization-aware attention
 * library libqat_attn.so.
 *
 * What it computes.  Fake-quant ("QAT") attention as in the FastVideo
 * attn_qat_train.py source page (functions _attn_fwd_inner, _attn_fwd,
 * _attn_bwd_preprocess, _attn_bwd_dkdv_cross, _attn_bwd_dq_cross and the
 * autograd wrapper _attention): the forward fake-quantizes the probability
 * tile P to fp8 (one absmax scale per query row and per group of
 * QAT_ATTN_P_GROUP key columns), keeps the quantized output O, a
 * high-precision straight-through copy O_hp and the log-sum-exp; the
 * backward rematerialises S and P from the log-sum-exp (the idea raised in
 * the "support for pytorch autograd" discussion) and returns straight-through
 * gradients dQ, dK, dV through every quantizer.
 *
 *   S    = sm_scale * Q^ K^T          (causal: keys j > query i masked)
 *   lse  = log sum_j exp(S)            (natural log, fp32)
 *   P    = exp(S - lse);  P^ = FQ(P)   per row, per QAT_ATTN_P_GROUP columns
 *   O_hp = P V^,   O = P^ V^
 *   Delta = rowsum(dO o O_hp), dS = P o (dO V^T - Delta)
 *   dV = P^T dO,  dQ = sm_scale dS K^,  dK = sm_scale dS^T Q^
 *
 * FQ(x) over a group: a = max|x|, s = fp32(a/FMAX), r = fp32(FMAX/a),
 * code = fp8 round-to-nearest-even, saturating (x*r), x^ = fp32(code*s);
 * an all-zero group gives zeros.  FMAX = 448 (e4m3fn) or 57344 (e5m2).
 *
 * Conventions shared by every entry point.
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    contiguous, layout [B, H, N, D] (row-major; D fastest), 16-byte aligned.
 *  - Storage dtype of q, k, v, dout, o, o_hp, dq, dk, dv is dims->dtype
 *    (bf16 or fp16); lse and v_scale are fp32.
 *  - `stream` is a hipStream_t (NULL: the default stream).  Every call only
 *    enqueues work on that stream; none synchronises, none allocates.
 *  - The caller owns every buffer, including the workspace.  Outputs are
 *    overwritten, never accumulated into.
 *  - Errors: validation happens before any launch and returns a nonzero
 *    status with nothing enqueued.  QAT_EHIP reports a failed launch.
 *  - Results are deterministic: no atomics, fixed reduction orders.
 */
#ifndef QAT_ATTN_H
#define QAT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define QAT_OK 0
#define QAT_EINVAL 1        /* null pointer, bad size, unknown flag bit      */
#define QAT_EUNSUPPORTED 2  /* valid request the library does not implement   */
#define QAT_EWORKSPACE 3    /* workspace pointer null or smaller than needed  */
#define QAT_EHIP 4          /* a kernel launch failed                         */
#define QAT_ESCRATCH 5      /* qat_attn_bwd_noalloc: beyond its static scratch */

/* storage dtypes */
#define QAT_DTYPE_BF16 0
#define QAT_DTYPE_FP16 1

/* quant_flags bits */
#define QAT_P_QUANT     (1u << 0) /* fake-quant P (else O == O_hp)                      */
#define QAT_P_E5M2      (1u << 1) /* P grid e5m2 (else e4m3fn)                          */
#define QAT_QKV_QUANT   (1u << 2) /* per-token e4m3fn fake quant of Q, K, V over D      */
#define QAT_V_FP8_E5M2  (1u << 3) /* v holds e5m2 codes (uint8) + v_scale[B,H,D] fp32  */
/*
 * K smoothing (FastVideo attn_qat_train.py, _attention.forward "smoothing k
 * from SageAttn", and the SMOOTH_K term of _attn_bwd_dq): k_mean[d], the mean
 * of K over every batch, head and token rounded to the dtype, is subtracted
 * from K (rounded to the dtype) before anything else, Q/K/V quantization
 * included.  Softmax does not change under that per-row score shift, so O,
 * O_hp and dV are those of the unsmoothed inputs (up to the rounding of
 * K - k_mean, and the K quantization then differs); lse is that of the
 * smoothed scores, i.e. shifted by -sm_scale * (q . k_mean).  dQ takes the
 * term sm_scale * rowsum(dS) k_mean, so it is the gradient for the original
 * K; dK is returned as computed for the smoothed K.
 */
#define QAT_SMOOTH_K    (1u << 4)

#define QAT_ATTN_P_GROUP 64       /* key columns per P-quant scale (absolute columns)   */

typedef struct qat_attn_dims {
    int32_t B, H;      /* batch, heads                                           */
    int32_t Nq, Nkv;   /* query and key/value sequence lengths (Nkv may != Nq)   */
    int32_t D;         /* head dim: 64 or 128                                    */
    int32_t dtype;     /* QAT_DTYPE_BF16 or QAT_DTYPE_FP16                        */
} qat_attn_dims;

/*
 * Forward (FastVideo attn_qat_train.py: _attention.forward driving the
 * fake_quantize_q / fake_quantize_kv pre-pass and _attn_fwd / _attn_fwd_inner).
 *
 *  q [B,H,Nq,D], k [B,H,Nkv,D]: dtype.
 *  v [B,H,Nkv,D]: dtype, or uint8 e5m2 codes with QAT_V_FP8_E5M2, in which
 *     case v_scale [B,H,D] (fp32) gives V^ = code * v_scale[b,h,d]; v_scale
 *     must be NULL otherwise.
 *  sm_scale: softmax scale (> 0, finite).  causal: nonzero for the causal
 *     mask (requires Nq == Nkv, top-left aligned, diagonal kept).
 *  o, o_hp [B,H,Nq,D] (dtype): quantized-P output and straight-through output.
 *  lse [B,H,Nq] (fp32): natural-log log-sum-exp of each query row.
 *  workspace: device scratch of at least qat_attn_workspace_bytes(dims,
 *     flags, 0) bytes (may be NULL when that is 0).
 *
 * Returns QAT_EINVAL (null/size/flag errors, v_scale presence not matching
 * the flag), QAT_EUNSUPPORTED (D not 64/128, causal with Nq != Nkv,
 * QAT_V_FP8_E5M2 together with QAT_QKV_QUANT or with fp16), QAT_EWORKSPACE,
 * QAT_EHIP, else QAT_OK.
 */
int qat_attn_fwd(const qat_attn_dims* dims, const void* q, const void* k, const void* v,
                 const float* v_scale, float sm_scale, int causal, uint32_t quant_flags,
                 void* o, void* o_hp, float* lse, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * Backward (FastVideo attn_qat_train.py: _attention.backward with
 * _attn_bwd_preprocess, _attn_bwd_dkdv_cross, _attn_bwd_dq_cross).
 *
 * Takes the same q, k, v, v_scale, sm_scale, causal and quant_flags as the
 * forward, the forward's o_hp and lse, and dout = dL/dO [B,H,Nq,D] (dtype).
 * With QAT_QKV_QUANT the inputs are fake-quantized again exactly as in the
 * forward (bit-identical), and the gradients are evaluated there.
 * Writes dq [B,H,Nq,D], dk, dv [B,H,Nkv,D] (dtype; dv is the gradient with
 * respect to the dequantized V^ when V is fp8) as straight-through gradients
 * of the un-quantized inputs.  Delta = rowsum(dout o o_hp) is kept in the
 * workspace (>= qat_attn_workspace_bytes(dims, flags, 1) bytes), and so are
 * fp32 partial sums of dk, dv when the last 128-key blocks of a launch are
 * split over query ranges to fill the device (added in a fixed order: the
 * result stays bitwise reproducible on a given device).
 * Errors as for qat_attn_fwd.
 */
int qat_attn_bwd(const qat_attn_dims* dims, const void* q, const void* k, const void* v,
                 const float* v_scale, const void* o_hp, const float* lse, const void* dout,
                 float sm_scale, int causal, uint32_t quant_flags,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * The backward as separately launchable stages, for callers that time,
 * interleave or overlap them.  Arguments and workspace are those of
 * qat_attn_bwd; `stages` is a mask of
 *   QAT_BWD_PREPARE  K smoothing and Q/K/V fake quant into the workspace
 *                    (QAT_SMOOTH_K, QAT_QKV_QUANT)
 *   QAT_BWD_DELTA    Delta = rowsum(dout o o_hp) into the workspace (together
 *                    with QAT_BWD_DQ the dQ kernel forms it, the same bits,
 *                    and no separate pass runs)
 *   QAT_BWD_DQ       dq, and with QAT_P_QUANT the P-quant absmax record
 *                    in the workspace (see QAT_P_ABSMAX_MAX_BYTES)
 *   QAT_BWD_DKDV     dk, dv (reads Delta and that record)
 * A stage reads what earlier stages left in the same workspace: run them in
 * this order, on one stream, with unchanged arguments.  qat_attn_bwd is
 * QAT_BWD_ALL.  Errors as for qat_attn_bwd; QAT_EINVAL for an empty or
 * unknown mask.
 */
#define QAT_BWD_PREPARE (1u << 0)
#define QAT_BWD_DELTA   (1u << 1)
#define QAT_BWD_DQ      (1u << 2)
#define QAT_BWD_DKDV    (1u << 3)
#define QAT_BWD_ALL     (QAT_BWD_PREPARE | QAT_BWD_DELTA | QAT_BWD_DQ | QAT_BWD_DKDV)

int qat_attn_bwd_stages(const qat_attn_dims* dims, const void* q, const void* k, const void* v,
                        const float* v_scale, const void* o_hp, const float* lse, const void* dout,
                        float sm_scale, int causal, uint32_t quant_flags,
                        void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        uint32_t stages, void* stream);

/*
 * The backward without allocation and without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Arguments, results
 * and errors are those of qat_attn_bwd, except that:
 *  - its scratch is a static device array of QAT_NOALLOC_SCRATCH_BYTES that
 *    the library holds on every GPU it runs on until the process ends (its
 *    address is looked up on the first call on each device); the call
 *    allocates nothing and needs none of its contents to start at zero;
 *  - problems whose scratch exceeds that size (qat_attn_workspace_bytes(dims,
 *    flags, 1) less the dK/dV partial sums and the P-quant absmax record)
 *    return QAT_ESCRATCH with nothing enqueued: e.g. the DiT image shape
 *    (B1 H24 N4608 D128, 0.4 MB) fits, per-token Q/K/V quantization at
 *    long-video size does not;
 *  - every dK/dV key block runs whole (no query-range split) and the dK/dV
 *    kernel forms the P-quant absmax itself, so dK and dV may differ from
 *    qat_attn_bwd's in the last bits (fp32 summation order, and the absmax
 *    taken from the dK/dV kernel's own scores);
 *  - all calls on one GPU share its scratch: calls that overlap on one GPU
 *    (other streams, other host threads) race and must be serialised by the
 *    caller.
 */
#define QAT_NOALLOC_SCRATCH_BYTES (64u << 20)
int qat_attn_bwd_noalloc(const qat_attn_dims* dims, const void* q, const void* k, const void* v,
                         const float* v_scale, const void* o_hp, const float* lse, const void* dout,
                         float sm_scale, int causal, uint32_t quant_flags,
                         void* dq, void* dk, void* dv, void* stream);

/*
 * Chunked-KV mode on one GPU: the local half of ring attention ("usp:
 * differentiable operators for training", the ring pass that merges partial
 * attention by log-sum-exp).  Run qat_attn_fwd on each KV chunk (keys of
 * chunk c as k, v; non-causal) into (o_c, o_hp_c, lse_c), then
 *   qat_attn_merge: lse = log sum_c exp(lse_c), o = sum_c exp(lse_c - lse) o_c,
 *                   o_hp likewise (fp32, chunk order; rounded to the dtype).
 * With chunk boundaries at multiples of QAT_ATTN_P_GROUP keys this is the
 * unchunked result up to rounding, the quantized o included (a group's
 * scale is invariant to the factor exp(lse_c - lse)).  For the backward run
 * qat_attn_bwd on each chunk with the merged o_hp and lse: its dk, dv are
 * those of the chunk's keys; the dq of the chunks are added by qat_attn_sum.
 * Flags: per-token Q/K/V quantization is per row, so chunking leaves it
 * unchanged; with fp8 V pass each chunk's codes with the unchunked v_scale.
 * QAT_SMOOTH_K does not carry over: each chunk would be smoothed by the mean
 * of its own keys, which shifts its lse_c by a different per-row constant
 * and so breaks the merge weights.  Subtract one mean over all keys from K
 * before chunking instead (softmax does not change; dQ then lacks the
 * rowsum(dS) * k_mean term, which the caller adds).
 *  dims: B, H, Nq, D, dtype of the parts (Nkv is not used); n_chunks in
 *  1..QAT_MERGE_MAX_CHUNKS; *_parts: host arrays of device pointers, each
 *  part [B,H,Nq,D] (dtype) and lse [B,H,Nq] (fp32), 16-byte aligned.  A row
 *  whose every lse_c is -inf gives lse = -inf and zero outputs.
 * qat_attn_sum: out = sum of n_parts tensors [B,H,Nq,D] (dtype), fp32 in part
 *  order.  Both: QAT_EINVAL for bad dims, counts or pointers; QAT_EHIP.
 */
#define QAT_MERGE_MAX_CHUNKS 16
int qat_attn_merge(const qat_attn_dims* dims, int n_chunks, const void* const* o_parts,
                   const void* const* o_hp_parts, const float* const* lse_parts,
                   void* o, void* o_hp, float* lse, void* stream);
int qat_attn_sum(const qat_attn_dims* dims, int n_parts, const void* const* parts, void* out, void* stream);

/*
 * Workspace bytes needed by the forward (pass 0) or the backward (pass 1).
 * No page defines this call: the FastVideo source's _attention.forward and
 * _attention.backward allocate their scratch tensors themselves (the
 * fake-quantized q, k, v copies, M, delta), while this library never
 * allocates, so the caller asks for the size and passes the buffer in.
 * Returns 0 for a null dims pointer, negative sizes or a pass other than
 * 0 or 1; otherwise the size for these dims and flags (it may be 0).
 */
size_t qat_attn_workspace_bytes(const qat_attn_dims* dims, uint32_t quant_flags, int pass);

/*
 * The backward's workspace holds, with QAT_P_QUANT, the dQ kernel's record of
 * the P-quant absmax per (query row, 64-key group), fp32 B*H*ceil(Nkv/64)*Nq,
 * for the dK/dV kernel, while that record takes at most this many bytes.
 * Beyond it the record is left out (the workspace stays linear in Nq and
 * Nkv) and the dK/dV kernel forms the absmax itself, at some cost in time.
 */
#define QAT_P_ABSMAX_MAX_BYTES ((size_t)1 << 30)

/*
 * Per-channel e5m2 quantization of V for the fp8-V path (the e5m2 value path
 * of _attn_fwd in the FastVideo source, with one absmax scale per
 * (b, h, d) over the Nkv tokens).  v [B,H,Nkv,D] dtype -> codes [B,H,Nkv,D]
 * uint8 and v_scale [B,H,D] fp32, by FQ with FMAX = 57344.
 * Errors: QAT_EINVAL, QAT_EUNSUPPORTED (D), QAT_EHIP.
 */
int qat_quant_v_fp8(const qat_attn_dims* dims, const void* v, uint8_t* codes, float* v_scale,
                    void* stream);

/*
 * FQ of a row-major fp32 matrix x [rows, cols] with one scale per row and
 * per `group` absolute columns, through the same device code the attention
 * kernels use (the fake_quantize call of _attn_fwd_inner).  fmt: 0 = e4m3fn,
 * 1 = e5m2.  Writes codes [rows, cols] uint8, scales [rows, ceil(cols/group)]
 * fp32 and xhat [rows, cols] fp32 (any of the three may be NULL).
 * Errors: QAT_EINVAL (x null, rows/cols/group <= 0, fmt not 0/1), QAT_EHIP.
 */
int qat_fake_quant_rows(const float* x, int32_t rows, int32_t cols, int32_t group, int32_t fmt,
                        uint8_t* codes, float* scales, float* xhat, void* stream);

/*
 * Self-test of a hardware property the kernels rely on.  The forward takes a
 * row's P-quant absmax as exp2 of the row group's largest argument rather
 * than as the max over the exp2 results; both are the same value exactly when
 * the exp2 instruction (v_exp_f32) never decreases between adjacent fp32
 * arguments.  Counts the adjacent fp32 pairs x < x' in [lo, hi] with
 * exp2(x') < exp2(x) into *violations (a device uint32, overwritten), over
 * every fp32 value in the range.  Errors: QAT_EINVAL (null pointer, NaN
 * bound, lo > hi), QAT_EHIP.
 */
int qat_selftest_exp2_monotone(float lo, float hi, uint32_t* violations, void* stream);

/*
 * Self-test of the quantizer's scale pair.  Every kernel computes a group's
 * s = a / FMAX and r = FMAX / a (correctly rounded fp32 quotients, both 0
 * when FMAX / a overflows; the quantizer definition above) without the
 * division instruction sequence: a reciprocal refined by a Newton step and a
 * remainder correction.  Counts into *mismatches (a device uint32,
 * overwritten) the positive finite fp32 values a, over all of them, for
 * which that pair differs in any bit from the one IEEE division gives.
 * fmt: 0 = e4m3fn (FMAX 448), 1 = e5m2 (FMAX 57344).  Errors: QAT_EINVAL
 * (null pointer, unknown fmt), QAT_EHIP.
 */
int qat_selftest_fq_scale(int32_t fmt, uint32_t* mismatches, void* stream);

/*
 * QAT_ATTN_P_GROUP as compiled into the kernels: the number of key columns
 * that share one P-quant scale per query row.  In the FastVideo source this
 * is the BLOCK_SIZE_QUANT_DIM argument of the fake_quantize call on the P
 * tile inside _attn_fwd_inner (the kernel's BLOCK_N, which differs between its
 * forward and backward variants); here one width serves both passes.  No
 * arguments, no errors.
 */
int qat_attn_p_group(void);

/*
 * Static description of a status code (never NULL; "unknown status" for a
 * value that is not one of the QAT_* codes).  No page defines it: the
 * source reports errors through Python exceptions (assert, ValueError in
 * _attention.forward); the C boundary returns codes instead.
 */
const char* qat_attn_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* QAT_ATTN_H */
