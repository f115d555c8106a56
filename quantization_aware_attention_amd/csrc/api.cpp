// C ABI of libqat_attn.so (declared in include/qat_attn.h): argument
// validation, workspace layout and kernel dispatch.  Every check runs before
// the first launch, so an error return means nothing was enqueued.
#include "../../include/qat_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "launch.hpp"
#include "api_internal.hpp"

namespace {

constexpr uint32_t KNOWN_FLAGS = QAT_P_QUANT | QAT_P_E5M2 | QAT_QKV_QUANT | QAT_V_FP8_E5M2 | QAT_SMOOTH_K;
constexpr size_t ALIGN = 256;

inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workspace layout (each piece 256-byte aligned, in this order):
//   bwd: delta fp32 [B,H,Nq]; with P quant, the dQ kernel's record of the
//   P-quant absmax fp32 [B,H,ceil(Nkv/64),Nq] while it takes at most
//   QAT_P_ABSMAX_MAX_BYTES (beyond that, the dK/dV kernel forms it itself);
//   fp32 partial dK/dV of key blocks split over query ranges
//   fwd and bwd, with K smoothing: the mean's partial sums fp32 [256, D], the
//   mean fp32 [D] and, without Q/K/V quantization, K - mean (dtype);
//   fwd and bwd, when Q/K/V quantization is on: the fp8 code values of Q and
//   K (dtype) with their per-token scales (fp32 [B,H,Nq], [B,H,Nkv]), and
//   V^ = code * scale rounded to the dtype
qat::Shape shape_of(const qat_attn_dims& d) { return qat::Shape{d.B, d.H, d.Nq, d.Nkv, d.D, d.dtype}; }

struct Layout {
  size_t delta = 0, amax = 0, part = 0, kpart = 0, kmean = 0, ksm = 0, qh = 0, kh = 0, vh = 0, qs = 0, ks = 0;
  size_t q8 = 0, k8 = 0, total = 0;
  bool side = false;   // the absmax record is part of the workspace
};

size_t p_absmax_bytes(const qat_attn_dims& d) {
  const size_t ng = ((size_t)d.Nkv + QAT_ATTN_P_GROUP - 1) / QAT_ATTN_P_GROUP;
  return (size_t)d.B * d.H * ng * d.Nq * sizeof(float);
}

// full = false (the static-scratch backward) leaves out the dK/dV tail-split
// partial sums (every key block then runs whole) and the absmax record
Layout layout(const qat_attn_dims& d, uint32_t flags, int pass, bool full = true) {
  Layout L;
  const size_t BH = (size_t)d.B * d.H;
  size_t off = 0;
  if (pass == 1) {
    L.delta = off;
    off += align_up(BH * d.Nq * sizeof(float));
    L.side = full && (flags & QAT_P_QUANT) && p_absmax_bytes(d) <= QAT_P_ABSMAX_MAX_BYTES;
    if (L.side) {
      L.amax = off;
      off += align_up(p_absmax_bytes(d));
    }
    L.part = off;
    if (full) off += align_up(qat::dkdv_part_bytes(shape_of(d)));
  }
  if (flags & QAT_SMOOTH_K) {
    L.kpart = off;
    off += align_up((size_t)qat::KMEAN_BLOCKS * d.D * sizeof(float));
    L.kmean = off;
    off += align_up((size_t)d.D * sizeof(float));
    if (!(flags & QAT_QKV_QUANT)) {
      L.ksm = off;
      off += align_up(BH * d.Nkv * d.D * 2);
    }
  }
  if (flags & QAT_QKV_QUANT) {
    L.qh = off;
    off += align_up(BH * d.Nq * d.D * 2);
    L.kh = off;
    off += align_up(BH * d.Nkv * d.D * 2);
    L.vh = off;
    off += align_up(BH * d.Nkv * d.D * 2);
    L.qs = off;
    off += align_up(BH * d.Nq * sizeof(float));
    L.ks = off;
    off += align_up(BH * d.Nkv * sizeof(float));
    L.q8 = off;
    off += align_up(BH * d.Nq * d.D);
    L.k8 = off;
    off += align_up(BH * d.Nkv * d.D);
  }
  L.total = off;
  return L;
}

// Shared validation.  Returns QAT_OK and sets *empty when there is no work.
int check_common(const qat_attn_dims* dims, float sm_scale, int causal, uint32_t flags,
                 const float* v_scale, bool* empty) {
  if (!dims) return QAT_EINVAL;
  const qat_attn_dims& d = *dims;
  if (d.B < 0 || d.H < 0 || d.Nq < 0 || d.Nkv < 0 || d.D <= 0) return QAT_EINVAL;
  if (d.dtype != QAT_DTYPE_BF16 && d.dtype != QAT_DTYPE_FP16) return QAT_EINVAL;
  if (flags & ~KNOWN_FLAGS) return QAT_EINVAL;
  if ((flags & QAT_P_E5M2) && !(flags & QAT_P_QUANT)) return QAT_EINVAL;
  if (!(std::isfinite(sm_scale) && sm_scale > 0.0f)) return QAT_EINVAL;
  const bool vfp8 = (flags & QAT_V_FP8_E5M2) != 0;
  if (vfp8 != (v_scale != nullptr)) return QAT_EINVAL;
  if (d.D != 64 && d.D != 128) return QAT_EUNSUPPORTED;
  if (causal && d.Nq != d.Nkv) return QAT_EUNSUPPORTED;
  if (vfp8 && (d.dtype != QAT_DTYPE_BF16 || (flags & QAT_QKV_QUANT))) return QAT_EUNSUPPORTED;
  // one workgroup per 128-row tile per (b, h): the launch must fit a 31-bit grid
  const long long tiles = ((long long)(d.Nq > d.Nkv ? d.Nq : d.Nkv) + 127) / 128;
  if ((long long)d.B * d.H > 65535 || tiles * d.B * d.H > 0x7fffffffLL) return QAT_EUNSUPPORTED;
  // one head's [N, D] tensor must be addressable by 32-bit byte offsets (the
  // kernels read tiles through buffer descriptors sized to one head)
  if ((long long)(d.Nq > d.Nkv ? d.Nq : d.Nkv) * d.D * 2 > 0x7fffffffLL) return QAT_EUNSUPPORTED;
  *empty = (d.B == 0 || d.H == 0 || d.Nq == 0);
  if (!*empty && d.Nkv == 0) return QAT_EINVAL;   // softmax over no keys
  return QAT_OK;
}

int check_ptr(const void* p) { return (p && aligned16(p)) ? QAT_OK : QAT_EINVAL; }


int pfmt_of(uint32_t flags) {
  if (!(flags & QAT_P_QUANT)) return -1;
  return (flags & QAT_P_E5M2) ? 1 : 0;
}

#define QAT_TRY(expr)                                  \
  do {                                                 \
    if ((expr) != hipSuccess) return QAT_EHIP;         \
  } while (0)

// The inputs the attention kernels read: the caller's tensors, or for Q/K/V
// quantization the pre-pass outputs in the workspace (run here).
int prepare_inputs(const qat_attn_dims& d, const Layout& L, uint32_t flags, const void* q, const void* k,
                   const void* v, const float* v_scale, char* ws, hipStream_t st, qat::Inputs* in) {
  *in = qat::Inputs{q, k, v, v_scale, nullptr, nullptr, qat::IN_PLAIN, nullptr};
  if (flags & QAT_V_FP8_E5M2) in->mode = qat::IN_VFP8;
  const long BH = (long)d.B * d.H;
  float* kmean = nullptr;
  if (flags & QAT_SMOOTH_K) {   // k_mean, and K - k_mean unless the quant pre-pass subtracts it
    kmean = reinterpret_cast<float*>(ws + L.kmean);
    void* ksm = (flags & QAT_QKV_QUANT) ? nullptr : ws + L.ksm;
    QAT_TRY(qat::launch_k_smooth(d.dtype, d.D, BH * d.Nkv, k, reinterpret_cast<float*>(ws + L.kpart), kmean, ksm, st));
    in->k_mean = kmean;
    if (ksm) in->k = ksm;
  }
  if (flags & QAT_QKV_QUANT) {
    float* qs = reinterpret_cast<float*>(ws + L.qs);
    float* ks = reinterpret_cast<float*>(ws + L.ks);
    QAT_TRY(qat::launch_token_quant(d.dtype, d.D, BH * d.Nq, q, ws + L.qh, qs, nullptr, ws + L.q8, st));
    QAT_TRY(qat::launch_token_quant(d.dtype, d.D, BH * d.Nkv, k, ws + L.kh, ks, kmean, ws + L.k8, st));
    QAT_TRY(qat::launch_token_quant(d.dtype, d.D, BH * d.Nkv, v, ws + L.vh, nullptr, nullptr, nullptr, st));
    *in = qat::Inputs{ws + L.qh, ws + L.kh, ws + L.vh, nullptr, qs, ks, qat::IN_QKS, kmean, ws + L.q8, ws + L.k8};
  }
  return QAT_OK;
}

// The inputs of the attention stages when the pre-passes ran earlier (their
// outputs are in the workspace).
qat::Inputs prepared_inputs(const Layout& L, uint32_t flags, const void* q, const void* k, const void* v,
                            const float* v_scale, char* ws) {
  qat::Inputs in{q, k, v, v_scale, nullptr, nullptr, qat::IN_PLAIN, nullptr};
  if (flags & QAT_V_FP8_E5M2) in.mode = qat::IN_VFP8;
  if (flags & QAT_SMOOTH_K) {
    in.k_mean = reinterpret_cast<float*>(ws + L.kmean);
    if (!(flags & QAT_QKV_QUANT)) in.k = ws + L.ksm;
  }
  if (flags & QAT_QKV_QUANT)
    in = qat::Inputs{ws + L.qh, ws + L.kh, ws + L.vh, nullptr, reinterpret_cast<float*>(ws + L.qs),
                     reinterpret_cast<float*>(ws + L.ks), qat::IN_QKS, in.k_mean, ws + L.q8, ws + L.k8};
  return in;
}

}  // namespace

size_t qat::bwd_bytes_whole(const qat_attn_dims* dims, uint32_t quant_flags) {
  if (!dims) return 0;
  const qat_attn_dims& d = *dims;
  if (d.B < 0 || d.H < 0 || d.Nq < 0 || d.Nkv < 0 || d.D <= 0) return 0;
  return layout(d, quant_flags, 1, false).total;
}

int qat::bwd_impl(const qat_attn_dims* dims, const void* q, const void* k, const void* v,
                  const float* v_scale, const void* o_hp, const float* lse, const void* dout,
                  float sm_scale, int causal, uint32_t quant_flags,
                  void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                  uint32_t stages, bool split_tail, void* stream) {
  if (stages == 0 || (stages & ~QAT_BWD_ALL)) return QAT_EINVAL;
  bool empty = false;
  int rc = check_common(dims, sm_scale, causal, quant_flags, v_scale, &empty);
  if (rc != QAT_OK) return rc;
  if (empty) return QAT_OK;
  const void* need[] = {q, k, v, o_hp, lse, dout, dq, dk, dv};
  for (const void* p : need)
    if ((rc = check_ptr(p)) != QAT_OK) return rc;
  if (v_scale && !aligned16(v_scale)) return QAT_EINVAL;
  const qat_attn_dims& d = *dims;
  const Layout L = layout(d, quant_flags, 1, split_tail);
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return QAT_EWORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const qat::Shape s = shape_of(d);
  char* ws = static_cast<char*>(workspace);
  qat::Inputs in;
  if (stages & QAT_BWD_PREPARE) {
    if ((rc = prepare_inputs(d, L, quant_flags, q, k, v, v_scale, ws, st, &in)) != QAT_OK) return rc;
  } else {   // later stages read what the prepare stage left in the workspace
    in = prepared_inputs(L, quant_flags, q, k, v, v_scale, ws);
  }
  float* delta = reinterpret_cast<float*>(ws + L.delta);
  float* amax = L.side ? reinterpret_cast<float*>(ws + L.amax) : nullptr;
  const int pfmt = pfmt_of(quant_flags);
  // Delta together with dQ: the dQ kernel forms it for its rows (bit for bit
  // as the separate pass) and publishes it for dK/dV, one launch fewer
  const bool delta_in_dq = (stages & QAT_BWD_DELTA) && (stages & QAT_BWD_DQ);
  if ((stages & QAT_BWD_DELTA) && !delta_in_dq) QAT_TRY(qat::launch_bwd_delta(s, o_hp, dout, delta, st));
  if (stages & QAT_BWD_DQ)
    QAT_TRY(qat::launch_bwd_dq(s, in, dout, lse, delta, delta_in_dq ? o_hp : nullptr, sm_scale, causal != 0, pfmt,
                               dq, amax, st));
  if (stages & QAT_BWD_DKDV)
    QAT_TRY(qat::launch_bwd_dkdv(s, in, dout, lse, delta, amax, sm_scale, causal != 0, pfmt, dk, dv,
                                 split_tail ? reinterpret_cast<float*>(ws + L.part) : nullptr, st));
  return QAT_OK;
}

extern "C" {

size_t qat_attn_workspace_bytes(const qat_attn_dims* dims, uint32_t quant_flags, int pass) {
  if (!dims || (pass != 0 && pass != 1)) return 0;
  const qat_attn_dims& d = *dims;
  if (d.B < 0 || d.H < 0 || d.Nq < 0 || d.Nkv < 0 || d.D <= 0) return 0;
  return layout(d, quant_flags, pass).total;
}

int qat_attn_fwd(const qat_attn_dims* dims, const void* q, const void* k, const void* v,
                 const float* v_scale, float sm_scale, int causal, uint32_t quant_flags,
                 void* o, void* o_hp, float* lse, void* workspace, size_t workspace_bytes,
                 void* stream) {
  bool empty = false;
  int rc = check_common(dims, sm_scale, causal, quant_flags, v_scale, &empty);
  if (rc != QAT_OK) return rc;
  if (empty) return QAT_OK;
  const void* need[] = {q, k, v, o, o_hp, lse};
  for (const void* p : need)
    if ((rc = check_ptr(p)) != QAT_OK) return rc;
  if (v_scale && !aligned16(v_scale)) return QAT_EINVAL;
  const qat_attn_dims& d = *dims;
  const Layout L = layout(d, quant_flags, 0);
  if (L.total > 0 && (!workspace || workspace_bytes < L.total || !aligned16(workspace))) return QAT_EWORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const qat::Shape s = shape_of(d);
  qat::Inputs in;
  if ((rc = prepare_inputs(d, L, quant_flags, q, k, v, v_scale, static_cast<char*>(workspace), st, &in)) != QAT_OK)
    return rc;
  QAT_TRY(qat::launch_fwd(s, in, sm_scale, causal != 0, pfmt_of(quant_flags), o, o_hp, lse, st));
  return QAT_OK;
}

int qat_attn_bwd_stages(const qat_attn_dims* dims, const void* q, const void* k, const void* v,
                        const float* v_scale, const void* o_hp, const float* lse, const void* dout,
                        float sm_scale, int causal, uint32_t quant_flags,
                        void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        uint32_t stages, void* stream) {
  return qat::bwd_impl(dims, q, k, v, v_scale, o_hp, lse, dout, sm_scale, causal, quant_flags, dq, dk, dv,
                       workspace, workspace_bytes, stages, true, stream);
}

int qat_attn_bwd(const qat_attn_dims* dims, const void* q, const void* k, const void* v,
                 const float* v_scale, const void* o_hp, const float* lse, const void* dout,
                 float sm_scale, int causal, uint32_t quant_flags,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return qat_attn_bwd_stages(dims, q, k, v, v_scale, o_hp, lse, dout, sm_scale, causal, quant_flags, dq, dk,
                             dv, workspace, workspace_bytes, QAT_BWD_ALL, stream);
}

static_assert(QAT_MERGE_MAX_CHUNKS == qat::MERGE_MAX, "merge chunk limit");

static int check_parts_dims(const qat_attn_dims* dims, int n) {
  if (!dims || n < 1 || n > QAT_MERGE_MAX_CHUNKS) return QAT_EINVAL;
  const qat_attn_dims& d = *dims;
  if (d.B < 0 || d.H < 0 || d.Nq < 0 || (d.D != 64 && d.D != 128)) return QAT_EINVAL;
  if (d.dtype != QAT_DTYPE_BF16 && d.dtype != QAT_DTYPE_FP16) return QAT_EINVAL;
  return QAT_OK;
}

int qat_attn_merge(const qat_attn_dims* dims, int n_chunks, const void* const* o_parts,
                   const void* const* o_hp_parts, const float* const* lse_parts,
                   void* o, void* o_hp, float* lse, void* stream) {
  int rc = check_parts_dims(dims, n_chunks);
  if (rc != QAT_OK) return rc;
  if (!o_parts || !o_hp_parts || !lse_parts) return QAT_EINVAL;
  const long rows = (long)dims->B * dims->H * dims->Nq;
  if (rows == 0) return QAT_OK;
  qat::MergeArgs a = {};
  a.n = n_chunks;
  for (int c = 0; c < n_chunks; ++c) {
    if (check_ptr(o_parts[c]) || check_ptr(o_hp_parts[c]) || check_ptr(lse_parts[c])) return QAT_EINVAL;
    a.o[c] = o_parts[c];
    a.o_hp[c] = o_hp_parts[c];
    a.lse[c] = lse_parts[c];
  }
  if (check_ptr(o) || check_ptr(o_hp) || check_ptr(lse)) return QAT_EINVAL;
  a.out_o = o;
  a.out_o_hp = o_hp;
  a.out_lse = lse;
  QAT_TRY(qat::launch_merge(dims->dtype, dims->D, rows, a, static_cast<hipStream_t>(stream)));
  return QAT_OK;
}

int qat_attn_sum(const qat_attn_dims* dims, int n_parts, const void* const* parts, void* out, void* stream) {
  int rc = check_parts_dims(dims, n_parts);
  if (rc != QAT_OK) return rc;
  if (!parts) return QAT_EINVAL;
  const long n = (long)dims->B * dims->H * dims->Nq * dims->D;
  if (n == 0) return QAT_OK;
  qat::MergeArgs a = {};
  a.n = n_parts;
  for (int c = 0; c < n_parts; ++c) {
    if (check_ptr(parts[c])) return QAT_EINVAL;
    a.o[c] = parts[c];
  }
  if (check_ptr(out)) return QAT_EINVAL;
  a.out_o = out;
  QAT_TRY(qat::launch_sum(dims->dtype, n, a, static_cast<hipStream_t>(stream)));
  return QAT_OK;
}

int qat_quant_v_fp8(const qat_attn_dims* dims, const void* v, uint8_t* codes, float* v_scale,
                    void* stream) {
  if (!dims) return QAT_EINVAL;
  const qat_attn_dims& d = *dims;
  if (d.B < 0 || d.H < 0 || d.Nkv < 0 || d.D <= 0) return QAT_EINVAL;
  if (d.dtype != QAT_DTYPE_BF16 && d.dtype != QAT_DTYPE_FP16) return QAT_EINVAL;
  if (d.D != 64 && d.D != 128) return QAT_EUNSUPPORTED;
  if ((long long)d.B * d.H > 0x7fffffff) return QAT_EUNSUPPORTED;
  if ((long long)d.B * d.H * d.Nkv == 0) return QAT_OK;
  if (!v || !codes || !v_scale || !aligned16(v) || !aligned16(codes) || !aligned16(v_scale)) return QAT_EINVAL;
  QAT_TRY(qat::launch_v_quant(d.dtype, d.D, d.B * d.H, d.Nkv, v, codes, v_scale,
                              static_cast<hipStream_t>(stream)));
  return QAT_OK;
}

int qat_fake_quant_rows(const float* x, int32_t rows, int32_t cols, int32_t group, int32_t fmt,
                        uint8_t* codes, float* scales, float* xhat, void* stream) {
  if (!x || rows <= 0 || cols <= 0 || group <= 0 || (fmt != 0 && fmt != 1)) return QAT_EINVAL;
  QAT_TRY(qat::launch_fq_rows(x, rows, cols, group, fmt, codes, scales, xhat,
                              static_cast<hipStream_t>(stream)));
  return QAT_OK;
}

int qat_selftest_exp2_monotone(float lo, float hi, uint32_t* violations, void* stream) {
  if (!violations || !(lo <= hi) || std::isnan(lo) || std::isnan(hi)) return QAT_EINVAL;
  QAT_TRY(qat::launch_exp2_selftest(lo, hi, violations, static_cast<hipStream_t>(stream)));
  return QAT_OK;
}

int qat_selftest_fq_scale(int32_t fmt, uint32_t* mismatches, void* stream) {
  if (!mismatches || (fmt != 0 && fmt != 1)) return QAT_EINVAL;
  QAT_TRY(qat::launch_fq_scale_selftest(fmt, mismatches, static_cast<hipStream_t>(stream)));
  return QAT_OK;
}

int qat_attn_p_group(void) { return QAT_ATTN_P_GROUP; }

const char* qat_attn_strerror(int status) {
  switch (status) {
    case QAT_OK: return "ok";
    case QAT_EINVAL: return "invalid argument";
    case QAT_EUNSUPPORTED: return "unsupported configuration";
    case QAT_EWORKSPACE: return "workspace missing or too small";
    case QAT_EHIP: return "HIP launch failure";
    case QAT_ESCRATCH: return "problem needs more than the static scratch of qat_attn_bwd_noalloc holds";
    default: return "unknown status";
  }
}

}  // extern "C"
