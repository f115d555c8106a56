// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qat {

struct Shape {
  int B, H, Nq, Nkv, D;
  int dtype;   // 0 bf16, 1 fp16
};

// Input modes of the attention kernels.
//  IN_PLAIN: q, k, v hold the values (dtype).
//  IN_VFP8:  v holds e5m2 codes, V^ = code * v_scale[b, h, d].
//  IN_QKS:   q, k hold fp8 code values (dtype) with one fp32 scale per token
//            (q_scale [B,H,Nq], k_scale [B,H,Nkv]); v holds values.
enum InMode { IN_PLAIN = 0, IN_VFP8 = 1, IN_QKS = 2 };

struct Inputs {
  const void* q;
  const void* k;
  const void* v;
  const float* v_scale;   // IN_VFP8
  const float* q_scale;   // IN_QKS
  const float* k_scale;   // IN_QKS
  int mode;
  const float* k_mean;    // K smoothing: the mean subtracted from K (dQ correction), or null
  const void* q8;         // IN_QKS: e4m3 code bytes of Q and K [BH, N, D] (the fp8 MFMA operands of S)
  const void* k8;
};

// pfmt: -1 = P not quantized, 0 = e4m3fn, 1 = e5m2
hipError_t launch_fwd(const Shape& s, const Inputs& in, float sm_scale, bool causal, int pfmt,
                      void* o, void* o_hp, float* lse, hipStream_t st);

// Per-token e4m3 fake quant: x [rows, D] -> xhat [rows, D] (same dtype); with
// scale_out the code values and the per-row scales are stored separately, and
// with codes8 also the e4m3 code bytes [rows, D].
hipError_t launch_token_quant(int dtype, int D, long rows, const void* x, void* xhat, float* scale_out,
                              const float* shift, void* codes8, hipStream_t st);

// K smoothing: mean[D] = dtype-rounded mean of K [rows, D] over all rows
// (part: KMEAN_BLOCKS x D fp32 scratch); with k_smooth, also K - mean rounded
// to the dtype.
constexpr int KMEAN_BLOCKS = 256;
hipError_t launch_k_smooth(int dtype, int D, long rows, const void* k, float* part, float* mean, void* k_smooth,
                           hipStream_t st);

// Per-channel e5m2 quant of V [BH, N, D] -> codes [BH, N, D], v_scale [BH, D].
hipError_t launch_v_quant(int dtype, int D, int BH, int N, const void* v, uint8_t* codes,
                          float* v_scale, hipStream_t st);

// Chunked-KV merge: up to MERGE_MAX chunks, pointers by value.
constexpr int MERGE_MAX = 16;
struct MergeArgs {
  int n;
  const void* o[MERGE_MAX];      // merge: O_c; sum: the parts
  const void* o_hp[MERGE_MAX];
  const float* lse[MERGE_MAX];
  void* out_o;
  void* out_o_hp;
  float* out_lse;
};
// rows = B*H*Nq; tensors [rows, D] (dtype), lse [rows]
hipError_t launch_merge(int dtype, int D, long rows, const MergeArgs& a, hipStream_t st);
// out_o[i] = sum_c o[c][i] over n elements (a multiple of 8; dtype)
hipError_t launch_sum(int dtype, long n, const MergeArgs& a, hipStream_t st);

// FQ test hook on fp32 rows.
hipError_t launch_fq_rows(const float* x, int rows, int cols, int group, int fmt, uint8_t* codes,
                          float* scales, float* xhat, hipStream_t st);

// Self-test: count decreasing adjacent pairs of v_exp_f32 over fp32 [lo, hi].
hipError_t launch_exp2_selftest(float lo, float hi, uint32_t* violations, hipStream_t st);
hipError_t launch_fq_scale_selftest(int fmt, uint32_t* mismatches, hipStream_t st);

// Backward pieces.
hipError_t launch_bwd_delta(const Shape& s, const void* o_hp, const void* dout, float* delta,
                            hipStream_t st);
// o_hp non-null: the kernel forms Delta itself (as launch_bwd_delta would) and
// writes it to delta; null: it reads delta.
hipError_t launch_bwd_dq(const Shape& s, const Inputs& in, const void* dout, const float* lse,
                         float* delta, const void* o_hp, float sm_scale, bool causal, int pfmt,
                         void* dq, float* p_amax, hipStream_t st);
// part_ws: fp32 scratch of dkdv_part_bytes(s) for the partial sums of key
// blocks split over query ranges (null: no block is split).
hipError_t launch_bwd_dkdv(const Shape& s, const Inputs& in, const void* dout, const float* lse,
                           const float* delta, const float* p_amax, float sm_scale, bool causal,
                           int pfmt, void* dk, void* dv, float* part_ws, hipStream_t st);

// dK/dV tail split: at most DKDV_MAX_SPLIT query ranges per key block and
// DKDV_PART_SLOTS partial blocks in all (three rounds of quarter blocks on
// 256 compute units).
constexpr int DKDV_MAX_SPLIT = 4;
constexpr int DKDV_PART_SLOTS = 768;
size_t dkdv_part_bytes(const Shape& s);

}  // namespace qat
