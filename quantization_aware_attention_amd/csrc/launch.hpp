// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qat {

struct Shape {
  int B, H, Nq, Nkv, D;
  int dtype;   // 0 bf16, 1 fp16
};

// pfmt: -1 = P not quantized, 0 = e4m3fn, 1 = e5m2
hipError_t launch_fwd(const Shape& s, const void* q, const void* k, const void* v,
                      const float* v_scale, float sm_scale, bool causal, int pfmt, bool v_fp8,
                      void* o, void* o_hp, float* lse, hipStream_t st);

// Per-token e4m3 fake quant: x [rows, D] -> xhat [rows, D] (same dtype).
hipError_t launch_token_quant(int dtype, int D, long rows, const void* x, void* xhat, hipStream_t st);

// Per-channel e5m2 quant of V [BH, N, D] -> codes [BH, N, D], v_scale [BH, D].
hipError_t launch_v_quant(int dtype, int D, int BH, int N, const void* v, uint8_t* codes,
                          float* v_scale, hipStream_t st);

// FQ test hook on fp32 rows.
hipError_t launch_fq_rows(const float* x, int rows, int cols, int group, int fmt, uint8_t* codes,
                          float* scales, float* xhat, hipStream_t st);

// Backward pieces.
hipError_t launch_bwd_delta(const Shape& s, const void* o_hp, const void* dout, float* delta,
                            hipStream_t st);
hipError_t launch_bwd_dq(const Shape& s, const void* q, const void* k, const void* v,
                         const float* v_scale, const void* dout, const float* lse,
                         const float* delta, float sm_scale, bool causal, int pfmt, bool v_fp8,
                         void* dq, float* p_amax, hipStream_t st);
hipError_t launch_bwd_dkdv(const Shape& s, const void* q, const void* k, const void* v,
                           const float* v_scale, const void* dout, const float* lse,
                           const float* delta, const float* p_amax, float sm_scale, bool causal,
                           int pfmt, bool v_fp8, void* dk, void* dv, hipStream_t st);

}  // namespace qat
