// Chunked-KV mode on one GPU (the local half of ring attention on the
// "usp: differentiable operators for training" page, and the merge of
// partial attention results by their log-sum-exp): the forward runs on each
// KV chunk, giving (O_c, O_hp_c, lse_c); merge_kernel combines them as
//   lse = log sum_c exp(lse_c),  O = sum_c exp(lse_c - lse) O_c  (O_hp alike),
// exact for the quantized O too when chunk boundaries are multiples of the
// 64-key P group (the per-row absmax scaling is invariant to the factor
// exp(lse_c - lse)).  In the backward every chunk's dK/dV come from the
// chunk itself with the merged lse and O_hp; its dQ parts are summed by
// sum_kernel.  Both add in chunk order (deterministic).
#include "common.hpp"
#include "launch.hpp"

namespace qat {

// One thread per (row, 8 consecutive d); 256 threads.
template <class DT, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a, long rows) {
  constexpr int CPR = D / 8;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * CPR) return;
  const long row = i / CPR;
  const int d0 = 8 * (int)(i % CPR);
  float m = -INFINITY;
  for (int c = 0; c < a.n; ++c) m = fmaxf(m, a.lse[c][row]);
  float w[MERGE_MAX];
  float sum = 0.0f;
  for (int c = 0; c < a.n; ++c) {
    w[c] = (m == -INFINITY) ? 0.0f : __expf(a.lse[c][row] - m);
    sum += w[c];
  }
  const float lse = (m == -INFINITY) ? -INFINITY : m + __logf(sum);
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
  float o[8] = {}, oh[8] = {};
  for (int c = 0; c < a.n; ++c) {
    const float wc = w[c] * inv;   // exp(lse_c - lse)
    const u32x4 x = *reinterpret_cast<const u32x4*>((const uint16_t*)a.o[c] + row * D + d0);
    const u32x4 y = *reinterpret_cast<const u32x4*>((const uint16_t*)a.o_hp[c] + row * D + d0);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      o[2 * h] += wc * DT::to_f32((uint16_t)(x[h] & 0xFFFFu));
      o[2 * h + 1] += wc * DT::to_f32((uint16_t)(x[h] >> 16));
      oh[2 * h] += wc * DT::to_f32((uint16_t)(y[h] & 0xFFFFu));
      oh[2 * h + 1] += wc * DT::to_f32((uint16_t)(y[h] >> 16));
    }
  }
  u32x4 ro, rh;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    ro[h] = DT::pack2(o[2 * h], o[2 * h + 1]);
    rh[h] = DT::pack2(oh[2 * h], oh[2 * h + 1]);
  }
  *reinterpret_cast<u32x4*>((uint16_t*)a.out_o + row * D + d0) = ro;
  *reinterpret_cast<u32x4*>((uint16_t*)a.out_o_hp + row * D + d0) = rh;
  if (d0 == 0) a.out_lse[row] = lse;
}

// out = sum_c part_c in fp32, chunk order; 8 elements per thread
template <class DT>
__global__ __launch_bounds__(256) void sum_kernel(MergeArgs a, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float s[8] = {};
  for (int c = 0; c < a.n; ++c) {
    const u32x4 x = *reinterpret_cast<const u32x4*>((const uint16_t*)a.o[c] + i * 8);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      s[2 * h] += DT::to_f32((uint16_t)(x[h] & 0xFFFFu));
      s[2 * h + 1] += DT::to_f32((uint16_t)(x[h] >> 16));
    }
  }
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 4; ++h) r[h] = DT::pack2(s[2 * h], s[2 * h + 1]);
  *reinterpret_cast<u32x4*>((uint16_t*)a.out_o + i * 8) = r;
}

hipError_t launch_merge(int dtype, int D, long rows, const MergeArgs& a, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const long threads = rows * (D / 8);
  dim3 grid((unsigned)((threads + 255) / 256));
  if (dtype == 0) {
    if (D == 128) hipLaunchKernelGGL((merge_kernel<BF16, 128>), grid, dim3(256), 0, st, a, rows);
    else hipLaunchKernelGGL((merge_kernel<BF16, 64>), grid, dim3(256), 0, st, a, rows);
  } else {
    if (D == 128) hipLaunchKernelGGL((merge_kernel<FP16, 128>), grid, dim3(256), 0, st, a, rows);
    else hipLaunchKernelGGL((merge_kernel<FP16, 64>), grid, dim3(256), 0, st, a, rows);
  }
  return hipGetLastError();
}

hipError_t launch_sum(int dtype, long n, const MergeArgs& a, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const long n8 = n / 8;
  dim3 grid((unsigned)((n8 + 255) / 256));
  if (dtype == 0) hipLaunchKernelGGL((sum_kernel<BF16>), grid, dim3(256), 0, st, a, n8);
  else hipLaunchKernelGGL((sum_kernel<FP16>), grid, dim3(256), 0, st, a, n8);
  return hipGetLastError();
}

}  // namespace qat
