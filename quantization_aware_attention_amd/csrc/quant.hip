// Stand-alone fake-quant kernels:
//  * per-token e4m3 fake quant of Q, K, V over the head dim (the
//    fake_quantize_q / fake_quantize_kv pre-pass that _attention.forward in
//    the FastVideo attn_qat_train.py source runs before the attention kernel;
//    like that source, the fake-quantized copy keeps the input dtype);
//  * per-channel e5m2 quantization of V to codes + scale (the fp8 V path);
//  * FQ of fp32 rows, a test hook that runs the very device code the
//    attention kernels use.
// All three are HBM-bound streaming kernels.
#include "common.hpp"
#include "launch.hpp"

namespace qat {

// 16 lanes per token row of D <= 128 elements: lane handles D/16 consecutive
// elements (8 for D = 128, 4 for D = 64).  With `scale_out` the row is stored
// split: the fp8 code values (exact in bf16 and fp16) and the fp32 scale s,
// so that x^ = code * s stays exact for the attention kernels; otherwise
// x^ = fp32(code * s) is rounded to the storage dtype.
// With `shift` (K smoothing) the row first becomes x - shift[d], rounded to
// the dtype: the smoothed K the attention sees.  With `codes8` (split only)
// the e4m3 code bytes are stored as well, for the fp8 MFMAs of S.
template <class DT, int D>
__global__ __launch_bounds__(256) void token_quant_kernel(const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ xhat,
                                                          float* __restrict__ scale_out, long rows,
                                                          const float* __restrict__ shift,
                                                          uint8_t* __restrict__ codes8) {
  constexpr int EPL = D / 16;   // elements per lane
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool valid = row < rows;
  float v[EPL];
  const uint16_t* src = x + (valid ? row : 0) * D + sub * EPL;
  if constexpr (EPL == 8) {
    const u32x4 w = valid ? *reinterpret_cast<const u32x4*>(src) : (u32x4){0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = DT::to_f32((uint16_t)(w[e >> 1] >> (16 * (e & 1))));
  } else {
    const u32x2 w = valid ? *reinterpret_cast<const u32x2*>(src) : (u32x2){0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = DT::to_f32((uint16_t)(w[e >> 1] >> (16 * (e & 1))));
  }
  if (shift) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] = DT::to_f32((uint16_t)DT::pack2(v[e] - shift[sub * EPL + e], 0.0f));
  }
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  const FqScale fs = fq_scale<0>(amax);
  const bool split = scale_out != nullptr;
  const FqScale unit = {1.0f, fs.r};   // code value times 1: the code itself
  uint32_t outw[EPL / 2], code2[EPL / 2];
#pragma unroll
  for (int e = 0; e < EPL; e += 2) {
    f32x2 xq = fq_pair<0>(v[e], v[e + 1], split ? unit : fs, &code2[e / 2]);
    if (fs.r == 0.0f) {   // zero group: +0, not -0
      xq = (f32x2){0.0f, 0.0f};
      code2[e / 2] = 0u;
    }
    outw[e / 2] = DT::pack2(xq[0], xq[1]);
  }
  if (!valid) return;
  if (split && sub == 0) scale_out[row] = fs.s;
  if (codes8) {   // two codes per conversion, in its low 16 bits
    uint32_t cw[EPL / 4];
#pragma unroll
    for (int h = 0; h < EPL / 4; ++h) cw[h] = (code2[2 * h] & 0xFFFFu) | (code2[2 * h + 1] << 16);
    uint8_t* cdst = codes8 + row * D + sub * EPL;
    if constexpr (EPL == 8) *reinterpret_cast<u32x2*>(cdst) = (u32x2){cw[0], cw[1]};
    else *reinterpret_cast<uint32_t*>(cdst) = cw[0];
  }
  uint16_t* dst = xhat + row * D + sub * EPL;
  if constexpr (EPL == 8) *reinterpret_cast<u32x4*>(dst) = (u32x4){outw[0], outw[1], outw[2], outw[3]};
  else *reinterpret_cast<u32x2*>(dst) = (u32x2){outw[0], outw[1]};
}

hipError_t launch_token_quant(int dtype, int D, long rows, const void* x, void* xhat, float* scale_out,
                              const float* shift, void* codes8, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 15) / 16));
  const uint16_t* xi = (const uint16_t*)x;
  uint16_t* xo = (uint16_t*)xhat;
  uint8_t* c8 = (uint8_t*)codes8;
  if (dtype == 0) {
    if (D == 128) hipLaunchKernelGGL((token_quant_kernel<BF16, 128>), grid, dim3(256), 0, st, xi, xo, scale_out, rows, shift, c8);
    else hipLaunchKernelGGL((token_quant_kernel<BF16, 64>), grid, dim3(256), 0, st, xi, xo, scale_out, rows, shift, c8);
  } else {
    if (D == 128) hipLaunchKernelGGL((token_quant_kernel<FP16, 128>), grid, dim3(256), 0, st, xi, xo, scale_out, rows, shift, c8);
    else hipLaunchKernelGGL((token_quant_kernel<FP16, 64>), grid, dim3(256), 0, st, xi, xo, scale_out, rows, shift, c8);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ K smoothing
// k_mean[d] = mean of K over every (batch, head, token) row, rounded to the
// dtype; two passes in a fixed order (deterministic): block b sums the rows
// [b*chunk, (b+1)*chunk) (thread t: the 8 channels of 16-byte chunk t % (D/8)
// over rows t / (D/8) + k * (256 / (D/8)), then the row phases in order), and
// one block adds the KMEAN_BLOCKS partial sums in block order.
template <int D, class DT>
__global__ __launch_bounds__(256) void kmean_partial_kernel(const uint16_t* __restrict__ k, long rows, long chunk,
                                                            float* __restrict__ part) {
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RPH = 256 / CPR;      // row phases
  __shared__ float acc[RPH][D];
  const int c = threadIdx.x % CPR, ph = threadIdx.x / CPR;
  const long r0 = (long)blockIdx.x * chunk, r1 = min(rows, r0 + chunk);
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const u32x4& w) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      s[2 * h] += DT::to_f32((uint16_t)(w[h] & 0xFFFFu));
      s[2 * h + 1] += DT::to_f32((uint16_t)(w[h] >> 16));
    }
  };
  // eight rows' loads in flight per thread (one at a time leaves the chip far
  // below HBM bandwidth); the additions keep the row order, so the sums do
  // not depend on the unrolling
  constexpr int UNR = 8;
  long r = r0 + ph;
  for (; r + (UNR - 1) * RPH < r1; r += UNR * RPH) {
    u32x4 w[UNR];
#pragma unroll
    for (int i = 0; i < UNR; ++i) w[i] = *reinterpret_cast<const u32x4*>(k + (r + i * RPH) * D + 8 * c);
#pragma unroll
    for (int i = 0; i < UNR; ++i) add(w[i]);
  }
  for (; r < r1; r += RPH) add(*reinterpret_cast<const u32x4*>(k + r * D + 8 * c));
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[ph][8 * c + e] = s[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float t = acc[0][d];
    for (int p = 1; p < RPH; ++p) t += acc[p][d];
    part[(size_t)blockIdx.x * D + d] = t;
  }
}

template <int D, class DT>
__global__ __launch_bounds__(256) void kmean_final_kernel(const float* __restrict__ part, int nblocks, long rows,
                                                          float* __restrict__ mean) {
  const int d = threadIdx.x;
  if (d >= D) return;
  // sixteen partials' loads in flight, added in block order
  constexpr int UNR = 16;
  float t = 0.0f;
  int b = 0;
  for (; b + UNR <= nblocks; b += UNR) {
    float v[UNR];
#pragma unroll
    for (int i = 0; i < UNR; ++i) v[i] = part[(size_t)(b + i) * D + d];
#pragma unroll
    for (int i = 0; i < UNR; ++i) t += v[i];
  }
  for (; b < nblocks; ++b) t += part[(size_t)b * D + d];
  mean[d] = DT::to_f32((uint16_t)DT::pack2(t / (float)rows, 0.0f));
}

// x - shift[d] rounded to the dtype, 8 elements per thread (D multiple of 8)
template <int D, class DT>
__global__ __launch_bounds__(256) void shift_rows_kernel(const uint16_t* __restrict__ x, const float* __restrict__ shift,
                                                         uint16_t* __restrict__ y, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int d0 = (int)((i * 8) % D);
  const u32x4 w = *reinterpret_cast<const u32x4*>(x + i * 8);
  u32x4 o;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float a = DT::to_f32((uint16_t)(w[h] & 0xFFFFu)) - shift[d0 + 2 * h];
    const float b = DT::to_f32((uint16_t)(w[h] >> 16)) - shift[d0 + 2 * h + 1];
    o[h] = DT::pack2(a, b);
  }
  *reinterpret_cast<u32x4*>(y + i * 8) = o;
}

template <int D, class DT>
static void launch_smooth_typed(long rows, const void* k, float* part, float* mean, void* k_smooth, hipStream_t st) {
  const int nb = (int)min((long)KMEAN_BLOCKS, rows);
  const long chunk = (rows + nb - 1) / nb;
  hipLaunchKernelGGL((kmean_partial_kernel<D, DT>), dim3(nb), dim3(256), 0, st, (const uint16_t*)k, rows, chunk, part);
  hipLaunchKernelGGL((kmean_final_kernel<D, DT>), dim3(1), dim3(256), 0, st, part, nb, rows, mean);
  if (k_smooth) {
    const long n8 = rows * D / 8;
    hipLaunchKernelGGL((shift_rows_kernel<D, DT>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                       (const uint16_t*)k, mean, (uint16_t*)k_smooth, n8);
  }
}

hipError_t launch_k_smooth(int dtype, int D, long rows, const void* k, float* part, float* mean, void* k_smooth,
                           hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (dtype == 0) {
    if (D == 128) launch_smooth_typed<128, BF16>(rows, k, part, mean, k_smooth, st);
    else launch_smooth_typed<64, BF16>(rows, k, part, mean, k_smooth, st);
  } else {
    if (D == 128) launch_smooth_typed<128, FP16>(rows, k, part, mean, k_smooth, st);
    else launch_smooth_typed<64, FP16>(rows, k, part, mean, k_smooth, st);
  }
  return hipGetLastError();
}

// One workgroup per (b, h): thread t owns channel d = t % D and walks the
// token rows t / D, t / D + 256 / D, ...; the column maxima are combined in
// LDS, then every element is encoded.
template <class DT, int D>
__global__ __launch_bounds__(256) void v_quant_kernel(const uint16_t* __restrict__ v, uint8_t* __restrict__ codes,
                                                      float* __restrict__ v_scale, int N) {
  constexpr int RPS = 256 / D;   // row phases
  __shared__ float part[RPS][D];
  __shared__ float scale_s[D], scale_r[D];
  const int bh = blockIdx.x;
  const int d = threadIdx.x % D, ph = threadIdx.x / D;
  const uint16_t* src = v + (size_t)bh * N * D;
  float amax = 0.0f;
  for (int n = ph; n < N; n += RPS) amax = fmaxf(amax, fabsf(DT::to_f32(src[(size_t)n * D + d])));
  part[ph][d] = amax;
  __syncthreads();
  if (ph == 0) {
    float m = part[0][d];
#pragma unroll
    for (int p = 1; p < RPS; ++p) m = fmaxf(m, part[p][d]);
    const FqScale fs = fq_scale<1>(m);
    scale_s[d] = fs.s;
    scale_r[d] = fs.r;
    v_scale[(size_t)bh * D + d] = fs.s;
  }
  __syncthreads();
  const FqScale fs = {scale_s[d], scale_r[d]};
  uint8_t* dst = codes + (size_t)bh * N * D;
  for (int n = ph; n < N; n += RPS) {
    uint32_t pk;
    fq_pair<1>(DT::to_f32(src[(size_t)n * D + d]), 0.0f, fs, &pk);
    dst[(size_t)n * D + d] = (fs.r == 0.0f) ? 0 : (uint8_t)(pk & 0xFF);
  }
}

hipError_t launch_v_quant(int dtype, int D, int BH, int N, const void* v, uint8_t* codes,
                          float* v_scale, hipStream_t st) {
  if (BH <= 0) return hipSuccess;
  const uint16_t* vi = (const uint16_t*)v;
  if (dtype == 0) {
    if (D == 128) hipLaunchKernelGGL((v_quant_kernel<BF16, 128>), dim3(BH), dim3(256), 0, st, vi, codes, v_scale, N);
    else hipLaunchKernelGGL((v_quant_kernel<BF16, 64>), dim3(BH), dim3(256), 0, st, vi, codes, v_scale, N);
  } else {
    if (D == 128) hipLaunchKernelGGL((v_quant_kernel<FP16, 128>), dim3(BH), dim3(256), 0, st, vi, codes, v_scale, N);
    else hipLaunchKernelGGL((v_quant_kernel<FP16, 64>), dim3(BH), dim3(256), 0, st, vi, codes, v_scale, N);
  }
  return hipGetLastError();
}

// Test hook: one thread per (row, group).
template <int FMT>
__global__ __launch_bounds__(256) void fq_rows_kernel(const float* __restrict__ x, int rows, int cols, int group,
                                                      uint8_t* codes, float* scales, float* xhat) {
  const int ng = (cols + group - 1) / group;
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  if (id >= (long)rows * ng) return;
  const int row = (int)(id / ng), gi = (int)(id % ng);
  const int c0 = gi * group, c1 = min(cols, c0 + group);
  const float* src = x + (size_t)row * cols;
  float amax = 0.0f;
  for (int c = c0; c < c1; ++c) amax = fmaxf(amax, fabsf(src[c]));
  const FqScale fs = fq_scale<FMT>(amax);
  if (scales) scales[(size_t)row * ng + gi] = fs.s;
  const bool zero = fs.r == 0.0f;
  for (int c = c0; c < c1; c += 2) {
    const bool two = c + 1 < c1;
    uint32_t pk;
    const f32x2 xq = fq_pair<FMT>(src[c], two ? src[c + 1] : 0.0f, fs, &pk);
    if (codes) {
      codes[(size_t)row * cols + c] = zero ? 0 : (uint8_t)(pk & 0xFF);
      if (two) codes[(size_t)row * cols + c + 1] = zero ? 0 : (uint8_t)((pk >> 8) & 0xFF);
    }
    if (xhat) {
      xhat[(size_t)row * cols + c] = zero ? 0.0f : xq[0];
      if (two) xhat[(size_t)row * cols + c + 1] = zero ? 0.0f : xq[1];
    }
  }
}

hipError_t launch_fq_rows(const float* x, int rows, int cols, int group, int fmt, uint8_t* codes,
                          float* scales, float* xhat, hipStream_t st) {
  const long n = (long)rows * ((cols + group - 1) / group);
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256));
  if (fmt == 0) hipLaunchKernelGGL((fq_rows_kernel<0>), grid, dim3(256), 0, st, x, rows, cols, group, codes, scales, xhat);
  else hipLaunchKernelGGL((fq_rows_kernel<1>), grid, dim3(256), 0, st, x, rows, cols, group, codes, scales, xhat);
  return hipGetLastError();
}

// Self-test: count adjacent fp32 pairs x < y (in value order, within
// [key_lo, key_hi] of the order-preserving integer key of fp32) whose
// v_exp_f32 results decrease.  Each thread walks one contiguous run of keys.
__device__ __forceinline__ float from_order_key(uint32_t k) {
  const uint32_t bits = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, bits);
}

__global__ __launch_bounds__(256) void exp2_monotone_kernel(uint32_t key_lo, uint32_t key_hi, uint32_t per_thread,
                                                            uint32_t* violations) {
  const uint64_t start = (uint64_t)key_lo + ((uint64_t)blockIdx.x * 256 + threadIdx.x) * per_thread;
  if (start >= key_hi) return;
  const uint64_t stop = min((uint64_t)key_hi, start + per_thread);
  uint32_t bad = 0;
  float prev = fast_exp2(from_order_key((uint32_t)start));
  for (uint64_t k = start + 1; k <= stop; ++k) {
    const float cur = fast_exp2(from_order_key((uint32_t)k));
    bad += cur < prev;
    prev = cur;
  }
  if (bad) atomicAdd(violations, bad);
}

__global__ void zero_u32(uint32_t* p) { *p = 0; }

// Self-test: count the positive finite fp32 values a whose fq_scale pair
// differs in any bit from (a/FMAX, FMAX/a) by IEEE division, or from (0, 0)
// where FMAX/a overflows.  Each thread walks one contiguous run of bit
// patterns of [1, 0x7F7FFFFF].
constexpr uint32_t FQS_LAST = 0x7F7FFFFFu;   // largest finite fp32
constexpr uint32_t FQS_PER_THREAD = 4096;

template <int FMT>
__global__ __launch_bounds__(256) void fq_scale_selftest_kernel(uint32_t* mismatches) {
  const uint64_t start = 1 + ((uint64_t)blockIdx.x * 256 + threadIdx.x) * FQS_PER_THREAD;
  if (start > FQS_LAST) return;
  const uint64_t stop = min((uint64_t)FQS_LAST, start + FQS_PER_THREAD - 1);
  constexpr float F = Fp8Fmt<FMT>::FMAX;
  uint32_t bad = 0;
  for (uint64_t u = start; u <= stop; ++u) {
    const float a = __builtin_bit_cast(float, (uint32_t)u);
    const float r_ref = F / a, s_ref = a / F;
    const bool ok = r_ref <= 3.402823466e38f;
    const FqScale q = fq_scale<FMT>(a);
    bad += (__builtin_bit_cast(uint32_t, q.s) != __builtin_bit_cast(uint32_t, ok ? s_ref : 0.0f)) ||
           (__builtin_bit_cast(uint32_t, q.r) != __builtin_bit_cast(uint32_t, ok ? r_ref : 0.0f));
  }
  if (bad) atomicAdd(mismatches, bad);
}

hipError_t launch_exp2_selftest(float lo, float hi, uint32_t* violations, hipStream_t st) {
  auto key = [](float f) {
    const uint32_t b = __builtin_bit_cast(uint32_t, f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  };
  const uint32_t klo = key(lo), khi = key(hi);
  hipLaunchKernelGGL(zero_u32, dim3(1), dim3(1), 0, st, violations);
  if (khi <= klo) return hipGetLastError();
  const uint32_t per = 4096;
  const uint64_t threads = ((uint64_t)khi - klo + per - 1) / per;
  hipLaunchKernelGGL(exp2_monotone_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, klo, khi, per,
                     violations);
  return hipGetLastError();
}

hipError_t launch_fq_scale_selftest(int fmt, uint32_t* mismatches, hipStream_t st) {
  hipLaunchKernelGGL(zero_u32, dim3(1), dim3(1), 0, st, mismatches);
  const uint64_t threads = (FQS_LAST + (uint64_t)FQS_PER_THREAD - 1) / FQS_PER_THREAD;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (fmt == 0) hipLaunchKernelGGL(fq_scale_selftest_kernel<0>, grid, dim3(256), 0, st, mismatches);
  else hipLaunchKernelGGL(fq_scale_selftest_kernel<1>, grid, dim3(256), 0, st, mismatches);
  return hipGetLastError();
}

}  // namespace qat
