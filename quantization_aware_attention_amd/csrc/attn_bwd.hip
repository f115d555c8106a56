// Straight-through backward of quantization-aware attention on gfx950.
//
// Follows _attention.backward of the FastVideo attn_qat_train.py source:
// Delta = rowsum(O_hp o dO) (_attn_bwd_preprocess, here with the
// straight-through output), then dQ (_attn_bwd_dq_cross) and dK/dV
// (_attn_bwd_dkdv_cross) in separate kernels that rematerialise
// S = Q^ K^T and P = exp2(S*c - M) from the saved log-sum-exp, with
// dV = P^T dO using the fake-quantized P, dP = dO V^T, dS = P o (dP - Delta),
// dQ = sm_scale dS K, dK = sm_scale dS^T Q.
//
// MI355X mapping:
//  * dQ kernel: a workgroup of 4 waves owns 128 query rows; like the forward,
//    each wave computes S^T = K Q^T and dP^T = V dO^T so every lane owns one
//    query row (Q^T, dO^T stay in registers, K/V tiles stream through LDS);
//    dQ^T = K^T dS^T reads K^T through ds_read_b64_tr_b16.  Because a lane
//    holds a query row's 64-key group, this kernel also records the P-quant
//    absmax of every (row, group) for the dK/dV kernel.
//  * dK/dV kernel: a workgroup of 8 waves owns 128 keys (two P groups);
//    each wave keeps its 32 keys' K^T (and V^T) in registers and computes
//    S = Q K^T (and dP = dO V^T) with one lane per key, so P^ and dS are
//    already the operands of dV^T = dO^T P^ and dK^T = Q^T dS (Q and dO
//    tiles go through LDS, read row-major for S/dP and transposed for dV/dK).
//    Half the waves accumulate dV, half dK, so each holds one accumulator.
//    A key-per-lane layout has a query's 64 keys spread over 64 lanes of two
//    waves; reading the absmax recorded by the dQ kernel replaces that
//    cross-lane reduction.
#include "common.hpp"
#include "launch.hpp"

namespace qat {

// ------------------------------------------------------------------ Delta
template <class DT, int D>
__global__ __launch_bounds__(256) void delta_kernel(const uint16_t* __restrict__ o_hp,
                                                    const uint16_t* __restrict__ dout,
                                                    float* __restrict__ delta, long rows) {
  constexpr int EPL = D / 16;
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const long r = row < rows ? row : 0;
  const uint16_t* a = o_hp + r * D + sub * EPL;
  const uint16_t* b = dout + r * D + sub * EPL;
  float acc = 0.0f;
  if constexpr (EPL == 8) {
    const u32x4 wa = *reinterpret_cast<const u32x4*>(a);
    const u32x4 wb = *reinterpret_cast<const u32x4*>(b);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc += DT::to_f32((uint16_t)(wa[e >> 1] >> (16 * (e & 1)))) * DT::to_f32((uint16_t)(wb[e >> 1] >> (16 * (e & 1))));
  } else {
    const u32x2 wa = *reinterpret_cast<const u32x2*>(a);
    const u32x2 wb = *reinterpret_cast<const u32x2*>(b);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc += DT::to_f32((uint16_t)(wa[e >> 1] >> (16 * (e & 1)))) * DT::to_f32((uint16_t)(wb[e >> 1] >> (16 * (e & 1))));
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < rows && sub == 0) delta[row] = acc;
}

hipError_t launch_bwd_delta(const Shape& s, const void* o_hp, const void* dout, float* delta,
                            hipStream_t st) {
  const long rows = (long)s.B * s.H * s.Nq;
  if (rows <= 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 15) / 16));
  const uint16_t* a = (const uint16_t*)o_hp;
  const uint16_t* b = (const uint16_t*)dout;
  if (s.dtype == 0) {
    if (s.D == 128) hipLaunchKernelGGL((delta_kernel<BF16, 128>), grid, dim3(256), 0, st, a, b, delta, rows);
    else hipLaunchKernelGGL((delta_kernel<BF16, 64>), grid, dim3(256), 0, st, a, b, delta, rows);
  } else {
    if (s.D == 128) hipLaunchKernelGGL((delta_kernel<FP16, 128>), grid, dim3(256), 0, st, a, b, delta, rows);
    else hipLaunchKernelGGL((delta_kernel<FP16, 64>), grid, dim3(256), 0, st, a, b, delta, rows);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ shared args
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* v_scale;   // IN_VFP8
  const float* q_scale;   // IN_QKS
  const float* k_scale;   // IN_QKS
  const void* dout;
  const float* lse;
  const float* delta;
  float* p_amax;        // [BH][NG][Nq]
  const float* p_amax_in;
  void* dq;
  void* dk;
  void* dv;
  int Nq, Nkv, NG;
  float sm_scale;
  float c;              // sm_scale * log2(e)
};

// Stage one [64 x D] tile of a key/value tensor into LDS (swizzled).  For fp8
// V the codes are dequantized with the per-channel scale and rounded to bf16.
template <class DT, int D, bool FP8V>
__device__ __forceinline__ void stage_kv_tile(char* dst, const uint8_t* src, const float* vscale, int key0,
                                              int Nkv, int tid) {
  constexpr int CH = D / 8;
  constexpr int LPT = 64 * CH / 256;
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int idx = tid + 256 * u, row = idx / CH, ch = idx % CH;
    const int key = key0 + row;
    u32x4 val = {0, 0, 0, 0};
    if (key < Nkv) {
      if constexpr (FP8V) {
        const u32x2 codes = *reinterpret_cast<const u32x2*>(src + (size_t)key * D + ch * 8);
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(vscale + ch * 8);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(vscale + ch * 8 + 4);
        const float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const f32x2 f = __builtin_amdgcn_cvt_pk_f32_bf8((int)(codes[h >> 1] >> (16 * (h & 1))), false);
          val[h] = BF16::pack2(f[0] * sc[2 * h], f[1] * sc[2 * h + 1]);
        }
      } else {
        val = *reinterpret_cast<const u32x4*>(src + ((size_t)key * D + ch * 8) * 2);
      }
    }
    *reinterpret_cast<u32x4*>(dst + tile_off<D>(row, ch)) = val;
  }
}

// ------------------------------------------------------------------ dQ
constexpr int DQ_BM = 128;
constexpr int DQ_BN = 64;

template <class DT, int D, bool CAUSAL, int PQ, int IN>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdArgs a) {
  constexpr bool VFP8 = IN == IN_VFP8;
  constexpr bool QKS = IN == IN_QKS;
  constexpr int TILE = DQ_BN * D * 2;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  constexpr int CH = D / 8;
  constexpr int LPT = DQ_BN * CH / 256;
  __shared__ __attribute__((aligned(16))) char smem[2][2][TILE];   // [buffer][K, V]
  __shared__ __attribute__((aligned(16))) float ks_s[2][DQ_BN];     // IN_QKS: key scales

  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int ntq = (a.Nq + DQ_BM - 1) / DQ_BM;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  const int bh = unit / ntq;
  const int qb = (CAUSAL ? ntq - 1 - unit % ntq : unit % ntq) * DQ_BM;
  const int q0 = qb + w * 32;
  const int qi = q0 + l32;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const uint16_t* qp = (const uint16_t*)a.q + (size_t)bh * Nq * D;
  const uint16_t* dop = (const uint16_t*)a.dout + (size_t)bh * Nq * D;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)bh * Nkv * D;
  const uint8_t* vp = (const uint8_t*)a.v + (size_t)bh * Nkv * D * (VFP8 ? 1 : 2);
  const float* vsc = VFP8 ? a.v_scale + (size_t)bh * D : nullptr;

  s16x8 qf[NKS], dof[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const bool ok = qi < Nq;
    qf[ks] = ok ? *reinterpret_cast<const s16x8*>(qp + (size_t)qi * D + 16 * ks + 8 * g) : (s16x8){};
    dof[ks] = ok ? *reinterpret_cast<const s16x8*>(dop + (size_t)qi * D + 16 * ks + 8 * g) : (s16x8){};
  }
  const float Mi = qi < Nq ? a.lse[(size_t)bh * Nq + qi] * LOG2E : 0.0f;
  const float Di = qi < Nq ? a.delta[(size_t)bh * Nq + qi] : 0.0f;
  float c_row = a.c;   // IN_QKS: s_q folds into the log2 scale (same rounding as dK/dV)
  if constexpr (QKS) c_row = a.c * (qi < Nq ? a.q_scale[(size_t)bh * Nq + qi] : 1.0f);

  f32x16 dq_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq_acc[db] = (f32x16){};

  // K tiles (and V, unless fp8) go HBM -> LDS directly, double-buffered; fp8
  // V codes and key scales take a register detour.
  u32x2 vcode[LPT];
  float ksreg = 0.0f;
  TileCopy<D, DQ_BN, 4> copy;
  copy.init(w, lane);
  auto issue_tile = [&](int t, int buf) {
    copy.issue(smem[buf][0], kp, t * DQ_BN, Nkv);
    if constexpr (VFP8) {
#pragma unroll
      for (int u = 0; u < LPT; ++u) {
        const int idx = tid + 256 * u, row = idx / CH, ch = idx % CH;
        const int key = min(t * DQ_BN + row, Nkv - 1);
        vcode[u] = *reinterpret_cast<const u32x2*>(vp + (size_t)key * D + ch * 8);
      }
    } else {
      copy.issue(smem[buf][1], (const uint16_t*)vp, t * DQ_BN, Nkv);
    }
    if constexpr (QKS) {
      const int key = t * DQ_BN + tid;
      if (tid < DQ_BN) ksreg = key < Nkv ? a.k_scale[(size_t)bh * Nkv + key] : 0.0f;
    }
  };
  auto finish_tile = [&](int buf) {
    if constexpr (VFP8) {   // V^ = code * v_scale[d], rounded to bf16
#pragma unroll
      for (int u = 0; u < LPT; ++u) {
        const int idx = tid + 256 * u, row = idx / CH, ch = idx % CH;
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(vsc + ch * 8);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(vsc + ch * 8 + 4);
        const float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        u32x4 vv;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const f32x2 f = __builtin_amdgcn_cvt_pk_f32_bf8((int)(vcode[u][h >> 1] >> (16 * (h & 1))), false);
          vv[h] = BF16::pack2(f[0] * sc[2 * h], f[1] * sc[2 * h + 1]);
        }
        *reinterpret_cast<u32x4*>(smem[buf][1] + tile_off<D>(row, ch)) = vv;
      }
    }
    if constexpr (QKS) {
      if (tid < DQ_BN) ks_s[buf][tid] = ksreg;
    }
  };

  const int kv_end = CAUSAL ? min(Nkv, qb + DQ_BM) : Nkv;
  const int ntiles = (kv_end + DQ_BN - 1) / DQ_BN;
  if (ntiles > 0) {
    issue_tile(0, 0);
    wait_vmem();
    finish_tile(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * DQ_BN;
    const int buf = t & 1;
    if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
    if (q0 < Nq && !(CAUSAL && kv0 > q0 + 31)) {
    const char* Kt = smem[buf][0];
    const char* Vt = smem[buf][1];
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (f32x16){};
      dp[kb] = (f32x16){};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        s[kb] = DT::mfma(lds_row8<D>(Kt, kb * 32 + l32, 2 * ks + g), qf[ks], s[kb]);
        dp[kb] = DT::mfma(lds_row8<D>(Vt, kb * 32 + l32, 2 * ks + g), dof[ks], dp[kb]);
      }
    }
    const bool need_mask = (kv0 + DQ_BN > Nkv) || (CAUSAL && kv0 + DQ_BN - 1 > q0);
    if constexpr (QKS) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4 v4 = *reinterpret_cast<const f32x4*>(&ks_s[buf][kb * 32 + 8 * u + 4 * g]);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kb][4 * u + e] *= v4[e];
        }
    }
    float p[2][16];
    float pmax = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = fast_exp2(__builtin_fmaf(s[kb][r], c_row, -Mi));
        if (need_mask) {
          const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= Nkv || (CAUSAL && key > qi)) x = 0.0f;
        }
        p[kb][r] = x;
        pmax = fmaxf(pmax, x);
      }
    if constexpr (PQ >= 0) {
      pmax = fmaxf(pmax, shfl_xor32(pmax));
      if (g == 0 && qi < Nq) a.p_amax[((size_t)bh * a.NG + t) * Nq + qi] = pmax;
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kb = kk >> 1, h = kk & 1;
      uint32_t w4[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r0 = 8 * h + 2 * jj;
        float d0 = p[kb][r0] * (dp[kb][r0] - Di), d1 = p[kb][r0 + 1] * (dp[kb][r0 + 1] - Di);
        if constexpr (QKS) {   // dQ = sm_scale sum_j dS_ij s_k[j] code_k[j]
          const f32x2 k2 = *reinterpret_cast<const f32x2*>(&ks_s[buf][kb * 32 + 8 * (r0 >> 2) + 4 * g + (r0 & 3)]);
          d0 *= k2[0];
          d1 *= k2[1];
        }
        w4[jj] = DT::pack2(d0, d1);
      }
      const s16x8 ds_op = __builtin_bit_cast(s16x8, (u32x4){w4[0], w4[1], w4[2], w4[3]});
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        dq_acc[db] = DT::mfma(lds_tr8<D>(Kt, kk * 16, db * 32, lane), ds_op, dq_acc[db]);
    }
    }
    wait_vmem();
    if (t + 1 < ntiles) finish_tile(buf ^ 1);
    __syncthreads();
  }
  // causal rows whose every later tile was skipped still record zero-free
  // groups only for tiles they visited; the dK/dV kernel never reads the
  // others (the keys are masked there).
  if (qi >= Nq) return;
  uint16_t* dqp = (uint16_t*)a.dq + (size_t)bh * Nq * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = db * 32 + 8 * u + 4 * g;
      const float x[4] = {dq_acc[db][4 * u], dq_acc[db][4 * u + 1], dq_acc[db][4 * u + 2], dq_acc[db][4 * u + 3]};
      *reinterpret_cast<u32x2*>(dqp + (size_t)qi * D + d) =
          (u32x2){DT::pack2(x[0] * a.sm_scale, x[1] * a.sm_scale), DT::pack2(x[2] * a.sm_scale, x[3] * a.sm_scale)};
    }
}

// ------------------------------------------------------------------ dK / dV
// Eight waves share one block of 128 keys (two P groups) and the staged Q /
// dO tiles: waves 0-3 ("dV waves") form S, P and the fake-quantized P^ for
// their 32 keys and accumulate dV^T = dO^T P^; waves 4-7 ("dK waves") form S,
// P, dP = dO V^T and dS and accumulate dK^T = Q^T dS.  S is formed by both
// halves (identically), which costs one extra QK^T per block but leaves every
// wave a single 64-register accumulator, so two waves fit on each SIMD.
constexpr int DKV_BN = 128;   // keys per workgroup
constexpr int DKV_BQ = 64;    // queries per staged tile

template <class DT, int D, bool CAUSAL, int PQ, int IN>
__global__ __launch_bounds__(512, 1) void dkdv_kernel(BwdArgs a) {
  constexpr bool VFP8 = IN == IN_VFP8;
  constexpr bool QKS = IN == IN_QKS;
  constexpr int TILE = DKV_BQ * D * 2;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  __shared__ __attribute__((aligned(16))) char qt_s[2][TILE];
  __shared__ __attribute__((aligned(16))) char dot_s[2][TILE];
  __shared__ __attribute__((aligned(16))) float m_s[2][DKV_BQ];
  __shared__ __attribute__((aligned(16))) float d_s[2][DKV_BQ];
  __shared__ __attribute__((aligned(16))) float sq_s[2][DKV_BQ];      // IN_QKS: query scales
  __shared__ __attribute__((aligned(16))) float qs_s[2][2][DKV_BQ];   // P-quant s per (group, query)
  __shared__ __attribute__((aligned(16))) float qr_s[2][2][DKV_BQ];   // P-quant r

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const bool dk_wave = w >= 4;
  const int kw = w & 3;
  const int nkb = (a.Nkv + DKV_BN - 1) / DKV_BN;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  const int bh = unit / nkb;
  const int k0 = (unit % nkb) * DKV_BN;   // causal: key block 0 sees every query: longest first
  const int k0w = k0 + kw * 32;
  const int kj = k0w + l32;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const int grp0 = k0 / 64;
  const int mygrp = kw >> 1;
  const uint16_t* qp = (const uint16_t*)a.q + (size_t)bh * Nq * D;
  const uint16_t* dop = (const uint16_t*)a.dout + (size_t)bh * Nq * D;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)bh * Nkv * D;

  // K^T (every wave) and V^T (dK waves) operands of this wave's 32 keys:
  // lane holds key kj, d = 16ks + 8g .. +7
  s16x8 kf[NKS], vf[NKS];
  {
    const bool ok = kj < Nkv;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kf[ks] = ok ? *reinterpret_cast<const s16x8*>(kp + (size_t)kj * D + 16 * ks + 8 * g) : (s16x8){};
      vf[ks] = (s16x8){};
      if (dk_wave && ok) {
        if constexpr (VFP8) {
          const uint8_t* vp = (const uint8_t*)a.v + (size_t)bh * Nkv * D;
          const float* vsc = a.v_scale + (size_t)bh * D + 16 * ks + 8 * g;
          const u32x2 codes = *reinterpret_cast<const u32x2*>(vp + (size_t)kj * D + 16 * ks + 8 * g);
          uint32_t wv[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const f32x2 f = __builtin_amdgcn_cvt_pk_f32_bf8((int)(codes[h >> 1] >> (16 * (h & 1))), false);
            wv[h] = BF16::pack2(f[0] * vsc[2 * h], f[1] * vsc[2 * h + 1]);
          }
          vf[ks] = __builtin_bit_cast(s16x8, (u32x4){wv[0], wv[1], wv[2], wv[3]});
        } else {
          const uint16_t* vp = (const uint16_t*)a.v + (size_t)bh * Nkv * D;
          vf[ks] = *reinterpret_cast<const s16x8*>(vp + (size_t)kj * D + 16 * ks + 8 * g);
        }
      }
    }
  }
  const float sk_lane = QKS ? (kj < Nkv ? a.k_scale[(size_t)bh * Nkv + kj] : 0.0f) : 1.0f;

  f32x16 acc[NDB];   // dV^T (dV waves) or dK^T (dK waves)
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = (f32x16){};

  // Q and dO tiles go HBM -> LDS directly (double-buffered); the per-query
  // vectors (log2-domain LSE, Delta, Q scales, P-quant scales of this
  // workgroup's two key groups) are staged through registers.
  float vec0 = 0.0f, vec1 = 0.0f, vec2 = 0.0f;
  auto issue_tile = [&](int t, int buf) {
    const int qt0 = t * DKV_BQ;
    TileCopy<D, DKV_BQ, 8> copy;   // offsets recomputed per tile: registers are tight here
    copy.init(wave_id(), lane);
    copy.issue(qt_s[buf], qp, qt0, Nq);
    copy.issue(dot_s[buf], dop, qt0, Nq);
    if (tid < DKV_BQ) {
      const int q = qt0 + tid;
      vec0 = q < Nq ? a.lse[(size_t)bh * Nq + q] * LOG2E : 0.0f;
      vec1 = q < Nq ? a.delta[(size_t)bh * Nq + q] : 0.0f;
      if constexpr (QKS) vec2 = q < Nq ? a.q_scale[(size_t)bh * Nq + q] : 1.0f;
    } else if constexpr (PQ >= 0) {
      if (tid < 3 * DKV_BQ) {
        const int e = tid - DKV_BQ, gi = e / DKV_BQ, qq = e % DKV_BQ;
        const int q = qt0 + qq, grp = grp0 + gi;
        vec0 = (q < Nq && grp < a.NG) ? a.p_amax_in[((size_t)bh * a.NG + grp) * Nq + q] : 0.0f;
      }
    }
  };
  auto finish_tile = [&](int buf) {
    if (tid < DKV_BQ) {
      m_s[buf][tid] = vec0;
      d_s[buf][tid] = vec1;
      if constexpr (QKS) sq_s[buf][tid] = vec2;
    } else if constexpr (PQ >= 0) {
      if (tid < 3 * DKV_BQ) {
        const int e = tid - DKV_BQ, gi = e / DKV_BQ, qq = e % DKV_BQ;
        const FqScale fs = fq_scale(vec0, Fp8Fmt<(PQ >= 0 ? PQ : 0)>::FMAX);
        qs_s[buf][gi][qq] = fs.s;
        qr_s[buf][gi][qq] = fs.r;
      }
    }
  };

  const int qt_begin = CAUSAL ? (k0 / DKV_BQ) : 0;
  const int ntq = (Nq + DKV_BQ - 1) / DKV_BQ;
  const bool wave_live = k0w < Nkv;
  if (qt_begin < ntq) {
    issue_tile(qt_begin, qt_begin & 1);
    wait_vmem();
    finish_tile(qt_begin & 1);
  }
  __syncthreads();
  for (int t = qt_begin; t < ntq; ++t) {
    const int qt0 = t * DKV_BQ;
    const int buf = t & 1;
    if (t + 1 < ntq) issue_tile(t + 1, buf ^ 1);
    if (wave_live) {
      const char* Qt = qt_s[buf];
      const char* dOt = dot_s[buf];
#pragma unroll
      for (int qb2 = 0; qb2 < DKV_BQ / 32; ++qb2) {
        const int qs = qt0 + qb2 * 32;          // first query of this 32-block
        if (qs >= Nq) break;
        if (CAUSAL && qs + 31 < k0w) continue;  // every key of the wave is after every query
        // ---- S = Q K^T (lane: key kj, registers: 16 queries)
        f32x16 sacc = (f32x16){};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) sacc = DT::mfma(lds_row8<D>(Qt, qb2 * 32 + l32, 2 * ks + g), kf[ks], sacc);
        const bool need_mask = (qs + 32 > Nq) || (k0w + 32 > Nkv) || (CAUSAL && qs < k0w + 31);
        // ---- P = exp2(S c - M), formed exactly as in the dQ kernel
        float p[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ql = qb2 * 32 + 8 * u + 4 * g;   // local query of registers 4u..4u+3
          const f32x4 mv = *reinterpret_cast<const f32x4*>(&m_s[buf][ql]);
          f32x4 sq4 = {1.0f, 1.0f, 1.0f, 1.0f};
          if constexpr (QKS) sq4 = *reinterpret_cast<const f32x4*>(&sq_s[buf][ql]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * u + e;
            const float sr = QKS ? sacc[r] * sk_lane : sacc[r];
            const float cr = QKS ? a.c * sq4[e] : a.c;
            p[r] = fast_exp2(__builtin_fmaf(sr, cr, -mv[e]));
          }
        }
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = qs + 8 * (r >> 2) + 4 * g + (r & 3);
            if (q >= Nq || kj >= Nkv || (CAUSAL && kj > q)) p[r] = 0.0f;
          }
        }
        if (!dk_wave) {
          // ---- dV waves: P^ = FQ(P) per (query, 64-key group); dV^T += dO^T P^
          uint32_t wp[8];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int ql = qb2 * 32 + 8 * u + 4 * g;
            if constexpr (PQ >= 0) {
              const f32x4 sv = *reinterpret_cast<const f32x4*>(&qs_s[buf][mygrp][ql]);
              const f32x4 rv = *reinterpret_cast<const f32x4*>(&qr_s[buf][mygrp][ql]);
              const FqScale f4[4] = {{sv[0], rv[0]}, {sv[1], rv[1]}, {sv[2], rv[2]}, {sv[3], rv[3]}};
              const f32x4 xq = fq_quad<(PQ >= 0 ? PQ : 0)>(&p[4 * u], f4);
              wp[2 * u] = DT::pack2(xq[0], xq[1]);
              wp[2 * u + 1] = DT::pack2(xq[2], xq[3]);
            } else {
              wp[2 * u] = DT::pack2(p[4 * u], p[4 * u + 1]);
              wp[2 * u + 1] = DT::pack2(p[4 * u + 2], p[4 * u + 3]);
            }
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const s16x8 p_op = __builtin_bit_cast(s16x8, (u32x4){wp[4 * h], wp[4 * h + 1], wp[4 * h + 2], wp[4 * h + 3]});
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              acc[db] = DT::mfma(lds_tr8<D>(dOt, qb2 * 32 + 16 * h, db * 32, lane), p_op, acc[db]);
          }
        } else {
          // ---- dK waves: dP = dO V^T, dS = P o (dP - Delta); dK^T += Q^T dS
          f32x16 dp = (f32x16){};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) dp = DT::mfma(lds_row8<D>(dOt, qb2 * 32 + l32, 2 * ks + g), vf[ks], dp);
          uint32_t wd[8];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int ql = qb2 * 32 + 8 * u + 4 * g;
            const f32x4 dv4 = *reinterpret_cast<const f32x4*>(&d_s[buf][ql]);
            f32x4 sq4 = {1.0f, 1.0f, 1.0f, 1.0f};
            if constexpr (QKS) sq4 = *reinterpret_cast<const f32x4*>(&sq_s[buf][ql]);
            float dsv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              dsv[e] = p[4 * u + e] * (dp[4 * u + e] - dv4[e]);
              if constexpr (QKS) dsv[e] *= sq4[e];   // dK = sm_scale sum_i dS_ij s_q[i] code_q[i]
            }
            wd[2 * u] = DT::pack2(dsv[0], dsv[1]);
            wd[2 * u + 1] = DT::pack2(dsv[2], dsv[3]);
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const s16x8 ds_op = __builtin_bit_cast(s16x8, (u32x4){wd[4 * h], wd[4 * h + 1], wd[4 * h + 2], wd[4 * h + 3]});
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              acc[db] = DT::mfma(lds_tr8<D>(Qt, qb2 * 32 + 16 * h, db * 32, lane), ds_op, acc[db]);
          }
        }
      }
    }
    wait_vmem();
    if (t + 1 < ntq) finish_tile(buf ^ 1);
    __syncthreads();
  }

  if (kj >= Nkv) return;
  uint16_t* outp = (uint16_t*)(dk_wave ? a.dk : a.dv) + (size_t)bh * Nkv * D;
  const float scale = dk_wave ? a.sm_scale : 1.0f;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = db * 32 + 8 * u + 4 * g;
      const float x[4] = {acc[db][4 * u] * scale, acc[db][4 * u + 1] * scale, acc[db][4 * u + 2] * scale,
                          acc[db][4 * u + 3] * scale};
      *reinterpret_cast<u32x2*>(outp + (size_t)kj * D + d) = (u32x2){DT::pack2(x[0], x[1]), DT::pack2(x[2], x[3])};
    }
}

// ------------------------------------------------------------------ dispatch
template <class DT, int D, bool CAUSAL, int PQ, int IN>
struct DqK {
  static void run(dim3 g, const BwdArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((dq_kernel<DT, D, CAUSAL, PQ, IN>), g, dim3(256), 0, st, a);
  }
};
template <class DT, int D, bool CAUSAL, int PQ, int IN>
struct DkvK {
  static void run(dim3 g, const BwdArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((dkdv_kernel<DT, D, CAUSAL, PQ, IN>), g, dim3(512), 0, st, a);
  }
};

template <template <class, int, bool, int, int> class K, class DT, int D, bool CAUSAL, int IN>
static void pick_pq(dim3 g, const BwdArgs& a, int pfmt, hipStream_t st) {
  if (pfmt == 0) K<DT, D, CAUSAL, 0, IN>::run(g, a, st);
  else if (pfmt == 1) K<DT, D, CAUSAL, 1, IN>::run(g, a, st);
  else K<DT, D, CAUSAL, -1, IN>::run(g, a, st);
}

template <template <class, int, bool, int, int> class K, class DT, int D, int IN>
static void pick_causal(dim3 g, const BwdArgs& a, bool causal, int pfmt, hipStream_t st) {
  if (causal) pick_pq<K, DT, D, true, IN>(g, a, pfmt, st);
  else pick_pq<K, DT, D, false, IN>(g, a, pfmt, st);
}

template <template <class, int, bool, int, int> class K, class DT, int D>
static void pick_rest(dim3 g, const BwdArgs& a, bool causal, int pfmt, int mode, hipStream_t st) {
  if (mode == IN_VFP8) {
    if constexpr (__is_same(DT, BF16)) pick_causal<K, DT, D, IN_VFP8>(g, a, causal, pfmt, st);
    return;
  }
  if (mode == IN_QKS) pick_causal<K, DT, D, IN_QKS>(g, a, causal, pfmt, st);
  else pick_causal<K, DT, D, IN_PLAIN>(g, a, causal, pfmt, st);
}

template <template <class, int, bool, int, int> class K>
static hipError_t pick_all(const Shape& s, dim3 g, const BwdArgs& a, bool causal, int pfmt, int mode,
                           hipStream_t st) {
  if (s.dtype == 0) {
    if (s.D == 128) pick_rest<K, BF16, 128>(g, a, causal, pfmt, mode, st);
    else pick_rest<K, BF16, 64>(g, a, causal, pfmt, mode, st);
  } else {
    if (s.D == 128) pick_rest<K, FP16, 128>(g, a, causal, pfmt, mode, st);
    else pick_rest<K, FP16, 64>(g, a, causal, pfmt, mode, st);
  }
  return hipGetLastError();
}

static BwdArgs make_args(const Shape& s, const Inputs& in, const void* dout, const float* lse,
                         const float* delta, float sm_scale) {
  BwdArgs a = {};
  a.q = in.q; a.k = in.k; a.v = in.v;
  a.v_scale = in.v_scale; a.q_scale = in.q_scale; a.k_scale = in.k_scale;
  a.dout = dout; a.lse = lse; a.delta = delta;
  a.Nq = s.Nq; a.Nkv = s.Nkv; a.NG = (s.Nkv + P_GROUP - 1) / P_GROUP;
  a.sm_scale = sm_scale;
  a.c = sm_scale * LOG2E;
  return a;
}

hipError_t launch_bwd_dq(const Shape& s, const Inputs& in, const void* dout, const float* lse,
                         const float* delta, float sm_scale, bool causal, int pfmt,
                         void* dq, float* p_amax, hipStream_t st) {
  BwdArgs a = make_args(s, in, dout, lse, delta, sm_scale);
  a.dq = dq;
  a.p_amax = p_amax;
  dim3 grid(((s.Nq + DQ_BM - 1) / DQ_BM) * s.B * s.H);
  return pick_all<DqK>(s, grid, a, causal, pfmt, in.mode, st);
}

hipError_t launch_bwd_dkdv(const Shape& s, const Inputs& in, const void* dout, const float* lse,
                           const float* delta, const float* p_amax, float sm_scale, bool causal,
                           int pfmt, void* dk, void* dv, hipStream_t st) {
  BwdArgs a = make_args(s, in, dout, lse, delta, sm_scale);
  a.p_amax_in = p_amax;
  a.dk = dk;
  a.dv = dv;
  dim3 grid(((s.Nkv + DKV_BN - 1) / DKV_BN) * s.B * s.H);
  return pick_all<DkvK>(s, grid, a, causal, pfmt, in.mode, st);
}

}  // namespace qat
