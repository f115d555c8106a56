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
      acc = __builtin_fmaf(DT::to_f32((uint16_t)(wa[e >> 1] >> (16 * (e & 1)))),
                           DT::to_f32((uint16_t)(wb[e >> 1] >> (16 * (e & 1)))), acc);
  } else {
    const u32x2 wa = *reinterpret_cast<const u32x2*>(a);
    const u32x2 wb = *reinterpret_cast<const u32x2*>(b);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_fmaf(DT::to_f32((uint16_t)(wa[e >> 1] >> (16 * (e & 1)))),
                           DT::to_f32((uint16_t)(wb[e >> 1] >> (16 * (e & 1)))), acc);
  }
  // (the dQ kernel reproduces this order when it forms Delta itself: row_delta)
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
  float* dkdv_part;     // fp32 partial dK/dV of split key blocks
  const float* k_mean;  // K smoothing: dQ += rowsum(dS) k_mean (null: off)
  const void* o_hp;     // dQ: with delta_out, Delta is formed in the kernel
  float* delta_out;     //   from o_hp and dout and written here
  int n_whole;          // dK/dV: key blocks run whole by one workgroup each
  int n_split;          // dK/dV: query-range parts of each remaining key block
  int Nq, Nkv, NG;
  float sm_scale;
  float c;              // sm_scale * log2(e)
};


// ------------------------------------------------------------------ dQ
// Delta of one query row from the dQ kernel's operand layout (lane half g
// holds d = 16 ks + 8 g + j, j = 0..7), in exactly delta_kernel's order: 16
// chunks of D/16 consecutive products summed in sequence (each product of two
// 16-bit values is exact in fp32), then pair sums of chunks 8, 4, 2 and 1
// apart.  At D = 128 chunk 2 ks + g is one fragment and only the last pair
// step crosses lane halves; at D = 64 chunk 4 ks + 2 g + h is half a fragment
// and the step at distance 2 crosses.  Float addition commutes, so the
// symmetric exchanges reproduce every partial sum bit for bit.
template <class DT, int D>
__device__ __forceinline__ float row_delta(const s16x8 (&ohf)[D / 16], const s16x8 (&dof)[D / 16]) {
  constexpr int NKS = D / 16;
  float t[NKS][2];   // chunk sums: [ks][half of the fragment] (D = 128 uses the whole fragment)
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const u32x4 wa = __builtin_bit_cast(u32x4, ohf[ks]), wb = __builtin_bit_cast(u32x4, dof[ks]);
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int h = D == 128 ? 0 : (j >> 2);
      acc[h] = __builtin_fmaf(DT::to_f32((uint16_t)(wa[j >> 1] >> (16 * (j & 1)))),
                              DT::to_f32((uint16_t)(wb[j >> 1] >> (16 * (j & 1)))), acc[h]);
    }
    t[ks][0] = acc[0];
    t[ks][1] = acc[1];
  }
  if constexpr (D == 128) {   // chunk c = 2 ks + g
    float s1[4], s2[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) s1[i] = t[i][0] + t[i + 4][0];   // distance 8
#pragma unroll
    for (int i = 0; i < 2; ++i) s2[i] = s1[i] + s1[i + 2];       // distance 4
    return sum_xor32(s2[0] + s2[1]);                             // distance 2, then 1 (lane halves)
  } else {                    // chunk c = 4 ks + 2 g + h
    float s1[2][2], s2[2], s3[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) s1[i][h] = t[i][h] + t[i + 2][h];   // distance 8
#pragma unroll
    for (int h = 0; h < 2; ++h) s2[h] = s1[0][h] + s1[1][h];         // distance 4
#pragma unroll
    for (int h = 0; h < 2; ++h) s3[h] = sum_xor32(s2[h]);            // distance 2 (lane halves)
    return s3[0] + s3[1];                                            // distance 1
  }
}

constexpr int DQ_BM = 128;
constexpr int DQ_BN = 64;

// SMK: K smoothing, dQ += sm_scale rowsum(dS) k_mean (a separate instance, so
// that the plain kernel is not burdened with the extra row sum)
template <class DT, int D, bool CAUSAL, int PQ, int IN, bool SMK>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdArgs a) {
  constexpr bool VFP8 = IN == IN_VFP8;
  constexpr bool QKS = IN == IN_QKS;
  constexpr int TILE = DQ_BN * D * 2;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  __shared__ __attribute__((aligned(16))) char smem[2][2][TILE];   // [buffer][K, V]
  __shared__ __attribute__((aligned(16))) float ks_s[2][DQ_BN];     // IN_QKS: key scales
  // IN_VFP8: the next tile's V codes, copied HBM -> LDS by DMA
  constexpr int VC_BYTES = VFP8 ? DQ_BN * D : 16;
  constexpr int VC_PER_THREAD = DQ_BN * D / (256 * 16);   // 16-byte chunks per thread
  __shared__ __attribute__((aligned(16))) char vc_s[VC_BYTES];

  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int ntq = (a.Nq + DQ_BM - 1) / DQ_BM;
  int bh, rank;   // causal: the longest rows (last blocks) first
  work_unit(blockIdx.x, gridDim.x, ntq, CAUSAL, &bh, &rank);
  const int qb = (CAUSAL ? ntq - 1 - rank : rank) * DQ_BM;
  const int q0 = qb + w * 32;
  const int qi = q0 + l32;
  const int lane_g4 = 4 * g, lane_dq = 4 * g - l32;   // mask terms (key - kv0 - c, key - qi + q0 - kv0 - c)
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
  float Di;
  if (a.delta_out) {   // Delta of this row (from dO as given), bit for bit as delta_kernel forms it, published for dK/dV
    s16x8 ohf[NKS];
    const uint16_t* ohp = (const uint16_t*)a.o_hp + (size_t)bh * Nq * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      ohf[ks] = qi < Nq ? *reinterpret_cast<const s16x8*>(ohp + (size_t)qi * D + 16 * ks + 8 * g) : (s16x8){};
    Di = row_delta<DT, D>(ohf, dof);
    if (g == 0 && qi < Nq) a.delta_out[(size_t)bh * Nq + qi] = Di;
  } else {
    Di = qi < Nq ? a.delta[(size_t)bh * Nq + qi] : 0.0f;
  }
  if constexpr (VFP8) {   // dP = (dO * v_scale) code^T: the per-channel V scale moves onto dO
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(vsc + 16 * ks + 8 * g);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(vsc + 16 * ks + 8 * g + 4);
      const float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      const u32x4 wd = __builtin_bit_cast(u32x4, dof[ks]);
      u32x4 ws;
#pragma unroll
      for (int h = 0; h < 4; ++h)
        ws[h] = BF16::pack2(BF16::to_f32((uint16_t)(wd[h] & 0xFFFFu)) * sc[2 * h],
                            BF16::to_f32((uint16_t)(wd[h] >> 16)) * sc[2 * h + 1]);
      dof[ks] = __builtin_bit_cast(s16x8, ws);
    }
  }
  float c_row = a.c;   // IN_QKS: s_q folds into the log2 scale (same rounding as dK/dV)
  // (a zero scale, all-zero row, is raised to the smallest normal so that a
  // masked score stays -inf after the product)
  if constexpr (QKS) c_row = a.c * fmaxf(qi < Nq ? a.q_scale[(size_t)bh * Nq + qi] : 1.0f, 1.17549435e-38f);

  f32x16 dq_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq_acc[db] = (f32x16){};
  constexpr bool smooth = SMK;
  float ds_rowsum = 0.0f;   // this lane's half of sum_j dS_ij (K smoothing)

  // K tiles (and V, unless fp8) go HBM -> LDS directly, double-buffered.  fp8
  // V codes go HBM -> LDS by DMA too, into one 8-bit tile in plain row order:
  // chunk u of a thread is the 16 bytes at P = (4u + wave) KiB + 16 lane,
  // and the same thread decodes exactly those bytes after its own copies
  // completed, so the decode needs no barrier.  Key scales take a register
  // detour.
  float ksreg = 0.0f;
  TileCopy<D, DQ_BN, 4> copy;
  copy.init(w, lane);
  auto issue_tile = [&](int t, int buf) {
    copy.issue(smem[buf][0], kp, t * DQ_BN, Nkv);
    if constexpr (VFP8) {
#pragma unroll
      for (int u = 0; u < VC_PER_THREAD; ++u) {
        const int blk = u * 4 + w, P = blk * 1024 + lane * 16;
        const int key = min(t * DQ_BN + P / D, Nkv - 1);   // tail rows repeat the last key (masked)
        __builtin_amdgcn_global_load_lds((const void*)(vp + (size_t)key * D + P % D),
                                         (lds_void*)(vc_s + blk * 1024), 16, 0, 0);
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
    if constexpr (VFP8) {   // the code values themselves (exact in bf16); v_scale is on dO
#pragma unroll
      for (int u = 0; u < VC_PER_THREAD; ++u) {
        const int P = (u * 4 + w) * 1024 + lane * 16, row = P / D, c0 = P % D;
        const u32x4 codes = *reinterpret_cast<const u32x4*>(vc_s + P);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {   // 8 codes -> one 16-byte chunk of the bf16 tile
          u32x4 vv;
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const f32x2 f = __builtin_amdgcn_cvt_pk_f32_bf8((int)(codes[2 * h2 + (h >> 1)] >> (16 * (h & 1))), false);
            vv[h] = BF16::pack2(f[0], f[1]);
          }
          *reinterpret_cast<u32x4*>(smem[buf][1] + tile_off<D>(row, c0 / 8 + h2)) = vv;
        }
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
    // masks (key tail, causal diagonal) zero p.  With key = kv0 + c + 4g (c
    // the element's offset) and qi = q0 + l32, each test compares one
    // per-lane value with a wave-uniform bound.
    float p[2][16];
    float pmax = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], c_row, -Mi));
    if (need_mask) {
      // an opaque statement keeps this a branch: otherwise the masks are
      // if-converted into selects that every tile executes
      asm volatile("");
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
          if (lane_g4 >= Nkv - kv0 - c || (CAUSAL && lane_dq > q0 - kv0 - c)) p[kb][r] = 0.0f;
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pmax = fmaxf(pmax, p[kb][r]);
    if constexpr (PQ >= 0) {
      pmax = max_xor32(pmax);
      if (g == 0 && qi < Nq) a.p_amax[((size_t)bh * a.NG + t) * Nq + qi] = pmax;
    }
    if constexpr (smooth) {   // K smoothing: sum_j dS_ij (fp32, before any key scale)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) ds_rowsum += p[kb][r] * (dp[kb][r] - Di);
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
  // K smoothing: dQ is taken for the original K = (K - k_mean) + k_mean
  float rs = 0.0f;
  if constexpr (smooth) rs = sum_xor32(ds_rowsum);
  if (qi >= Nq) return;
  uint16_t* dqp = (uint16_t*)a.dq + (size_t)bh * Nq * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = db * 32 + 8 * u + 4 * g;
      float x[4] = {dq_acc[db][4 * u], dq_acc[db][4 * u + 1], dq_acc[db][4 * u + 2], dq_acc[db][4 * u + 3]};
      if constexpr (smooth) {
        const f32x4 km = *reinterpret_cast<const f32x4*>(a.k_mean + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] += rs * km[e];
      }
      *reinterpret_cast<u32x2*>(dqp + (size_t)qi * D + d) =
          (u32x2){DT::pack2(x[0] * a.sm_scale, x[1] * a.sm_scale), DT::pack2(x[2] * a.sm_scale, x[3] * a.sm_scale)};
    }
}

// ---------------------------------------------------------------------------
// Software-pipelined dK/dV: one wave per SIMD.
//
// Four waves own 128 keys (32 each) and produce dK and dV for them, walking
// the query range in blocks of 32.  Each wave holds the whole 512-entry
// register file: the dK/dV accumulators, the K and V operands of its keys,
// two S/dP buffers and two sets of packed P^/dS operands.  Iteration b
// issues as one instruction stream
//   the matrix work  dV^T += dO^T P^(b-1), dK^T += Q^T dS(b-1),
//                    S(b+1) = Q K^T, dP(b+1) = dO V^T, and
//   the vector work of block b: P = exp2(S c - M), P^ = FQ(P) with the
//                    (query, 64-key group) scales, dS = P o (dP - Delta),
//                    packed as the next iteration's operands,
// in eight fenced groups of MFMAs plus a slice of the vector work, so the
// matrix core runs under the vector work of the same wave.  Q/dO blocks are
// staged through registers: loaded from HBM in iteration b-5, written to LDS
// slot b%8 in iteration b-4, read in iterations b-1 .. b+1.  A barrier ends
// every third iteration only (b % 3 == 2): a block written in iteration c is
// first read in c + 3, after a barrier that ends one of c .. c + 2, and the
// block its slot held before was last read in c - 3, before a barrier that
// ends one of c - 3 .. c - 1.
constexpr int DSP_BN = 128;    // keys per workgroup
constexpr int DSP_BQ = 32;     // queries per block
constexpr int DSP_SLOTS = 8;   // LDS block slots

template <class DT, int D, bool CAUSAL, int PQ, int IN>
__global__ __launch_bounds__(256, 1) void dkdv_sp_kernel(BwdArgs a) {
  constexpr bool VFP8 = IN == IN_VFP8;
  constexpr bool QKS = IN == IN_QKS;
  constexpr int TILE = DSP_BQ * D * 2;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  constexpr int FQF = PQ >= 0 ? PQ : 0;
  constexpr int NGW = DSP_BN / 64;          // 64-key P groups of the workgroup
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int NCH = DSP_BQ * CPR / 256;   // staged chunks per thread per tile
  constexpr int NST2 = 4 * NDB;             // dV/dK MFMAs of a block
  constexpr int NST = NST2 + 2 * NKS;       // + S/dP MFMAs
  constexpr int NGRP = 8;                   // fenced groups per iteration
  constexpr int GSZ = NST / NGRP;           // MFMAs per group
  constexpr int AHEAD = 4;                  // MFMA steps whose LDS operand is in flight
  static_assert(NST % NGRP == 0 && NCH >= 1, "shape");
  __shared__ __attribute__((aligned(16))) char q_s[DSP_SLOTS][TILE];
  __shared__ __attribute__((aligned(16))) char do_s[DSP_SLOTS][TILE];
  __shared__ __attribute__((aligned(16))) float m_s[DSP_SLOTS][DSP_BQ];
  __shared__ __attribute__((aligned(16))) float d_s[DSP_SLOTS][DSP_BQ];
  __shared__ __attribute__((aligned(16))) float sq_s[DSP_SLOTS][DSP_BQ];
  __shared__ __attribute__((aligned(16))) float cq_s[QKS ? DSP_SLOTS : 1][DSP_BQ];   // c * s_q (exponent scale)
  __shared__ __attribute__((aligned(16))) float qs_s[DSP_SLOTS][NGW][DSP_BQ];
  __shared__ __attribute__((aligned(16))) float qr_s[DSP_SLOTS][NGW][DSP_BQ];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int nkb = (a.Nkv + DSP_BN - 1) / DSP_BN;
  // Workgroups [0, n_whole) take whole key blocks; the rest take one of
  // n_split query ranges of the last key blocks, which would otherwise run
  // alone in a last, mostly idle round of the chip.
  int unit, part = 0, nparts = 1;
  if (CAUSAL) {   // never split; key block 0 sees every query: longest first
    int bh_c, rank;
    work_unit(blockIdx.x, gridDim.x, nkb, true, &bh_c, &rank);
    unit = bh_c * nkb + rank;
  } else if ((int)blockIdx.x < a.n_whole) {
    unit = xcd_unit(blockIdx.x, a.n_whole);
  } else {
    const int j = xcd_unit(blockIdx.x - a.n_whole, gridDim.x - a.n_whole);
    unit = a.n_whole + j / a.n_split;
    part = j % a.n_split;
    nparts = a.n_split;
  }
  const int bh = unit / nkb;
  const int k0 = (unit % nkb) * DSP_BN;
  const int k0w = k0 + w * 32;
  const int kj = k0w + l32;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const int lgrp = w >> 1;                // this wave's 64-key group within the workgroup
  const int grp0 = k0 / 64;
  const uint16_t* qp = (const uint16_t*)a.q + (size_t)bh * Nq * D;
  const uint16_t* dop = (const uint16_t*)a.dout + (size_t)bh * Nq * D;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)bh * Nkv * D;

  // K^T and V^T operands of this wave's 32 keys: lane holds key kj, d = 16ks + 8g .. +7
  s16x8 kf[NKS], vf[NKS];
  {
    const bool ok = kj < Nkv;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kf[ks] = ok ? *reinterpret_cast<const s16x8*>(kp + (size_t)kj * D + 16 * ks + 8 * g) : (s16x8){};
      vf[ks] = (s16x8){};
      if (ok) {
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
  // per-key scale in the exponent; raised to the smallest normal (and 1 for
  // absent keys) so that a masked score stays -inf after the product
  const float sk_lane = QKS ? (kj < Nkv ? fmaxf(a.k_scale[(size_t)bh * Nkv + kj], 1.17549435e-38f) : 1.0f) : 1.0f;
  // these loads complete here, so that no wait for them lands inside the loop
  // (where it would also drain the block loads in flight)
  wait_vmem();

  const int qb_first = CAUSAL ? k0 / DSP_BQ : 0;
  const int nqb = (Nq + DSP_BQ - 1) / DSP_BQ;
  const int NB_all = nqb > qb_first ? nqb - qb_first : 0;
  const int qb_begin = qb_first + NB_all * part / nparts;
  const int NB = qb_first + NB_all * (part + 1) / nparts - qb_begin;   // query blocks of this workgroup
  const bool wave_live = k0w < Nkv;
  auto qstart = [&](int b) { return (qb_begin + b) * DSP_BQ; };
  // some (query, key) pair of block b and this wave's keys is unmasked
  auto active = [&](int b) { return wave_live && (!CAUSAL || qstart(b) + DSP_BQ - 1 >= k0w); };

  // ---- staging of a block: thread tid holds chunks tid + 256i of the Q and
  // dO tiles and vector entry tid (kind tid/32: 0 LSE, 1 Delta, 2 query
  // scale, 3.. P-quant absmax of local group kind-3; query tid%32)
  u32x4 stq[NCH], sto[NCH];
  float stv = 0.0f;
  const int e_kind = tid >> 5, e_q = tid & 31;
  // source row of this thread's vector entry (loop-invariant); entries that
  // are not used read LSE and are discarded, so the load is unconditional
  // and nothing waits on it before the block is written to LDS
  const int e_grp = grp0 + e_kind - 3;
  const bool e_used = e_kind < 2 || (e_kind == 2 && QKS) || (PQ >= 0 && e_kind >= 3 && e_kind < 3 + NGW && e_grp < a.NG);
  const float* e_src = a.lse + (size_t)bh * Nq;
  if (e_used && e_kind == 1) e_src = a.delta + (size_t)bh * Nq;
  if (e_used && e_kind == 2) e_src = a.q_scale + (size_t)bh * Nq;
  if (e_used && e_kind >= 3) e_src = a.p_amax_in + ((size_t)bh * a.NG + e_grp) * Nq;
  auto load_stage = [&](int b) __attribute__((always_inline)) {
    const int q0 = qstart(b);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + 256 * i, row = c / CPR, ch = c % CPR;
      const size_t rr = (size_t)min(q0 + row, Nq - 1);
      stq[i] = *reinterpret_cast<const u32x4*>(qp + rr * D + 8 * ch);
      sto[i] = *reinterpret_cast<const u32x4*>(dop + rr * D + 8 * ch);
    }
    stv = e_src[min(q0 + e_q, Nq - 1)];
  };
  auto write_tiles = [&](int b) __attribute__((always_inline)) {
    const int slot = b & (DSP_SLOTS - 1);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + 256 * i, row = c / CPR, ch = c % CPR;
      *reinterpret_cast<u32x4*>(q_s[slot] + tile_off<D>(row, ch)) = stq[i];
      *reinterpret_cast<u32x4*>(do_s[slot] + tile_off<D>(row, ch)) = sto[i];
    }
  };
  auto write_vec = [&](int b) __attribute__((always_inline)) {
    const int slot = b & (DSP_SLOTS - 1);
    const bool ok = e_used && qstart(b) + e_q < Nq;
    if (e_kind == 0) m_s[slot][e_q] = ok ? stv * LOG2E : 0.0f;
    else if (e_kind == 1) d_s[slot][e_q] = ok ? stv : 0.0f;
    else if (e_kind == 2) {
      sq_s[slot][e_q] = ok ? stv : 1.0f;
      // a zero scale (all-zero row) is raised to the smallest normal so that a
      // masked score stays -inf after the product
      if constexpr (QKS) cq_s[slot][e_q] = a.c * fmaxf(ok ? stv : 1.0f, 1.17549435e-38f);
    }
    else if (PQ >= 0 && e_kind < 3 + NGW) {
      const FqScale fs = fq_scale<FQF>(ok ? stv : 0.0f);
      qs_s[slot][e_kind - 3][e_q] = fs.s;
      qr_s[slot][e_kind - 3][e_q] = fs.r;
    }
  };

  f32x16 acc_dv[NDB], acc_dk[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    acc_dv[db] = (f32x16){};
    acc_dk[db] = (f32x16){};
  }
  // S/dP of a block (lane: key kj, registers: queries 8(r/4) + 4g + r%4) and
  // its packed P^ / dS operands (query half h = words 4h .. 4h+3)
  f32x16 sA, dpA, sB, dpB;
  uint32_t pA[8], dsA[8], pB[8], dsB[8];

  // MFMA step st of iteration b: first the k-steps of S and dP of block b+1,
  // interleaved (Q or dO row fragment against K or V), so that they are
  // complete when the next iteration reads them; then st >= NST1: half h,
  // column block db, {dV, dK} of block b-1 (transposed dO or Q fragment).
  constexpr int NST1 = NST - NST2;
  auto fetch = [&](int b, int st_) __attribute__((always_inline)) {
    const int st = st_ < NST1 ? st_ + NST2 : st_ - NST1;
    if (st < NST2) {
      const int h = st / (2 * NDB), r = st % (2 * NDB), db = r >> 1, which = r & 1;
      const int slot = (b - 1) & (DSP_SLOTS - 1);
      return lds_tr8<D>(which ? q_s[slot] : do_s[slot], 16 * h, 32 * db, lane);
    }
    const int k = st - NST2, ks = k >> 1, which = k & 1;
    const int slot = (b + 1) & (DSP_SLOTS - 1);
    return lds_row8<D>(which ? do_s[slot] : q_s[slot], l32, 2 * ks + g);
  };
  auto step = [&](const s16x8& frag, int st_, const uint32_t (&Pp)[8], const uint32_t (&DSp)[8], f32x16& S2,
                  f32x16& DP2) __attribute__((always_inline)) {
    const int st = st_ < NST1 ? st_ + NST2 : st_ - NST1;
    if (st < NST2) {
      const int h = st / (2 * NDB), r = st % (2 * NDB), db = r >> 1, which = r & 1;
      if (which == 0) {
        const s16x8 op = __builtin_bit_cast(s16x8, (u32x4){Pp[4 * h], Pp[4 * h + 1], Pp[4 * h + 2], Pp[4 * h + 3]});
        acc_dv[db] = DT::mfma(frag, op, acc_dv[db]);
      } else {
        const s16x8 op = __builtin_bit_cast(s16x8, (u32x4){DSp[4 * h], DSp[4 * h + 1], DSp[4 * h + 2], DSp[4 * h + 3]});
        acc_dk[db] = DT::mfma(frag, op, acc_dk[db]);
      }
    } else {
      const int k = st - NST2, ks = k >> 1, which = k & 1;
      if (k == 0) {
        S2 = (f32x16){};
        DP2 = (f32x16){};
      }
      if (which == 0) S2 = DT::mfma(frag, kf[ks], S2);
      else DP2 = DT::mfma(frag, vf[ks], DP2);
    }
  };
  // vector work of block b, per quarter u (registers 4u .. 4u+3): read the
  // per-query vectors, form P, then quantize, form dS and pack both operands.
  // The reads of a quarter are issued a group or more before their use.
  float p[16];
  f32x4 mvv[4], dvv[4], sqv[4], cqv[4], svv[4], rvv[4];
  auto readvec = [&](int u, int b) __attribute__((always_inline)) {
    const int slot = b & (DSP_SLOTS - 1), ql = 8 * u + 4 * g;
    mvv[u] = *reinterpret_cast<const f32x4*>(&m_s[slot][ql]);
    dvv[u] = *reinterpret_cast<const f32x4*>(&d_s[slot][ql]);
    sqv[u] = (f32x4){1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (QKS) {
      sqv[u] = *reinterpret_cast<const f32x4*>(&sq_s[slot][ql]);
      cqv[u] = *reinterpret_cast<const f32x4*>(&cq_s[slot][ql]);
    }
    if constexpr (PQ >= 0) {
      svv[u] = *reinterpret_cast<const f32x4*>(&qs_s[slot][lgrp][ql]);
      rvv[u] = *reinterpret_cast<const f32x4*>(&qr_s[slot][lgrp][ql]);
    }
  };
  auto form_p = [&](int u, const f32x16& S) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * u + e;
      const float sr = QKS ? S[r] * sk_lane : S[r];
      const float cr = QKS ? cqv[u][e] : a.c;
      p[r] = fast_exp2(__builtin_fmaf(sr, cr, -mvv[u][e]));
    }
  };
  auto finish = [&](int u, const f32x16& DP, uint32_t (&Pn)[8], uint32_t (&DSn)[8]) __attribute__((always_inline)) {
    uint32_t w0, w1;
    if constexpr (PQ >= 0) {   // P^ = FQ(P) per (query, 64-key group)
      const FqScale f4[4] = {{svv[u][0], rvv[u][0]}, {svv[u][1], rvv[u][1]}, {svv[u][2], rvv[u][2]},
                             {svv[u][3], rvv[u][3]}};
      const f32x4 xq = fq_quad<FQF>(&p[4 * u], f4);
      w0 = DT::pack2(xq[0], xq[1]);
      w1 = DT::pack2(xq[2], xq[3]);
    } else {
      w0 = DT::pack2(p[4 * u], p[4 * u + 1]);
      w1 = DT::pack2(p[4 * u + 2], p[4 * u + 3]);
    }
    float dsv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dsv[e] = p[4 * u + e] * (DP[4 * u + e] - dvv[u][e]);
      if constexpr (QKS) dsv[e] *= sqv[u][e];   // dK = sm_scale sum_i dS_ij s_q[i] code_q[i]
    }
    Pn[2 * u] = w0;
    Pn[2 * u + 1] = w1;
    DSn[2 * u] = DT::pack2(dsv[0], dsv[1]);
    DSn[2 * u + 1] = DT::pack2(dsv[2], dsv[3]);
  };
  // slice j of the vector work, placed in fenced group j (NGRP == 8):
  //   0: read 0 | 1: P 0, read 1 | 2: finish 0, read 2 | 3: P 1
  //   4: finish 1, read 3 | 5: P 2 | 6: finish 2, P 3 | 7: finish 3
  auto valu_piece = [&](int j, int b, const f32x16& S, const f32x16& DP, uint32_t (&Pn)[8],
                        uint32_t (&DSn)[8]) __attribute__((always_inline)) {
    switch (j) {
      case 0: readvec(0, b); break;
      case 1: form_p(0, S); readvec(1, b); break;
      case 2: finish(0, DP, Pn, DSn); readvec(2, b); break;
      case 3: form_p(1, S); break;
      case 4: finish(1, DP, Pn, DSn); readvec(3, b); break;
      case 5: form_p(2, S); break;
      case 6: finish(2, DP, Pn, DSn); form_p(3, S); break;
      default: finish(3, DP, Pn, DSn); break;
    }
  };

  // iteration b: S, DP = block b (in), S2, DP2 = block b+1 (out);
  // Pp, DSp = operands of block b-1 (in), Pn, DSn = operands of block b (out)
  auto iteration = [&](int b, f32x16& S, f32x16& DP, f32x16& S2, f32x16& DP2, const uint32_t (&Pp)[8],
                       const uint32_t (&DSp)[8], uint32_t (&Pn)[8], uint32_t (&DSn)[8],
                       bool sync) __attribute__((always_inline)) {
    const bool do2 = b >= 1 && active(b - 1);
    const bool do1 = b + 1 < NB && active(b + 1);
    const bool dov = b < NB && active(b);
    const bool full = do2 && do1 && dov;
    // staging of block b+4 (loaded in iteration b-1) and loads of block b+5:
    // inside the first fenced groups on the full path, up front otherwise
    const bool stw = b + 4 < NB, stl = b + 5 < NB;
    if (!full) {
      if (stw) {
        write_tiles(b + 4);
        write_vec(b + 4);
      }
      if (stl) load_stage(b + 5);
    }
    if (dov) {   // masked scores -> -inf before the exponent
      const int q0 = qstart(b);
      if ((q0 + DSP_BQ > Nq) || (k0w + 32 > Nkv) || (CAUSAL && q0 < k0w + 31)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (q >= Nq || kj >= Nkv || (CAUSAL && kj > q)) S[r] = -INFINITY;
        }
      }
    }
    if (full) {
      s16x8 ring[AHEAD];
#pragma unroll
      for (int st = 0; st < AHEAD; ++st) ring[st] = fetch(b, st);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NGRP; ++j) {
#pragma unroll
        for (int i = 0; i < GSZ; ++i) {
          const int st = j * GSZ + i;
          const s16x8 cur = ring[st % AHEAD];
          if (st + AHEAD < NST) ring[st % AHEAD] = fetch(b, st + AHEAD);
          step(cur, st, Pp, DSp, S2, DP2);
        }
        valu_piece(j, b, S, DP, Pn, DSn);
        if (j == 0 && stw) write_tiles(b + 4);
        if (j == 1 && stw) write_vec(b + 4);
        if (j == 2 && stl) load_stage(b + 5);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      if (do1) {
#pragma unroll
        for (int st = 0; st < NST1; ++st) step(fetch(b, st), st, Pp, DSp, S2, DP2);
      }
      if (do2) {
#pragma unroll
        for (int st = NST1; st < NST; ++st) step(fetch(b, st), st, Pp, DSp, S2, DP2);
      }
      if (dov) {
#pragma unroll
        for (int j = 0; j < NGRP; ++j) valu_piece(j, b, S, DP, Pn, DSn);
      }
    }
    if (sync) __syncthreads();
  };

  // prologue: blocks 0 .. 3 in LDS, block 4 staged, S/dP of block 0
#pragma unroll
  for (int b0 = 0; b0 < 4; ++b0) {
    if (NB > b0) {
      load_stage(b0);
      write_tiles(b0);
      write_vec(b0);
    }
  }
  if (NB > 4) load_stage(4);
  __syncthreads();
  if (NB > 0 && active(0)) {
#pragma unroll
    for (int st = 0; st < NST1; ++st) step(fetch(-1, st), st, pB, dsB, sA, dpA);
  }
  for (int b = 0; b <= NB; b += 2) {
    iteration(b, sA, dpA, sB, dpB, pB, dsB, pA, dsA, b % 3 == 2);
    if (b + 1 <= NB) iteration(b + 1, sB, dpB, sA, dpA, pA, dsA, pB, dsB, (b + 1) % 3 == 2);
  }

  if (kj >= Nkv) return;
  if (nparts > 1) {   // unscaled fp32 partials [slot][dK, dV][key of the block][D]
    float* pw = a.dkdv_part + (size_t)((unit - a.n_whole) * nparts + part) * 2 * DSP_BN * D;
    const int kl = w * 32 + l32;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = db * 32 + 8 * u + 4 * g;
        *reinterpret_cast<f32x4*>(pw + (size_t)kl * D + d) =
            (f32x4){acc_dk[db][4 * u], acc_dk[db][4 * u + 1], acc_dk[db][4 * u + 2], acc_dk[db][4 * u + 3]};
        *reinterpret_cast<f32x4*>(pw + (size_t)(DSP_BN + kl) * D + d) =
            (f32x4){acc_dv[db][4 * u], acc_dv[db][4 * u + 1], acc_dv[db][4 * u + 2], acc_dv[db][4 * u + 3]};
      }
    return;
  }
  uint16_t* dkp = (uint16_t*)a.dk + (size_t)bh * Nkv * D;
  uint16_t* dvp = (uint16_t*)a.dv + (size_t)bh * Nkv * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = db * 32 + 8 * u + 4 * g;
      float x[4], y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = acc_dk[db][4 * u + e] * a.sm_scale;
        y[e] = acc_dv[db][4 * u + e];
      }
      *reinterpret_cast<u32x2*>(dkp + (size_t)kj * D + d) = (u32x2){DT::pack2(x[0], x[1]), DT::pack2(x[2], x[3])};
      *reinterpret_cast<u32x2*>(dvp + (size_t)kj * D + d) = (u32x2){DT::pack2(y[0], y[1]), DT::pack2(y[2], y[3])};
    }
}

// Sum of the query-range partials of each split key block, in part order
// (deterministic), scaled and rounded like the whole-block epilogue.  Thread
// t of workgroup (block, z) handles four consecutive d of one key.
template <class DT, int D>
__global__ __launch_bounds__(256) void dkdv_merge_kernel(BwdArgs a, int nkb) {
  constexpr int PER_BLOCK = DSP_BN * D / 4;   // threads per key block
  const int i = blockIdx.y * 256 + threadIdx.x;
  if (i >= PER_BLOCK) return;
  const int kl = i / (D / 4), d = 4 * (i % (D / 4));
  const int unit = a.n_whole + blockIdx.x;
  const int bh = unit / nkb, key = (unit % nkb) * DSP_BN + kl;
  if (key >= a.Nkv) return;
  const float* pw = a.dkdv_part + (size_t)blockIdx.x * a.n_split * 2 * DSP_BN * D;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.n_split; ++p) {
    const float* q = pw + (size_t)p * 2 * DSP_BN * D;
    sk += *reinterpret_cast<const f32x4*>(q + (size_t)kl * D + d);
    sv += *reinterpret_cast<const f32x4*>(q + (size_t)(DSP_BN + kl) * D + d);
  }
  const size_t o = ((size_t)bh * a.Nkv + key) * D + d;
  *reinterpret_cast<u32x2*>((uint16_t*)a.dk + o) =
      (u32x2){DT::pack2(sk[0] * a.sm_scale, sk[1] * a.sm_scale), DT::pack2(sk[2] * a.sm_scale, sk[3] * a.sm_scale)};
  *reinterpret_cast<u32x2*>((uint16_t*)a.dv + o) = (u32x2){DT::pack2(sv[0], sv[1]), DT::pack2(sv[2], sv[3])};
}

// ------------------------------------------------------------------ dispatch
template <class DT, int D, bool CAUSAL, int PQ, int IN>
struct DqK {
  static void run(dim3 g, const BwdArgs& a, hipStream_t st) {
    if (a.k_mean) hipLaunchKernelGGL((dq_kernel<DT, D, CAUSAL, PQ, IN, true>), g, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((dq_kernel<DT, D, CAUSAL, PQ, IN, false>), g, dim3(256), 0, st, a);
  }
};
template <class DT, int D, bool CAUSAL, int PQ, int IN>
struct DkvK {
  static void run(dim3 g, const BwdArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((dkdv_sp_kernel<DT, D, CAUSAL, PQ, IN>), g, dim3(256), 0, st, a);
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
  a.k_mean = in.k_mean;
  a.sm_scale = sm_scale;
  a.c = sm_scale * LOG2E;
  return a;
}

hipError_t launch_bwd_dq(const Shape& s, const Inputs& in, const void* dout, const float* lse,
                         float* delta, const void* o_hp, float sm_scale, bool causal, int pfmt,
                         void* dq, float* p_amax, hipStream_t st) {
  BwdArgs a = make_args(s, in, dout, lse, delta, sm_scale);
  a.dq = dq;
  a.p_amax = p_amax;
  if (o_hp) {
    a.o_hp = o_hp;
    a.delta_out = delta;
  }
  dim3 grid(((s.Nq + DQ_BM - 1) / DQ_BM) * s.B * s.H);
  return pick_all<DqK>(s, grid, a, causal, pfmt, in.mode, st);
}

size_t dkdv_part_bytes(const Shape& s) {
  const long long units = (long long)((s.Nkv + DSP_BN - 1) / DSP_BN) * s.B * s.H;
  const long long slots = units * DKDV_MAX_SPLIT < DKDV_PART_SLOTS ? units * DKDV_MAX_SPLIT : DKDV_PART_SLOTS;
  return (size_t)slots * 2 * DSP_BN * s.D * sizeof(float);
}

// Tail split: with U key blocks on C compute units, the last rem = U mod C
// blocks would run in a round of their own, mostly or partly idle.  They are
// cut into k query ranges each (2 <= k <= DKDV_MAX_SPLIT), whose partial sums
// a merge kernel adds up, with the k whose ceil(rem k / C) rounds of 1/k of
// a block finish first (the smaller k on a tie): 96 leftover blocks of 256
// take k = 2 (half a round), 192 take k = 4 (three quarter rounds).  Causal
// launches already order their blocks longest first and are left whole.
static void plan_dkdv(const Shape& s, bool causal, int cus, BwdArgs* a) {
  const int nkb = (s.Nkv + DSP_BN - 1) / DSP_BN;
  const int units = nkb * s.B * s.H;
  const int nqb = (s.Nq + DSP_BQ - 1) / DSP_BQ;
  a->n_whole = units;
  a->n_split = 1;
  if (causal || cus <= 0 || !a->dkdv_part) return;
  const int rem = units % cus;
  if (rem == 0) return;
  int best = 1, best_rounds = 1;   // rounds of 1/best of a block: compare rounds / k across k
  for (int k = 2; k <= DKDV_MAX_SPLIT && k <= nqb; ++k) {
    if ((long long)rem * k > DKDV_PART_SLOTS) break;
    const int rounds = (rem * k + cus - 1) / cus;
    if (rounds * best < best_rounds * k) {   // rounds / k < best_rounds / best
      best = k;
      best_rounds = rounds;
    }
  }
  if (best < 2) return;
  a->n_whole = units - rem;
  a->n_split = best;
}

template <class DT, int D>
static void launch_merge(const BwdArgs& a, int nkb, int nblocks, hipStream_t st) {
  dim3 grid((unsigned)nblocks, (unsigned)((DSP_BN * D / 4 + 255) / 256));
  hipLaunchKernelGGL((dkdv_merge_kernel<DT, D>), grid, dim3(256), 0, st, a, nkb);
}

hipError_t launch_bwd_dkdv(const Shape& s, const Inputs& in, const void* dout, const float* lse,
                           const float* delta, const float* p_amax, float sm_scale, bool causal,
                           int pfmt, void* dk, void* dv, float* part_ws, hipStream_t st) {
  BwdArgs a = make_args(s, in, dout, lse, delta, sm_scale);
  a.p_amax_in = p_amax;
  a.dk = dk;
  a.dv = dv;
  a.dkdv_part = part_ws;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  plan_dkdv(s, causal, cus, &a);
  const int nkb = (s.Nkv + DSP_BN - 1) / DSP_BN;
  const int units = nkb * s.B * s.H;
  const int split_blocks = units - a.n_whole;
  dim3 grid((unsigned)(a.n_whole + split_blocks * a.n_split));
  hipError_t e = pick_all<DkvK>(s, grid, a, causal, pfmt, in.mode, st);
  if (e != hipSuccess || split_blocks == 0) return e;
  if (s.dtype == 0) {
    if (s.D == 128) launch_merge<BF16, 128>(a, nkb, split_blocks, st);
    else launch_merge<BF16, 64>(a, nkb, split_blocks, st);
  } else {
    if (s.D == 128) launch_merge<FP16, 128>(a, nkb, split_blocks, st);
    else launch_merge<FP16, 64>(a, nkb, split_blocks, st);
  }
  return hipGetLastError();
}

}  // namespace qat
