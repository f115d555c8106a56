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
//    dQ^T = K^T dS^T reads K^T through ds_read_b64_tr_b16.  A lane holds a
//    query row's 64-key group, so this kernel can record the P-quant absmax
//    of every (row, group) for the dK/dV kernel (when that record is kept).
//  * dK/dV kernel: a workgroup of 8 waves owns 128 keys (two P groups);
//    each wave keeps its 32 keys' K^T (and V^T) in registers and computes
//    S = Q K^T (and dP = dO V^T) with one lane per key, so P^ and dS are
//    already the operands of dV^T = dO^T P^ and dK^T = Q^T dS (Q and dO
//    tiles go through LDS, read row-major for S/dP and transposed for dV/dK).
//    Half the waves accumulate dV, half dK, so each holds one accumulator.
//    A query's 64-key P group spans the 32 keys of two waves: the kernel
//    reads the dQ kernel's absmax record, or (AMX, when the record would be
//    too large to keep) each wave reduces its half over lanes, the two
//    exchange the halves through LDS across the workgroup barrier, and the
//    P^ and dV of a block follow one iteration later.
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

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
  const uint8_t* q8;      // IN_QKS: e4m3 code bytes of Q and K (S on the fp8 MFMA)
  const uint8_t* k8;
  const void* dout;
  const float* lse;
  const float* delta;
  float* p_amax;        // dQ: P-quant absmax per (row, 64-key group) [BH][NG][Nq], or null
  const float* p_amax_in;   // dK/dV: the same, or null (formed in the dK/dV kernel)
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


// Power-of-two scale for a row of fp16 MFMA operands whose absolute maximum
// is m: x * up lands the largest at [2^14, 2^15) (every fp16 keeps 11
// significant bits down to 2^-10 of that maximum), and down = 1 / up undoes
// it on the fp32 product.  Both exact; m == 0 gives up = down = 1.
struct Pow2Scale { float up, down; };
__device__ __forceinline__ Pow2Scale pow2_scale(float m) {
  int e = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xFF) - 127;   // exponent of m (m >= 0)
  e = m > 0.0f ? min(max(e, -100), 100) : 14;
  Pow2Scale r;
  r.up = __builtin_bit_cast(float, (uint32_t)(127 + 14 - e) << 23);
  r.down = __builtin_bit_cast(float, (uint32_t)(127 - 14 + e) << 23);
  return r;
}

constexpr int DQ_BM = 128;
constexpr int DQ_BN = 64;
// Waves of a dQ workgroup (32 query rows each).  Eight (256 rows, one
// workgroup per CU) load each K/V tile once for twice the rows: the DiT image
// dQ 0.397 -> 0.376 ms.  Causal launches keep four (finer blocks balance the
// unequal row lengths better: causal LM dQ 0.237 -> 0.247 ms with eight),
// and so does fp8 V (its workgroups see few key tiles, 8 at the
// cross-attention shape, and two per CU overlap one's prologue with the
// other's tiles: dQ 0.213 -> 0.234 ms with eight).  Per-token codes need
// eight (LDS for the K code tiles; see dq_kernel).
constexpr int dq_waves(int in, bool causal) {
  return in == IN_QKS ? 8 : (causal || in == IN_VFP8 ? 4 : 8);
}

// SMK: K smoothing, dQ += sm_scale rowsum(dS) k_mean (a separate instance, so
// that the plain kernel is not burdened with the extra row sum)
// IN_QKS: S on the fp8 MFMA from the e4m3 code bytes, whose K tiles take
// LDS beside the 16-bit K tiles of dQ; the workgroup is then eight waves (256
// rows, one per CU), since two four-wave workgroups would not fit one CU's LDS.
template <class DT, int D, bool CAUSAL, int PQ, int IN, bool SMK>
__global__ __launch_bounds__(dq_waves(IN, CAUSAL) * 64, dq_waves(IN, CAUSAL) == 8 ? 1 : 2) void dq_kernel(BwdArgs a) {
  constexpr bool VFP8 = IN == IN_VFP8;
  constexpr bool QKS = IN == IN_QKS;
  constexpr int TILE = DQ_BN * D * 2;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  constexpr int NW = dq_waves(IN, CAUSAL);   // waves
  constexpr int BM = NW * 32;        // query rows per workgroup
  __shared__ __attribute__((aligned(16))) char smem[2][2][TILE];   // [buffer][K, V]
  __shared__ __attribute__((aligned(16))) float ks_s[2][DQ_BN];     // IN_QKS: key scales
  __shared__ __attribute__((aligned(16))) char k8_s[QKS ? 2 : 1][QKS ? DQ_BN * D : 16];   // IN_QKS: K codes
  // IN_VFP8: the next tile's V codes, copied HBM -> LDS by DMA
  constexpr int VC_BYTES = VFP8 ? DQ_BN * D : 16;
  constexpr int VC_KIB = DQ_BN * D / 1024;                    // KiB of a code tile
  constexpr int VCW = VC_KIB < dq_waves(IN, CAUSAL) ? VC_KIB : dq_waves(IN, CAUSAL);   // waves copying it
  constexpr int VC_PER_THREAD = VC_KIB / VCW;                 // 16-byte chunks per thread of those waves
  __shared__ __attribute__((aligned(16))) char vc_s[VC_BYTES];

  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int ntq = (a.Nq + BM - 1) / BM;
  int bh, rank;   // causal: the longest rows (last blocks) first
  work_unit(blockIdx.x, gridDim.x, ntq, CAUSAL, &bh, &rank);
  const int qb = (CAUSAL ? ntq - 1 - rank : rank) * BM;
  const int q0 = qb + w * 32;
  const int qi = q0 + l32;
  const int lane_g4 = 4 * g, lane_dq = 4 * g - l32;   // mask terms (key - kv0 - c, key - qi + q0 - kv0 - c)
  const int Nq = a.Nq, Nkv = a.Nkv;
  const uint16_t* qp = (const uint16_t*)a.q + (size_t)bh * Nq * D;
  const uint16_t* dop = (const uint16_t*)a.dout + (size_t)bh * Nq * D;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)bh * Nkv * D;
  const uint8_t* vp = (const uint8_t*)a.v + (size_t)bh * Nkv * D * (VFP8 ? 1 : 2);
  const float* vsc = VFP8 ? a.v_scale + (size_t)bh * D : nullptr;

  // Q^T (B operand of S^T = K Q^T): 16-bit values, or with per-token codes
  // the e4m3 bytes d = 64 ks + 32 g + 0..31 of the row in two 16-byte halves
  s16x8 qf[QKS ? 2 * (D / 64) : NKS], dof[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const bool ok = qi < Nq;
    if constexpr (QKS) {
      if (ks < 2 * (D / 64))
        qf[ks] = ok ? *reinterpret_cast<const s16x8*>(a.q8 + ((size_t)bh * Nq + qi) * D + 64 * (ks >> 1) + 32 * g +
                                                      16 * (ks & 1))
                    : (s16x8){};
    } else {
      qf[ks] = ok ? *reinterpret_cast<const s16x8*>(qp + (size_t)qi * D + 16 * ks + 8 * g) : (s16x8){};
    }
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
  // fp8 V: dP = (dO * v_scale) code^T on the fp16 MFMA.  The per-channel V
  // scale moves onto dO, the row is scaled by a power of two (its largest
  // product near 2^14) and rounded to fp16 (11 significant bits), and the
  // codes are exact fp16 values; dp_down undoes the row scale on the result.
  float dp_down = 1.0f;
  if constexpr (VFP8) {
    float prod[NKS][8];
    float mx = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(vsc + 16 * ks + 8 * g);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(vsc + 16 * ks + 8 * g + 4);
      const float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      const u32x4 wd = __builtin_bit_cast(u32x4, dof[ks]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        prod[ks][e] = BF16::to_f32((uint16_t)(wd[e >> 1] >> (16 * (e & 1)))) * sc[e];
        mx = fmaxf(mx, fabsf(prod[ks][e]));
      }
    }
    const Pow2Scale ps = pow2_scale(max_xor32(mx));
    dp_down = ps.down;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 ws;
#pragma unroll
      for (int h = 0; h < 4; ++h) ws[h] = FP16::pack2(prod[ks][2 * h] * ps.up, prod[ks][2 * h + 1] * ps.up);
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
  // lane offsets of the K^T reads of k-step 0 per column block (a k-step adds 16 rows: an immediate offset)
  int kt_lane[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h) kt_lane[db][h] = tr8_off<D>(8 * h, db * 32, lane);
  constexpr bool smooth = SMK;
  float ds_rowsum = 0.0f;   // this lane's half of sum_j dS_ij (K smoothing)

  // K tiles (and V, unless fp8) go HBM -> LDS directly, double-buffered.  fp8
  // V codes go HBM -> LDS by DMA too, into one 8-bit tile in plain row order:
  // chunk u of a thread of the VCW copying waves is the 16 bytes at
  // P = (VCW u + wave) KiB + 16 lane, and the same thread decodes exactly
  // those bytes after its own copies
  // completed, so the decode needs no barrier.  Key scales take a register
  // detour.
  float ksreg = 0.0f;
  TileCopy<D, DQ_BN, NW> copy;
  copy.init(w, lane);
  constexpr int K8W = DQ_BN * D / 1024 < NW ? DQ_BN * D / 1024 : NW;   // waves copying the K code tile
  CodeCopy<D, DQ_BN, K8W, true> kcopy8;
  if constexpr (QKS) kcopy8.init(w % K8W, lane);
  auto issue_tile = [&](int t, int buf) {
    copy.issue(smem[buf][0], kp, t * DQ_BN, Nkv);
    if constexpr (QKS) {
      if (w < K8W) kcopy8.issue(k8_s[QKS ? buf : 0], a.k8 + (size_t)bh * Nkv * D, t * DQ_BN, Nkv);
    }
    if constexpr (VFP8) {
#pragma unroll
      for (int u = 0; u < VC_PER_THREAD; ++u) {
        if (w >= VCW) break;
        const int blk = u * VCW + w, P = blk * 1024 + lane * 16;
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
    if constexpr (VFP8) {   // the code values themselves as fp16 (exact: an e5m2 code is an fp16's high byte)
#pragma unroll
      for (int u = 0; u < VC_PER_THREAD; ++u) {
        if (w >= VCW) break;
        const int P = (u * VCW + w) * 1024 + lane * 16, row = P / D, c0 = P % D;
        const u32x4 codes = *reinterpret_cast<const u32x4*>(vc_s + P);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)   // 8 codes -> one 16-byte chunk of the fp16 tile
          *reinterpret_cast<s16x8*>(smem[buf][1] + tile_off<D>(row, c0 / 8 + h2)) =
              e5m2x8_to_f16((int)codes[2 * h2], (int)codes[2 * h2 + 1]);
      }
    }
    if constexpr (QKS) {
      if (tid < DQ_BN) ks_s[buf][tid] = ksreg;
    }
  };

  const int kv_end = CAUSAL ? min(Nkv, qb + BM) : Nkv;
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
    if constexpr (!QKS) {
      // S and dP as one stream of single-fragment steps (step f: key block
      // f / 2NKS, k-step (f % 2NKS) / 2, K for S or V for dP), each fragment
      // read DQ_AHEAD steps before its MFMA (fenced)
      constexpr int NSD = 4 * NKS, DQ_AHEAD = 2;
      auto fetch_sd = [&](int f) __attribute__((always_inline)) {
        return lds_row8<D>((f & 1) ? Vt : Kt, (f / (2 * NKS)) * 32 + l32, 2 * ((f % (2 * NKS)) >> 1) + g);
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = (f32x16){};
        dp[kb] = (f32x16){};
      }
      s16x8 ring[DQ_AHEAD];
#pragma unroll
      for (int f = 0; f < DQ_AHEAD; ++f) {
        ring[f] = fetch_sd(f);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int f = 0; f < NSD; ++f) {
        const s16x8 cur = ring[f % DQ_AHEAD];
        if (f + DQ_AHEAD < NSD) ring[f % DQ_AHEAD] = fetch_sd(f + DQ_AHEAD);
        __builtin_amdgcn_sched_barrier(0);
        const int kb = f / (2 * NKS), ks = (f % (2 * NKS)) >> 1;
        if (f & 1) {
          if constexpr (VFP8) dp[kb] = FP16::mfma(cur, dof[ks], dp[kb]);
          else dp[kb] = DT::mfma(cur, dof[ks], dp[kb]);
        } else {
          s[kb] = DT::mfma(cur, qf[ks], s[kb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {   // per-token codes: S from the K codes against the Q codes, 64 d per MFMA
      const char* K8t = k8_s[QKS ? buf : 0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = (f32x16){};
        dp[kb] = (f32x16){};
#pragma unroll
        for (int ks = 0; ks < D / 64; ++ks)
          s[kb] = mfma_e4m3(lds_f8row<D>(K8t, kb * 32 + l32, 4 * ks + 2 * g),
                            lds_f8row<D>(K8t, kb * 32 + l32, 4 * ks + 2 * g + 1), qf[2 * ks], qf[2 * ks + 1], s[kb]);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) dp[kb] = DT::mfma(lds_row8<D>(Vt, kb * 32 + l32, 2 * ks + g), dof[ks], dp[kb]);
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
    if (PQ >= 0 && a.p_amax) {   // the P-quant absmax of the row's group, for the dK/dV kernel
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) pmax = fmaxf(pmax, p[kb][r]);
      pmax = max_xor32(pmax);
      if (g == 0 && qi < Nq) a.p_amax[((size_t)bh * a.NG + t) * Nq + qi] = pmax;
    }
    if constexpr (smooth) {   // K smoothing: sum_j dS_ij (fp32, before any key scale)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) ds_rowsum += p[kb][r] * __builtin_fmaf(dp[kb][r], dp_down, -Di);
    }
    // dQ^T += K^T dS^T, the K^T fragments read two steps ahead
    auto fetch_kt = [&](int f) __attribute__((always_inline)) {
      const char* kk16 = Kt + (f / NDB) * 16 * D * 2;
      return lds_tr8_at(kk16 + kt_lane[f % NDB][0], kk16 + kt_lane[f % NDB][1]);
    };
    s16x8 kr[2];
    kr[0] = fetch_kt(0);
    kr[1] = fetch_kt(1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kb = kk >> 1, h = kk & 1;
      uint32_t w4[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r0 = 8 * h + 2 * jj;
        float d0, d1;
        if constexpr (VFP8) {
          d0 = p[kb][r0] * __builtin_fmaf(dp[kb][r0], dp_down, -Di);
          d1 = p[kb][r0 + 1] * __builtin_fmaf(dp[kb][r0 + 1], dp_down, -Di);
        } else {
          d0 = p[kb][r0] * (dp[kb][r0] - Di);
          d1 = p[kb][r0 + 1] * (dp[kb][r0 + 1] - Di);
        }
        if constexpr (QKS) {   // dQ = sm_scale sum_j dS_ij s_k[j] code_k[j]
          const f32x2 k2 = *reinterpret_cast<const f32x2*>(&ks_s[buf][kb * 32 + 8 * (r0 >> 2) + 4 * g + (r0 & 3)]);
          d0 *= k2[0];
          d1 *= k2[1];
        }
        w4[jj] = DT::pack2(d0, d1);
      }
      const s16x8 ds_op = __builtin_bit_cast(s16x8, (u32x4){w4[0], w4[1], w4[2], w4[3]});
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int f = kk * NDB + db;
        const s16x8 cur = kr[f & 1];
        if (f + 2 < 4 * NDB) kr[f & 1] = fetch_kt(f + 2);
        __builtin_amdgcn_sched_barrier(0);
        dq_acc[db] = DT::mfma(cur, ds_op, dq_acc[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    }
    wait_vmem();
    if (t + 1 < ntiles) finish_tile(buf ^ 1);
    __syncthreads();
  }
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
// dK/dV in split roles: two waves per SIMD.
//
// A workgroup of eight waves owns 128 keys and walks the query range in
// blocks of 32.  Waves w < 4 ("P waves") and w + 4 ("dS waves") share a SIMD
// and the same 32 keys (lane = key, so every product below is the operand
// layout of the next one):
//   P wave:  S = Q K^T, P = exp2(S c - M) (masks), P^ = FQ(P) with the
//            (query, 64-key group) scales, dV^T += dO^T P^; it hands the
//            high-precision P to its partner through LDS;
//   dS wave: dP = dO V^T, dS = P o (dP - Delta) with that P,
//            dK^T += Q^T dS.
// Each wave holds one accumulator (dV or dK, 64 registers at D = 128) and one
// of the K^T / V^T operands, which fits the 256 registers of two waves per
// SIMD: while one wave waits on an MFMA or an LDS read the other issues, and
// the two waves' vector work runs under each other's matrix work.
// The absmax of a (query, 64-key group) needs the keys of two P waves (kw,
// kw ^ 1).  With the dQ kernel's record, wave 1 stages its scale pairs with
// the block.  Without it (AMX), each P wave publishes its 32-key maximum
// per query of block i, and after the barrier both form the group's scales
// and quantize P(i), read back from LDS.
// Iteration i (one workgroup barrier at its end):
//   P wave:  S(i+1) MFMAs; P(i) to LDS; P^ and dV MFMAs of block i, or
//            (AMX) the 32-key maxima of block i, and scales, P^ and dV
//            MFMAs of block i-1;
//   dS wave: dP(i) MFMAs; vector work of block i-1 (P(i-1) from LDS, written
//            in iteration i-1); dK MFMAs of block i-1;
//   all:     block i+2 (loaded in iteration i-1) written to LDS slot
//            (i+2) % 4 in the second half of the iteration, then block i+3
//            loaded into the staging registers.
// LDS slot reads in iteration i touch blocks i-1 .. i+1 only, so the slot
// written in iteration i was last read in iteration i-1, before the barrier;
// the P buffer and the maxima of parity i&1 are rewritten in iteration i+2,
// after the barrier that ends their reads in iteration i+1.
// Maximum over aligned groups of N consecutive lanes (N = 8 or 16) by DPP:
// the partner exchanges lane ^ 1, lane ^ 2, the mirror within eight lanes and
// (N = 16) the mirror within sixteen leave every lane with its group's max.
template <int N>
__device__ __forceinline__ float row_max_dpp(float x) {
  static_assert(N == 8 || N == 16, "group");
  auto step = [](float v, auto CTRL) {
    constexpr int c = decltype(CTRL)::value;
    const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), c, 0xF, 0xF, false);
    return fmaxf(v, __builtin_bit_cast(float, o));
  };
  x = step(x, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
  x = step(x, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
  x = step(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
  if constexpr (N == 16) x = step(x, std::integral_constant<int, 0x140>{});   // row_mirror
  return x;
}

// Maximum over the 32 lanes of each lane half, for each of the 16 registers
// of x (probabilities: >= 0 and never NaN, so the unsigned order of their
// bit patterns is their order), by a transposing reduction that halves the
// register count at every step: v_permlane16_swap pairs the two 16-lane rows
// of a half (lane ^ 16), then DPP pairs lane ^ 8 (row rotation by 8),
// l <-> 7 - l within eight lanes (half-row mirror), lane ^ 2 and lane ^ 1
// (quad permutations).  At each step a lane keeps the register of the pair
// that its lane bit selects, combined with the same register of its
// partner, whose bit is the other one.  Lane l ends with the maximum of
// register (l >> 1) & 15 of its half.
__device__ __forceinline__ float half_max16(const f32x16& x, int lane) {
  uint32_t t[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {   // bit 4: lanes < 16 of a half keep x[k], the others x[k + 8]
    // (elements copied out first: a bit cast of a vector element expression
    // reads the vector's first element in this compiler)
    const float lo = x[k], hi = x[k + 8];
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, lo),
                                                    __builtin_bit_cast(uint32_t, hi), false, false);
    t[k] = max((uint32_t)r[0], (uint32_t)r[1]);
  }
  auto pair = [](uint32_t lo, uint32_t hi, bool bit, auto CTRL) {
    constexpr int c = decltype(CTRL)::value;
    const uint32_t ml = max(lo, (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, c, 0xF, 0xF, true));
    const uint32_t mh = max(hi, (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, c, 0xF, 0xF, true));
    return bit ? mh : ml;
  };
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
  uint32_t u[4], v[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] = pair(t[k], t[k + 4], b3, std::integral_constant<int, 0x128>{});   // row_ror:8
#pragma unroll
  for (int k = 0; k < 2; ++k) v[k] = pair(u[k], u[k + 2], b2, std::integral_constant<int, 0x141>{});   // row_half_mirror
  const uint32_t m = pair(v[0], v[1], b1, std::integral_constant<int, 0x4E>{});                        // quad_perm [2,3,0,1]
  return __builtin_bit_cast(float, max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, true)));
}

constexpr int DPR_BN = 128;    // keys per workgroup
constexpr int DPR_BQ = 32;     // queries per block
constexpr int DPR_SLOTS = 4;   // LDS slots of Q/dO blocks

// AMX (P quant only): the P waves form the group absmax themselves (above);
// otherwise they read the absmax the dQ kernel recorded per (query, group).
// Lanes of a 32-query score register with query offset c that the causal
// mask hides in a wave's diagonal block: lane l (key l % 32 of the wave's
// 32, query 4 (l / 32) + c of the block) when its key follows the query.
constexpr uint64_t diag_lane_mask(int c) {
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l)
    if ((l & 31) - 4 * (l >> 5) > c) m |= 1ull << l;
  return m;
}

template <class DT, int D, bool CAUSAL, int PQ, int IN, bool AMX>
__global__ __launch_bounds__(512, 1) void dkdv_pair_kernel(BwdArgs a) {
  static_assert(!AMX || PQ >= 0, "in-kernel absmax is for P quant");
  constexpr bool VFP8 = IN == IN_VFP8;
  constexpr bool QKS = IN == IN_QKS;
  constexpr int TILE = DPR_BQ * D * 2;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  constexpr int FQF = PQ >= 0 ? PQ : 0;
  constexpr int NGW = DPR_BN / 64;          // 64-key P groups of the workgroup
  constexpr bool SIDE = PQ >= 0 && !AMX;    // P-quant absmax read from the dQ kernel's record
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int CHUNKS = DPR_BQ * CPR;      // chunks per tensor and block
  constexpr int NCH = 2 * CHUNKS / 512;     // staged chunks per thread (Q and dO together)
  constexpr int NGRP = 8;                   // fenced groups per iteration
  constexpr int AHEAD = 2;                  // MFMA steps whose LDS operand is in flight
  static_assert(NCH >= 1 && 2 * CHUNKS % 512 == 0, "shape");
  __shared__ __attribute__((aligned(16))) char q_s[DPR_SLOTS][TILE];
  // IN_QKS: the block's e4m3 Q code bytes (the P wave's fp8 MFMA operand of
  // S), converted from the staged Q code values as they are written
  __shared__ __attribute__((aligned(16))) char q8_s[QKS ? DPR_SLOTS : 1][QKS ? DPR_BQ * D : 16];
  __shared__ __attribute__((aligned(16))) char do_s[DPR_SLOTS][TILE];
  __shared__ __attribute__((aligned(16))) float m_s[DPR_SLOTS][DPR_BQ];
  __shared__ __attribute__((aligned(16))) float d_s[DPR_SLOTS][DPR_BQ];
  __shared__ __attribute__((aligned(16))) float sq_s[QKS ? DPR_SLOTS : 1][DPR_BQ];
  __shared__ __attribute__((aligned(16))) float cq_s[QKS ? DPR_SLOTS : 1][DPR_BQ];   // c * s_q (exponent scale)
  // rows of +inf read as M by key lanes past Nkv, so that their p is 0 (and
  // stays out of the P-quant absmax)
  __shared__ __attribute__((aligned(16))) float minf_s[DPR_SLOTS][DPR_BQ];
  // SIDE: the P-quant scale pairs of the workgroup's two 64-key groups per
  // staged block.  AMX: each P wave's maximum over its 32 keys per query
  // ([block parity][wave][query]), and the scale pair of the wave's 64-key
  // group that the wave forms from its own and its partner's maxima.
  __shared__ __attribute__((aligned(16))) float qs_s[SIDE ? DPR_SLOTS : 1][NGW][DPR_BQ];
  __shared__ __attribute__((aligned(16))) float qr_s[SIDE ? DPR_SLOTS : 1][NGW][DPR_BQ];
  __shared__ __attribute__((aligned(16))) float pm_s[AMX ? 2 : 1][4][DPR_BQ];
  __shared__ __attribute__((aligned(16))) float qsw_s[AMX ? 4 : 1][DPR_BQ];
  __shared__ __attribute__((aligned(16))) float qrw_s[AMX ? 4 : 1][DPR_BQ];
  __shared__ __attribute__((aligned(16))) f32x4 p_s[2][4][4][64];   // [block parity][key quarter][reg quarter][lane]
  // fp8 V: dO * v_scale rows scaled by a power of two and rounded to fp16 (the
  // dS wave's dP operand; dV keeps the plain dO tile), and each row's inverse
  // scale
  __shared__ __attribute__((aligned(16))) char dos_s[VFP8 ? DPR_SLOTS : 1][VFP8 ? TILE : 16];
  __shared__ __attribute__((aligned(16))) float es_s[VFP8 ? DPR_SLOTS : 1][DPR_BQ];
  __shared__ __attribute__((aligned(16))) float vs_s[VFP8 ? D : 1];

  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int kw = w & 3;   // this wave's 32 keys within the workgroup
  const int nkb = (a.Nkv + DPR_BN - 1) / DPR_BN;
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
  const int k0 = (unit % nkb) * DPR_BN;
  const int k0w = k0 + kw * 32;
  const int kj = k0w + l32;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const int lgrp = kw >> 1;               // this wave's 64-key group within the workgroup
  const uint16_t* qp = (const uint16_t*)a.q + (size_t)bh * Nq * D;
  const uint16_t* dop = (const uint16_t*)a.dout + (size_t)bh * Nq * D;

  const int qb_first = CAUSAL ? k0 / DPR_BQ : 0;
  const int nqb = (Nq + DPR_BQ - 1) / DPR_BQ;
  const int NB_all = nqb > qb_first ? nqb - qb_first : 0;
  const int qb_begin = qb_first + NB_all * part / nparts;
  const int NB = qb_first + NB_all * (part + 1) / nparts - qb_begin;   // query blocks of this workgroup
  const bool wave_live = k0w < Nkv;
  auto qstart = [&](int b) { return (qb_begin + b) * DPR_BQ; };
  // some (query, key) pair of block b and this wave's keys is unmasked
  auto active = [&](int b) { return wave_live && (!CAUSAL || qstart(b) + DPR_BQ - 1 >= k0w); };

  // ---- staging of a block, loaded into registers one iteration before it
  // is written to LDS.  Q and dO tiles: thread tid holds chunks tid + 512 j
  // (the Q tile, then the dO tile), read with buffer loads whose range is the
  // head's Nq rows, so rows past Nq read as zeros and each address is a fixed
  // per-thread offset plus the block's uniform row offset.  Per-query
  // vectors, one wave each so that control flow stays uniform: wave 0 LSE
  // (lanes 0-31) and Delta (lanes 32-63), wave 1 (SIDE) the P-quant absmax
  // of the workgroup's two 64-key groups (group lane / 32), wave 2 the
  // per-token query scale (per-token codes only).
  u32x4 stg[NCH];
  float stv = 0.0f;
  const __amdgpu_buffer_rsrc_t rsrc_q = __builtin_amdgcn_make_buffer_rsrc((void*)qp, 0, Nq * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_do = __builtin_amdgcn_make_buffer_rsrc((void*)dop, 0, Nq * D * 2, 0x00020000);
  // tensor of chunk j: with D = 128 chunk j of every thread is tensor j; with
  // D = 64 waves 0-3 hold the Q tile and waves 4-7 the dO tile
  auto st_tensor = [&](int j) { return CHUNKS == 512 ? j == 1 : w >= 4; };
  auto st_within = [&](int j) { return (tid + 512 * j) % CHUNKS; };
  if constexpr (VFP8) {   // fp8 V: the head's v_scale in LDS (read where the dO copy is scaled)
    if (tid < D) vs_s[tid] = a.v_scale[(size_t)bh * D + tid];
    __syncthreads();
  }
  const float* v_src = nullptr;   // waves 0-2: this lane's vector source (per head), else unused
  bool v_live = false;            // the lane's vector entry exists (wave 1: group inside the keys)
  if (w == 0) {
    v_src = (lane < 32 ? a.lse : a.delta) + (size_t)bh * Nq;
    v_live = true;
  } else if (w == 1 && SIDE) {
    const int gq = k0 / 64 + g;
    v_live = g < NGW && gq < a.NG;
    v_src = a.p_amax_in + ((size_t)bh * a.NG + (v_live ? gq : 0)) * Nq;
  } else if (w == 2 && QKS && lane < 32) {
    v_src = a.q_scale + (size_t)bh * Nq;
    v_live = true;
  }
  auto load_stage = [&](int b) __attribute__((always_inline)) {
    const int q0 = qstart(b);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int within = st_within(j), row = within / CPR, ch = within % CPR;
      stg[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            st_tensor(j) ? rsrc_do : rsrc_q, row * D * 2 + ch * 16, q0 * D * 2, 0));
    }
    if (v_live) stv = v_src[min(q0 + l32, Nq - 1)];
  };
  // chunks [jlo, jhi) of the staged block (slot: compile-time b % DPR_SLOTS,
  // so the LDS addresses fold into offsets)
  auto write_tiles = [&](auto SLOTc, int jlo, int jhi) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOTc)::value;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (j < jlo || j >= jhi) continue;
      const int within = st_within(j), row = within / CPR, ch = within % CPR;
      *reinterpret_cast<u32x4*>((st_tensor(j) ? do_s[slot] : q_s[slot]) + tile_off<D>(row, ch)) = stg[j];
      if constexpr (QKS) {   // the chunk's 8 Q code values (exact e4m3 values) as code bytes, for the fp8 S
        if (!st_tensor(j)) {
          float f[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = DT::to_f32((uint16_t)(stg[j][e >> 1] >> (16 * (e & 1))));
          int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
          lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
          int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
          hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
          *reinterpret_cast<u32x2*>(q8_s[QKS ? slot : 0] + f8_off<D>(row, ch >> 1) + 8 * (ch & 1)) =
              (u32x2){(uint32_t)lo, (uint32_t)hi};
        }
      }
      if constexpr (VFP8) {
        if (st_tensor(j)) {   // the row's CPR chunks sit in CPR consecutive lanes
          const f32x4 va = *reinterpret_cast<const f32x4*>(&vs_s[8 * ch]);
          const f32x4 vb = *reinterpret_cast<const f32x4*>(&vs_s[8 * ch + 4]);
          const float vs8[8] = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
          float x[8], m = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[e] = BF16::to_f32((uint16_t)(stg[j][e >> 1] >> (16 * (e & 1)))) * vs8[e];
            m = fmaxf(m, fabsf(x[e]));
          }
          m = row_max_dpp<CPR>(m);
          const Pow2Scale ps = pow2_scale(m);
          u32x4 h;
#pragma unroll
          for (int k2 = 0; k2 < 4; ++k2) h[k2] = FP16::pack2(x[2 * k2] * ps.up, x[2 * k2 + 1] * ps.up);
          *reinterpret_cast<u32x4*>(dos_s[slot] + tile_off<D>(row, ch)) = h;
          if (ch == 0) es_s[slot][row] = ps.down;
        }
      }
    }
  };
  auto write_vec = [&](int b, auto SLOTc) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOTc)::value;
    const float v = stv;
    const bool ok = v_live && qstart(b) + l32 < Nq;
    if (w == 0) {
      // M = +inf for rows past Nq: their p = exp2(S c - M) is exactly 0
      float* dst = lane < 32 ? &m_s[slot][l32] : &d_s[slot][l32];
      *dst = lane < 32 ? (ok ? v * LOG2E : INFINITY) : (ok ? v : 0.0f);
    } else if (w == 1 && SIDE) {
      const FqScale fs = fq_scale<FQF>(ok ? v : 0.0f);
      if (g < NGW) {
        qs_s[SIDE ? slot : 0][g][l32] = fs.s;
        qr_s[SIDE ? slot : 0][g][l32] = fs.r;
      }
    } else if (w == 2 && QKS && lane < 32) {
      sq_s[slot][l32] = ok ? v : 1.0f;
      // a zero scale (all-zero row) is raised to the smallest normal so that
      // a masked score stays -inf after the product
      cq_s[slot][l32] = a.c * fmaxf(ok ? v : 1.0f, 1.17549435e-38f);
    }
  };

  // prologue: the slots the prologue does not fill (2, 3, and 0, 1 when
  // the workgroup has fewer blocks) and the P buffers are zeroed: the first
  // and last iterations' MFMAs read them before or without any block landing
  // there, so their data must be finite; then blocks 0, 1 in LDS and block 2
  // in the staging registers
  {
    const int z0 = min(NB, 2);   // first slot the prologue leaves empty
    constexpr int WPS = TILE / 16;   // 16-byte words per slot
    for (int k = tid; k < 2 * DPR_SLOTS * WPS; k += 512) {
      const int t = k / (DPR_SLOTS * WPS), sl = (k / WPS) % DPR_SLOTS, o = (k % WPS) * 16;
      if (sl >= z0) *reinterpret_cast<u32x4*>((t ? do_s[sl] : q_s[sl]) + o) = (u32x4){0u, 0u, 0u, 0u};
      if constexpr (QKS) {
        if (sl >= z0 && !t && o < DPR_BQ * D) *reinterpret_cast<u32x4*>(q8_s[QKS ? sl : 0] + o) = (u32x4){0u, 0u, 0u, 0u};
      }
      if constexpr (VFP8) {
        if (sl >= z0 && t) *reinterpret_cast<u32x4*>(dos_s[VFP8 ? sl : 0] + o) = (u32x4){0u, 0u, 0u, 0u};
      }
    }
    f32x4* pz = &p_s[0][0][0][0];
    for (int k = tid; k < 2 * 4 * 4 * 64; k += 512) pz[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (AMX && tid < 2 * 4 * DPR_BQ) (&pm_s[0][0][0])[tid] = 0.0f;
    if (tid < DPR_SLOTS * DPR_BQ) (&minf_s[0][0])[tid] = INFINITY;
    if (tid < DPR_BQ) {
      for (int sl = z0; sl < DPR_SLOTS; ++sl) {
        m_s[sl][tid] = 0.0f;
        d_s[sl][tid] = 0.0f;
        if constexpr (SIDE) {
#pragma unroll
          for (int gq = 0; gq < NGW; ++gq) qs_s[SIDE ? sl : 0][gq][tid] = qr_s[SIDE ? sl : 0][gq][tid] = 0.0f;
        }
        if constexpr (QKS) sq_s[sl][tid] = cq_s[sl][tid] = 0.0f;
        if constexpr (VFP8) es_s[VFP8 ? sl : 0][tid] = 0.0f;
      }
    }
  }
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if (NB > 0) { load_stage(0); write_tiles(I0{}, 0, NCH); write_vec(0, I0{}); }
  if (NB > 1) { load_stage(1); write_tiles(I1{}, 0, NCH); write_vec(1, I1{}); }
  if (NB > 2) load_stage(2);

  // one wave role for the whole kernel: R = 0 P wave, R = 1 dS wave
  auto run = [&](auto ROLE) __attribute__((always_inline)) {
    constexpr int R = decltype(ROLE)::value;
    // per-token codes: the P wave forms S on the fp8 MFMA, 64 d per step
    constexpr bool F8S = QKS && R == 0;
    constexpr int NSS = F8S ? 2 * (D / 64) : NKS;   // score steps (fp8: two 16-byte halves per MFMA)
    constexpr int NST = NSS + 2 * NDB;              // MFMA-operand steps per iteration
    constexpr int GMAX = (NSS + 3) / 4 > (2 * NDB + 3) / 4 ? (NSS + 3) / 4 : (2 * NDB + 3) / 4;
    // steps [gb(j), gb(j + 1)) run in fenced group j: the score steps in
    // groups 0-3, the accumulator steps in groups 4-7
    auto gb = [](int j) { return j < 4 ? j * NSS / 4 : NSS + (j - 4) * (2 * NDB) / 4; };
    // K^T (P wave) or V^T (dS wave) of this wave's 32 keys: lane holds key
    // kj, d = 16 ks + 8 g .. +7; fp8 K^T: half h holds the code bytes
    // d = 64 (h / 2) + 32 g + 16 (h % 2) .. +15
    s16x8 kv[NKS];
    {
      const bool ok = kj < Nkv;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        kv[ks] = (s16x8){};
        if (!ok) continue;
        if constexpr (F8S) {
          if (ks < NSS)
            kv[ks] = *reinterpret_cast<const s16x8*>(a.k8 + ((size_t)bh * Nkv + kj) * D + 64 * (ks >> 1) + 32 * g +
                                                     16 * (ks & 1));
        } else if constexpr (R == 0) {
          const uint16_t* kp = (const uint16_t*)a.k + (size_t)bh * Nkv * D;
          kv[ks] = *reinterpret_cast<const s16x8*>(kp + (size_t)kj * D + 16 * ks + 8 * g);
        } else if constexpr (VFP8) {   // the e5m2 codes as fp16 values (exact); v_scale is on dO
          const uint8_t* vp = (const uint8_t*)a.v + (size_t)bh * Nkv * D;
          const u32x2 codes = *reinterpret_cast<const u32x2*>(vp + (size_t)kj * D + 16 * ks + 8 * g);
          kv[ks] = e5m2x8_to_f16((int)codes[0], (int)codes[1]);
        } else {
          const uint16_t* vp = (const uint16_t*)a.v + (size_t)bh * Nkv * D;
          kv[ks] = *reinterpret_cast<const s16x8*>(vp + (size_t)kj * D + 16 * ks + 8 * g);
        }
      }
    }
    // per-key scale in the exponent; raised to the smallest normal (and 1 for
    // absent keys) so that a masked score stays -inf after the product
    const float sk_lane =
        (QKS && R == 0) ? (kj < Nkv ? fmaxf(a.k_scale[(size_t)bh * Nkv + kj], 1.17549435e-38f) : 1.0f) : 1.0f;
    // these loads complete here, so that no wait for them lands inside the
    // loop (where it would also drain the block loads in flight)
    wait_vmem();
    __syncthreads();

    f32x16 acc[NDB];   // dV^T (P wave) or dK^T (dS wave): lane key, registers d
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = (f32x16){};
    // score buffers: P wave S(i) / S(i+1), dS wave dP(i-1) / dP(i), by parity
    f32x16 sb[2] = {(f32x16){}, (f32x16){}};
    uint32_t op[8];   // packed P^ (P wave) or dS (dS wave) of block i-1: query half h = words 4h .. 4h+3
#pragma unroll
    for (int j = 0; j < 8; ++j) op[j] = 0u;
    // per-query vectors of a register quarter, double-buffered by quarter
    // parity: P wave M and c s_q (per-token codes) of block i, P-quant s, r
    // and the quarter's P of block i-1 (from LDS); dS wave Delta, s_q
    // (per-token codes) and the quarter's P of block i-1
    f32x4 v0[2], v1[2], v2[2], v3[2], pq[2];
    // P wave: M rows of this lane's key (+inf rows past Nkv)
    const float* m_lane = kj < Nkv ? &m_s[0][0] : &minf_s[0][0];

    // MFMA step st of iteration i: st < NKS the score k-step st (Q or dO row
    // fragment against the K^T or V^T registers), else the accumulator step
    // (h, db) (transposed dO or Q fragment against the packed operand).
    auto tiles = [&](auto SLOTc, const char*& X, const char*& Y) __attribute__((always_inline)) {
      constexpr int SL = decltype(SLOTc)::value;   // slot of block i
      if constexpr (R == 0) {   // dV of block i - 1 (AMX) or i
        X = F8S ? q8_s[QKS ? (SL + 1) & (DPR_SLOTS - 1) : 0] : q_s[(SL + 1) & (DPR_SLOTS - 1)];
        Y = do_s[AMX ? (SL + DPR_SLOTS - 1) & (DPR_SLOTS - 1) : SL];
      } else {
        X = VFP8 ? dos_s[VFP8 ? SL : 0] : do_s[SL];
        Y = q_s[(SL + DPR_SLOTS - 1) & (DPR_SLOTS - 1)];
      }
    };
    auto fetch = [&](const char* X, const char* Y, int st) __attribute__((always_inline)) {
      if (st < NSS) {
        if constexpr (F8S) return lds_f8row<D>(X, l32, 4 * (st >> 1) + 2 * g + (st & 1));
        else return lds_row8<D>(X, l32, 2 * st + g);
      }
      const int k = st - NSS, h = k / NDB, db = k % NDB;
      return lds_tr8<D>(Y, 16 * h, 32 * db, lane);
    };
    s16x8 qlo8;   // fp8 S: the first half of the Q operand
    auto step = [&](const s16x8& frag, int st, f32x16& SO) __attribute__((always_inline)) {
      if (st < NSS) {
        if (st == 0) SO = (f32x16){};
        if constexpr (F8S) {
          if ((st & 1) == 0) qlo8 = frag;
          else SO = mfma_e4m3(qlo8, frag, kv[st - 1], kv[st], SO);
        } else if constexpr (VFP8 && R == 1) {
          SO = FP16::mfma(frag, kv[st], SO);
        } else {
          SO = DT::mfma(frag, kv[st], SO);
        }
      } else {
        const int k = st - NSS, h = k / NDB, db = k % NDB;
        const s16x8 o = __builtin_bit_cast(s16x8, (u32x4){op[4 * h], op[4 * h + 1], op[4 * h + 2], op[4 * h + 3]});
        acc[db] = DT::mfma(frag, o, acc[db]);
      }
    };
    // ---- vector work of a register quarter u (registers 4u .. 4u+3: queries
    // 8u + 4g + 0..3 of the block), its vectors in buffer u & 1
    auto read_quarter = [&](int u, int slot, int par) __attribute__((always_inline)) {   // dS wave, block i-1
      const int ql = 8 * u + 4 * g, bsel = u & 1;
      v0[bsel] = *reinterpret_cast<const f32x4*>(&d_s[slot][ql]);
      if constexpr (QKS) v1[bsel] = *reinterpret_cast<const f32x4*>(&sq_s[slot][ql]);
      if constexpr (VFP8) v1[bsel] = *reinterpret_cast<const f32x4*>(&es_s[VFP8 ? slot : 0][ql]);
      v2[bsel] = p_s[par][kw][u][lane];   // P of block i-1, written by the P wave
    };
    auto read_m = [&](int u, int slot) __attribute__((always_inline)) {   // P wave, block i
      const int ql = 8 * u + 4 * g, bsel = u & 1;
      v0[bsel] = *reinterpret_cast<const f32x4*>(m_lane + slot * DPR_BQ + ql);
      if constexpr (QKS) v1[bsel] = *reinterpret_cast<const f32x4*>(&cq_s[slot][ql]);
      if constexpr (SIDE) {   // and the staged scale pairs of block i
        v2[bsel] = *reinterpret_cast<const f32x4*>(&qs_s[SIDE ? slot : 0][lgrp][ql]);
        v3[bsel] = *reinterpret_cast<const f32x4*>(&qr_s[SIDE ? slot : 0][lgrp][ql]);
      }
    };
    auto read_pq = [&](int u, int par) __attribute__((always_inline)) {   // P wave, P of block i-1
      pq[u & 1] = p_s[par][kw][u][lane];
    };
    auto read_sc = [&](int u) __attribute__((always_inline)) {   // P wave, scales of block i-1
      const int ql = 8 * u + 4 * g, bsel = u & 1;
      if constexpr (AMX) {
        v2[bsel] = *reinterpret_cast<const f32x4*>(&qsw_s[kw][ql]);
        v3[bsel] = *reinterpret_cast<const f32x4*>(&qrw_s[kw][ql]);
      }
    };
    // P wave: p = exp2(S c - M) in place (S of block i)
    auto form_p = [&](int u, f32x16& S) __attribute__((always_inline)) {
      const int bsel = u & 1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * u + e;
        const float sr = QKS ? S[r] * sk_lane : S[r];
        const float cr = QKS ? v1[bsel][e] : a.c;
        S[r] = fast_exp2(__builtin_fmaf(sr, cr, -v0[bsel][e]));
      }
    };
    // P wave: P of block i to LDS (the dS wave's operand in iteration i+1,
    // and this wave's P^ of block i in iteration i+1)
    auto store_p = [&](int u, const f32x16& S, int par) __attribute__((always_inline)) {
      p_s[par][kw][u][lane] = (f32x4){S[4 * u], S[4 * u + 1], S[4 * u + 2], S[4 * u + 3]};
    };
    // P wave: the 64-key group absmax of block i-1 per query from the two
    // P waves' 32-key maxima, and its scale pair for this wave's quarters
    uint32_t pm_own = 0u, pm_par = 0u;
    auto read_pm = [&](int par) __attribute__((always_inline)) {
      if constexpr (AMX) {
        pm_own = __builtin_bit_cast(uint32_t, pm_s[par][kw][l32]);
        pm_par = __builtin_bit_cast(uint32_t, pm_s[par][kw ^ 1][l32]);
      }
    };
    auto group_scales = [&]() __attribute__((always_inline)) {
      if constexpr (AMX) {
        const FqScale fs = fq_scale<FQF>(__builtin_bit_cast(float, max(pm_own, pm_par)));   // p >= 0
        if (g == 0) {
          qsw_s[kw][l32] = fs.s;
          qrw_s[kw][l32] = fs.r;
        }
        // lane-to-lane through this wave's own LDS words: in order within
        // the wave, kept in order by the compiler
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    };
    // P wave: P^ = FQ(P) per (query, 64-key group) of quarter u, packed, from
    // P of block i-1 read back (AMX) or of block i in registers
    auto quantize = [&](int u, const f32x4& x4) __attribute__((always_inline)) {
      const int bsel = u & 1;
      uint32_t w0, w1;
      if constexpr (PQ >= 0) {
        const FqScale f4[4] = {{v2[bsel][0], v3[bsel][0]}, {v2[bsel][1], v3[bsel][1]},
                               {v2[bsel][2], v3[bsel][2]}, {v2[bsel][3], v3[bsel][3]}};
        const float x[4] = {x4[0], x4[1], x4[2], x4[3]};
        const f32x4 xq = fq_quad<FQF>(x, f4);
        w0 = DT::pack2(xq[0], xq[1]);
        w1 = DT::pack2(xq[2], xq[3]);
      } else {
        w0 = DT::pack2(x4[0], x4[1]);
        w1 = DT::pack2(x4[2], x4[3]);
      }
      op[2 * u] = w0;
      op[2 * u + 1] = w1;
    };
    // P wave: this wave's 32-key maximum per query of block i, for both P
    // waves of the group (p >= 0, masked entries are 0)
    auto publish_max = [&](const f32x16& S, int par) __attribute__((always_inline)) {
      if constexpr (AMX) {
        const float m = half_max16(S, lane);
        const int r = (lane >> 1) & 15;
        pm_s[par][kw][4 * g + 8 * (r >> 2) + (r & 3)] = m;
      }
    };
    // dS wave: dS = P o (dP - Delta) for block i-1
    auto finish_ds = [&](int u, const f32x16& DP) __attribute__((always_inline)) {
      const int bsel = u & 1;
      float dsv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (VFP8) dsv[e] = v2[bsel][e] * __builtin_fmaf(DP[4 * u + e], v1[bsel][e], -v0[bsel][e]);
        else dsv[e] = v2[bsel][e] * (DP[4 * u + e] - v0[bsel][e]);
        if constexpr (QKS) dsv[e] *= v1[bsel][e];   // dK = sm_scale sum_i dS_ij s_q[i] code_q[i]
      }
      op[2 * u] = DT::pack2(dsv[0], dsv[1]);
      op[2 * u + 1] = DT::pack2(dsv[2], dsv[3]);
    };
    // slice j of the vector work, placed after the MFMAs of fenced group j
    // (the accumulator MFMAs of query half h, groups 4 + 2h and 5 + 2h, find
    // their operand words written by then); the vectors of a quarter are read
    // a slice or more before their use
    auto slice = [&](int j, auto SLOTc, f32x16& CUR, int par) __attribute__((always_inline)) {
      constexpr int SL = decltype(SLOTc)::value;
      if constexpr (R == 0) {
        // block i: P to LDS and this wave's maximum (par = i & 1); block i-1:
        // scales, P^ for the dV MFMAs of this iteration (par ^ 1)
        constexpr int slot = SL;
        auto cur4 = [&](int u) {
          return (f32x4){CUR[4 * u], CUR[4 * u + 1], CUR[4 * u + 2], CUR[4 * u + 3]};
        };
        if constexpr (AMX) {
          switch (j) {
            case 0: read_pm(par ^ 1); read_m(0, slot); read_m(1, slot); form_p(0, CUR); break;
            case 1: group_scales(); read_pq(0, par ^ 1); read_pq(1, par ^ 1); form_p(1, CUR);
                    store_p(0, CUR, par); store_p(1, CUR, par); read_m(2, slot); read_m(3, slot); break;
            case 2: read_sc(0); read_sc(1); form_p(2, CUR); break;
            case 3: quantize(0, pq[0]); quantize(1, pq[1]); read_sc(2); read_sc(3); read_pq(2, par ^ 1);
                    read_pq(3, par ^ 1); form_p(3, CUR); store_p(2, CUR, par); store_p(3, CUR, par); break;
            case 4: quantize(2, pq[0]); quantize(3, pq[1]); break;
            case 5: publish_max(CUR, par); break;
            default: break;
          }
        } else {   // block i throughout: P to LDS and P^ in the same iteration
          switch (j) {
            case 0: read_m(0, slot); read_m(1, slot); form_p(0, CUR); break;
            case 1: store_p(0, CUR, par); quantize(0, cur4(0)); form_p(1, CUR); read_m(2, slot); break;
            case 2: store_p(1, CUR, par); quantize(1, cur4(1)); read_m(3, slot); break;
            case 3: form_p(2, CUR); break;
            case 4: store_p(2, CUR, par); quantize(2, cur4(2)); form_p(3, CUR); break;
            case 5: store_p(3, CUR, par); quantize(3, cur4(3)); break;
            default: break;
          }
        }
      } else {
        constexpr int slot = (SL + DPR_SLOTS - 1) & (DPR_SLOTS - 1);   // block i - 1
        switch (j) {
          case 0: read_quarter(0, slot, par); read_quarter(1, slot, par); break;
          case 1: finish_ds(0, CUR); read_quarter(2, slot, par); break;
          case 2: finish_ds(1, CUR); read_quarter(3, slot, par); break;
          case 3: finish_ds(2, CUR); break;
          case 4: finish_ds(3, CUR); break;
          default: break;
        }
      }
    };
    // Masks (P wave, block i).  Query rows past Nq have M = +inf (write_vec),
    // so their p is exactly 0; key lanes past Nkv are left unmasked (their K^T
    // registers are zero), since every MFMA output column belongs to one key
    // and those columns are never stored.  Only the causal diagonal block
    // needs a per-element mask: register r holds query q0 + 4g + c_r,
    // c_r = 8(r/4) + r%4, and lane l the key k0w + l % 32.  With off = q0 -
    // k0w (a multiple of 32, the same for the whole wave) a block before the
    // wave's diagonal (off < 0) has every key past every query, the diagonal
    // block (off = 0) masks the lanes with l % 32 - 4 (l / 32) > c_r, and later
    // blocks mask nothing: so register r's mask over the 64 lanes is one of
    // three wave-uniform 64-bit values, chosen by scalar instructions, and
    // the select takes it as its lane condition (one vector instruction per
    // register).  It runs unconditionally (a branch around it makes the
    // register allocator copy S between the two paths).
    auto mask = [&](int i, f32x16& S) __attribute__((always_inline)) {
      if constexpr (CAUSAL) {
        const int off = qstart(i) - k0w;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint64_t m = off < 0 ? ~0ull : (off == 0 ? diag_lane_mask(8 * (r >> 2) + (r & 3)) : 0ull);
          S[r] = __builtin_amdgcn_inverse_ballot_w64(m) ? -INFINITY : S[r];
        }
      }
    };

    // iteration i; SLOTc = i % DPR_SLOTS at compile time (the loop is
    // unrolled by DPR_SLOTS), so every LDS address is a per-lane register
    // plus an immediate offset
    auto iteration = [&](int i, auto SLOTc) __attribute__((always_inline)) {
      constexpr int SL = decltype(SLOTc)::value;
      constexpr int PAR = SL & 1;
      // P wave: scores S(i+1) into sb[PAR^1], vector work on S(i) in sb[PAR];
      // dS wave: dP(i) into sb[PAR], vector work on dP(i-1) in sb[PAR^1]
      f32x16& SO = R == 0 ? sb[PAR ^ 1] : sb[PAR];
      f32x16& CUR = R == 0 ? sb[PAR] : sb[PAR ^ 1];
      constexpr int pb = R == 0 ? PAR : PAR ^ 1;   // P buffer written (P wave) / read (dS wave)
      // the block of the accumulator MFMAs (i for the P wave without AMX,
      // else i - 1) exists for this wave (else its operand words are zeroed,
      // and the accumulator MFMAs add nothing)
      const bool ok = (R == 0 && !AMX) ? (i < NB && active(i)) : (i >= 1 && active(i - 1));
      const bool stw = i + 2 < NB, stl = i + 3 < NB;
      const char *X, *Y;
      tiles(SLOTc, X, Y);
      if (R == 0) mask(i, CUR);
      // Every iteration runs the same instruction stream: at the edges
      // (before the first block, after the last, blocks outside the causal
      // range of this wave's keys) the MFMAs work on finite stale or zeroed
      // LDS data whose results are never used, or on zero operands, so the
      // accumulators need no branches (which would make the register
      // allocator copy them between paths).
      s16x8 ring[AHEAD];
#pragma unroll
      for (int st = 0; st < AHEAD; ++st) ring[st] = fetch(X, Y, st);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NGRP; ++j) {
#pragma unroll
        for (int k = 0; k < GMAX; ++k) {
          const int st = gb(j) + k;
          if (st >= gb(j + 1)) continue;
          const s16x8 cur = ring[st % AHEAD];
          if (st + AHEAD < NST) ring[st % AHEAD] = fetch(X, Y, st + AHEAD);
          step(cur, st, SO);
        }
        slice(j, SLOTc, CUR, pb);
        // operand words of an absent block: zero after they are formed and
        // before the accumulator MFMAs of query half 0 (group 4) and half 1
        // (group 6) read them
        constexpr int zlo = (R == 0 && AMX) ? 3 : 2;
        if ((j == zlo || j == 5) && !ok) {
#pragma unroll
          for (int w4 = 0; w4 < 4; ++w4) op[(j == zlo ? 0 : 4) + w4] = 0u;
        }
        // Block i+2 goes to LDS in groups 4 (chunk 0: the Q tile, or both
        // tiles at D = 64) and 6 (the dO tile), whose own LDS traffic is the
        // lightest (group 0 carries the dS wave's P and Delta reads and the
        // P wave's M and scale reads); block i+3 is loaded after both.
        using W2 = std::integral_constant<int, (SL + 2) & (DPR_SLOTS - 1)>;
        if (j == 4 && stw) write_tiles(W2{}, 0, NCH > 1 ? 1 : NCH);
        if (j == 6 && stw && NCH > 1) write_tiles(W2{}, 1, NCH);
        if (j == 1 && stw) write_vec(i + 2, W2{});
        if (j == 7 && stl) load_stage(i + 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
    };

    // P wave: S(0) before the first iteration
    if (R == 0 && NB > 0 && active(0)) {
      const char* X0 = F8S ? q8_s[0] : q_s[0];
#pragma unroll
      for (int st = 0; st < NSS; ++st) step(fetch(X0, X0, st), st, sb[0]);
    }
    for (int i = 0; i <= NB; i += DPR_SLOTS) {
      static_assert(DPR_SLOTS == 4, "the loop is unrolled by the slot count");
      iteration(i, I0{});
      if (i + 1 <= NB) iteration(i + 1, I1{});
      if (i + 2 <= NB) iteration(i + 2, std::integral_constant<int, 2>{});
      if (i + 3 <= NB) iteration(i + 3, std::integral_constant<int, 3>{});
    }

    // ---- epilogue: the P wave writes dV, the dS wave dK (times sm_scale)
    if (kj >= Nkv) return;
    if (nparts > 1) {   // unscaled fp32 partials [slot][dK, dV][key of the block][D]
      float* pw = a.dkdv_part + (size_t)((unit - a.n_whole) * nparts + part) * 2 * DPR_BN * D +
                  (R == 0 ? (size_t)DPR_BN * D : 0);
      const int kl = kw * 32 + l32;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int d = db * 32 + 8 * u + 4 * g;
          *reinterpret_cast<f32x4*>(pw + (size_t)kl * D + d) =
              (f32x4){acc[db][4 * u], acc[db][4 * u + 1], acc[db][4 * u + 2], acc[db][4 * u + 3]};
        }
      return;
    }
    uint16_t* outp = (uint16_t*)(R == 0 ? a.dv : a.dk) + (size_t)bh * Nkv * D;
    const float scale = R == 0 ? 1.0f : a.sm_scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = db * 32 + 8 * u + 4 * g;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * u + e] * scale;
        *reinterpret_cast<u32x2*>(outp + (size_t)kj * D + d) = (u32x2){DT::pack2(x[0], x[1]), DT::pack2(x[2], x[3])};
      }
  };
  if (w < 4) run(I0{});
  else run(I1{});
}

// Sum of the query-range partials of each split key block, in part order
// (deterministic), scaled and rounded like the whole-block epilogue.  Thread
// t of workgroup (block, z) handles four consecutive d of one key.
template <class DT, int D>
__global__ __launch_bounds__(256) void dkdv_merge_kernel(BwdArgs a, int nkb) {
  constexpr int PER_BLOCK = DPR_BN * D / 4;   // threads per key block
  const int i = blockIdx.y * 256 + threadIdx.x;
  if (i >= PER_BLOCK) return;
  const int kl = i / (D / 4), d = 4 * (i % (D / 4));
  const int unit = a.n_whole + blockIdx.x;
  const int bh = unit / nkb, key = (unit % nkb) * DPR_BN + kl;
  if (key >= a.Nkv) return;
  const float* pw = a.dkdv_part + (size_t)blockIdx.x * a.n_split * 2 * DPR_BN * D;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.n_split; ++p) {
    const float* q = pw + (size_t)p * 2 * DPR_BN * D;
    sk += *reinterpret_cast<const f32x4*>(q + (size_t)kl * D + d);
    sv += *reinterpret_cast<const f32x4*>(q + (size_t)(DPR_BN + kl) * D + d);
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
    const dim3 blk(dq_waves(IN, CAUSAL) * 64);
    if (a.k_mean) hipLaunchKernelGGL((dq_kernel<DT, D, CAUSAL, PQ, IN, true>), g, blk, 0, st, a);
    else hipLaunchKernelGGL((dq_kernel<DT, D, CAUSAL, PQ, IN, false>), g, blk, 0, st, a);
  }
};
template <class DT, int D, bool CAUSAL, int PQ, int IN>
struct DkvK {
  static void run(dim3 g, const BwdArgs& a, hipStream_t st) {
    if constexpr (PQ >= 0) {
      if (!a.p_amax_in) {
        hipLaunchKernelGGL((dkdv_pair_kernel<DT, D, CAUSAL, PQ, IN, true>), g, dim3(512), 0, st, a);
        return;
      }
    }
    hipLaunchKernelGGL((dkdv_pair_kernel<DT, D, CAUSAL, PQ, IN, false>), g, dim3(512), 0, st, a);
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
  a.q8 = (const uint8_t*)in.q8; a.k8 = (const uint8_t*)in.k8;
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
  const int bm = dq_waves(in.mode, causal) * 32;   // rows per workgroup (dq_kernel's BM)
  dim3 grid(((s.Nq + bm - 1) / bm) * s.B * s.H);
  return pick_all<DqK>(s, grid, a, causal, pfmt, in.mode, st);
}

size_t dkdv_part_bytes(const Shape& s) {
  const long long units = (long long)((s.Nkv + DPR_BN - 1) / DPR_BN) * s.B * s.H;
  const long long slots = units * DKDV_MAX_SPLIT < DKDV_PART_SLOTS ? units * DKDV_MAX_SPLIT : DKDV_PART_SLOTS;
  return (size_t)slots * 2 * DPR_BN * s.D * sizeof(float);
}

// Tail split: with U key blocks on C compute units, the last rem = U mod C
// blocks would run in a round of their own, mostly or partly idle.  They are
// cut into k query ranges each (2 <= k <= DKDV_MAX_SPLIT), whose partial sums
// a merge kernel adds up, with the k whose ceil(rem k / C) rounds of 1/k of
// a block finish first (the smaller k on a tie): 96 leftover blocks of 256
// take k = 2 (half a round), 192 take k = 4 (three quarter rounds).  Causal
// launches already order their blocks longest first and are left whole.
static void plan_dkdv(const Shape& s, bool causal, int cus, BwdArgs* a) {
  const int nkb = (s.Nkv + DPR_BN - 1) / DPR_BN;
  const int units = nkb * s.B * s.H;
  const int nqb = (s.Nq + DPR_BQ - 1) / DPR_BQ;
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
  dim3 grid((unsigned)nblocks, (unsigned)((DPR_BN * D / 4 + 255) / 256));
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
  const int nkb = (s.Nkv + DPR_BN - 1) / DPR_BN;
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
