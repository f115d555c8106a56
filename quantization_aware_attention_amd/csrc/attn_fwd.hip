// Forward of quantization-aware attention on gfx950.
//
// Follows the tile loop of _attn_fwd / _attn_fwd_inner in the FastVideo
// attn_qat_train.py source: for every key/value tile the scores are formed,
// the running row maximum updated, the un-normalised probability tile
// p = exp2(S*c - m) fake-quantized per row (one scale per 64-key group,
// here exactly one tile), both accumulators rescaled, and
// O += P^ V, O_hp += P V, l += rowsum(P) (from the high-precision P).
// The epilogue divides both accumulators by l and stores the log-sum-exp.
//
// Mapping onto the MI355X (two kernels: the ping-pong fwd_pp_kernel for
// value or per-token-code inputs, fwd_f8v_kernel for fp8 V codes):
//  * every wave owns 32 query rows and computes S^T = K Q^T with
//    v_mfma_f32_32x32x16, so every lane owns one query row and 32 of the
//    tile's 64 keys in registers: the row maximum, the P-quant absmax and
//    the row sum are in-lane reductions plus one exchange with the lane 32
//    apart;
//  * K and V tiles of 64 keys are double-buffered through LDS (XOR-swizzled
//    16-byte chunks), copied HBM -> LDS by DMA;
//  * O^T = V^T P^T: the P registers are already in the B-operand layout, V^T
//    comes from LDS through transposing reads; the quantized and the
//    straight-through P@V share that V operand (with fp8 V the quantized one
//    runs on the fp8 MFMA from the codes of P^ and V);
//  * the accumulators are rescaled only when the running maximum grows by
//    more than 2^8 (exact in real arithmetic: every tile is scaled by the
//    same stale maximum, and the P-quant absmax scaling is invariant to it).
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace qat {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* v_scale;   // IN_VFP8: [BH, D]
  const float* q_scale;   // IN_QKS: [BH, Nq]
  const float* k_scale;   // IN_QKS: [BH, Nkv]
  const uint8_t* q8;      // IN_QKS: e4m3 code bytes of Q and K (S^T on the fp8 MFMA)
  const uint8_t* k8;
  void* o;
  void* o_hp;
  float* lse;
  int Nq, Nkv;
  float c;          // sm_scale * log2(e)
};

constexpr int FWD_BM = 128;      // query rows per workgroup
constexpr int FWD_BN = 64;       // keys per tile (= P_GROUP)
constexpr float RESCALE_SLACK = 8.0f;

// ---------------------------------------------------------------------------
// Forward with fp8 V: e5m2 codes [B,H,Nkv,D] and a per-(b, h, d) scale.
//
// V never leaves its 8-bit codes: tiles go HBM -> LDS by DMA and are read
// back with ds_read_b64_tr_b8 as V^T operands; v_scale[d] factors out of
// every key contraction and is applied in the epilogue.
//  * O (P quant on): P^ = code_P * s, so per tile and column block one
//    32x32x64 fp8 MFMA of the V codes with the P^ codes forms the exact code
//    products, and the row's group scale s multiplies the result;
//  * O_hp: 32x32x16 fp16 MFMAs of P_hp (rounded to fp16) with the same V
//    operand bytes, widened to fp16 exactly (an e5m2 code is the high byte of
//    the equal fp16).
// Four waves own 32 query rows each; Q rows are held in registers as the B
// operand of S^T = K Q^T; K (bf16) and V tiles are double-buffered in
// separate LDS arrays selected at compile time, so the reads of one buffer
// never wait for the copies into the other.
template <int D, bool CAUSAL, int PQ>
__global__ __launch_bounds__(256, 2) void fwd_f8v_kernel(FwdArgs a) {
  using DT = BF16;
  constexpr int TILE = FWD_BN * D * 2;      // bytes per K tile
  constexpr int VTILE = FWD_BN * D;         // bytes per V code tile
  constexpr int NDB = D / 32;               // 32-wide d blocks
  constexpr int NKS = D / 16;               // 16-deep k steps over D
  constexpr int FQF = PQ >= 0 ? PQ : 0;
  __shared__ __attribute__((aligned(16))) char k_s0[TILE];
  __shared__ __attribute__((aligned(16))) char k_s1[TILE];
  __shared__ __attribute__((aligned(16))) char v_s0[VTILE];
  __shared__ __attribute__((aligned(16))) char v_s1[VTILE];

  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int ntq = (a.Nq + FWD_BM - 1) / FWD_BM;
  int bh, rank;   // causal: the longest rows (last blocks) first
  work_unit(blockIdx.x, gridDim.x, ntq, CAUSAL, &bh, &rank);
  const int qb = (CAUSAL ? ntq - 1 - rank : rank) * FWD_BM;
  const int q0 = qb + w * 32;
  const int qi = q0 + l32;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const uint16_t* qp = (const uint16_t*)a.q + (size_t)bh * Nq * D;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)bh * Nkv * D;
  const uint8_t* vp = (const uint8_t*)a.v + (size_t)bh * Nkv * D;
  const float c_row = a.c;

  // Q^T operand: lane holds row qi, d = 16ks + 8g .. +7
  s16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (qi < Nq) qf[ks] = *reinterpret_cast<const s16x8*>(qp + (size_t)qi * D + 16 * ks + 8 * g);
    else qf[ks] = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
  }

  const int kv_end = CAUSAL ? min(Nkv, qb + FWD_BM) : Nkv;
  const int ntiles = (kv_end + FWD_BN - 1) / FWD_BN;
  TileCopy<D, FWD_BN, 4> kcopy;
  CodeCopy<D, FWD_BN, 4> vcopy;
  kcopy.init(w, lane);
  vcopy.init(w, lane);
  // per-lane parts of the LDS operand addresses (tile_off and vc_off with
  // the tile-independent terms folded): K row l32, and the V-code row and
  // 8-byte half of lds_vcode_tr
  const int vrow = 8 * ((lane & 15) >> 3) + 4 * g + ((lane & 15) >> 1 & 3);
  const int k_off0 = l32 * (D * 2), k_sw0 = swz<D>(l32);
  const int v_off0 = vrow * D + ((lane & 1) << 3), v_sw0 = vc_swz<D>(vrow), v_c16 = (lane >> 4) & 1;

  float m_used = -INFINITY;   // stale running maximum (scaled log2 units)
  float l_part = 0.0f;        // this lane's share of the row sum
  f32x16 o_acc[NDB], oh_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    o_acc[db] = (f32x16){};
    oh_acc[db] = (f32x16){};
  }

  // one tile from buffer BUF (compile-time), copies of the next into the other
  auto tile_step = [&](auto BUF, int t) __attribute__((always_inline)) {
    constexpr int bsel = decltype(BUF)::value;
    char* Kt = bsel ? k_s1 : k_s0;
    char* Vc = bsel ? v_s1 : v_s0;
    // recomputed per tile rather than kept live across the loop (which
    // spills them, and every reload would then wait for the tile copies)
    int k_off = k_off0, k_sw = k_sw0, v_off = v_off0, v_sw = v_sw0;
    asm volatile("" : "+v"(k_off), "+v"(k_sw), "+v"(v_off), "+v"(v_sw));
    if (t + 1 < ntiles) {
      kcopy.issue(bsel ? k_s0 : k_s1, kp, (t + 1) * FWD_BN, Nkv);
      vcopy.issue(bsel ? v_s0 : v_s1, vp, (t + 1) * FWD_BN, Nkv);
    }
    const int kv0 = t * FWD_BN;
    const bool active = (q0 < Nq) && (!CAUSAL || kv0 <= q0 + 31);
    if (active) {
      // ---- S^T = K Q^T (two 32-key blocks)
      prio_mfma();
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = (f32x16){};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const s16x8 ka = *reinterpret_cast<const s16x8*>(Kt + kb * 32 * (D * 2) + k_off + (((2 * ks + g) ^ k_sw) << 4));
          s[kb] = DT::mfma(ka, qf[ks], s[kb]);
        }
      }
      prio_valu();
      // ---- masks: key tail, causal diagonal
      const bool need_mask = (kv0 + FWD_BN > Nkv) || (CAUSAL && kv0 + FWD_BN - 1 > q0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= Nkv || (CAUSAL && key > qi)) s[kb][r] = -INFINITY;
          }
      }
      // ---- running maximum with lazy rescale
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max_xor32(mx);
      const float t_new = mx * c_row;
      const bool resc = t_new > m_used + RESCALE_SLACK;
      if (__any(resc)) {
        const float m_new = resc ? t_new : m_used;
        const float alpha = resc ? fast_exp2(m_used - m_new) : 1.0f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          if constexpr (PQ >= 0) o_acc[db] *= alpha;
          oh_acc[db] *= alpha;
        }
        l_part *= alpha;
        m_used = m_new;
      }
      const float m_sub = (m_used == -INFINITY) ? 0.0f : m_used;
      // ---- P-quant scale of this row's 64-key group: the absmax of p is
      // exp2 of the largest argument (exp2 is monotone; mx is the row max)
      FqScale fs = {0.0f, 0.0f};
      if constexpr (PQ >= 0) {
        const float pmax = (mx == -INFINITY) ? 0.0f : fast_exp2(__builtin_fmaf(mx, c_row, -m_sub));
        fs = fq_scale<FQF>(pmax);
      }
      // ---- p = exp2(S*c - m); operands: P^ codes (dword 4kb + u = keys
      // 32kb + 8u + 4g + 0..3) and P_hp in fp16 (k step kk = 2kb + h)
      float psum = 0.0f;
      i32x8 pcode;
      uint32_t phw[4][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(__builtin_fmaf(s[kb][r], c_row, -m_sub));
          psum += p[r];
        }
        if constexpr (PQ >= 0) {
#pragma unroll
          for (int u = 0; u < 4; ++u) pcode[4 * kb + u] = fq_codes4<FQF>(&p[4 * u], fs.r);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) phw[2 * kb + h][jj] = FP16::pack2(p[8 * h + 2 * jj], p[8 * h + 2 * jj + 1]);
      }
      l_part += psum;
      // ---- O^T += s (V^T codes . P^ codes^T);  O_hp^T += V^T P_hp^T
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        // lds_vcode_tr with the lane terms precomputed
        i32x8 vc;
        const char* vb = Vc + v_off + (((2 * db + v_c16) ^ v_sw) << 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const i32x2 t2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vb + (32 * (r >> 1) + 16 * (r & 1)) * D));
          vc[2 * r] = t2[0];
          vc[2 * r + 1] = t2[1];
        }
        if constexpr (PQ >= 0) {
          const f32x16 t8 = mfma_f8_bf8a<FQF>(vc, pcode, (f32x16){});
          o_acc[db] += t8 * fs.s;
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const s16x8 bop = __builtin_bit_cast(s16x8, (u32x4){phw[kk][0], phw[kk][1], phw[kk][2], phw[kk][3]});
          oh_acc[db] = FP16::mfma(e5m2x8_to_f16(vc[2 * kk], vc[2 * kk + 1]), bop, oh_acc[db]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };

  if (ntiles > 0) {
    kcopy.issue(k_s0, kp, 0, Nkv);
    vcopy.issue(v_s0, vp, 0, Nkv);
  }
  wait_vmem();
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    tile_step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < ntiles) tile_step(std::integral_constant<int, 1>{}, t + 1);
  }

  // ---- epilogue: O = O_acc / l * v_scale[d] (O_hp likewise)
  if (q0 >= Nq) return;
  const float l = sum_xor32(l_part);
  const float inv_l = 1.0f / l;
  uint16_t* op = (uint16_t*)a.o + (size_t)bh * Nq * D;
  uint16_t* ohp = (uint16_t*)a.o_hp + (size_t)bh * Nq * D;
  if (qi < Nq) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = db * 32 + 8 * u + 4 * g;
        const f32x4 vs = *reinterpret_cast<const f32x4*>(a.v_scale + (size_t)bh * D + d);
        float x[4], y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[e] = oh_acc[db][4 * u + e] * inv_l * vs[e];
          x[e] = PQ >= 0 ? o_acc[db][4 * u + e] * inv_l * vs[e] : y[e];
        }
        *reinterpret_cast<u32x2*>(op + (size_t)qi * D + d) = (u32x2){DT::pack2(x[0], x[1]), DT::pack2(x[2], x[3])};
        *reinterpret_cast<u32x2*>(ohp + (size_t)qi * D + d) = (u32x2){DT::pack2(y[0], y[1]), DT::pack2(y[2], y[3])};
      }
    if (g == 0) a.lse[(size_t)bh * Nq + qi] = (m_used + __builtin_log2f(l)) * LN2;
  }
}

// ---------------------------------------------------------------------------
// Ping-pong forward (values or per-token-scaled codes as inputs).
//
// Eight waves own 256 query rows (32 each); waves w and w+4 share a SIMD.
// The waves form two groups that alternate between an MFMA phase
// (P@V of the previous tile, then S^T of this tile) and a VALU phase
// (masks, running maximum, exp2, P fake quant, operand packing), separated
// by workgroup barriers: while one group keeps the SIMD's matrix core busy
// the other works through its vector instructions.  Phase p:
//   group 0: p = 2t   -> MFMA(t),   p = 2t+1 -> VALU(t)
//   group 1: p = 2t+1 -> MFMA(t),   p = 2t+2 -> VALU(t)
// with MFMA(T) = P@V of the last tile only.  K(t) is read in phases 2t and
// 2t+1, V(t) in phases 2t+2 and 2t+3 (both double-buffered).  The block's Q
// rows stay in LDS; the MFMA phase is one software-pipelined stream whose
// LDS operands are read two steps ahead of their MFMAs.  Tile copies are
// issued by group 0 in its VALU phases and waited for before the barrier,
// so no MFMA phase ever waits on global memory.
constexpr int PP_BM = 256;

template <class DT, int D, bool CAUSAL, int PQ, int IN>
__global__ __launch_bounds__(512, 1) void fwd_pp_kernel(FwdArgs a) {
  static_assert(IN != IN_VFP8, "fp8 V uses fwd_f8v_kernel");
  constexpr bool QKS = IN == IN_QKS;
  constexpr int TILE = FWD_BN * D * 2;
  constexpr int QKB = QKS ? 1 : 2;   // bytes per Q / K element in LDS: e4m3 codes with per-token scales
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  constexpr int FQF = PQ >= 0 ? PQ : 0;
  constexpr int NPV = 4 * NDB;   // P@V steps of an MFMA phase
  // fragments in flight ahead of their MFMAs: five (no spills; six spilled
  // and ran slower), four with per-token codes (which need more registers)
  constexpr int PP_AHEAD = QKS ? 4 : 5;
  __shared__ __attribute__((aligned(16))) char kbuf[2][FWD_BN * D * QKB];
  __shared__ __attribute__((aligned(16))) char vbuf[2][TILE];
  __shared__ __attribute__((aligned(16))) float ks_s[3][FWD_BN];   // IN_QKS: key scales of K(t)
  __shared__ __attribute__((aligned(16))) char qbuf[PP_BM * D * QKB];   // the block's Q rows

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int grp = w >> 2;
  const int ntq = (a.Nq + PP_BM - 1) / PP_BM;
  int bh, rank;   // causal: the longest rows (last blocks) first
  work_unit(blockIdx.x, gridDim.x, ntq, CAUSAL, &bh, &rank);
  const int qb = (CAUSAL ? ntq - 1 - rank : rank) * PP_BM;
  const int q0 = qb + w * 32;
  const int qi = q0 + l32;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const uint16_t* qp = (const uint16_t*)a.q + (size_t)bh * Nq * D;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)bh * Nkv * D;
  const uint16_t* vp = (const uint16_t*)a.v + (size_t)bh * Nkv * D;

  const uint8_t* k8p = QKS ? a.k8 + (size_t)bh * Nkv * D : nullptr;
  {   // Q rows [qb, qb + PP_BM) into LDS (rows past Nq repeat the last row)
    if constexpr (QKS) {
      CodeCopy<D, PP_BM, 8, true> qcopy;
      qcopy.init(wave_id(), lane);
      qcopy.issue(qbuf, a.q8 + (size_t)bh * Nq * D, qb, Nq);
    } else {
      TileCopy<D, PP_BM, 8> qcopy;
      qcopy.init(wave_id(), lane);
      qcopy.issue(qbuf, qp, qb, Nq);
    }
  }
  // exponent scale of this row; a zero per-token Q scale (all-zero row, every
  // score 0) is raised to the smallest normal so that masked scores stay -inf
  float c_row = a.c;
  if constexpr (QKS) c_row = a.c * fmaxf(qi < Nq ? a.q_scale[(size_t)bh * Nq + qi] : 1.0f, 1.17549435e-38f);
  const float* ksp = QKS ? a.k_scale + (size_t)bh * Nkv : nullptr;

  const int kv_end = CAUSAL ? min(Nkv, qb + PP_BM) : Nkv;
  const int T = (kv_end + FWD_BN - 1) / FWD_BN;
  TileCopy<D, FWD_BN, 4> copy;   // used by group 0 only (K and V, or V only)
  copy.init(wave_id() & 3, lane);
  CodeCopy<D, FWD_BN, 4, true> kcopy8;   // IN_QKS: K codes
  if constexpr (QKS) kcopy8.init(wave_id() & 3, lane);
  auto issue_k = [&](int t) __attribute__((always_inline)) {
    if constexpr (QKS) kcopy8.issue(kbuf[t & 1], k8p, t * FWD_BN, Nkv);
    else copy.issue(kbuf[t & 1], kp, t * FWD_BN, Nkv);
  };
  float ksreg = 0.0f;

  float m_used = -INFINITY, l_part = 0.0f;
  f32x16 o_acc[NDB], oh_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    o_acc[db] = (f32x16){};
    oh_acc[db] = (f32x16){};
  }
  // S^T of a tile from its MFMA phase to its VALU phase; the VALU phase then
  // overwrites it in place with the packed operands of P@V: for k-step kk
  // (keys 16kk..16kk+15) words s[kk/2][8(kk%2) + 0..3] hold P^ and
  // words + 4..7 hold P_hp, until the next MFMA phase consumes them.
  f32x16 s[2];
  const bool live_rows = q0 < Nq;
  auto active = [&](int t) { return live_rows && (!CAUSAL || t * FWD_BN <= q0 + 31); };

  auto scale_keys = [&](int t) __attribute__((always_inline)) {   // IN_QKS: S^T *= per-key scales
    if constexpr (QKS) {
      // the lane's half (g) recomputed here from the lane counter: held from
      // the kernel's start, its address was spilled, and the reload's vmcnt
      // wait also waited for the tile copies just issued
      // (an opaque all-ones mask keeps the count from being hoisted out of
      // the loop and spilled in turn)
      uint32_t ones = ~0u;
      asm volatile("" : "+s"(ones));
      const int gh = (int)__builtin_amdgcn_mbcnt_hi(ones, __builtin_amdgcn_mbcnt_lo(ones, 0u)) >> 5;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4 sk = *reinterpret_cast<const f32x4*>(&ks_s[t % 3][kb * 32 + 8 * u + 4 * gh]);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kb][4 * u + e] *= sk[e];
        }
    }
  };
  // The MFMA phase as one stream of single-fragment steps: NPV steps of
  // P@V (a V fragment feeding the O and O_hp MFMAs of a 16-key by 32-column
  // block), then for each k-step of S^T = K Q^T a Q fragment and the two K
  // fragments (one MFMA each, against the last Q fragment).  With per-token
  // codes a k-step spans 64 d on the fp8 MFMA and every operand is two
  // 16-byte halves, so the step order is Q, Q, K0, K0 (MFMA), K1, K1 (MFMA).
  // Step f reads the fragment of step f + PP_AHEAD; scheduling fences keep
  // that order, so every MFMA finds its LDS operand already loaded.
  constexpr int NSS = QKS ? 6 * (D / 64) : 3 * NKS;   // S^T steps
  constexpr int NFR = NPV + NSS;
  // Operand addresses formed once: the lane offsets of the V^T reads of
  // k-step 0 per column block (k-step kk adds 16kk rows, a constant that the
  // reads take as an immediate offset), and those of the wave's Q fragments,
  // which never move.  Formed per read, they cost a vector add or two in
  // front of each read of the MFMA phase.
  int vt_lane[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h) vt_lane[db][h] = tr8_off<D>(8 * h, db * 32, lane);
  int q_lane[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) q_lane[ks] = tile_off<D>(w * 32 + l32, 2 * ks + g);
  auto fetch = [&](const char* Vt, const char* Kt, int f) __attribute__((always_inline)) {
    if (f < NPV) {
      const char* vk = Vt + (f / NDB) * 16 * D * 2;
      return lds_tr8_at(vk + vt_lane[f % NDB][0], vk + vt_lane[f % NDB][1]);
    }
    const int k = f - NPV;
    if constexpr (QKS) {   // e4m3 codes: chunk 4ks + 2g + half of the row, d = 64ks + 32g + 0..31
      const int ks = k / 6, part = k % 6, obj = part >> 1, chunk = 4 * ks + 2 * g + (part & 1);
      if (obj == 0) return lds_f8row<D>(qbuf, w * 32 + l32, chunk);
      return lds_f8row<D>(Kt, (obj - 1) * 32 + l32, chunk);
    } else {
      const int ks = k / 3, part = k % 3;
      if (part == 0) return *reinterpret_cast<const s16x8*>(qbuf + q_lane[ks]);
      return lds_row8<D>(Kt, (part - 1) * 32 + l32, 2 * ks + g);
    }
  };
  s16x8 qcur, qcur2, kcur;
  auto step = [&](const s16x8& frag, int f) __attribute__((always_inline)) {
    if (f < NPV) {   // O^T += V^T P^T, k-step kk, column block db
      const int kk = f / NDB, db = f % NDB, kb = kk >> 1, o8 = 8 * (kk & 1);
      const s16x8 bhp = __builtin_bit_cast(s16x8, (f32x4){s[kb][o8 + 4], s[kb][o8 + 5], s[kb][o8 + 6], s[kb][o8 + 7]});
      if constexpr (PQ >= 0) {
        const s16x8 bq = __builtin_bit_cast(s16x8, (f32x4){s[kb][o8], s[kb][o8 + 1], s[kb][o8 + 2], s[kb][o8 + 3]});
        o_acc[db] = DT::mfma(frag, bq, o_acc[db]);
        oh_acc[db] = DT::mfma(frag, bhp, oh_acc[db]);
      } else {
        o_acc[db] = DT::mfma(frag, bhp, o_acc[db]);
      }
    } else {          // S^T = K Q^T, k-step ks
      const int k = f - NPV;
      if (k == 0) {
        s[0] = (f32x16){};
        s[1] = (f32x16){};
      }
      if constexpr (QKS) {
        const int part = k % 6;
        if (part == 0) qcur = frag;
        else if (part == 1) qcur2 = frag;
        else if (part == 2 || part == 4) kcur = frag;
        else s[(part - 3) >> 1] = mfma_e4m3(kcur, frag, qcur, qcur2, s[(part - 3) >> 1]);
      } else {
        const int part = k % 3;
        if (part == 0) qcur = frag;
        else s[part - 1] = DT::mfma(frag, qcur, s[part - 1]);
      }
    }
  };
  auto mfma_phase = [&](int t) __attribute__((always_inline)) {
    const bool do_pv = t >= 1 && active(t - 1);
    const bool do_qk = t < T && active(t);
    const char* Vt = vbuf[(t - 1) & 1];
    const char* Kt = kbuf[t & 1];
    if (do_pv && do_qk) {
      s16x8 ring[PP_AHEAD];
#pragma unroll
      for (int f = 0; f < PP_AHEAD; ++f) {   // fenced, so that they issue in step order
        ring[f] = fetch(Vt, Kt, f);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < NFR; ++f) {
        const s16x8 cur = ring[f % PP_AHEAD];
        if (f + PP_AHEAD < NFR) ring[f % PP_AHEAD] = fetch(Vt, Kt, f + PP_AHEAD);
        __builtin_amdgcn_sched_barrier(0);
        step(cur, f);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {          // first and last phases, causal edges: the same steps unpipelined
      if (do_pv) {
#pragma unroll
        for (int f = 0; f < NPV; ++f) step(fetch(Vt, Kt, f), f);
      }
      if (do_qk) {
#pragma unroll
        for (int f = NPV; f < NFR; ++f) step(fetch(Vt, Kt, f), f);
      }
    }
  };
  auto valu_phase = [&](int t) __attribute__((always_inline)) {
    if (!active(t)) return;
    // IN_QKS: the key scales of tile t are in ks_s[t % 3], written at the end
    // of group 0's copy phase 2t - 1 and read in phases 2t + 1 (group 0) and
    // 2t + 2 (group 1); the buffer is next rewritten at the end of phase
    // 2t + 5, after the barrier that follows phase 2t + 3
    scale_keys(t);
    const int kv0 = t * FWD_BN;
    if ((kv0 + FWD_BN > Nkv) || (CAUSAL && kv0 + FWD_BN - 1 > q0)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= Nkv || (CAUSAL && key > qi)) s[kb][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_xor32(mx);
    const float t_new = mx * c_row;
    const bool resc = t_new > m_used + RESCALE_SLACK;
    if (__any(resc)) {
      const float m_new = resc ? t_new : m_used;
      const float alpha = resc ? fast_exp2(m_used - m_new) : 1.0f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        o_acc[db] *= alpha;
        if constexpr (PQ >= 0) oh_acc[db] *= alpha;
      }
      l_part *= alpha;
      m_used = m_new;
    }
    const float m_sub = (m_used == -INFINITY) ? 0.0f : m_used;
    FqScale fs = {0.0f, 0.0f};
    if constexpr (PQ >= 0) {   // absmax of the row group = exp2 of its largest argument
      const float pmax = (mx == -INFINITY) ? 0.0f : fast_exp2(__builtin_fmaf(mx, c_row, -m_sub));
      fs = fq_scale<FQF>(pmax);
    }
    const FqScale f4[4] = {fs, fs, fs, fs};
    float psum = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kb = kk >> 1, h = kk & 1;
      float p8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p8[j] = fast_exp2(__builtin_fmaf(s[kb][8 * h + j], c_row, -m_sub));
        psum += p8[j];
      }
      uint32_t w8[8];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) w8[4 + jj] = DT::pack2(p8[2 * jj], p8[2 * jj + 1]);
      if constexpr (PQ >= 0) {
#pragma unroll
        for (int jq = 0; jq < 2; ++jq) {
          const f32x4 xq = fq_quad<FQF>(&p8[4 * jq], f4);
          w8[2 * jq] = DT::pack2(xq[0], xq[1]);
          w8[2 * jq + 1] = DT::pack2(xq[2], xq[3]);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) w8[jj] = w8[4 + jj];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) s[kb][8 * h + j] = __builtin_bit_cast(float, w8[j]);
    }
    l_part += psum;
  };

  // prologue: K(0) (and its scales) resident before phase 0
  if (T > 0 && grp == 0) {
    issue_k(0);
    if constexpr (QKS) {
      if (tid < FWD_BN) ksreg = tid < Nkv ? ksp[tid] : 0.0f;
    }
  }
  wait_vmem();
  if constexpr (QKS) {
    if (T > 0 && tid < FWD_BN) ks_s[0][tid] = ksreg;
  }
  __syncthreads();
  // Tile copies are issued only by group 0, in its VALU phases (2t+1: K(t+1)
  // and V(t), into the buffers last read in phase 2t-1), and waited for
  // before that phase's barrier: no wave ever reads LDS while a copy of its
  // own is in flight, so the MFMA phases carry no wait on global memory.
  const int nphase = 2 * T + 2;
  for (int ph_i = 0; ph_i < nphase; ++ph_i) {
    // group 0: MFMA on even phases, VALU on odd; group 1 one phase later
    const bool mfma_now = ((ph_i + grp) & 1) == 0;
    const int t_work = (ph_i - grp) >> 1;
    // The VALU part comes first in program order and ends with the wait for
    // this wave's copies, so the LDS reads of the MFMA part (executed under
    // the complementary lane mask) never wait on global memory.
    if (!mfma_now) {
      const int t = ph_i >> 1;
      if (grp == 0) {
        if (t + 1 < T) {
          issue_k(t + 1);
          if constexpr (QKS) {
            const int key = (t + 1) * FWD_BN + tid;
            if (tid < FWD_BN) ksreg = key < Nkv ? ksp[key] : 0.0f;
          }
        }
        if (t < T) copy.issue(vbuf[t & 1], vp, t * FWD_BN, Nkv);
      }
      if (t_work >= 0 && t_work < T) valu_phase(t_work);
    }
    wait_vmem();
    if constexpr (QKS) {
      const int t = ph_i >> 1;
      if (grp == 0 && !mfma_now && t + 1 < T && tid < FWD_BN) ks_s[(t + 1) % 3][tid] = ksreg;
    }
    if (mfma_now) {   // raised issue priority: the MFMAs go first, the other wave's VALU work fills in
      prio_mfma();
      mfma_phase(t_work);
      prio_valu();
    }
    // Barriers: after every odd phase (group 0's VALU phase) only.  That
    // barrier publishes the tiles (and key scales) group 0 copied in the
    // phase, and orders each copy after the last reads of the buffer it
    // overwrites: K/V buffers were last read in the odd phase two earlier,
    // and the three key-scale buffers in the phases before that (the VALU
    // phases read no other LDS), so even phases need no barrier.
    if (ph_i + 1 < nphase && (ph_i & 1)) __syncthreads();
  }

  // ---- epilogue
  if (qi >= Nq) return;
  const float l = sum_xor32(l_part);
  const float inv_l = 1.0f / l;
  uint16_t* op = (uint16_t*)a.o + (size_t)bh * Nq * D;
  uint16_t* ohp = (uint16_t*)a.o_hp + (size_t)bh * Nq * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = db * 32 + 8 * u + 4 * g;
      float x[4], y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = o_acc[db][4 * u + e] * inv_l;
        y[e] = (PQ >= 0 ? oh_acc[db][4 * u + e] : o_acc[db][4 * u + e]) * inv_l;
      }
      *reinterpret_cast<u32x2*>(op + (size_t)qi * D + d) = (u32x2){DT::pack2(x[0], x[1]), DT::pack2(x[2], x[3])};
      *reinterpret_cast<u32x2*>(ohp + (size_t)qi * D + d) = (u32x2){DT::pack2(y[0], y[1]), DT::pack2(y[2], y[3])};
    }
  if (g == 0) a.lse[(size_t)bh * Nq + qi] = (m_used + __builtin_log2f(l)) * LN2;
}

template <class DT, int D, bool CAUSAL, int PQ, int IN>
static hipError_t fwd_launch(const Shape& s, const FwdArgs& a, hipStream_t st) {
  if constexpr (IN == IN_VFP8) {
    dim3 grid(((s.Nq + FWD_BM - 1) / FWD_BM) * s.B * s.H);
    hipLaunchKernelGGL((fwd_f8v_kernel<D, CAUSAL, PQ>), grid, dim3(256), 0, st, a);
  } else {
    dim3 grid(((s.Nq + PP_BM - 1) / PP_BM) * s.B * s.H);
    hipLaunchKernelGGL((fwd_pp_kernel<DT, D, CAUSAL, PQ, IN>), grid, dim3(512), 0, st, a);
  }
  return hipGetLastError();
}

template <class DT, int D, bool CAUSAL, int IN>
static hipError_t fwd_pick_pq(const Shape& s, const FwdArgs& a, int pfmt, hipStream_t st) {
  if (pfmt == 0) return fwd_launch<DT, D, CAUSAL, 0, IN>(s, a, st);
  if (pfmt == 1) return fwd_launch<DT, D, CAUSAL, 1, IN>(s, a, st);
  return fwd_launch<DT, D, CAUSAL, -1, IN>(s, a, st);
}

template <class DT, int D, int IN>
static hipError_t fwd_pick_causal(const Shape& s, const FwdArgs& a, bool causal, int pfmt, hipStream_t st) {
  return causal ? fwd_pick_pq<DT, D, true, IN>(s, a, pfmt, st) : fwd_pick_pq<DT, D, false, IN>(s, a, pfmt, st);
}

template <class DT, int D>
static hipError_t fwd_pick(const Shape& s, const FwdArgs& a, bool causal, int pfmt, int mode, hipStream_t st) {
  if (mode == IN_VFP8) {
    if constexpr (__is_same(DT, BF16)) return fwd_pick_causal<DT, D, IN_VFP8>(s, a, causal, pfmt, st);
    return hipErrorInvalidValue;
  }
  if (mode == IN_QKS) return fwd_pick_causal<DT, D, IN_QKS>(s, a, causal, pfmt, st);
  return fwd_pick_causal<DT, D, IN_PLAIN>(s, a, causal, pfmt, st);
}

hipError_t launch_fwd(const Shape& s, const Inputs& in, float sm_scale, bool causal, int pfmt,
                      void* o, void* o_hp, float* lse, hipStream_t st) {
  FwdArgs a;
  a.q = in.q; a.k = in.k; a.v = in.v;
  a.v_scale = in.v_scale; a.q_scale = in.q_scale; a.k_scale = in.k_scale;
  a.q8 = (const uint8_t*)in.q8; a.k8 = (const uint8_t*)in.k8;
  a.o = o; a.o_hp = o_hp; a.lse = lse;
  a.Nq = s.Nq; a.Nkv = s.Nkv;
  a.c = sm_scale * LOG2E;
  if (s.dtype == 0) {
    return s.D == 128 ? fwd_pick<BF16, 128>(s, a, causal, pfmt, in.mode, st)
                      : fwd_pick<BF16, 64>(s, a, causal, pfmt, in.mode, st);
  }
  return s.D == 128 ? fwd_pick<FP16, 128>(s, a, causal, pfmt, in.mode, st)
                    : fwd_pick<FP16, 64>(s, a, causal, pfmt, in.mode, st);
}

}  // namespace qat
