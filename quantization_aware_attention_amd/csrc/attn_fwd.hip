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
// Mapping onto the MI355X:
//  * a workgroup of 4 waves owns 128 query rows (32 per wave); each wave
//    computes S^T = K Q^T with v_mfma_f32_32x32x16, so every lane owns one
//    query row and 32 of the tile's 64 keys in registers: the row maximum,
//    the P-quant absmax and the row sum are in-lane reductions plus one
//    exchange with the lane 32 apart;
//  * Q^T stays in registers for the whole loop; K and V tiles of 64 keys are
//    double-buffered through LDS (XOR-swizzled 16-byte chunks);
//  * O^T = V^T P^T: the P registers are already in the B-operand layout, V^T
//    comes from LDS through ds_read_b64_tr_b16; the quantized and the
//    straight-through P@V share that V operand;
//  * the accumulators are rescaled only when the running maximum grows by
//    more than 2^8 (exact in real arithmetic: every tile is scaled by the
//    same stale maximum, and the P-quant absmax scaling is invariant to it).
#include "common.hpp"
#include "launch.hpp"

namespace qat {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* v_scale;   // IN_VFP8: [BH, D]
  const float* q_scale;   // IN_QKS: [BH, Nq]
  const float* k_scale;   // IN_QKS: [BH, Nkv]
  void* o;
  void* o_hp;
  float* lse;
  int Nq, Nkv;
  float c;          // sm_scale * log2(e)
};

constexpr int FWD_BM = 128;      // query rows per workgroup
constexpr int FWD_BN = 64;       // keys per tile (= P_GROUP)
constexpr float RESCALE_SLACK = 8.0f;

template <class DT, int D, bool CAUSAL, int PQ, int IN>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  constexpr bool VFP8 = IN == IN_VFP8;
  constexpr bool QKS = IN == IN_QKS;
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = FWD_BN * D * 2;      // bytes per K or V tile
  constexpr int LPT = FWD_BN * CH / 256;    // chunks per thread per tile
  constexpr int NDB = D / 32;               // 32-wide d blocks
  constexpr int NKS = D / 16;               // 16-deep k steps over D
  __shared__ __attribute__((aligned(16))) char smem[2][2][TILE];
  __shared__ __attribute__((aligned(16))) float ks_s[2][FWD_BN];   // IN_QKS: key scales of the tile

  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int ntq = (a.Nq + FWD_BM - 1) / FWD_BM;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  const int bh = unit / ntq;
  // causal: the longest rows first, so short tiles fill the tail of the launch
  const int qb = (CAUSAL ? ntq - 1 - unit % ntq : unit % ntq) * FWD_BM;
  const int q0 = qb + w * 32;
  const int qi = q0 + l32;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const uint16_t* qp = (const uint16_t*)a.q + (size_t)bh * Nq * D;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)bh * Nkv * D;
  const uint8_t* vp8 = (const uint8_t*)a.v + (size_t)bh * Nkv * D * (VFP8 ? 1 : 2);

  // Q^T operand: lane holds row qi, d = 16ks + 8g .. +7
  s16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (qi < Nq) qf[ks] = *reinterpret_cast<const s16x8*>(qp + (size_t)qi * D + 16 * ks + 8 * g);
    else qf[ks] = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
  }

  // IN_QKS: S = s_q[i] s_k[j] (code_q . code_k); s_q folds into the log2 scale
  float c_row = a.c;
  if constexpr (QKS) c_row = a.c * (qi < Nq ? a.q_scale[(size_t)bh * Nq + qi] : 1.0f);
  const float* ksp = QKS ? a.k_scale + (size_t)bh * Nkv : nullptr;

  const int kv_end = CAUSAL ? min(Nkv, qb + FWD_BM) : Nkv;
  const int ntiles = (kv_end + FWD_BN - 1) / FWD_BN;

  // V codes of the fp8-V path take a register detour (decoded to bf16 on the
  // way into LDS); every other tile goes HBM -> LDS directly.
  u32x2 vcode[LPT];
  float ksreg = 0.0f;
  TileCopy<D, FWD_BN, 4> copy;
  copy.init(w, lane);
  auto issue_tile = [&](int t, int buf) {
    copy.issue(smem[buf][0], kp, t * FWD_BN, Nkv);
    if constexpr (VFP8) {
#pragma unroll
      for (int u = 0; u < LPT; ++u) {
        const int idx = tid + 256 * u, row = idx / CH, ch = idx % CH;
        const int key = min(t * FWD_BN + row, Nkv - 1);
        vcode[u] = *reinterpret_cast<const u32x2*>(vp8 + (size_t)key * D + ch * 8);
      }
    } else {
      copy.issue(smem[buf][1], (const uint16_t*)vp8, t * FWD_BN, Nkv);
    }
    if constexpr (QKS) {
      const int key = t * FWD_BN + tid;
      if (tid < FWD_BN) ksreg = key < Nkv ? ksp[key] : 0.0f;
    }
  };
  // register-staged parts of a tile: written after the loads landed
  auto finish_tile = [&](int buf) {
    if constexpr (VFP8) {
#pragma unroll
      for (int u = 0; u < LPT; ++u) {
        const int idx = tid + 256 * u, row = idx / CH, ch = idx % CH;
        u32x4 vv;   // e5m2 codes -> bf16 (exact: every e5m2 value is a bf16 value)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t word = vcode[u][h >> 1] >> (16 * (h & 1));
          const f32x2 f = __builtin_amdgcn_cvt_pk_f32_bf8((int)word, false);
          vv[h] = BF16::pack2(f[0], f[1]);
        }
        *reinterpret_cast<u32x4*>(smem[buf][1] + tile_off<D>(row, ch)) = vv;
      }
    }
    if constexpr (QKS) {
      if (tid < FWD_BN) ks_s[buf][tid] = ksreg;
    }
  };

  float m_used = -INFINITY;   // stale running maximum (scaled log2 units)
  float l_part = 0.0f;        // this lane's share of the row sum
  f32x16 o_acc[NDB], oh_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    o_acc[db] = (f32x16){};
    oh_acc[db] = (f32x16){};
  }

  if (ntiles > 0) {
    issue_tile(0, 0);
    wait_vmem();
    finish_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
    const int kv0 = t * FWD_BN;
    const bool active = (q0 < Nq) && (!CAUSAL || kv0 <= q0 + 31);
    if (active) {
      const char* Kt = smem[buf][0];
      const char* Vt = smem[buf][1];
      // ---- S^T = K Q^T (two 32-key blocks)
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = (f32x16){};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const s16x8 ka = lds_row8<D>(Kt, kb * 32 + l32, 2 * ks + g);
          s[kb] = DT::mfma(ka, qf[ks], s[kb]);
        }
      }
      if constexpr (QKS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const f32x4 sk = *reinterpret_cast<const f32x4*>(&ks_s[buf][kb * 32 + 8 * u + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[kb][4 * u + e] *= sk[e];
          }
      }
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
      mx = fmaxf(mx, shfl_xor32(mx));
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
      // ---- P-quant scale of this row's 64-key group: the absmax of p is
      // exp2 of the largest argument (exp2 is monotone; mx is the row max)
      FqScale fs = {0.0f, 0.0f};
      if constexpr (PQ >= 0) {
        const float pmax = (mx == -INFINITY) ? 0.0f : fast_exp2(__builtin_fmaf(mx, c_row, -m_sub));
        fs = fq_scale(pmax, Fp8Fmt<(PQ >= 0 ? PQ : 0)>::FMAX);
      }
      // ---- p = exp2(S*c - m)
      float p[2][16];
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], c_row, -m_sub));
          psum += p[kb][r];
        }
      l_part += psum;
      // ---- O^T += V^T P^T  (4 k-steps of 16 keys)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int kb = kk >> 1, h = kk & 1;
        uint32_t ph[4], pq[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) ph[jj] = DT::pack2(p[kb][8 * h + 2 * jj], p[kb][8 * h + 2 * jj + 1]);
        if constexpr (PQ >= 0) {
          const FqScale f4[4] = {fs, fs, fs, fs};
#pragma unroll
          for (int jq = 0; jq < 2; ++jq) {
            const f32x4 xq = fq_quad<(PQ >= 0 ? PQ : 0)>(&p[kb][8 * h + 4 * jq], f4);
            pq[2 * jq] = DT::pack2(xq[0], xq[1]);
            pq[2 * jq + 1] = DT::pack2(xq[2], xq[3]);
          }
        }
        const s16x8 bh_op = __builtin_bit_cast(s16x8, (u32x4){ph[0], ph[1], ph[2], ph[3]});
        s16x8 bq_op = bh_op;
        if constexpr (PQ >= 0) bq_op = __builtin_bit_cast(s16x8, (u32x4){pq[0], pq[1], pq[2], pq[3]});
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const s16x8 va = lds_tr8<D>(Vt, kk * 16, db * 32, lane);
          o_acc[db] = DT::mfma(va, bq_op, o_acc[db]);
          if constexpr (PQ >= 0) oh_acc[db] = DT::mfma(va, bh_op, oh_acc[db]);
        }
      }
    }
    wait_vmem();
    if (t + 1 < ntiles) finish_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  if (q0 >= Nq) return;
  const float l = l_part + shfl_xor32(l_part);
  const float inv_l = 1.0f / l;
  uint16_t* op = (uint16_t*)a.o + (size_t)bh * Nq * D;
  uint16_t* ohp = (uint16_t*)a.o_hp + (size_t)bh * Nq * D;
  if (qi < Nq) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = db * 32 + 8 * u + 4 * g;
        float vs[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if constexpr (VFP8) {
          const f32x4 sc = *reinterpret_cast<const f32x4*>(a.v_scale + (size_t)bh * D + d);
          vs[0] = sc[0]; vs[1] = sc[1]; vs[2] = sc[2]; vs[3] = sc[3];
        }
        float x[4], y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = o_acc[db][4 * u + e] * inv_l * vs[e];
          y[e] = (PQ >= 0 ? oh_acc[db][4 * u + e] : o_acc[db][4 * u + e]) * inv_l * vs[e];
        }
        *reinterpret_cast<u32x2*>(op + (size_t)qi * D + d) = (u32x2){DT::pack2(x[0], x[1]), DT::pack2(x[2], x[3])};
        *reinterpret_cast<u32x2*>(ohp + (size_t)qi * D + d) = (u32x2){DT::pack2(y[0], y[1]), DT::pack2(y[2], y[3])};
      }
    if (g == 0) a.lse[(size_t)bh * Nq + qi] = (m_used + __builtin_log2f(l)) * LN2;
  }
}

template <class DT, int D, bool CAUSAL, int PQ, int IN>
static hipError_t fwd_launch(const Shape& s, const FwdArgs& a, hipStream_t st) {
  dim3 grid(((s.Nq + FWD_BM - 1) / FWD_BM) * s.B * s.H);
  hipLaunchKernelGGL((fwd_kernel<DT, D, CAUSAL, PQ, IN>), grid, dim3(256), 0, st, a);
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
