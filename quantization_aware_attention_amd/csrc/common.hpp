// Shared device helpers for the gfx950 quantization-aware attention kernels:
// vector types, MFMA wrappers, the LDS tile swizzle, the transposing LDS read,
// dtype packing and the fake quantizer FQ.
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_{bf16,f16}),
// lane l in 0..63, g = l / 32:
//   A[m][k]: lane holds m = l % 32, k = 8g + j (j = 0..7, one 16-byte operand)
//   B[k][n]: lane holds n = l % 32, k = 8g + j
//   C[m][n]: lane holds n = l % 32, m = 8(r/4) + 4g + r%4 (r = 0..15)
// An accumulator block therefore gives each lane one column n and 16 rows m;
// the 16 rows of registers 8h..8h+7 (h = 0, 1) are the rows
// 16h + 8(j/4) + 4g + j%4, which is exactly the k order a 16-deep operand
// needs when those registers are reused as an A or B operand ("permuted k").
// Tiles read from LDS as the other operand follow the same permuted k order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qat {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int P_GROUP = 64;          // key columns per P-quant scale
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------- dtypes
struct BF16 {
  typedef __bf16 scalar;
  typedef bf16x8 vec8;
  __device__ static inline f32x16 mfma(const s16x8& a, const s16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16((bf16x8)a, (bf16x8)b, c, 0, 0, 0);
  }
  // two fp32 -> packed pair (round to nearest even)
  __device__ static inline uint32_t pack2(float x, float y) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static inline float to_f32(uint16_t bits) {
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
  }
};

struct FP16 {
  typedef _Float16 scalar;
  typedef f16x8 vec8;
  __device__ static inline f32x16 mfma(const s16x8& a, const s16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16((f16x8)a, (f16x8)b, c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float x, float y) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 v = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static inline float to_f32(uint16_t bits) {
    return (float)__builtin_bit_cast(_Float16, bits);
  }
};

// ---------------------------------------------------------------- LDS tiles
// A tile of R rows x D 16-bit elements lives in LDS as rows of D*2 bytes,
// split into 16-byte chunks; chunk c of row R is stored at chunk position
// c ^ swz(R).  With D = 128 this makes both access patterns conflict-free:
//  * 16 consecutive rows, one chunk each (row-major operand reads), and
//  * 4 consecutive rows x 4 consecutive chunks (transposing reads).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (row >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {  // byte offset
  return row * (D * 2) + ((chunk ^ swz<D>(row)) << 4);
}

// Row-major operand: 8 consecutive elements (one chunk) of `row`.
template <int D>
__device__ __forceinline__ s16x8 lds_row8(const char* tile, int row, int chunk) {
  return *reinterpret_cast<const s16x8*>(tile + tile_off<D>(row, chunk));
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed operand for a 16-deep k step: lane l receives the elements
// (row0 + 8(j/4) + 4g + j%4, col0 + l%32) for j = 0..7, i.e. one column of
// the tile over the permuted k order, from two ds_read_b64_tr_b16.
// Within each 16-lane group the instruction hands lane i, slot s, element
// i%4 of the 8 bytes read by lane 4s + i/4; so lane (4s + q) of the group
// reads row (base + s), columns col0 + 16*(group%2) + 4q .. +3.
// Byte offset in the tile of lane `lane`'s 8-byte read of rows row0..row0+7;
// the second read of the step is at tr8_off(row0 + 8, ...).  Moving row0 by
// a multiple of 16 moves the offset by as many rows (the swizzle depends on
// the row's low four bits only).
template <int D>
__device__ __forceinline__ int tr8_off(int row0, int col0, int lane) {
  const int G = lane >> 4, i = lane & 15, g = lane >> 5;
  const int row = row0 + 4 * g + (i >> 2);
  const int col = col0 + 16 * (G & 1) + 4 * (i & 3);
  return tile_off<D>(row, col >> 3) + (col & 7) * 2;
}
__device__ __forceinline__ s16x8 lds_tr8_at(const char* p0, const char* p1) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  return (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <int D>
__device__ __forceinline__ s16x8 lds_tr8(const char* tile, int row0, int col0, int lane) {
  return lds_tr8_at(tile + tr8_off<D>(row0, col0, lane), tile + tr8_off<D>(row0 + 8, col0, lane));
}

typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous copy of [BN x D] 16-bit tiles from HBM into the swizzled LDS
// layout with buffer_load_dwordx4 ... lds: every wave instruction fills one
// contiguous KiB of LDS (lane l -> bytes 16l..16l+15), so lane l fetches the
// global chunk that belongs at that LDS position.  The per-lane source
// offsets are fixed for the whole loop; each copy only adds a wave-uniform
// base.  Rows past `nrows` are clamped to the last valid row (finite data;
// the kernels mask those rows).  The buffer resource spans the tile, so an
// offset outside it would read zeros rather than fault.  (The compiler counts
// the global_load_lds form as a flat access that may touch LDS, and while one
// is in flight it waits for every LDS read with lgkmcnt(0), which serialises
// an operand stream behind the latest read.)  Each of the NW waves issues
// (BN*D*2/1024)/NW instructions.  Only the offset of the wave's first KiB is
// held: the swizzles split into a part of the KiB index and a part of the
// lane (disjoint bits), so KiB u of the wave is that offset with the chunk
// bits XORed by a wave-uniform term, plus u KiB.
template <int D, int BN, int NW>
struct TileCopy {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CPR = ROW_BYTES / 16;                 // chunks per row
  static constexpr int ROWS_PER_KIB = 1024 / ROW_BYTES;
  static constexpr int KIB = BN * ROW_BYTES / 1024;
  static constexpr int PER_WAVE = KIB / NW;
  static_assert(KIB % NW == 0, "tile must split evenly over the waves");
  uint32_t off0;   // byte offset of this lane's source chunk in the wave's first KiB
  int wave;        // wave index (uniform)

  __device__ __forceinline__ void init(int wave_uniform, int lane) {
    wave = wave_uniform;
    const int row = wave * PER_WAVE * ROWS_PER_KIB + lane / CPR;
    off0 = (uint32_t)(row * ROW_BYTES + (((lane % CPR) ^ swz<D>(row)) * 16));
  }
  __device__ __forceinline__ uint32_t offset(int u) const {
    const int b0 = wave * PER_WAVE * ROWS_PER_KIB, bu = b0 + u * ROWS_PER_KIB;
    return (off0 ^ (uint32_t)((swz<D>(bu) ^ swz<D>(b0)) << 4)) + u * 1024;
  }
  // Copy rows [row0, row0 + BN) of src ([nrows x D]) into lds_tile.
  __device__ __forceinline__ void issue(char* lds_tile, const uint16_t* src, int row0, int nrows) const {
    const char* base = reinterpret_cast<const char*>(src + (size_t)row0 * D);
    const bool full = row0 + BN <= nrows;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, KIB * 1024, 0x00020000);
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      uint32_t o = offset(u);
      if (!full) {   // tail tile: clamp the row, keep the column
        const int row = (int)(o / ROW_BYTES);
        const int r = min(row0 + row, nrows - 1) - row0;
        o = (uint32_t)(r * ROW_BYTES) + (o % ROW_BYTES);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_tile + (wave * PER_WAVE + u) * 1024), 16, o, 0,
                                               0, 0);
    }
  }
};

// Wait for this wave's outstanding global loads (including LDS DMA).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// ---------------------------------------------------------------- FQ
struct FqScale { float s, r; };

// FMT: 0 = e4m3fn (FMAX 448), 1 = e5m2 (FMAX 57344)
template <int FMT> struct Fp8Fmt;
template <> struct Fp8Fmt<0> {
  static constexpr float FMAX = 448.0f;
  __device__ static inline uint32_t cvt2(float a, float b) {   // RNE onto the e4m3 grid
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
  }
  __device__ static inline f32x2 val2(uint32_t pk) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)pk, false);
  }
};
template <> struct Fp8Fmt<1> {
  static constexpr float FMAX = 57344.0f;
  __device__ static inline uint32_t cvt2(float a, float b) {   // RNE onto the e5m2 grid
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false) & 0xFFFFu;
  }
  __device__ static inline f32x2 val2(uint32_t pk) {
    return __builtin_amdgcn_cvt_pk_f32_bf8((int)pk, false);
  }
};

// One group's scale pair from its absmax a: s = a/FMAX and r = FMAX/a, each
// the correctly rounded fp32 quotient; a == 0 or an r that overflows gives
// s = r = 0 (the group quantizes to zeros).  Computed without the division
// sequence (a dependent chain of about a dozen instructions per quotient):
//  * s: s0 = a*z with z = RN(1/FMAX); the remainder a - s0*FMAX is exact in
//    one fma, and s0 + remainder*z rounds to the correctly rounded quotient;
//  * r: the hardware reciprocal of a refined by one Newton step (y1), then
//    q = FMAX*y1 corrected by its exact remainder FMAX - a*q (Markstein's
//    correction).  From a = 2^64 up, a and FMAX are both scaled by 2^-32
//    first (exact), which keeps 1/a out of the subnormal range.
// Both FMAX values are 1.75 * 2^k.  For every positive finite fp32 a, s, r
// and the flush decision equal those of the two IEEE divisions: checked
// exhaustively, for both formats, by qat_selftest_fq_scale.
template <int FMT>
__device__ __forceinline__ FqScale fq_scale(float a) {
  constexpr float F = Fp8Fmt<FMT>::FMAX;
  constexpr float z = 1.0f / F;
  const float s0 = a * z;
  const float s = __builtin_fmaf(__builtin_fmaf(-s0, F, a), z, s0);
  const bool big = a >= 0x1p64f;
  const float as = big ? a * 0x1p-32f : a;
  const float fs = big ? F * 0x1p-32f : F;
  const float y = __builtin_amdgcn_rcpf(as);
  const float y1 = __builtin_fmaf(__builtin_fmaf(-as, y, 1.0f), y, y);
  const float q = fs * y1;
  const float r = __builtin_fmaf(__builtin_fmaf(-as, q, fs), y1, q);
  const bool ok = (a > 0.0f) && (r <= 3.402823466e38f);
  FqScale out;
  out.s = ok ? s : 0.0f;
  out.r = ok ? r : 0.0f;
  return out;
}

// Fake-quantize a pair of values: v = fp32(x*r), code = RNE(v), x^ = fp32(code*s).
// The two values may belong to different groups (scales q0, q1).  Returns
// the dequantized pair; *codes gets the two 8-bit codes (low byte first).
template <int FMT>
__device__ __forceinline__ f32x2 fq_pair2(float x0, float x1, FqScale q0, FqScale q1,
                                          uint32_t* codes = nullptr) {
  const float v0 = x0 * q0.r;
  const float v1 = x1 * q1.r;
  const uint32_t pk = Fp8Fmt<FMT>::cvt2(v0, v1);
  if (codes) *codes = pk;
  const f32x2 c = Fp8Fmt<FMT>::val2(pk);
  f32x2 out;
  out[0] = c[0] * q0.s;
  out[1] = c[1] * q1.s;
  return out;
}
template <int FMT>
__device__ __forceinline__ f32x2 fq_pair(float x0, float x1, FqScale q, uint32_t* codes = nullptr) {
  return fq_pair2<FMT>(x0, x1, q, q, codes);
}

// Four values, each with its own scale pair: the four codes share one dword
// (low word first), so no register clearing or masking is needed.
template <int FMT>
__device__ __forceinline__ f32x4 fq_quad(const float x[4], const FqScale q[4]) {
  // The first conversion writes the low half of its destination and keeps the
  // high half of its third operand, which the second conversion overwrites:
  // passing a product that dies there lets the destination take its register
  // (no copy of a live value into a fresh one).
  const float v0 = x[0] * q[0].r, v1 = x[1] * q[1].r, v2 = x[2] * q[2].r, v3 = x[3] * q[3].r;
  int pk;
  if constexpr (FMT == 0) {
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, __builtin_bit_cast(int, v0), false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, pk, true);
  } else {
    pk = __builtin_amdgcn_cvt_pk_bf8_f32(v0, v1, __builtin_bit_cast(int, v0), false);
    pk = __builtin_amdgcn_cvt_pk_bf8_f32(v2, v3, pk, true);
  }
  f32x2 lo, hi;
  if constexpr (FMT == 0) {
    lo = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
    hi = __builtin_amdgcn_cvt_pk_f32_fp8(pk, true);
  } else {
    lo = __builtin_amdgcn_cvt_pk_f32_bf8(pk, false);
    hi = __builtin_amdgcn_cvt_pk_f32_bf8(pk, true);
  }
  return (f32x4){lo[0] * q[0].s, lo[1] * q[1].s, hi[0] * q[2].s, hi[1] * q[3].s};
}

// The four 8-bit codes of fq_quad (same conversions, byte e = code of x[e]),
// for callers that feed the codes themselves to an fp8 MFMA.
template <int FMT>
__device__ __forceinline__ int fq_codes4(const float x[4], float r) {
  const float v0 = x[0] * r, v1 = x[1] * r, v2 = x[2] * r, v3 = x[3] * r;
  int pk;   // (third operand of the first conversion: as in fq_quad)
  if constexpr (FMT == 0) {
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, __builtin_bit_cast(int, v0), false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, pk, true);
  } else {
    pk = __builtin_amdgcn_cvt_pk_bf8_f32(v0, v1, __builtin_bit_cast(int, v0), false);
    pk = __builtin_amdgcn_cvt_pk_bf8_f32(v2, v3, pk, true);
  }
  return pk;
}

// ---------------------------------------------------------------- fp8 MFMA
// v_mfma_f32_32x32x64_f8f6f4 with A = e5m2 codes and B = FMT codes (0 e4m3fn,
// 1 e5m2), unit block scales (E8M0 127).  Operand: 32 bytes per lane; lane l
// supplies row m (A) or column n (B) = l % 32 and 32 of the 64 k values, the
// half selected by l / 32.  Any assignment of those 32 k values to bytes works
// as long as A and B use the same one.  C has the 32x32x16 layout.
template <int FMT>
__device__ __forceinline__ f32x16 mfma_f8_bf8a(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 1, FMT, 0, 127, 0, 127);
}

// LDS tile of 8-bit codes: rows of D bytes in 16-byte chunks, chunk c of row
// R stored at c ^ vc_swz(R).  A half-wave of transposing reads touches eight
// rows (R0 + 0..3, R0 + 8..11; R0 a multiple of 4 with bit 3 clear) at two
// adjacent chunks (2k, 2k + 1); rows of equal parity share a 256-byte bank
// line, so the four of each parity get the even offsets 0, 2, 4, 6 and their
// 4 x 2 chunks fall on eight distinct bank groups.
template <int D>
__device__ __forceinline__ int vc_swz(int row) {
  return (2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1))) & (D / 16 - 1);
}
// byte offset of the 8-byte half `h8` (0..2D/16-1 over the row) of row `row`
template <int D>
__device__ __forceinline__ int vc_off(int row, int h8) {
  return row * D + (((h8 >> 1) ^ vc_swz<D>(row)) << 4) + ((h8 & 1) << 3);
}

typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// A operand of the fp8 MFMA holding V^T codes for columns 32*db .. +31 of a
// 64-key code tile: byte j = 8r + s of lane l (column d = 32db + l%32, half
// g = l/32) is the code of key 32(r/2) + 16(r%2) + 8(s/4) + 4g + s%4, from
// four ds_read_b64_tr_b8.  Within a 16-lane group that instruction hands
// lane i, slot s, byte i%8 of the 8 bytes read by lane 2s + i/8; so lane
// 2s + b of the group reads that key's row at 8-byte half 4db + 2((l/16)%2) + b.
// The matching B operand holds in dword 4kb + u, bytes e = 0..3, the codes of
// keys 32kb + 8u + 4g + e: the keys a query lane owns in the S^T layout.
// Dwords 2r, 2r+1 alone are the 16-deep k step r in the permuted k order of
// the 16-bit MFMAs (element j = slot j).
template <int D>
__device__ __forceinline__ i32x8 lds_vcode_tr(const char* tile, int db, int lane) {
  const int G = lane >> 4, L = lane & 15, g = lane >> 5, s = L >> 1;
  const int h8 = 4 * db + 2 * (G & 1) + (L & 1);
  i32x8 out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 32 * (r >> 1) + 16 * (r & 1) + 8 * (s >> 2) + 4 * g + (s & 3);
    const i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(tile + vc_off<D>(row, h8)));
    out[2 * r] = t[0];
    out[2 * r + 1] = t[1];
  }
  return out;
}

// Eight e5m2 codes (two dwords, byte j = element j) -> eight fp16 values:
// an e5m2 code is the high byte of the fp16 with the same value.
__device__ __forceinline__ s16x8 e5m2x8_to_f16(int lo, int hi) {
  const uint32_t a = __builtin_amdgcn_perm(lo, lo, 0x010c000cu), b = __builtin_amdgcn_perm(lo, lo, 0x030c020cu);
  const uint32_t c = __builtin_amdgcn_perm(hi, hi, 0x010c000cu), d = __builtin_amdgcn_perm(hi, hi, 0x030c020cu);
  return __builtin_bit_cast(s16x8, (u32x4){a, b, c, d});
}

// LDS tile of 8-bit codes that is read row-major (the fp8 MFMA operands of
// per-token Q and K codes): rows of D bytes in 16-byte chunks, chunk c of row
// R stored at c ^ f8_swz(R).  Eight consecutive rows reading one chunk each
// fall on eight distinct 16-byte bank groups of a 128-byte line, and so do
// the even and the odd rows of sixteen consecutive ones.
template <int D>
__device__ __forceinline__ int f8_swz(int row) {
  if constexpr (D == 128) return (row ^ (row >> 3)) & 7;
  else return (row ^ (row >> 2)) & 3;
}
template <int D>
__device__ __forceinline__ int f8_off(int row, int chunk) {
  return row * D + ((chunk ^ f8_swz<D>(row)) << 4);
}
// One 16-byte chunk of a row of codes (half of an fp8 MFMA operand).
template <int D>
__device__ __forceinline__ s16x8 lds_f8row(const char* tile, int row, int chunk) {
  return *reinterpret_cast<const s16x8*>(tile + f8_off<D>(row, chunk));
}
// C += A B over 64 k of e4m3 codes (v_mfma_f32_32x32x64_f8f6f4, unit block
// scales): lane l holds row or column l % 32 and, in its two 16-byte halves,
// the 32 codes k = 32 (l / 32) + 0..31 of the k step, for A and B alike.
__device__ __forceinline__ f32x16 mfma_e4m3(const s16x8& alo, const s16x8& ahi, const s16x8& blo,
                                            const s16x8& bhi, const f32x16& c) {
  const u32x4 a0 = __builtin_bit_cast(u32x4, alo), a1 = __builtin_bit_cast(u32x4, ahi);
  const u32x4 b0 = __builtin_bit_cast(u32x4, blo), b1 = __builtin_bit_cast(u32x4, bhi);
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Asynchronous copy of [BN x D] 8-bit code tiles from HBM into the vc_swz
// layout (ROWMAJOR: the f8_swz layout) with buffer_load_dwordx4 ... lds (same
// scheme as TileCopy).
template <int D, int BN, int NW, bool ROWMAJOR = false>
struct CodeCopy {
  static constexpr int CPR = D / 16;                   // 16-byte chunks per row
  static constexpr int ROWS_PER_KIB = 1024 / D;
  static constexpr int KIB = BN * D / 1024;
  static constexpr int PER_WAVE = KIB / NW;
  static_assert(KIB % NW == 0, "tile must split evenly over the waves");
  uint32_t off0;   // as in TileCopy: the first KiB's offset, the others derived
  int wave;

  __device__ __forceinline__ static int sw(int row) { return ROWMAJOR ? f8_swz<D>(row) : vc_swz<D>(row); }
  __device__ __forceinline__ void init(int wave_uniform, int lane) {
    wave = wave_uniform;
    const int row = wave * PER_WAVE * ROWS_PER_KIB + lane / CPR;
    off0 = (uint32_t)(row * D + (((lane % CPR) ^ sw(row)) * 16));
  }
  __device__ __forceinline__ uint32_t offset(int u) const {
    const int b0 = wave * PER_WAVE * ROWS_PER_KIB, bu = b0 + u * ROWS_PER_KIB;
    return (off0 ^ (uint32_t)((sw(bu) ^ sw(b0)) << 4)) + u * 1024;
  }
  __device__ __forceinline__ void issue(char* lds_tile, const uint8_t* src, int row0, int nrows) const {
    const char* base = reinterpret_cast<const char*>(src + (size_t)row0 * D);
    const bool full = row0 + BN <= nrows;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, KIB * 1024, 0x00020000);
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      uint32_t o = offset(u);
      if (!full) {
        const int row = (int)(o / D);
        const int r = min(row0 + row, nrows - 1) - row0;
        o = (uint32_t)(r * D) + (o % D);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_tile + (wave * PER_WAVE + u) * 1024), 16, o, 0,
                                               0, 0);
    }
  }
};

// ---------------------------------------------------------------- work order
// MI355X deals the workgroups of a launch to its 8 XCDs round-robin by linear
// id, and each XCD has its own L2.  xcd_unit() renumbers the launch so that
// every XCD receives one contiguous range of work units: the tiles of one
// (batch, head) then run on the same XCD and share its L2 for the K/V (or
// Q/dO) tiles they all stream.  Bijective on [0, total).
constexpr int NUM_XCD = 8;
__device__ __forceinline__ int xcd_unit(int linear, int total) {
  const int x = linear % NUM_XCD, idx = linear / NUM_XCD;
  const int base = total / NUM_XCD, rem = total % NUM_XCD;
  return x * base + min(x, rem) + idx;
}

// Work order of a launch over BH (batch, head) pairs x nblk blocks per pair.
// Equal blocks (non-causal): xcd_unit's XCD-contiguous, head-major order, so
// the blocks of one head share an L2.  Causal blocks differ in length up to
// nblk-fold, and greedy dispatch of a head-by-head sequence can start long
// blocks last; they are ordered longest first across the whole launch (all
// heads' longest blocks, then the next longest, ...), and the round-robin
// dealing of workgroups to XCDs mixes the lengths on every XCD.
// Sets the head and the block's rank (causal: 0 = longest).
__device__ __forceinline__ void work_unit(int linear, int total, int nblk, bool longest_first, int* bh,
                                          int* rank) {
  if (longest_first) {
    const int nbh = total / nblk;
    *bh = linear % nbh;
    *rank = linear / nbh;
  } else {
    const int unit = xcd_unit(linear, total);
    *bh = unit / nblk;
    *rank = unit % nblk;
  }
}

// ---------------------------------------------------------------- misc
// Combine a value with the one held by lane l ^ 32.  v_permlane32_swap
// exchanges the upper 32 lanes of its first operand with the lower 32 lanes
// of its second; with x in both, each lane ends up holding its own value in
// one result and its partner's in the other, so a symmetric combination of
// the two takes two VALU instructions: no LDS round trip (ds_bpermute, which
// waits behind the other waves' operand reads) and no lane select.  The two
// results are read straight from the builtin's return value: copied into a
// vector first, the second one is lost in code generation.
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// v_exp_f32.  The kernels take a row group's P absmax as exp2 of the largest
// argument (instead of a max over the exp2 results); that is exact because
// this instruction is monotone non-decreasing over every fp32 argument the
// kernels can produce (checked exhaustively by qat_selftest_exp2_monotone).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Issue priority of this wave relative to the other wave on its SIMD: raised
// around runs of MFMAs so that they issue as soon as their operands are
// ready, while the other wave's VALU work fills the gaps.
__device__ __forceinline__ void prio_mfma() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void prio_valu() { __builtin_amdgcn_s_setprio(0); }

// Wave index as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

}  // namespace qat
