// Shared device helpers for the LoLA HIP kernels (gfx950 / CDNA4).
//
// MFMA conventions used throughout (checked on the device by a layout probe):
//   v_mfma_f32_32x32x16_{bf16,f16}: A is 32 x 16 (M x K), B is 16 x 32 (K x N).
//     Lane l supplies row/column (l % 32) and 8 K-values; half h = l / 32
//     supplies the K-slots of its half.  Output lane l holds column (l % 32)
//     and rows 8*(i/4) + 4*h + (i%4), i = 0..15.
// Because a contraction may permute its K index freely (as long as A and B
// agree), a C-layout result can feed the next MFMA directly: within a 16-wide
// K-block the lane's K-slots are then
//     sigma_h(j) = 4h + j (j < 4),  8 + 4h + (j - 4) (j >= 4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lola {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int WAVE = 64;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ---- scalar conversions -------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}
// round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950), two at
// a time: a in the low half, b in the high half
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  return cvt_pk_bf16(x, 0.f) & 0xFFFFu;
}
__device__ __forceinline__ __bf16 bits_to_bf16(uint32_t b) {
  return __builtin_bit_cast(__bf16, (uint16_t)b);
}
// x = hi + lo with hi, lo bf16; |x - hi - lo| <= 2^-16 |x|
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(x);
  lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

// Pack 8 bf16 bit patterns held as uint32 (low 16 bits) into an operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(const uint32_t* b) {
  u32x4 w;
  w[0] = b[0] | (b[1] << 16);
  w[1] = b[2] | (b[3] << 16);
  w[2] = b[4] | (b[5] << 16);
  w[3] = b[6] | (b[7] << 16);
  return __builtin_bit_cast(bf16x8, w);
}
// Split 8 floats into hi and lo bf16 operands.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) split_bf16(x[j], h[j], l[j]);
  hi = pack_bf16x8(h);
  lo = pack_bf16x8(l);
}

// x = hi + lo with hi, lo fp16; |x - hi - lo| <= 2^-22 |x| for |x| in the
// fp16 normal range (absolute error <= 2^-25 below it); |x| < 65504 required.
__device__ __forceinline__ void split_f16(float x, uint32_t& hi, uint32_t& lo) {
  _Float16 h = (_Float16)x;
  _Float16 l = (_Float16)(x - (float)h);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ u32x4 pack8(const uint32_t* b) {
  u32x4 w;
  w[0] = b[0] | (b[1] << 16);
  w[1] = b[2] | (b[3] << 16);
  w[2] = b[4] | (b[5] << 16);
  w[3] = b[6] | (b[7] << 16);
  return w;
}

// ---- element types of the inputs --------------------------------------
// The tag fixes the storage dtype and the 16-bit format that fp32 quantities
// are split into for MFMA (x = hi + lo, products hi*hi + hi*lo + lo*hi):
//  * BF16 inputs: inputs are exact in one bf16 operand; fp32 quantities
//    (phi, H, s) split into bf16 hi/lo (full fp32 range, ~2^-16 per product).
//  * F32 inputs: every operand splits into fp16 hi/lo (~2^-22 per product,
//    magnitudes below 65504).
struct BF16 {
  using T = uint16_t;
  static constexpr bool kSplit = false;     // inputs are exact in one pass
  __device__ static __forceinline__ float to_f32(T x) { return bf16_bits_to_f32(x); }
  __device__ static __forceinline__ void split(float x, uint32_t& hi, uint32_t& lo) {
    split_bf16(x, hi, lo);
  }
  __device__ static __forceinline__ float from_bits(uint32_t b) { return bf16_bits_to_f32(b); }
  __device__ static __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return mfma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c);
  }
};
struct F32 {
  using T = float;
  static constexpr bool kSplit = true;      // inputs need hi + lo
  __device__ static __forceinline__ float to_f32(T x) { return x; }
  __device__ static __forceinline__ void split(float x, uint32_t& hi, uint32_t& lo) {
    split_f16(x, hi, lo);
  }
  __device__ static __forceinline__ float from_bits(uint32_t b) { return f16_bits_to_f32(b); }
  __device__ static __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return mfma_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c);
  }
};

// Split 8 floats into hi and lo operands in the tag's 16-bit format.
template <class DT>
__device__ __forceinline__ void splitop(const float* x, u32x4& hi, u32x4& lo) {
  if constexpr (DT::kSplit) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) DT::split(x[j], h[j], l[j]);
    hi = pack8(h);
    lo = pack8(l);
  } else {
    // bf16 pairs: hi = RNE(x), lo = RNE(x - hi), both exact RNE as split_bf16
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t hp = cvt_pk_bf16(x[2 * j], x[2 * j + 1]);
      hi[j] = hp;
      lo[j] = cvt_pk_bf16(x[2 * j] - __uint_as_float(hp << 16),
                          x[2 * j + 1] - __uint_as_float(hp & 0xFFFF0000u));
    }
  }
}
__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Load 8 consecutive input elements as float.
__device__ __forceinline__ void load8_f32(const uint16_t* p, float* o) {
  u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = __uint_as_float(w[j] << 16);
    o[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8_f32(const float* p, float* o) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) { o[j] = a[j]; o[4 + j] = b[j]; }
}
// Load 8 consecutive bf16 input elements directly as an operand.
__device__ __forceinline__ bf16x8 load8_bf16op(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// ---- wave reductions ---------------------------------------------------
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
// One DPP move of a 64-bit value (both halves); lanes without a source (or
// in rows outside ROWMASK) get `ident`.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x, uint64_t ident) {
  const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)ident, (int)(uint32_t)x, CTRL, ROWMASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(ident >> 32), (int)(uint32_t)(x >> 32), CTRL, ROWMASK, 0xf, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
// Wave minimum and maximum of 64-bit keys, valid in lane 63 (the scan steps
// of wave_incl_scan below with min / max in place of +).
__device__ __forceinline__ void wave_minmax_u64(uint64_t& mn, uint64_t& mx) {
  auto step = [&](uint64_t a, uint64_t b) { mn = a < mn ? a : mn; mx = b > mx ? b : mx; };
  step(dpp_u64<0x111, 0xf>(mn, ~0ull), dpp_u64<0x111, 0xf>(mx, 0ull));
  step(dpp_u64<0x112, 0xf>(mn, ~0ull), dpp_u64<0x112, 0xf>(mx, 0ull));
  step(dpp_u64<0x114, 0xf>(mn, ~0ull), dpp_u64<0x114, 0xf>(mx, 0ull));
  step(dpp_u64<0x118, 0xf>(mn, ~0ull), dpp_u64<0x118, 0xf>(mx, 0ull));
  step(dpp_u64<0x142, 0xa>(mn, ~0ull), dpp_u64<0x142, 0xa>(mx, 0ull));
  step(dpp_u64<0x143, 0xc>(mn, ~0ull), dpp_u64<0x143, 0xc>(mx, 0ull));
}

// inclusive prefix sum over the wave, with DPP moves (no LDS round trips):
// shifts by 1, 2, 4, 8 within each row of 16 lanes (lanes shifted in from
// outside the row add 0), then the last lane of row 0 is added to row 1 and
// that of row 2 to row 3 (row_bcast:15), then lane 31 to rows 2 and 3
// (row_bcast:31)
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// Staging of rows of 16-bit elements in LDS for transposing reads: a row of
// P 16-byte pieces is stored unpadded with its pieces permuted (XOR of the
// piece index with a function of the row), so that the four consecutive rows
// one transposing read touches fall on distinct banks.  Element offset of
// (row, col), col % 4 == 0.
template <int P>
__device__ __forceinline__ int stg_off(int row, int col) {
  static_assert(P == 4 || P == 8 || P == 16, "rows of 64, 128 or 256 bytes");
  const int x = P == 16 ? 4 * (row & 3) : P == 8 ? 4 * ((row >> 1) & 1) : 0;
  return row * (8 * P) + ((((col >> 3) ^ x)) << 3) + (col & 7);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i names 4 16-bit elements of row i / 4, columns 4 (i % 4) .. of a
// 4 x 16 block, and receives column i of the block (its 4 rows, in order).
__device__ __forceinline__ u32x2 ld_tr(const uint16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)p));
}

}  // namespace lola
