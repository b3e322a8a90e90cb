// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 XCDs, blocks are dealt round-robin
// s_getreg_b32 operand for HW_REG_XCC_ID (register 20, bits 3:0): the XCD
// the wave runs on.
constexpr int kHwRegXccId = 20 | (3 << 11);

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
  return __uint_as_float(packed & 0xFFFF0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Eight OCP e4m3 codes (k order: byte 0 first) -> eight bf16, exactly (every
// e4m3 value is a bf16 value); v_cvt_scalef32_pk_bf16_fp8 with scale 1.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// ------------------------------------------------------------------ math

__device__ __forceinline__ float sigmoid_f32(float v) { return 1.0f / (1.0f + expf(-v)); }

// SiLU(g) * u with the optional clamp: g <= L, -L <= u <= L when L > 0.
// SiLU(g) = g / (1 + e^-g) with e^-g = 2^(-g log2 e) from v_exp_f32 and the
// reciprocal from v_rcp_f32 (each about 1 ulp): the result is rounded to
// bf16 right after, so the approximation is far below that rounding.
// Large negative g: 2^(large) = inf, 1/inf = 0, SiLU -> -0.
__device__ __forceinline__ float swiglu_f32(float g, float u, float limit) {
  if (limit > 0.0f) {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
  }
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// ------------------------------------------------------------------ MFMA
// v_mfma_f32_32x32x16_bf16: A 32x16, B 16x32, C 32x32.  Lane l supplies row
// (l % 32) of A and column (l % 32) of B, eight consecutive k each, lanes
// 32..63 the upper eight.  C: lane l holds column l % 32, register r holds
// row 8 * (r / 4) + 4 * (l / 32) + (r % 4).
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// ---------------------------------------------------------- XCD mapping
// Blocks are dispatched to XCDs round-robin (block b -> XCD b % 8).  Given
// `nvalid` units of work, give each XCD a contiguous range of units so that
// blocks sharing operands share an L2.  Returns -1 for a block without work.
__host__ __device__ __forceinline__ int xcd_remap(int bid, int nvalid) {
  const int per = (nvalid + kNumXcd - 1) / kNumXcd;
  const int xcd = bid % kNumXcd;
  const int slot = bid / kNumXcd;
  if (slot >= per) return -1;
  const int u = xcd * per + slot;
  return u < nvalid ? u : -1;
}

// As xcd_remap, but the last `nlast` units (0 <= nlast <= nvalid) are dealt
// over the XCDs one at a time and come first in each XCD's order, while the
// others keep contiguous ranges: each XCD runs at most ceil(nlast / 8) of
// them, all in its first round.  Needs ceil(nvalid / 8) + 1 blocks per XCD.
__host__ __device__ __forceinline__ int xcd_remap_dealt(int bid, int nvalid, int nlast) {
  const int nr = nvalid - nlast;
  const int xcd = bid % kNumXcd;
  const int slot = bid / kNumXcd;
  const int mine = nlast / kNumXcd + (xcd < nlast % kNumXcd ? 1 : 0);
  if (slot < mine) return nr + slot * kNumXcd + xcd;
  const int per = (nr + kNumXcd - 1) / kNumXcd;
  const int s = slot - mine;
  if (s >= per) return -1;
  const int u = xcd * per + s;
  return u < nr ? u : -1;
}

__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

}  // namespace moe
