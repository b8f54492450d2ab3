// 16x16 MFMA tiles for gfx950 with two precision policies.
//
// Output layout of every 16x16 tile (v_mfma_f32_16x16x*): lane l holds rows
// 4*(l/16) + r (r = 0..3) of column l%16. Operand A is read by rows (lane l: row l%16),
// operand B by columns (lane l: column l%16). Which k a lane supplies in a step is our
// choice, as long as A and B use the same assignment: here lane l supplies k in
// [KPL*(l/16) + KSTEP*v, +KPL) in step v, so each lane reads KPL contiguous values of a
// row of A and of a column of B (a row of B^T).
//
//  FP32   : v_mfma_f32_16x16x4_f32, KPL = 4 (one float4 per lane per step, KSTEP 16).
//  BF16X3 : v_mfma_f32_16x16x32_bf16, KPL = 8 (KSTEP 32). Each fp32 operand value x is
//           split into hi = bf16_rne(x) and lo = bf16_rne(x - hi); the product is
//           lo*hi + hi*lo + hi*hi accumulated in fp32 (the "bf16x3" scheme of Henry,
//           Tang & Heinecke, ARITH 2019), about 16 significant bits per operand.
#pragma once

#include "device_common.h"

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kPolFP32 = 1;
constexpr int kPolBF16X3 = 2;

template <int POL>
struct Mma;

template <>
struct Mma<kPolFP32> {
  static constexpr int KPL = 4;
  static constexpr int KSTEP = 16;
  __device__ __forceinline__ static void step(f32x4& acc, const float* a, const float* b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  }
};

template <>
struct Mma<kPolBF16X3> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 32;
  __device__ __forceinline__ static void split(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 h = static_cast<__bf16>(x[e]);
      hi[e] = h;
      lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
    }
  }
  __device__ __forceinline__ static void step(f32x4& acc, const float* a, const float* b) {
    bf16x8 ah, al, bh, bl;
    split(a, ah, al);
    split(b, bh, bl);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  }
};

// KPL contiguous floats from p (16-byte aligned): global or LDS.
template <int KPL>
__device__ __forceinline__ void load_k(const float* p, float* out) {
#pragma unroll
  for (int i = 0; i < KPL / 4; ++i) {
    const float4 v = reinterpret_cast<const float4*>(p)[i];
    out[4 * i] = v.x;
    out[4 * i + 1] = v.y;
    out[4 * i + 2] = v.z;
    out[4 * i + 3] = v.w;
  }
}

}  // namespace gdn
