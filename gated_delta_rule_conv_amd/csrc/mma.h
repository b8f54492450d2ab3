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
  // an operand fragment: the lane's KPL values of one step
  struct Frag {
    float v[4];
  };
  __device__ __forceinline__ static Frag frag(const float* x) {
    Frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[e] = x[e];
    return f;
  }
  __device__ __forceinline__ static void mma(f32x4& acc, const Frag& a, const Frag& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void step(f32x4& acc, const float* a, const float* b) {
    mma(acc, frag(a), frag(b));
  }
  // three independent accumulator chains (summed by total()) instead of one dependent chain
  __device__ __forceinline__ static void mma3(f32x4 (&acc)[3], const Frag& a, const Frag& b) {
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[1], b.v[1], acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[2], b.v[2], acc[2], 0, 0, 0);
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[3], b.v[3], acc[0], 0, 0, 0);
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
  struct Frag {
    bf16x8 hi, lo;
  };
  __device__ __forceinline__ static Frag frag(const float* x) {
    Frag f;
    split(x, f.hi, f.lo);
    return f;
  }
  __device__ __forceinline__ static void mma(f32x4& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void step(f32x4& acc, const float* a, const float* b) {
    mma(acc, frag(a), frag(b));
  }
  // the three products on three independent accumulator chains (summed by total())
  __device__ __forceinline__ static void mma3(f32x4 (&acc)[3], const Frag& a, const Frag& b) {
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc[2], 0, 0, 0);
  }
};

__device__ __forceinline__ void zero3(f32x4 (&acc)[3]) {
#pragma unroll
  for (int i = 0; i < 3; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}
// acc[0] + (acc[1] + acc[2]): the main products plus the two correction chains
__device__ __forceinline__ f32x4 total(const f32x4 (&acc)[3]) { return acc[0] + (acc[1] + acc[2]); }

// Operand matrices stored "pre-split": for BF16X3 an R x Cc matrix is two bf16 planes
// (hi, then lo), for FP32 one fp32 plane; both take R*Cc*4 bytes. A fragment is the
// lane's KPL values starting at (row, col); col is a multiple of KPL.
template <int POL>
struct Split;

template <>
struct Split<kPolFP32> {
  using M = Mma<kPolFP32>;
  __device__ __forceinline__ static M::Frag load(const void* base, int rows, int cols, int row, int col) {
    (void)rows;
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + (int64_t)row * cols + col);
    M::Frag f;
    f.v[0] = v.x; f.v[1] = v.y; f.v[2] = v.z; f.v[3] = v.w;
    return f;
  }
  __device__ __forceinline__ static M::Frag zero() {
    M::Frag f;
    f.v[0] = f.v[1] = f.v[2] = f.v[3] = 0.f;
    return f;
  }
  // store n (<= 8, multiple of 4) consecutive values of one row
  __device__ __forceinline__ static void store(void* base, int rows, int cols, int row, int col, const float* x, int n) {
    (void)rows;
    float* p = static_cast<float*>(base) + (int64_t)row * cols + col;
    for (int i = 0; i < n; i += 4) *reinterpret_cast<float4*>(p + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
  }
  __device__ __forceinline__ static void store1(void* base, int rows, int cols, int row, int col, float x) {
    (void)rows;
    static_cast<float*>(base)[(int64_t)row * cols + col] = x;
  }
};

template <>
struct Split<kPolBF16X3> {
  using M = Mma<kPolBF16X3>;
  __device__ __forceinline__ static M::Frag load(const void* base, int rows, int cols, int row, int col) {
    const __bf16* hi = static_cast<const __bf16*>(base) + (int64_t)row * cols + col;
    const __bf16* lo = hi + (int64_t)rows * cols;
    M::Frag f;
    f.hi = *reinterpret_cast<const bf16x8*>(hi);
    f.lo = *reinterpret_cast<const bf16x8*>(lo);
    return f;
  }
  __device__ __forceinline__ static M::Frag zero() {
    M::Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.hi[e] = f.lo[e] = static_cast<__bf16>(0.f);
    return f;
  }
  // store n (4 or 8) consecutive values of one row (8 or 16 bytes per plane)
  __device__ __forceinline__ static void store(void* base, int rows, int cols, int row, int col, const float* x, int n) {
    __bf16* hi = static_cast<__bf16*>(base) + (int64_t)row * cols + col;
    __bf16* lo = hi + (int64_t)rows * cols;
    if (n == 8) {
      bf16x8 h, l;
      M::split(x, h, l);
      *reinterpret_cast<bf16x8*>(hi) = h;
      *reinterpret_cast<bf16x8*>(lo) = l;
    } else {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 h, l;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 t = static_cast<__bf16>(x[e]);
        h[e] = t;
        l[e] = static_cast<__bf16>(x[e] - static_cast<float>(t));
      }
      *reinterpret_cast<bf16x4*>(hi) = h;
      *reinterpret_cast<bf16x4*>(lo) = l;
    }
  }
  __device__ __forceinline__ static void store1(void* base, int rows, int cols, int row, int col, float x) {
    __bf16* hi = static_cast<__bf16*>(base) + (int64_t)row * cols + col;
    const __bf16 t = static_cast<__bf16>(x);
    hi[0] = t;
    hi[(int64_t)rows * cols] = static_cast<__bf16>(x - static_cast<float>(t));
  }
};

// Operands in fragment order (global workspace). An R x K operand (row r, contraction
// index k) is cut into 16 x KSTEP fragments; fragment (rt, ks) is a block of BYTES bytes at
// block index rt * nks + ks. Inside a block, lane l's KPL values (row 16 rt + l % 16, k from
// ks * KSTEP + KPL * (l / 16)) are 16 contiguous bytes at l * 16 -- for bf16x3 the hi values,
// with the lo values 1 KiB further on. One load instruction of a wave is then one
// contiguous KiB, which the gfx950 load path moves about twice as fast as the same bytes
// gathered as 16 half cache lines.
template <int POL>
struct FragIO;

template <>
struct FragIO<kPolFP32> {
  using M = Mma<kPolFP32>;
  static constexpr int BYTES = 1024;
  __device__ __forceinline__ static M::Frag load(const char* blk, int lane) {
    const float4 v = *reinterpret_cast<const float4*>(blk + lane * 16);
    M::Frag f;
    f.v[0] = v.x; f.v[1] = v.y; f.v[2] = v.z; f.v[3] = v.w;
    return f;
  }
  __device__ __forceinline__ static void store(char* blk, int lane, const float* x) {
    *reinterpret_cast<float4*>(blk + lane * 16) = make_float4(x[0], x[1], x[2], x[3]);
  }
  __device__ __forceinline__ static void store_frag(char* blk, int lane, const M::Frag& f) { store(blk, lane, f.v); }
};

template <>
struct FragIO<kPolBF16X3> {
  using M = Mma<kPolBF16X3>;
  static constexpr int BYTES = 2048;
  __device__ __forceinline__ static M::Frag load(const char* blk, int lane) {
    M::Frag f;
    f.hi = *reinterpret_cast<const bf16x8*>(blk + lane * 16);
    f.lo = *reinterpret_cast<const bf16x8*>(blk + 1024 + lane * 16);
    return f;
  }
  __device__ __forceinline__ static void store(char* blk, int lane, const float* x) {
    bf16x8 h, l;
    M::split(x, h, l);
    *reinterpret_cast<bf16x8*>(blk + lane * 16) = h;
    *reinterpret_cast<bf16x8*>(blk + 1024 + lane * 16) = l;
  }
  // an already split fragment
  __device__ __forceinline__ static void store_frag(char* blk, int lane, const M::Frag& f) {
    *reinterpret_cast<bf16x8*>(blk + lane * 16) = f.hi;
    *reinterpret_cast<bf16x8*>(blk + 1024 + lane * 16) = f.lo;
  }
};

// Block index and lane of the fragment slot holding (row r, k0), k0 a multiple of KPL.
template <int POL>
__device__ __forceinline__ void frag_slot(int r, int k0, int nks, int& blk, int& lane) {
  using M = Mma<POL>;
  blk = (r / 16) * nks + k0 / M::KSTEP;
  lane = r % 16 + 16 * ((k0 % M::KSTEP) / M::KPL);
}

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
