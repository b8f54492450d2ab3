// Device helpers shared by the gfx950 kernels of the GDN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kWave = 64;  // CDNA wavefront width

// Native clang vector (the nontemporal builtins and MFMA operands need these).
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Waits until every vector memory load and store this wave has issued is complete:
// s_waitcnt with vmcnt = 0 and the export and LDS/scalar counters at their maxima (7, 15),
// i.e. not waited on (gfx9 field layout: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Waits until at most N vector memory operations of this wave are outstanding (the N
// issued last may still be in flight; on gfx9 a wave's loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_leaving() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Load 8 consecutive elements of dtype T as fp32 (16-byte aligned for bf16,
// 32 bytes for fp32).
template <typename T>
struct Vec8;

template <>
struct Vec8<float> {
  // raw = the 8 values as loaded (two 16-byte vectors), converted later
  struct Raw {
    f32x4 a, b;
  };
  typedef __attribute__((address_space(1))) float GT;
  __device__ __forceinline__ static Raw load_raw(const float* p) {
    return Raw{reinterpret_cast<const f32x4*>(p)[0], reinterpret_cast<const f32x4*>(p)[1]};
  }
  __device__ __forceinline__ static Raw load_raw_g(const GT* p) {
    typedef __attribute__((address_space(1))) const f32x4 G4;
    return Raw{((G4*)p)[0], ((G4*)p)[1]};
  }
  __device__ __forceinline__ static void store_raw_g(GT* p, const Raw& r) {
    typedef __attribute__((address_space(1))) f32x4 G4;
    ((G4*)p)[0] = r.a;
    ((G4*)p)[1] = r.b;
  }
  // element e (compile-time) of a raw vector, as fp32
  __device__ __forceinline__ static float elem(const Raw& r, int e) { return e < 4 ? r.a[e] : r.b[e - 4]; }
  __device__ __forceinline__ static void convert(const Raw& r, float (&v)[8]) {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
  __device__ __forceinline__ static void load(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store(float* p, const float (&v)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

template <>
struct Vec8<uint16_t> {
  typedef uint32_t Raw __attribute__((ext_vector_type(4)));  // 8 bf16 as loaded
  typedef __attribute__((address_space(1))) uint16_t GT;
  __device__ __forceinline__ static Raw load_raw(const uint16_t* p) { return *reinterpret_cast<const Raw*>(p); }
  __device__ __forceinline__ static Raw load_raw_g(const GT* p) {
    typedef __attribute__((address_space(1))) const Raw G4;
    return *(G4*)p;
  }
  __device__ __forceinline__ static void store_raw_g(GT* p, const Raw& r) {
    typedef __attribute__((address_space(1))) Raw G4;
    *(G4*)p = r;
  }
  __device__ __forceinline__ static float elem(const Raw& a, int e) {
    return (e & 1) ? __uint_as_float(a[e >> 1] & 0xFFFF0000u) : __uint_as_float(a[e >> 1] << 16);
  }
  __device__ __forceinline__ static void convert(const Raw& a, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static void load(const uint16_t* p, float (&v)[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static void store(uint16_t* p, const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16_rne(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16_rne(v[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// 4 consecutive elements of dtype T as loaded: 8 bytes (bf16) or 16 bytes (fp32), aligned
// to their size.
template <typename T>
struct Vec4;

template <>
struct Vec4<float> {
  typedef f32x4 Raw;
  typedef __attribute__((address_space(1))) float GT;
  __device__ __forceinline__ static Raw load_raw(const float* p) { return *reinterpret_cast<const Raw*>(p); }
  __device__ __forceinline__ static Raw load_raw_g(const GT* p) {
    typedef __attribute__((address_space(1))) const Raw G4;
    return *(G4*)p;
  }
  __device__ __forceinline__ static void store_raw_g(GT* p, const Raw& r) {
    typedef __attribute__((address_space(1))) Raw G4;
    *(G4*)p = r;
  }
  __device__ __forceinline__ static float elem(const Raw& r, int e) { return r[e]; }
};

template <>
struct Vec4<uint16_t> {
  typedef uint32_t Raw __attribute__((ext_vector_type(2)));  // 4 bf16 as loaded
  typedef __attribute__((address_space(1))) uint16_t GT;
  __device__ __forceinline__ static Raw load_raw(const uint16_t* p) { return *reinterpret_cast<const Raw*>(p); }
  __device__ __forceinline__ static Raw load_raw_g(const GT* p) {
    typedef __attribute__((address_space(1))) const Raw G2;
    return *(G2*)p;
  }
  __device__ __forceinline__ static void store_raw_g(GT* p, const Raw& r) {
    typedef __attribute__((address_space(1))) Raw G2;
    *(G2*)p = r;
  }
  __device__ __forceinline__ static float elem(const Raw& a, int e) {
    return (e & 1) ? __uint_as_float(a[e >> 1] & 0xFFFF0000u) : __uint_as_float(a[e >> 1] << 16);
  }
};

// ---------------------------------------------------------------- DPP reductions
// dpp_ctrl encodings (GCN/CDNA DPP): quad_perm [1,0,3,2] = 0xB1 (lane ^ 1),
// quad_perm [2,3,0,1] = 0x4E (lane ^ 2), row_half_mirror = 0x141 (lane i <-> 7 - i
// inside each group of 8), row_mirror = 0x140 (lane i <-> 15 - i inside each row of 16).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G in {1, 2, 4, 8, 16}); every lane of the group
// ends with the same bits (fp add is commutative), and the order of the additions
// depends only on G, never on the launch shape.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
  if constexpr (G >= 2) v += dpp_f32<0xB1>(v);
  if constexpr (G >= 4) v += dpp_f32<0x4E>(v);
  if constexpr (G >= 8) v += dpp_f32<0x141>(v);
  if constexpr (G >= 16) v += dpp_f32<0x140>(v);
  return v;
}

}  // namespace gdn
