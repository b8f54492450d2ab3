// The taps of the depthwise causal conv for 8 adjacent channels, and the conv of one
// token: y[c] = act(b[c] + sum_{j<K} w[c][j] z_j[c]), z_0 .. z_{K-2} the preceding rows
// (oldest first) and z_{K-1} the current token. Shared by the conv kernels and the fused
// decode kernel so that both produce the same bits.
#pragma once

#include "device_common.h"

namespace gdn {

constexpr int kConvVec = 8;  // channels per thread

// x * sigmoid(x) = x / (1 + e^-x), with e^-x = 2^(-x * log2 e) from the hardware base-2
// exponential and the division as a hardware reciprocal (each about 1 ulp; the result is
// within a few ulp of the correctly rounded value). Outside the exponent range 2^(..)
// saturates to 0 or +inf, which gives x or -0, the limits of the function.
__device__ __forceinline__ float silu(float x) {
  const float e = __builtin_amdgcn_exp2f(-x * 1.44269504088896341f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// 4 consecutive elements as fp32: 8 bytes (bf16, 8-byte aligned) or 16 bytes (fp32, 16-byte aligned)
template <typename T>
__device__ __forceinline__ void load4(const T* p, float* v) {
  if constexpr (sizeof(T) == 2) {
    const uint2 r = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(r.x << 16);
    v[1] = __uint_as_float(r.x & 0xFFFF0000u);
    v[2] = __uint_as_float(r.y << 16);
    v[3] = __uint_as_float(r.y & 0xFFFF0000u);
  } else {
    const float4 r = *reinterpret_cast<const float4*>(p);
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
}

template <typename T, int K>
struct ConvTaps {
  float w[K][kConvVec];
  float b[kConvVec];

  __device__ __forceinline__ void load(const T* __restrict__ wp, const T* __restrict__ bp, int ch0) {
    // w is [C][K]: the 8*K taps of channels ch0..ch0+7 are contiguous and 16-byte aligned.
    float flat[K * kConvVec];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      float tmp[kConvVec];
      Vec8<T>::load(wp + static_cast<int64_t>(ch0) * K + i * kConvVec, tmp);
#pragma unroll
      for (int e = 0; e < kConvVec; ++e) flat[i * kConvVec + e] = tmp[e];
    }
#pragma unroll
    for (int c = 0; c < kConvVec; ++c)
#pragma unroll
      for (int j = 0; j < K; ++j) w[j][c] = flat[c * K + j];
    if (bp) {
      Vec8<T>::load(bp + ch0, b);
    } else {
#pragma unroll
      for (int c = 0; c < kConvVec; ++c) b[c] = 0.f;
    }
  }

  // The same for two groups of 4 channels, chA..chA+3 (as channels 0-3) and chB..chB+3
  // (as 4-7): their 4*K taps each are contiguous and at least 8-byte aligned.
  __device__ __forceinline__ void load_halves(const T* __restrict__ wp, const T* __restrict__ bp, int chA, int chB) {
    float flat[2][4 * K];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const T* src = wp + static_cast<int64_t>(hh ? chB : chA) * K;
#pragma unroll
      for (int i = 0; i < K; ++i) load4<T>(src + 4 * i, &flat[hh][4 * i]);
    }
#pragma unroll
    for (int c = 0; c < kConvVec; ++c)
#pragma unroll
      for (int j = 0; j < K; ++j) w[j][c] = flat[c / 4][(c % 4) * K + j];
    if (bp) {
      load4<T>(bp + chA, &b[0]);
      load4<T>(bp + chB, &b[4]);
    } else {
#pragma unroll
      for (int c = 0; c < kConvVec; ++c) b[c] = 0.f;
    }
  }

  // the same from raw (unconverted) tap and bias vectors
  __device__ __forceinline__ void from_raw(const typename Vec8<T>::Raw (&wr)[K], const typename Vec8<T>::Raw& br,
                                           bool has_b) {
    float flat[K * kConvVec];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      float tmp[kConvVec];
      Vec8<T>::convert(wr[i], tmp);
#pragma unroll
      for (int e = 0; e < kConvVec; ++e) flat[i * kConvVec + e] = tmp[e];
    }
#pragma unroll
    for (int c = 0; c < kConvVec; ++c)
#pragma unroll
      for (int j = 0; j < K; ++j) w[j][c] = flat[c * K + j];
    if (has_b) {
      Vec8<T>::convert(br, b);
    } else {
#pragma unroll
      for (int c = 0; c < kConvVec; ++c) b[c] = 0.f;
    }
  }

  // win[0..K-2] = z rows preceding the current token (oldest first), cur = current token.
  __device__ __forceinline__ void apply(const float (&win)[K - 1][kConvVec], const float (&cur)[kConvVec], bool silu,
                                        float (&out)[kConvVec]) const {
#pragma unroll
    for (int c = 0; c < kConvVec; ++c) {
      float acc = b[c];
#pragma unroll
      for (int j = 0; j < K - 1; ++j) acc = fmaf(w[j][c], win[j][c], acc);
      acc = fmaf(w[K - 1][c], cur[c], acc);
      if (silu) acc = gdn::silu(acc);
      out[c] = acc;
    }
  }
};

// The conv of 4 adjacent channels straight from the loaded (raw) vectors: the taps
// [4][K] as K vectors of 4, the bias, the K-1 preceding rows and the current token. The
// operations and their order are those of ConvTaps::apply (acc = b; acc = fma(w_j, z_j,
// acc) for j = 0 .. K-1; then the activation), so both give the same bits.
template <typename T, int K>
__device__ __forceinline__ void conv4_raw(const typename Vec4<T>::Raw (&wr)[K], const typename Vec4<T>::Raw& br,
                                          bool has_b, const typename Vec4<T>::Raw (&rows)[K - 1],
                                          const typename Vec4<T>::Raw& cur, bool silu, float (&out)[4]) {
  using V4 = Vec4<T>;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float acc = has_b ? V4::elem(br, c) : 0.f;
#pragma unroll
    for (int j = 0; j < K - 1; ++j) acc = fmaf(V4::elem(wr[(c * K + j) / 4], (c * K + j) % 4), V4::elem(rows[j], c), acc);
    acc = fmaf(V4::elem(wr[(c * K + K - 1) / 4], (c * K + K - 1) % 4), V4::elem(cur, c), acc);
    if (silu) acc = gdn::silu(acc);
    out[c] = acc;
  }
}

}  // namespace gdn
