// Depthwise causal conv1d with per-sequence conv state, gfx950.
//
// For a sequence with conv state cs (K-1 rows, oldest first) and tokens x_0..x_{L-1},
// z = [cs ; x] and y_t[c] = act(b[c] + sum_{j<K} w[c][j] z_{t+j}[c]); the new conv
// state is the last K-1 rows of z. ("System Design" (project_6), "GDN Kernel Dispatch
// Detail": the depthwise causal Conv1d ahead of the L2 norm, and the conv state update
// that opens the decode branch; aprender #5279, "Where concurrency is lost": conv
// kernels with a sequence dimension and per-sequence conv state.)
//
// Layout: x / y rows are tokens, channels contiguous. Each thread owns 8 adjacent
// channels (one 16-byte bf16 load or two 16-byte fp32 loads per row), so a wave
// streams 512 channels = 1 KiB (bf16) of a row per load and stores 2 KiB of fp32.
// The op is purely HBM-bound (8 flops per element), so there is no LDS staging: a
// thread walks a strip of tokens keeping the K-1 previous rows of z in registers.

#include "conv_taps.h"
#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kDecThreads = 64;  // decode: one wave per workgroup
constexpr int kVec = kConvVec;
constexpr int kStrip = 8;  // tokens per block in prefill mode

template <typename T, int K>
__global__ __launch_bounds__(kThreads) void conv_prefill_kernel(ConvArgs a) {
  const int ch0 = (blockIdx.x * kThreads + threadIdx.x) * kVec;
  if (ch0 >= a.channels) return;
  const int C = a.channels;
  const T* __restrict__ x = static_cast<const T*>(a.x);
  const int* __restrict__ cu = a.cu_seqlens;
  const int t0 = blockIdx.y * kStrip;
  const int nt = min(kStrip, a.total_tokens - t0);

  // every x row of the strip is loaded up front (rows past the end repeat the last one),
  // so the strip's loads are all in flight together
  typename Vec8<T>::Raw xr[kStrip];
#pragma unroll
  for (int u = 0; u < kStrip; ++u) xr[u] = Vec8<T>::load_raw(x + static_cast<int64_t>(t0 + min(u, nt - 1)) * a.x_stride + ch0);

  ConvTaps<T, K> taps;
  taps.load(static_cast<const T*>(a.w), static_cast<const T*>(a.b), ch0);

  // sequence holding t0: largest s with cu[s] <= t0 (cu[n] = total_tokens > t0)
  int lo = 0, hi = a.n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t0) lo = mid; else hi = mid;
  }
  int s = lo;
  int seq_start = cu[s];
  int seq_end = cu[s + 1];

  float win[K - 1][kVec];
  bool reload = true;
#pragma unroll
  for (int u = 0; u < kStrip; ++u) {
    if (u < nt) {  // (a guard, not a break: the loop must unroll fully to keep xr in registers)
      const int t = t0 + u;
      while (t >= seq_end) {  // next non-empty sequence starts at t
        ++s;
        seq_start = seq_end;
        seq_end = cu[s + 1];
        reload = true;
      }
      if (reload) {
        const int p = t - seq_start;  // position of t in its sequence
        const T* cs = reinterpret_cast<const T*>(a.state_ptrs[s]);
#pragma unroll
        for (int i = 0; i < K - 1; ++i) {
          const int r = p + i;  // z row feeding tap i of token t
          if (r < K - 1)
            Vec8<T>::load(cs + static_cast<int64_t>(r) * C + ch0, win[i]);
          else
            Vec8<T>::load(x + static_cast<int64_t>(seq_start + r - (K - 1)) * a.x_stride + ch0, win[i]);
        }
        reload = false;
      }
      float cur[kVec], out[kVec];
      Vec8<T>::convert(xr[u], cur);
      taps.apply(win, cur, a.silu != 0, out);
      Vec8<float>::store(a.y + static_cast<int64_t>(t) * a.y_stride + ch0, out);
#pragma unroll
      for (int i = 0; i < K - 2; ++i)
#pragma unroll
        for (int c = 0; c < kVec; ++c) win[i][c] = win[i + 1][c];
#pragma unroll
      for (int c = 0; c < kVec; ++c) win[K - 2][c] = cur[c];
    }
  }
}

// After conv_prefill_kernel (stream order): each sequence's conv state becomes the last
// K-1 rows of its z. A thread reads every row it needs before it writes any, and owns
// its (sequence, channel group) column, so the in-place update cannot race.
template <typename T, int K>
__global__ __launch_bounds__(kThreads) void conv_commit_kernel(ConvArgs a) {
  const int ch0 = (blockIdx.x * kThreads + threadIdx.x) * kVec;
  if (ch0 >= a.channels) return;
  const int s = blockIdx.y;
  const int start = a.cu_seqlens[s];
  const int L = a.cu_seqlens[s + 1] - start;
  if (L <= 0) return;
  const int C = a.channels;
  const T* __restrict__ x = static_cast<const T*>(a.x);
  T* cs = reinterpret_cast<T*>(a.state_ptrs[s]);
  float nz[K - 1][kVec];
#pragma unroll
  for (int i = 0; i < K - 1; ++i) {
    const int r = L + i;  // row of z that becomes new state row i
    if (r < K - 1)
      Vec8<T>::load(cs + static_cast<int64_t>(r) * C + ch0, nz[i]);
    else
      Vec8<T>::load(x + static_cast<int64_t>(start + r - (K - 1)) * a.x_stride + ch0, nz[i]);
  }
#pragma unroll
  for (int i = 0; i < K - 1; ++i) Vec8<T>::store(cs + static_cast<int64_t>(i) * C + ch0, nz[i]);
}

// Decode mode: token i belongs to slot i (sequence length 1); conv and state shift in one
// pass, in place. A zero state pointer marks an inactive slot. The slot pointer is a
// scalar load; the taps, the K-1 state rows and the token are all loaded before any of
// them is used (one memory round trip), and the state goes through global-address-space
// accesses. Small workgroups spread a slot over many CUs.
template <typename T, int K>
__global__ __launch_bounds__(kDecThreads) void conv_decode_kernel(ConvArgs a) {
  typedef __attribute__((address_space(4))) const uint64_t cu64;
  const int ch0 = (blockIdx.x * kDecThreads + threadIdx.x) * kVec;
  if (ch0 >= a.channels) return;
  const int i = blockIdx.y;
  const uint64_t sp = ((cu64*)a.state_ptrs)[i];
  if (sp == 0) return;
  const int C = a.channels;
  using GT = __attribute__((address_space(1))) T;
  GT* cs = (GT*)reinterpret_cast<T*>(sp);
  typename Vec8<T>::Raw wr[K], sr[K - 1], xr, br;
#pragma unroll
  for (int j = 0; j < K; ++j) wr[j] = Vec8<T>::load_raw(static_cast<const T*>(a.w) + static_cast<int64_t>(ch0) * K + j * kVec);
#pragma unroll
  for (int r = 0; r < K - 1; ++r) sr[r] = Vec8<T>::load_raw_g(cs + static_cast<int64_t>(r) * C + ch0);
  xr = Vec8<T>::load_raw(static_cast<const T*>(a.x) + static_cast<int64_t>(i) * a.x_stride + ch0);
  const bool has_b = a.b != nullptr;
  br = Vec8<T>::load_raw(static_cast<const T*>(has_b ? a.b : a.w) + ch0);  // (taps as a stand-in when no bias)
  ConvTaps<T, K> taps;
  taps.from_raw(wr, br, has_b);
  float win[K - 1][kVec], cur[kVec], out[kVec];
#pragma unroll
  for (int r = 0; r < K - 1; ++r) Vec8<T>::convert(sr[r], win[r]);
  Vec8<T>::convert(xr, cur);
  taps.apply(win, cur, a.silu != 0, out);
  Vec8<float>::store(a.y + static_cast<int64_t>(i) * a.y_stride + ch0, out);
#pragma unroll
  for (int r = 0; r < K - 2; ++r) Vec8<T>::store_raw_g(cs + static_cast<int64_t>(r) * C + ch0, sr[r + 1]);
  Vec8<T>::store_raw_g(cs + static_cast<int64_t>(K - 2) * C + ch0, xr);
}

template <typename T>
hipError_t launch_all(const ConvArgs& a, hipStream_t s, bool decode) {
  const unsigned gx = (a.channels / kVec + kThreads - 1) / kThreads;
  if (decode) {
    if (a.n == 0) return hipSuccess;
    dim3 grid((a.channels / kVec + kDecThreads - 1) / kDecThreads, a.n);
    switch (a.width) {
      case 2: conv_decode_kernel<T, 2><<<grid, kDecThreads, 0, s>>>(a); break;
      case 3: conv_decode_kernel<T, 3><<<grid, kDecThreads, 0, s>>>(a); break;
      default: conv_decode_kernel<T, 4><<<grid, kDecThreads, 0, s>>>(a); break;
    }
    return hipGetLastError();
  }
  if (a.total_tokens > 0) {
    dim3 grid(gx, (a.total_tokens + kStrip - 1) / kStrip);
    switch (a.width) {
      case 2: conv_prefill_kernel<T, 2><<<grid, kThreads, 0, s>>>(a); break;
      case 3: conv_prefill_kernel<T, 3><<<grid, kThreads, 0, s>>>(a); break;
      default: conv_prefill_kernel<T, 4><<<grid, kThreads, 0, s>>>(a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n == 0) return hipSuccess;
  dim3 grid(gx, a.n);
  switch (a.width) {
    case 2: conv_commit_kernel<T, 2><<<grid, kThreads, 0, s>>>(a); break;
    case 3: conv_commit_kernel<T, 3><<<grid, kThreads, 0, s>>>(a); break;
    default: conv_commit_kernel<T, 4><<<grid, kThreads, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_prefill(const ConvArgs& a, hipStream_t s) {
  return a.bf16 ? launch_all<uint16_t>(a, s, false) : launch_all<float>(a, s, false);
}

hipError_t launch_conv_decode(const ConvArgs& a, hipStream_t s) {
  return a.bf16 ? launch_all<uint16_t>(a, s, true) : launch_all<float>(a, s, true);
}

}  // namespace gdn
