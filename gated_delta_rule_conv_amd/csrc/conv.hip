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

#include <type_traits>

#include "conv_taps.h"
#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kDecThreads = 64;  // decode: one wave per workgroup
constexpr int kVec = kConvVec;
constexpr int kStrip = 8;  // tokens per block in prefill mode

// Prefill mode. A wave covers 512 channels: lane l owns channels 4l..4l+3 and
// 256+4l..256+4l+3 of them, so each of its loads (4 channels) and stores (4 fp32) is one
// contiguous run across the wave -- 512 B of bf16 input and 1 KiB of fp32 output per
// instruction. A thread walks a strip of kStrip tokens.
template <typename T>
struct Half4 {
  // raw storage of 4 elements: uint2 for bf16, float4 for fp32
  typedef typename std::conditional<sizeof(T) == 2, uint2, float4>::type Raw;
  __device__ __forceinline__ static Raw load(const T* p) { return *reinterpret_cast<const Raw*>(p); }
  __device__ __forceinline__ static void convert(const Raw& r, float* v) {
    if constexpr (sizeof(T) == 2) {
      v[0] = __uint_as_float(r.x << 16);
      v[1] = __uint_as_float(r.x & 0xFFFF0000u);
      v[2] = __uint_as_float(r.y << 16);
      v[3] = __uint_as_float(r.y & 0xFFFF0000u);
    } else {
      v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    }
  }
};

template <typename T, int K>
__global__ __launch_bounds__(kThreads) void conv_prefill_kernel(ConvArgs a) {
  using H = Half4<T>;
  const int C = a.channels;
  const int lane = threadIdx.x & 63;
  const int wbase = (blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 512;
  if (wbase >= C) return;
  // channel groups of this lane; past the channel count the loads are clamped to the last
  // group (valid memory) and the stores are skipped
  const int chA = wbase + 4 * lane, chB = chA + 256;
  const bool okA = chA < C, okB = chB < C;
  const int ldA = min(chA, C - 4), ldB = min(chB, C - 4);
  const T* __restrict__ x = static_cast<const T*>(a.x);
  const int* __restrict__ cu = a.cu_seqlens;
  const int t0 = blockIdx.y * kStrip;
  const int nt = min(kStrip, a.total_tokens - t0);

  // every x row of the strip is loaded up front (rows past the end repeat the last one),
  // so the strip's loads are all in flight together; then the K-1 rows before the strip,
  // on the guess that they belong to the sequence of the strip's first token (true unless
  // that sequence starts less than K-1 tokens before it; checked below), so the common
  // case needs no second round trip
  typename H::Raw xa[kStrip], xb[kStrip], ha[K - 1], hb[K - 1];
#pragma unroll
  for (int u = 0; u < kStrip; ++u) {
    const T* row = x + static_cast<int64_t>(t0 + min(u, nt - 1)) * a.x_stride;
    xa[u] = H::load(row + ldA);
    xb[u] = H::load(row + ldB);
  }
#pragma unroll
  for (int i = 0; i < K - 1; ++i) {
    const T* row = x + static_cast<int64_t>(max(t0 - (K - 1) + i, 0)) * a.x_stride;
    ha[i] = H::load(row + ldA);
    hb[i] = H::load(row + ldB);
  }

  ConvTaps<T, K> taps;
  taps.load_halves(static_cast<const T*>(a.w), static_cast<const T*>(a.b), ldA, ldB);

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
  bool reload = true, first = true;
#pragma unroll
  for (int u = 0; u < kStrip; ++u) {
    if (u < nt) {  // (a guard, not a break: the loop must unroll fully to keep the rows in registers)
      const int t = t0 + u;
      while (t >= seq_end) {  // next non-empty sequence starts at t
        ++s;
        seq_start = seq_end;
        seq_end = cu[s + 1];
        reload = true;
      }
      if (reload) {
        const int p = t - seq_start;  // position of t in its sequence
        if (first && p >= K - 1) {
          // the rows before the strip are this sequence's tokens t0-K+1 .. t0-1: loaded above
#pragma unroll
          for (int i = 0; i < K - 1; ++i) {
            H::convert(ha[i], &win[i][0]);
            H::convert(hb[i], &win[i][4]);
          }
        } else {
          const T* cs = reinterpret_cast<const T*>(a.state_ptrs[s]) + a.state_off;
#pragma unroll
          for (int i = 0; i < K - 1; ++i) {
            const int r = p + i;  // z row feeding tap i of token t
            const T* row = r < K - 1 ? cs + static_cast<int64_t>(r) * a.state_stride
                                     : x + static_cast<int64_t>(seq_start + r - (K - 1)) * a.x_stride;
            H::convert(H::load(row + ldA), &win[i][0]);
            H::convert(H::load(row + ldB), &win[i][4]);
          }
        }
        reload = false;
      }
      first = false;
      float cur[kVec], out[kVec];
      H::convert(xa[u], &cur[0]);
      H::convert(xb[u], &cur[4]);
      taps.apply(win, cur, a.silu != 0, out);
      float* yrow = a.y + static_cast<int64_t>(t) * a.y_stride;
      if (okA) *reinterpret_cast<float4*>(yrow + chA) = make_float4(out[0], out[1], out[2], out[3]);
      if (okB) *reinterpret_cast<float4*>(yrow + chB) = make_float4(out[4], out[5], out[6], out[7]);
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
  const int C = a.channels;
  const int cg = (blockIdx.x * kDecThreads + threadIdx.x) * kVec;
  const bool live = cg < C;
  const int ch0 = live ? cg : 0;  // (threads past the channels load channel 0 and store nothing)
  const int i = blockIdx.y;
  // the loads that do not need the slot pointer go first, so they overlap its load
  typename Vec8<T>::Raw wr[K], sr[K - 1], xr, br;
#pragma unroll
  for (int j = 0; j < K; ++j) wr[j] = Vec8<T>::load_raw(static_cast<const T*>(a.w) + static_cast<int64_t>(ch0) * K + j * kVec);
  xr = Vec8<T>::load_raw(static_cast<const T*>(a.x) + static_cast<int64_t>(i) * a.x_stride + ch0);
  const bool has_b = a.b != nullptr;
  br = Vec8<T>::load_raw(static_cast<const T*>(has_b ? a.b : a.w) + ch0);  // (taps as a stand-in when no bias)
  // An inactive slot (zero pointer) reads the taps in place of a state (C x K elements,
  // so K - 1 rows are in bounds) and stores nothing: no branch on the pointer keeps the
  // loads above free to issue before it arrives.
  const uint64_t sp = ((cu64*)a.state_ptrs)[i];
  const bool act = sp != 0 && live;
  using GT = __attribute__((address_space(1))) T;
  GT* cs = (GT*)reinterpret_cast<T*>(sp != 0 ? sp : reinterpret_cast<uint64_t>(a.w));
#pragma unroll
  for (int r = 0; r < K - 1; ++r) sr[r] = Vec8<T>::load_raw_g(cs + static_cast<int64_t>(r) * C + ch0);
  ConvTaps<T, K> taps;
  taps.from_raw(wr, br, has_b);
  float win[K - 1][kVec], cur[kVec], out[kVec];
#pragma unroll
  for (int r = 0; r < K - 1; ++r) Vec8<T>::convert(sr[r], win[r]);
  Vec8<T>::convert(xr, cur);
  taps.apply(win, cur, a.silu != 0, out);
  if (!act) return;
  Vec8<float>::store(a.y + static_cast<int64_t>(i) * a.y_stride + ch0, out);
#pragma unroll
  for (int r = 0; r < K - 2; ++r) Vec8<T>::store_raw_g(cs + static_cast<int64_t>(r) * C + ch0, sr[r + 1]);
  Vec8<T>::store_raw_g(cs + static_cast<int64_t>(K - 2) * C + ch0, xr);
}

// mode: 0 decode, 1 prefill conv + commit, 2 prefill conv only
template <typename T>
hipError_t launch_all(const ConvArgs& a, hipStream_t s, int mode) {
  const unsigned gx = (a.channels / kVec + kThreads - 1) / kThreads;
  const bool decode = mode == 0;
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
    dim3 grid((a.channels + 512 * (kThreads / 64) - 1) / (512 * (kThreads / 64)), (a.total_tokens + kStrip - 1) / kStrip);
    switch (a.width) {
      case 2: conv_prefill_kernel<T, 2><<<grid, kThreads, 0, s>>>(a); break;
      case 3: conv_prefill_kernel<T, 3><<<grid, kThreads, 0, s>>>(a); break;
      default: conv_prefill_kernel<T, 4><<<grid, kThreads, 0, s>>>(a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mode == 2 || a.n == 0) return hipSuccess;
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
  return a.bf16 ? launch_all<uint16_t>(a, s, 1) : launch_all<float>(a, s, 1);
}

hipError_t launch_conv_prefill_only(const ConvArgs& a, hipStream_t s) {
  return a.bf16 ? launch_all<uint16_t>(a, s, 2) : launch_all<float>(a, s, 2);
}

hipError_t launch_conv_decode(const ConvArgs& a, hipStream_t s) {
  return a.bf16 ? launch_all<uint16_t>(a, s, 0) : launch_all<float>(a, s, 0);
}

}  // namespace gdn
