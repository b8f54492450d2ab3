// Chunked prefill of the gated delta rule over packed ragged sequences, gfx950.
//
// ("System Design" (project_6), "GDN Kernel Dispatch Detail": the prefill branch hands
// (q, k, v, g, beta, state) to a chunked gated-delta-rule kernel and updates the
// temporal state; aprender #5279, "Phase plan", P6: ragged lengths must give the
// per-slot result.)
//
// Per sequence and v-head the rule S_t = exp(g_t) S_{t-1}(I - beta_t k_t k_t^T) +
// beta_t v_t k_t^T, o_t = S_t q_t is rewritten over chunks of C tokens (chunks start at
// each sequence's own first token). With gam = inclusive cumsum of g in the chunk and
// S0 the state on entry:
//   A[t,s] = beta_t e^{gam_t - gam_s} (k_t . k_s)  (s < t),   T = (I + A)^-1
//   P[t,s] = e^{gam_t - gam_s} (q_t . k_s)          (s <= t)
//   U = T (diag(beta) V - diag(beta e^gam) K S0^T)
//   O = diag(e^gam) Q S0^T + P U
//   S = e^{gam_n} S0 + U^T diag(e^{gam_n - gam}) K
// Every decay factor is exp of gam_t - gam_s with t >= s (or gam alone, <= 0): nothing
// can overflow, so no clamp is needed.
//
// Launches, in stream order:
//   (fused entry point, chunk-parallel form or chunks other than 64 tokens: the conv of
//   the v channels into the workspace, a kernel of conv.hip)
//   chunk_table_kernel : cu_seqlens -> chunk table (sequence, start, length), per-sequence
//                        chunk offsets, a longest-first sequence order and (chunk-parallel
//                        form) the segment table, on the device. Not launched for whole
//                        sequences when there are at most 64: each intra-chunk workgroup
//                        then finds its chunk from cu_seqlens, and one of them writes the
//                        offsets and the order.
//   intra_chunk_kernel : one workgroup per (chunk, k-head), all chunks in parallel:
//                        K, Q in LDS (L2-normalised unless that is switched off); K K^T and Q K^T on MFMA; for each v-head
//                        sharing the k-head: the decay mask, A, T by blocked (16x16)
//                        forward substitution, and P. K^, Q^, T and P go to the workspace.
//                        Through the fused entry point it also convolves its chunk's q and
//                        k channels from x, and a sequence's first chunk commits the conv
//                        state of its k-head's q and k channels (and of its v-heads' v
//                        channels where those were convolved by the kernel above).
//   inter_chunk_kernel : one workgroup per (sequence, v-head, 16 state rows), walking the
//                        chunks of its sequence in order with its 16 x d slice of the
//                        state resident in registers/LDS; the contractions K S^T, Q S^T,
//                        T R, P U and U^T K run on MFMA (K^ is staged through LDS for the
//                        last one, whose contraction runs over tokens). The 16-row slices
//                        of one head are mapped to one XCD so they share K, Q, T and P
//                        through its L2. Each workgroup prefetches the next chunk's
//                        operands; where 16-row workgroups would be 512 or more, a
//                        workgroup takes two 16-row blocks of a head (one CU each).
//                        Through the fused entry point (whole sequences, 64-token chunks)
//                        it convolves its own v channels from x two chunks ahead, so v
//                        never goes through memory, and commits their conv state.
// In the chunk-parallel form the last launch is replaced by three: the inter-chunk kernel
// computing every segment's affine state map, segment_scan_kernel forming the segments'
// start states, and the inter-chunk kernel producing every segment's outputs.

#include <algorithm>
#include <type_traits>
#include <cmath>

#include "conv_taps.h"
#include "launch.h"
#include "mma.h"

// Multiply-adds are fused only within one source expression (a * b + c), never across
// statements: the compiler's cross-statement fusion depends on the surrounding code, and
// the inter-chunk kernel's variants (and the segmented form) must round the same
// arithmetic the same way to give bit-identical results.
#pragma clang fp contract(on)

namespace gdn {
namespace {

constexpr int kThreads = 512;      // intra-chunk workgroup: 8 waves
constexpr int kWaves = 8;
constexpr int kInterThreads = 512; // inter-chunk workgroup: 8 waves
constexpr int kDVB = 16;           // state rows per inter-chunk workgroup
// Inter-chunk variant choice: where 16-row workgroups would fill every CU (MI355X: 256)
// twice over, a workgroup takes two 16-row blocks; below that one (both prefetch).
constexpr int kInterPrefetchMaxCUs = 256;
constexpr int kMetaThreads = 1024;
constexpr int kLptMaxSeqs = 256;   // longest-first ordering only up to this many sequences

// Per-chunk operands the intra-chunk kernel hands to the inter-chunk kernel, stored in
// fragment order for the MFMA policy (FragIO<> in mma.h), zero-padded past the chunk:
//   per (chunk, k-head): K^ and Q^ (q already scaled) as A operands (rows = tokens,
//                        k = head dim)
//   per (chunk, v-head): T, then P, as A operands (rows and k = tokens); then the decay
//                        factors e^gam [C] (fp32, padded with e^{gam_{n-1}}), beta [C]
//                        (padded with 0) and e^{gam_{n-1} - gam} [C] (padded with 1)
//   chunk-parallel form only (segmented): per (segment, v-head) three d x d fp32
//   matrices: the segment's start state Z, the transposed linear part M^T of its affine
//   map S -> S M + B, and B.
struct Workspace {
  int* n_chunks;
  int4* table;  // (sequence, first token, length, index in sequence)
  int* chunk_off;
  int* order;
  char* kq;
  char* tp;
  int64_t kq_stride;  // bytes per (chunk, k-head)
  int64_t tp_stride;  // bytes per (chunk, v-head)
  int segmented;      // chunk-parallel form (else whole sequences)
  int* n_segs;
  int* seg_off;       // [N+1] first segment of each sequence
  int4* seg_table;    // (sequence, first chunk, end chunk, last segment of its sequence?)
  float* zs;
  float* mt;
  float* bt;
};

inline size_t up256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

inline size_t max_chunks_of(int chunk, int num_seqs, int total_tokens) {
  return static_cast<size_t>(total_tokens) / chunk + static_cast<size_t>(num_seqs);
}

// fragment counts: token tiles (C / 16), k-steps over the head dim (D / KSTEP) and over
// the chunk's tokens (nk, padded up to a whole k-step)
template <int POL>
struct FragCount {
  static constexpr int KSTEP = Mma<POL>::KSTEP;
  static constexpr int BYTES = FragIO<POL>::BYTES;
  __host__ __device__ static constexpr int nk(int C) { return (C + KSTEP - 1) / KSTEP; }
  __host__ __device__ static constexpr size_t kq(int D, int C) { return 2ull * (C / 16) * (D / KSTEP) * BYTES; }
  __host__ __device__ static constexpr size_t tp(int C) { return 2ull * (C / 16) * nk(C) * BYTES + 3ull * C * 4; }
};

// per-chunk strides of the two operand regions: the larger of the two policies' sizes
inline size_t kq_stride(int D, int C) {
  const size_t a = FragCount<kPolFP32>::kq(D, C), b = FragCount<kPolBF16X3>::kq(D, C);
  return a > b ? a : b;
}
inline size_t tp_stride(int C) {
  const size_t a = FragCount<kPolFP32>::tp(C), b = FragCount<kPolBF16X3>::tp(C);
  return a > b ? a : b;
}

// Chunk-parallel prefill. When a launch has fewer state-row workgroups than CUs (few
// heads, e.g. one GPU's share of a head-sharded layer, and few sequences), a sequence of
// n >= 8 chunks is cut into segments of sc chunks. Every segment's affine map
// S -> S M + B is computed in parallel (rows of the state evolve independently: M's rows
// are the recurrence run from identity rows with v = 0, B's from zero rows with the real
// v), a scan over segments gives each segment's start state, and then all segments
// produce their outputs in parallel: a chain of about 2 sc chunk steps plus one small
// product per segment instead of n chunk steps. sc is the largest k with k^2 <= n
// (within [2, 32]), which balances the two (a scan step costs about 0.8 of a chunk step:
// each streams a 64 KiB map through its CU); it depends on the sequence's own length
// only, so within this form packing does not change a sequence's segments.
constexpr int kSegmentBelowWGs = 256;  // MI355X CUs
constexpr int kSegmentMinChunks = 8;

// form: 0 auto, 1 whole sequences, 2 segments (gdn_prefill_form)
bool use_segments(int hv, int d, int num_seqs, int form) {
  if (form != 0) return form == 2;
  return static_cast<long>(d / kDVB) * hv * num_seqs < kSegmentBelowWGs;
}

// A sequence of nc chunks has at most ceil(nc / 2) segments (sc >= 2), or one; with
// sum nc <= T / C + N that is at most T / (2 C) + 1.5 N + 1 over a launch.
inline size_t max_segments_of(int chunk, int num_seqs, int total_tokens) {
  return static_cast<size_t>(total_tokens) / (2 * static_cast<size_t>(chunk)) + 2 * static_cast<size_t>(num_seqs) + 1;
}

__device__ __forceinline__ int segment_len(int nc) {
  if (nc < kSegmentMinChunks) return nc > 0 ? nc : 1;
  int k = 2;
  while (k < 32 && (k + 1) * (k + 1) <= nc) ++k;
  return k;
}

// The size covers every call with at most num_seqs sequences and total_tokens tokens:
// each term grows with both, and under AUTO the segment maps are counted whenever some
// call of this layer could take the chunk-parallel form (a single sequence would, i.e.
// (d / 16) * Hv < 256), not only when a call of exactly num_seqs sequences would.
size_t workspace_bytes(int hk, int hv, int d, int chunk, int num_seqs, int total_tokens, int form) {
  const size_t mc = max_chunks_of(chunk, num_seqs, total_tokens);
  size_t b = 256 + up256(mc * sizeof(int4)) + up256((static_cast<size_t>(num_seqs) + 1) * sizeof(int)) +
             up256(static_cast<size_t>(num_seqs) * sizeof(int) + 4) + up256(mc * hk * kq_stride(d, chunk)) +
             up256(mc * hv * tp_stride(chunk));
  if (use_segments(hv, d, form == 0 ? 1 : num_seqs, form)) {
    const size_t ns = max_segments_of(chunk, num_seqs, total_tokens);
    b += 256 + up256((static_cast<size_t>(num_seqs) + 1) * sizeof(int)) + up256(ns * sizeof(int4)) +
         3 * up256(ns * hv * static_cast<size_t>(d) * d * sizeof(float));
  }
  return b;
}

Workspace carve(void* base, int hk, int hv, int d, int chunk, int num_seqs, int total_tokens, int form) {
  char* p = static_cast<char*>(base);
  const size_t mc = max_chunks_of(chunk, num_seqs, total_tokens);
  Workspace w;
  w.n_chunks = reinterpret_cast<int*>(p);
  p += 256;
  w.table = reinterpret_cast<int4*>(p);
  p += up256(mc * sizeof(int4));
  w.chunk_off = reinterpret_cast<int*>(p);
  p += up256((static_cast<size_t>(num_seqs) + 1) * sizeof(int));
  w.order = reinterpret_cast<int*>(p);
  p += up256(static_cast<size_t>(num_seqs) * sizeof(int) + 4);
  w.kq = p;
  p += up256(mc * hk * kq_stride(d, chunk));
  w.tp = p;
  p += up256(mc * hv * tp_stride(chunk));
  w.kq_stride = static_cast<int64_t>(kq_stride(d, chunk));
  w.tp_stride = static_cast<int64_t>(tp_stride(chunk));
  w.segmented = use_segments(hv, d, num_seqs, form) ? 1 : 0;
  w.n_segs = nullptr;
  w.seg_off = nullptr;
  w.seg_table = nullptr;
  w.zs = w.mt = w.bt = nullptr;
  if (w.segmented) {
    const size_t ns = max_segments_of(chunk, num_seqs, total_tokens);
    const size_t mat = up256(ns * hv * static_cast<size_t>(d) * d * sizeof(float));
    w.n_segs = reinterpret_cast<int*>(p);
    p += 256;
    w.seg_off = reinterpret_cast<int*>(p);
    p += up256((static_cast<size_t>(num_seqs) + 1) * sizeof(int));
    w.seg_table = reinterpret_cast<int4*>(p);
    p += up256(ns * sizeof(int4));
    w.zs = reinterpret_cast<float*>(p);
    p += mat;
    w.mt = reinterpret_cast<float*>(p);
    p += mat;
    w.bt = reinterpret_cast<float*>(p);
  }
  return w;
}

// ------------------------------------------------------------------------ chunk table
// One workgroup. Each thread reads its sequence's bounds once (all reads independent),
// the chunk counts are scanned (in LDS; by shuffles within one wave up to 64
// sequences), and the chunk entries are written; the longest-first order is ranked from
// lengths kept on chip, so the kernel makes a single dependent round trip to global
// memory.
__global__ __launch_bounds__(kMetaThreads) void chunk_table_kernel(const int* __restrict__ cu, int N, int C,
                                                                  Workspace w) {
  __shared__ int scan[kMetaThreads];
  __shared__ int scan_seg[kMetaThreads];
  __shared__ int lens[kLptMaxSeqs];
  const int tid = threadIdx.x;
  const bool segmented = w.segmented != 0;
  if (N <= 64) {
    // Up to 64 sequences: one wave, lane s = sequence s; scans by shuffles (no LDS, no
    // barriers), and each sequence's entries written by all 64 lanes.
    if (tid >= 64) return;
    const int lane = tid;
    int start = 0, len = 0;
    if (lane < N) {
      start = cu[lane];
      len = cu[lane + 1] - start;
    }
    const int nc = (len + C - 1) / C;
    const int sc = segment_len(nc);
    const int ns = segmented ? (nc + sc - 1) / sc : 0;
    int inc = nc, inc_s = ns;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(inc, off, 64), us = __shfl_up(inc_s, off, 64);
      if (lane >= off) {
        inc += u;
        inc_s += us;
      }
    }
    const int first = inc - nc, first_seg = inc_s - ns;
    if (lane < N) {
      w.chunk_off[lane] = first;
      if (segmented) w.seg_off[lane] = first_seg;
    }
    if (lane == 0) {
      const int total = __builtin_amdgcn_readlane(inc, 63), total_s = __builtin_amdgcn_readlane(inc_s, 63);
      w.chunk_off[N] = total;
      *w.n_chunks = total;
      if (segmented) {
        w.seg_off[N] = total_s;
        *w.n_segs = total_s;
      }
    }
    for (int q = 0; q < N; ++q) {
      const int fq = __builtin_amdgcn_readlane(first, q), nq = __builtin_amdgcn_readlane(nc, q);
      const int sq = __builtin_amdgcn_readlane(start, q), lq = __builtin_amdgcn_readlane(len, q);
      for (int c = lane; c < nq; c += 64) w.table[fq + c] = make_int4(q, sq + c * C, min(C, lq - c * C), c);
      if (segmented) {
        const int gq = __builtin_amdgcn_readlane(first_seg, q), mq = __builtin_amdgcn_readlane(ns, q);
        const int scq = __builtin_amdgcn_readlane(sc, q);
        for (int g = lane; g < mq; g += 64) w.seg_table[gq + g] = make_int4(q, g * scq, min(nq, (g + 1) * scq), g == mq - 1);
      }
    }
    // longest sequence first (ties by index)
    if (lane < N) {
      int rank = 0;
      for (int q = 0; q < N; ++q) {
        const int lq = __builtin_amdgcn_readlane(len, q);
        rank += (lq > len) || (lq == len && q < lane);
      }
      w.order[rank] = lane;
    }
    return;
  }
  int carry = 0, carry_seg = 0;
  for (int base = 0; base < N; base += kMetaThreads) {
    const int s = base + tid;
    int start = 0, len = 0;
    if (s < N) {
      start = cu[s];
      len = cu[s + 1] - start;
    }
    const int nc = (len + C - 1) / C;
    const int sc = segment_len(nc);
    const int ns = segmented ? (nc + sc - 1) / sc : 0;  // segments of this sequence
    if (N <= kLptMaxSeqs && s < N) lens[s] = len;
    scan[tid] = nc;
    scan_seg[tid] = ns;
    __syncthreads();
    for (int off = 1; off < kMetaThreads; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      const int add_seg = tid >= off ? scan_seg[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      scan_seg[tid] += add_seg;
      __syncthreads();
    }
    const int first = carry + scan[tid] - nc;  // this sequence's first chunk index
    const int first_seg = carry_seg + scan_seg[tid] - ns;
    if (s < N) {
      w.chunk_off[s] = first;
      for (int c = 0; c < nc; ++c) w.table[first + c] = make_int4(s, start + c * C, min(C, len - c * C), c);
      if (segmented) {
        w.seg_off[s] = first_seg;
        for (int g = 0; g < ns; ++g)
          w.seg_table[first_seg + g] = make_int4(s, g * sc, min(nc, (g + 1) * sc), g == ns - 1);
      }
    }
    carry += scan[kMetaThreads - 1];
    carry_seg += scan_seg[kMetaThreads - 1];
    __syncthreads();
  }
  if (tid == 0) {
    w.chunk_off[N] = carry;
    *w.n_chunks = carry;
    if (segmented) {
      w.seg_off[N] = carry_seg;
      *w.n_segs = carry_seg;
    }
  }
  // longest sequence first, so its long chain of chunks starts with the first wave of
  // workgroups (ties by index)
  for (int s = tid; s < N; s += kMetaThreads) {
    if (N <= kLptMaxSeqs) {
      const int ls = lens[s];
      int rank = 0;
      for (int q = 0; q < N; ++q) {
        const int lq = lens[q];
        rank += (lq > ls) || (lq == ls && q < s);
      }
      w.order[rank] = s;
    } else {
      w.order[s] = s;
    }
  }
}

// Inclusive prefix sum over the 64 lanes of a wave (fixed order).
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// ------------------------------------------------------------------------ intra-chunk
// Step 1's thread mapping: thread e < ACTIVE owns 8 adjacent channels (group e % G; q's D/8
// groups, then k's) of the rows RPT (e / G) .. RPT (e / G) + RPT - 1 of the chunk, so one
// row of q (or k) is held by D/8 adjacent, aligned lanes.
template <int D, int C>
struct QKMap {
  static constexpr int G = 2 * D / kConvVec;                              // 8-channel groups
  static constexpr int RPT = (G * C >= kThreads) ? G * C / kThreads : 1;  // rows per thread
  static constexpr int NS = C / RPT;                                       // row strips
  static constexpr int ACTIVE = G * NS;
  __device__ __forceinline__ static bool is_q(int tid) { return tid % G < G / 2; }
  __device__ __forceinline__ static int col(int tid) { return (tid % G % (G / 2)) * kConvVec; }
  __device__ __forceinline__ static int row0(int tid) { return (tid / G) * RPT; }
};

// The fused entry point's q/k conv, inside the intra-chunk kernel: the thread's rows and
// channels (QKMap) of q and k of k-head h, convolved from x (and, before the sequence's
// first token, from its conv state) into registers, not yet normalised; rows >= n are zero.
// The per-channel arithmetic is ConvTaps::apply, as in the conv kernels, so the values are
// those the conv kernel would have written. The K-1 rows before the strip are loaded once.
template <typename T, int K, int D, int C, bool SILU>
__device__ __forceinline__ void conv_qk_rows_k(const PrefillArgs& a, int h, int t0, int n, int seq_start, int s,
                                               float (&out)[QKMap<D, C>::RPT][kConvVec], int tid) {
  using QM = QKMap<D, C>;
  constexpr int RPT = QM::RPT;
  using V8 = Vec8<T>;
  using GT = const typename V8::GT;
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int c = 0; c < kConvVec; ++c) out[i][c] = 0.f;
  if (tid >= QM::ACTIVE) return;
  // (global-address-space pointers: every load below is issued before any is used, in
  // one memory round trip)
  GT* x = (GT*)static_cast<const T*>(a.conv.x);
  GT* cs = (GT*)reinterpret_cast<const T*>(a.conv.state_ptrs[s]);
  GT* wt = (GT*)static_cast<const T*>(a.conv.w);
  const bool has_b = a.conv.b != nullptr;
  GT* bs = (GT*)static_cast<const T*>(has_b ? a.conv.b : a.conv.w);  // (taps stand in when there is no bias)
  const int64_t cstride = a.conv.channels;
  const int pos0 = t0 - seq_start;  // position of the chunk's first row in its sequence
  const int ch = (QM::is_q(tid) ? 0 : a.r.hk * D) + h * D + QM::col(tid);  // channel of x, the taps and the conv state
  typename V8::Raw wr[K], br;
#pragma unroll
  for (int t = 0; t < K; ++t) wr[t] = V8::load_raw_g(wt + static_cast<int64_t>(ch) * K + t * kConvVec);
  br = V8::load_raw_g(bs + ch);
  const int r0 = QM::row0(tid);
  typename V8::Raw z[RPT + K - 1];  // z rows r0 - (K-1) .. r0 + RPT - 1 (chunk coordinates)
  if (pos0 >= K - 1 && a.conv.x_stride <= 0x7FFFFFFF) {
    // (past a sequence's first K-1 tokens every row comes from x: one base row, t0 - (K-1),
    // and 32-bit row indices)
    GT* xb = x + static_cast<int64_t>(t0 - (K - 1)) * a.conv.x_stride + ch;
    const uint32_t xs = static_cast<uint32_t>(a.conv.x_stride);
#pragma unroll
    for (int i = 0; i < RPT + K - 1; ++i) {
      const uint32_t idx = min(r0 + i, n - 1 + (K - 1));  // rows past the chunk's end repeat its last
      z[i] = V8::load_raw_g(xb + static_cast<uint64_t>(idx) * xs);
    }
  } else {
#pragma unroll
    for (int i = 0; i < RPT + K - 1; ++i) {
      const int rr = min(r0 - (K - 1) + i, n - 1);  // rows past the chunk's end repeat its last
      const int p = pos0 + rr;                       // position in the sequence
      GT* src = p >= 0 ? x + static_cast<int64_t>(seq_start + p) * a.conv.x_stride + ch
                       : cs + static_cast<int64_t>(p + K - 1) * cstride + ch;
      z[i] = V8::load_raw_g(src);
    }
  }
  ConvTaps<T, K> taps;
  taps.from_raw(wr, br, has_b);
  // each z row converted once; row i's window is rows i .. i + K - 1
  float zf[RPT + K - 1][kConvVec];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) V8::convert(z[j], zf[j]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    V8::convert(z[i + K - 1], zf[i + K - 1]);
    if (r0 + i < n) {
      float win[K - 1][kConvVec], cur[kConvVec];
#pragma unroll
      for (int j = 0; j < K - 1; ++j)
#pragma unroll
        for (int c = 0; c < kConvVec; ++c) win[j][c] = zf[i + j][c];
#pragma unroll
      for (int c = 0; c < kConvVec; ++c) cur[c] = zf[i + K - 1][c];
      taps.apply(win, cur, SILU, out[i]);
    }
  }
}

template <typename T, int K, int D, int C>
__device__ __forceinline__ void conv_qk_rows_act(const PrefillArgs& a, int h, int t0, int n, int seq_start, int s,
                                                 float (&out)[QKMap<D, C>::RPT][kConvVec], int tid) {
  // (the activation as a template argument: no per-value select)
  if (a.conv.silu) {
    conv_qk_rows_k<T, K, D, C, true>(a, h, t0, n, seq_start, s, out, tid);
  } else {
    conv_qk_rows_k<T, K, D, C, false>(a, h, t0, n, seq_start, s, out, tid);
  }
}

template <int D, int C>
__device__ __forceinline__ void conv_qk_rows(const PrefillArgs& a, int h, int t0, int n, int seq_start, int s,
                                             float (&out)[QKMap<D, C>::RPT][kConvVec], int tid) {
  if (a.conv.bf16) {
    switch (a.conv.width) {
      case 2: conv_qk_rows_act<uint16_t, 2, D, C>(a, h, t0, n, seq_start, s, out, tid); break;
      case 3: conv_qk_rows_act<uint16_t, 3, D, C>(a, h, t0, n, seq_start, s, out, tid); break;
      default: conv_qk_rows_act<uint16_t, 4, D, C>(a, h, t0, n, seq_start, s, out, tid); break;
    }
  } else {
    switch (a.conv.width) {
      case 2: conv_qk_rows_act<float, 2, D, C>(a, h, t0, n, seq_start, s, out, tid); break;
      case 3: conv_qk_rows_act<float, 3, D, C>(a, h, t0, n, seq_start, s, out, tid); break;
      default: conv_qk_rows_act<float, 4, D, C>(a, h, t0, n, seq_start, s, out, tid); break;
    }
  }
}

// The same rows and channels of q and k as given (fp32), rows >= n zero.
template <int D, int C>
__device__ __forceinline__ void load_qk_rows(const RecurArgs& r, int h, int t0, int n,
                                             float (&out)[QKMap<D, C>::RPT][kConvVec], int tid) {
  using QM = QKMap<D, C>;
  const bool isq = QM::is_q(tid);
  const float* src = (isq ? r.q : r.k) + h * D + QM::col(tid);
  const int64_t stride = isq ? r.q_stride : r.k_stride;
  const int r0 = QM::row0(tid);
#pragma unroll
  for (int i = 0; i < QM::RPT; ++i) {
    if (tid < QM::ACTIVE && r0 + i < n) {
      load_k<kConvVec>(src + static_cast<int64_t>(t0 + r0 + i) * stride, out[i]);
    } else {
#pragma unroll
      for (int c = 0; c < kConvVec; ++c) out[i][c] = 0.f;
    }
  }
}

// The conv-state commit of the fused entry point, for one (sequence, k-head): the
// channels of q and k of k-head h and of v of its `group` v-heads become the last K-1
// rows of [old conv state | the sequence's x rows] (rows before the sequence come from
// the old state, as in the conv kernels). The chunk-0 workgroup of the pair runs it after
// its own loader, the only reader of the old q/k rows; the v rows were read by the v
// conv, which ran before. (group = 0 where the inter-chunk kernel convolves v: it
// commits the v channels itself.) A thread owns 8 channels.
template <typename T, int K, int D>
__device__ __forceinline__ void commit_conv_rows_k(const PrefillArgs& a, int h, int group, int s, int tid) {
  constexpr int NQ = sizeof(T) / 2;  // 16-byte pieces of 8 channels
  const int start = a.cu_seqlens[s];
  const int L = a.cu_seqlens[s + 1] - start;
  T* cs = reinterpret_cast<T*>(a.conv.state_ptrs[s]);
  const T* x = static_cast<const T*>(a.conv.x);
  const int64_t C = a.conv.channels;
  const int ng = (2 + group) * D / kConvVec;
  for (int e = tid; e < ng; e += kThreads) {
    const int c8 = e * kConvVec;  // position in [q of h | k of h | v of the group]
    const int ch = c8 < D ? h * D + c8
                 : c8 < 2 * D ? a.r.hk * D + h * D + (c8 - D)
                              : 2 * a.r.hk * D + h * group * D + (c8 - 2 * D);
    // New row i is row L + i of z; in increasing i an old state row is always read before
    // it is overwritten (L >= 1), so rows are copied one at a time.
#pragma unroll
    for (int i = 0; i < K - 1; ++i) {
      const int r = L + i;
      const T* src = r < K - 1 ? cs + static_cast<int64_t>(r) * C + ch
                               : x + static_cast<int64_t>(start + r - (K - 1)) * a.conv.x_stride + ch;
      T* dst = cs + static_cast<int64_t>(i) * C + ch;
#pragma unroll
      for (int q = 0; q < NQ; ++q) reinterpret_cast<uint4*>(dst)[q] = reinterpret_cast<const uint4*>(src)[q];
    }
  }
}

template <int D>
__device__ __forceinline__ void commit_conv_rows(const PrefillArgs& a, int h, int group, int s, int tid) {
  if (a.conv.bf16) {
    switch (a.conv.width) {
      case 2: commit_conv_rows_k<uint16_t, 2, D>(a, h, group, s, tid); break;
      case 3: commit_conv_rows_k<uint16_t, 3, D>(a, h, group, s, tid); break;
      default: commit_conv_rows_k<uint16_t, 4, D>(a, h, group, s, tid); break;
    }
  } else {
    switch (a.conv.width) {
      case 2: commit_conv_rows_k<float, 2, D>(a, h, group, s, tid); break;
      case 3: commit_conv_rows_k<float, 3, D>(a, h, group, s, tid); break;
      default: commit_conv_rows_k<float, 4, D>(a, h, group, s, tid); break;
    }
  }
}

// LDS of the intra-chunk kernel, in floats. K^ and Q^ live only until K K^T and Q K^T are
// in registers; then G and QK take K^'s place and A and T take Q^'s, so the peak is two
// areas, each the largest of K^ as fp32 rows, K^ as bf16 hi and lo planes and two C x C
// matrices (74 KB at C = 64, D = 128); with the decay terms of up to 8 v-heads (4 KB) two
// workgroups still fit on a CU.
template <int D, int C>
struct IntraLayout {
  // Row strides of K^ and Q^ are 32 bytes more than a multiple of 64 (fp32 rows D + 8
  // values, bf16 plane rows D + 16): the MFMA fragment reads of steps 1b and 2 (16 rows,
  // one 16-byte group per lane, groups 16 bytes apart across the four 16-lane quarters)
  // then meet no bank conflict on gfx950, where rows D + 4 (or D + 8) values long cost
  // twice the cycles (measured with per-pattern bank-conflict counters).
  static constexpr int KP = D + 8;  // padded row of K^/Q^
  static constexpr int CP = C + 4;  // padded row of C x C matrices
  static constexpr int KHF = D + 16;  // a row of K^ (or Q^) as bf16 hi and lo planes, in floats
  static constexpr int RS0 = (C * KP > 2 * C * CP) ? C * KP : 2 * C * CP;
  static constexpr int RS = (RS0 > C * KHF) ? RS0 : C * KHF;  // one area
  static constexpr int OFF_K = 0;        // K^   alias  G, QK
  static constexpr int OFF_G = 0;
  static constexpr int OFF_QK = C * CP;
  static constexpr int OFF_Q = RS;       // Q^   alias  A, T
  static constexpr int OFF_A = RS;
  static constexpr int OFF_T = RS + C * CP;
  static constexpr int NGB = 8;           // v-heads whose gam and beta are held at once
  static constexpr int OFF_GAM = 2 * RS;  // [NGB][C]
  static constexpr int OFF_BET = OFF_GAM + NGB * C;
  static constexpr int TOTAL = OFF_BET + NGB * C;
};

template <int POL, int D, int C>
__global__ __launch_bounds__(kThreads) void intra_chunk_kernel(PrefillArgs a, Workspace w) {
  using M = Mma<POL>;
  using FIO = FragIO<POL>;
  using Lo = IntraLayout<D, C>;
  using F32 = Mma<kPolFP32>;
  constexpr int NB = C / 16;
  constexpr int KP = Lo::KP, CP = Lo::CP;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP;
  constexpr int NVF = D / KSTEP;              // k-steps over the head dim
  constexpr int NKF = FragCount<POL>::nk(C);  // k-steps over the chunk (padded)
  constexpr bool kWholeK = NKF * KSTEP == C && KPL % 4 == 0;  // no fragment k range runs past the chunk
  __shared__ __attribute__((aligned(16))) float smem[Lo::TOTAL];
  float(*Kh)[KP] = reinterpret_cast<float(*)[KP]>(smem + Lo::OFF_K);
  float(*Qh)[KP] = reinterpret_cast<float(*)[KP]>(smem + Lo::OFF_Q);
  float(*Am)[CP] = reinterpret_cast<float(*)[CP]>(smem + Lo::OFF_A);
  float(*Tm)[CP] = reinterpret_cast<float(*)[CP]>(smem + Lo::OFF_T);
  float(*Gm)[CP] = reinterpret_cast<float(*)[CP]>(smem + Lo::OFF_G);
  float(*QKm)[CP] = reinterpret_cast<float(*)[CP]>(smem + Lo::OFF_QK);
  float* gam = smem + Lo::OFF_GAM;
  float* bet = smem + Lo::OFF_BET;

  const int chunk = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the chunk's (sequence, first token, tokens, index in its sequence): from the chunk
  // table, or -- whole sequences, at most 64 of them, no table launch -- from cu_seqlens,
  // by one scan in every wave (lane s = sequence s); then the chunk-(0, 0) workgroup writes
  // the sequences' chunk offsets and the longest-first order for the inter-chunk kernel
  int4 ent;
  if (a.table_free && a.num_seqs == 1) {
    // one sequence: cu_seqlens is [0, total_tokens], so the chunk's place needs no load
    const int T = a.total_tokens;
    const int total = (T + C - 1) / C;
    if (chunk == 0 && h == 0 && wave == 0 && lane == 0) {
      w.chunk_off[0] = 0;
      w.chunk_off[1] = total;
      *w.n_chunks = total;
      w.order[0] = 0;
    }
    if (chunk >= total) return;
    ent = make_int4(0, chunk * C, min(C, T - chunk * C), chunk);
  } else if (a.table_free) {
    const int N = a.num_seqs;
    int start = 0, len = 0;
    if (lane < N) {
      start = a.cu_seqlens[lane];
      len = a.cu_seqlens[lane + 1] - start;
    }
    const int nc = (len + C - 1) / C;
    int inc = nc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(inc, off, 64);
      if (lane >= off) inc += u;
    }
    const int first = inc - nc;
    const int total = __builtin_amdgcn_readlane(inc, 63);
    if (chunk == 0 && h == 0 && wave == 0) {
      if (lane < N) {
        w.chunk_off[lane] = first;
        int rank = 0;  // longest sequence first, ties by index
        for (int q = 0; q < N; ++q) {
          const int lq = __builtin_amdgcn_readlane(len, q);
          rank += (lq > len) || (lq == len && q < lane);
        }
        w.order[rank] = lane;
      }
      if (lane == 0) {
        w.chunk_off[N] = total;
        *w.n_chunks = total;
      }
    }
    if (chunk >= total) return;
    const uint64_t owner = __ballot(lane < N && chunk >= first && chunk < first + nc);
    const int sq = __builtin_ctzll(owner);
    const int fq = __builtin_amdgcn_readlane(first, sq), sst = __builtin_amdgcn_readlane(start, sq);
    const int sl = __builtin_amdgcn_readlane(len, sq);
    const int cq = chunk - fq;
    ent = make_int4(sq, sst + cq * C, min(C, sl - cq * C), cq);
  } else {
    if (chunk >= *w.n_chunks) return;
    ent = w.table[chunk];
  }
  const int t0 = ent.y, n = ent.z;
  const RecurArgs& r = a.r;
  const int l16 = lane & 15, lg = lane >> 4;
  const int group = r.hv / r.hk;
  // The decay terms of the group's v-heads are formed NGB v-heads at a time, v-head
  // jb + i of a batch on wave (i + 4) % 8 (waves 4-7 have one product fewer in step 2);
  // the first batch's g and beta are read here.
  constexpr int NGB = Lo::NGB;
  static_assert(NGB == kWaves, "one v-head per wave in a batch");
  const int my_gb = (wave + 4) % kWaves;  // this wave's v-head within a batch
  float g_in = 0.f, b_in = 0.f;
  auto load_gb = [&](int jb) {
    if (jb + my_gb < group) {
      const int tl = min(lane, n - 1);  // (a valid token; lanes >= n are masked at use)
      g_in = r.g[static_cast<int64_t>(t0 + tl) * r.hv + h * group + jb + my_gb];
      b_in = r.beta[static_cast<int64_t>(t0 + tl) * r.hv + h * group + jb + my_gb];
    }
  };
  load_gb(0);
  // gam (inclusive cumsum of g over the chunk) and beta into LDS, and the chunk's decay
  // factors for the inter-chunk kernel into the workspace (lanes >= n hold gam_{n-1})
  auto decay_terms = [&](int jb) {
    if (jb + my_gb >= group) return;
    const int j = h * group + jb + my_gb;
    float* gam_out = reinterpret_cast<float*>(w.tp + (static_cast<int64_t>(chunk) * r.hv + j) * w.tp_stride +
                                              2 * static_cast<size_t>(C / 16) * FragCount<POL>::nk(C) * FIO::BYTES);
    const float gv = wave_inclusive_scan(lane < n ? g_in : 0.f);
    const float bv = lane < n ? b_in : 0.f;
    const float gn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), C - 1));
    if (lane < C) {
      gam[my_gb * C + lane] = gv;
      bet[my_gb * C + lane] = bv;
      gam_out[lane] = expf(gv);
      gam_out[C + lane] = bv;
      gam_out[2 * C + lane] = expf(gn - gv);
    }
  };

  // 1. normalised K and Q rows of the chunk into LDS; rows >= n are zero. Each thread holds
  // its rows and channels (QKMap) in registers -- convolved from x through the fused entry
  // point, else read -- and a row's squared norm is the sum of the thread's 8 squares (in
  // channel order) summed over the D/8 lanes that hold the row. With bf16x3 products, K^
  // and Q^ are kept as bf16 hi and lo planes ([C][KH] each, the lo plane after the hi one):
  // split once here, then read as they are by the products and the export below.
  using QM = QKMap<D, C>;
  const bool fused = a.conv.x != nullptr;
  constexpr bool kPlanes = POL == kPolBF16X3;
  constexpr int KH = Lo::KHF;  // plane row length (elements)
  auto* Khp = reinterpret_cast<__bf16*>(smem + Lo::OFF_K);
  auto* Qhp = reinterpret_cast<__bf16*>(smem + Lo::OFF_Q);
  {
    float rows[QM::RPT][kConvVec];
    if (fused) {
      conv_qk_rows<D, C>(a, h, t0, n, t0 - ent.w * C, ent.x, rows, tid);
    } else {
      load_qk_rows<D, C>(r, h, t0, n, rows, tid);
    }
    const bool isq = QM::is_q(tid);
    const int col = QM::col(tid), r0 = QM::row0(tid);
    const float num = isq ? r.scale : 1.0f;
    // Squared norms of the thread's rows; every lane of a row's group holds the same bits
    // (group_sum). Where a row's group spans at least RPT lanes, lane l of each aligned run
    // of RPT lanes forms the factor of row l % RPT only and the RPT factors are gathered
    // from those lanes (the same bits as if each lane formed all of them), instead of every
    // lane taking RPT square roots and divisions.
    constexpr int RPT = QM::RPT;
    constexpr bool kShare = (RPT == 2 || RPT == 4) && D / kConvVec >= RPT;
    float ss[RPT], rs[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      ss[i] = 0.f;
#pragma unroll
      for (int c = 0; c < kConvVec; ++c) ss[i] = fmaf(rows[i][c], rows[i][c], ss[i]);
      ss[i] = group_sum<D / kConvVec>(ss[i]);
    }
    auto factor = [&](float sq) { return r.qk_norm ? num / sqrtf(sq + r.eps) : num; };
    if constexpr (kShare) {
      const int mine = lane % RPT;
      float sq = ss[0];
#pragma unroll
      for (int i = 1; i < RPT; ++i) sq = mine == i ? ss[i] : sq;
      const float f = factor(sq);
      auto from = [&](auto ctrl) {  // quad_perm DPP move
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(f), decltype(ctrl)::value, 0xF, 0xF, false));
      };
      if constexpr (RPT == 4) {  // lane i of the quad: quad_perm [i, i, i, i]
        rs[0] = from(std::integral_constant<int, 0x00>());
        rs[1] = from(std::integral_constant<int, 0x55>());
        rs[2] = from(std::integral_constant<int, 0xAA>());
        rs[3] = from(std::integral_constant<int, 0xFF>());
      } else {  // lane i of each pair: quad_perm [i, i, 2 + i, 2 + i]
        rs[0] = from(std::integral_constant<int, 0xA0>());
        rs[1] = from(std::integral_constant<int, 0xF5>());
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) rs[i] = factor(ss[i]);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = r0 + i;
      if (row >= n) rs[i] = 0.f;
      float v[kConvVec];
#pragma unroll
      for (int c = 0; c < kConvVec; ++c) v[c] = rows[i][c] * rs[i];
      if (tid < QM::ACTIVE) {
        if constexpr (kPlanes) {
          // (the split is Mma<>::split's)
          bf16x8 hi, lo;
#pragma unroll
          for (int c = 0; c < kConvVec; ++c) {
            hi[c] = static_cast<__bf16>(v[c]);
            lo[c] = static_cast<__bf16>(v[c] - static_cast<float>(hi[c]));
          }
          __bf16* dst = (isq ? Qhp : Khp) + row * KH + col;
          *reinterpret_cast<bf16x8*>(dst) = hi;
          *reinterpret_cast<bf16x8*>(dst + C * KH) = lo;
        } else {
          float* dst = isq ? &Qh[row][col] : &Kh[row][col];
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
      }
    }
  }
  // (here, while this wave's only memory operations in flight are loads: a later wait for
  // g and beta would also wait for the exports' stores)
  decay_terms(0);
  __syncthreads();
  // the A-operand fragment of row t, head-dim values d0 .. d0 + KPL - 1 of K^ (or Q^)
  auto frag_of = [&](bool isq, int t, int d0) {
    if constexpr (kPlanes) {
      const __bf16* base = (isq ? Qhp : Khp) + t * KH + d0;
      typename M::Frag f;
      f.hi = *reinterpret_cast<const bf16x8*>(base);
      f.lo = *reinterpret_cast<const bf16x8*>(base + C * KH);
      return f;
    } else {
      float x[KPL];
      load_k<KPL>(isq ? &Qh[t][d0] : &Kh[t][d0], x);
      return M::frag(x);
    }
  };

  // 1b. export K^ and Q^ as A operands in fragment order. Thread e writes lane e % 64 of
  // fragment block e / 64, so each wave stores whole contiguous KiBs.
  {
    char* kq = w.kq + (static_cast<int64_t>(chunk) * r.hk + h) * w.kq_stride;
    char* qq = kq + static_cast<size_t>(C / 16) * NVF * FIO::BYTES;
    for (int e = tid; e < (C / 16) * NVF * 64; e += kThreads) {
      const int blk = e / 64, ln = e % 64;
      const int t = (blk / NVF) * 16 + ln % 16, d0 = (blk % NVF) * KSTEP + KPL * (ln / 16);
      FIO::store_frag(kq + static_cast<size_t>(blk) * FIO::BYTES, ln, frag_of(false, t, d0));
      FIO::store_frag(qq + static_cast<size_t>(blk) * FIO::BYTES, ln, frag_of(true, t, d0));
    }
  }

  // 2. G = K^ K^T and QK = Q^ K^T on the lower-triangular 16x16 tiles, held in registers
  // until every wave is done reading K^ and Q^, then written over them
  {
    constexpr int NT = NB * (NB + 1) / 2;
    constexpr int MAXI = (2 * NT + kWaves - 1) / kWaves;  // tiles per wave
    const int kl = KPL * lg;
    f32x4 res[MAXI];
#pragma unroll
    for (int q = 0; q < MAXI; ++q) {
      const int item = wave + q * kWaves;
      if (item < 2 * NT) {
        const bool isq = item >= NT;
        const int it = isq ? item - NT : item;
        int ti = 0;
        while ((ti + 1) * (ti + 2) / 2 <= it) ++ti;
        const int tj = it - ti * (ti + 1) / 2;
        f32x4 a3[3];
        zero3(a3);
#pragma unroll
        for (int v = 0; v < NVF; ++v)
          M::mma3(a3, frag_of(isq, ti * 16 + l16, kl + v * KSTEP), frag_of(false, tj * 16 + l16, kl + v * KSTEP));
        res[q] = total(a3);
      }
    }
    __syncthreads();  // K^ and Q^ are dead
#pragma unroll
    for (int q = 0; q < MAXI; ++q) {
      const int item = wave + q * kWaves;
      if (item < 2 * NT) {
        const bool isq = item >= NT;
        const int it = isq ? item - NT : item;
        int ti = 0;
        while ((ti + 1) * (ti + 2) / 2 <= it) ++ti;
        const int tj = it - ti * (ti + 1) / 2;
        float(*Out)[CP] = isq ? QKm : Gm;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) Out[ti * 16 + 4 * lg + rr][tj * 16 + l16] = res[q][rr];
      }
    }
  }
  __syncthreads();

  // 3. per v-head of this k-head's group: decay mask, A, T = (I + A)^-1, P (the decay
  // terms of v-heads 8 and on are formed when their batch comes up)
  for (int jj = 0; jj < group; ++jj) {
    const int j = h * group + jj;
    char* tp = w.tp + (static_cast<int64_t>(chunk) * r.hv + j) * w.tp_stride;
    char* pp = tp + static_cast<size_t>(C / 16) * NKF * FIO::BYTES;
    if (jj > 0 && jj % NGB == 0) {
      load_gb(jj);
      decay_terms(jj);
      __syncthreads();
    }
    const float* gamj = gam + (jj % NGB) * C;
    const float* betj = bet + (jj % NGB) * C;

    // A (strictly lower) into LDS and P (lower incl. diagonal) to the workspace, one
    // fragment lane per thread; the k range runs to the padded NKF * KSTEP so the zero
    // padding of the P fragments is written too. Fragments wholly above the diagonal are
    // neither written nor read: the inter-chunk kernel skips their products (the same
    // test, kk * KSTEP >= 16 (row tile + 1)), and A's upper triangle is never read. Nor is
    // a lane's part of a fragment whose k range starts past its row (s0 > t, all zeros):
    // the inter-chunk kernel takes zeros for it (for T as well).
    for (int e = tid; e < (C / 16) * NKF * 64; e += kThreads) {
      const int blk = e / 64, ln = e % 64;
      if ((blk % NKF) * KSTEP >= (blk / NKF + 1) * 16) continue;
      const int t = (blk / NKF) * 16 + ln % 16, s0 = (blk % NKF) * KSTEP + KPL * (ln / 16);
      float pv[KPL];
      if constexpr (kWholeK) {
        // (the lane's k range lies inside the chunk: its LDS values are read as whole
        // 16-byte groups and the mask is applied by selection; the same arithmetic)
        const float gt = gamj[t], bt = betj[t];
        float gs[KPL], qk[KPL], gg[KPL];
        load_k<KPL>(gamj + s0, gs);
        load_k<KPL>(&QKm[t][s0], qk);
        load_k<KPL>(&Gm[t][s0], gg);
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const int s = s0 + i;
          const float dec = expf(gt - gs[i]);  // (s > t: unused, possibly inf)
          pv[i] = s <= t ? dec * qk[i] : 0.f;
          Am[t][s] = s < t ? bt * dec * gg[i] : 0.f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const int s = s0 + i;
          float av = 0.f;
          pv[i] = 0.f;
          if (s <= t) {
            const float dec = expf(gamj[t] - gamj[s]);
            pv[i] = dec * QKm[t][s];
            if (s < t) av = betj[t] * dec * Gm[t][s];
          }
          if (s < C) Am[t][s] = av;
        }
      }
      if (s0 <= t) FIO::store(pp + static_cast<size_t>(blk) * FIO::BYTES, ln, pv);
    }
    __syncthreads();

    // diagonal 16x16 blocks by forward substitution, all on one wave: lane 16 b + c owns
    // column c of block b. (One block per wave would issue the same instructions on four
    // waves with 16 lanes each; the kernel's time follows the total work of the two
    // workgroups sharing a CU, so the other waves leave the SIMDs to the other one.)
    static_assert(NB <= 4, "the diagonal blocks fit one wave");
    if (wave == 1 && lane < NB * 16) {
      const int b = lane >> 4, c = lane & 15;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
        for (int k = 0; k < i; ++k) acc = fmaf(-Am[b * 16 + i][b * 16 + k], x[k], acc);
        x[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) Tm[b * 16 + i][b * 16 + c] = x[i];
    }
    __syncthreads();

    // off-diagonal blocks by distance from the diagonal, one wave per block, on fp32 MFMA:
    //   Wb = sum_{k=jb}^{ib-1} A_{ib,k} T_{k,jb},   T_{ib,jb} = -T_{ib,ib} Wb.
    // Wb's accumulator layout (lane l: rows 4(l/16)+r, column l%16) is exactly the B
    // operand layout of the second product, so it feeds it without a round trip.
    for (int dd = 1; dd < NB; ++dd) {
      for (int jb = wave; jb < NB - dd; jb += kWaves) {
        const int ib = jb + dd;
        f32x4 wacc = {0.f, 0.f, 0.f, 0.f};
        for (int kb = jb; kb < ib; ++kb) {
          // one 16-deep step: lane l supplies k = 4(l/16) + e, e = 0..3
          F32::Frag fa, fb;
          const float4 av = *reinterpret_cast<const float4*>(&Am[ib * 16 + l16][kb * 16 + 4 * lg]);
          fa.v[0] = av.x; fa.v[1] = av.y; fa.v[2] = av.z; fa.v[3] = av.w;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) fb.v[e2] = Tm[kb * 16 + 4 * lg + e2][jb * 16 + l16];
          F32::mma(wacc, fa, fb);
        }
        F32::Frag ta, tb;
        const float4 tv = *reinterpret_cast<const float4*>(&Tm[ib * 16 + l16][ib * 16 + 4 * lg]);
        ta.v[0] = tv.x; ta.v[1] = tv.y; ta.v[2] = tv.z; ta.v[3] = tv.w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) tb.v[e2] = wacc[e2];
        f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
        F32::mma(tacc, ta, tb);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) Tm[ib * 16 + 4 * lg + rr][jb * 16 + l16] = -tacc[rr];
      }
      __syncthreads();
    }

    for (int e = tid; e < (C / 16) * NKF * 64; e += kThreads) {
      const int blk = e / 64, ln = e % 64;
      if ((blk % NKF) * KSTEP >= (blk / NKF + 1) * 16) continue;  // (above the diagonal, as P)
      const int t = (blk / NKF) * 16 + ln % 16, s0 = (blk % NKF) * KSTEP + KPL * (ln / 16);
      float tv[KPL];
      if constexpr (kWholeK) {
        float tr[KPL];
        load_k<KPL>(&Tm[t][s0], tr);
#pragma unroll
        for (int i = 0; i < KPL; ++i) tv[i] = (s0 + i <= t) ? tr[i] : 0.f;
      } else {
#pragma unroll
        for (int i = 0; i < KPL; ++i) tv[i] = (s0 + i <= t) ? Tm[t][s0 + i] : 0.f;
      }
      if (s0 <= t) FIO::store(tp + static_cast<size_t>(blk) * FIO::BYTES, ln, tv);
    }
    __syncthreads();
  }
  if (fused && ent.w == 0) commit_conv_rows<D>(a, h, a.v_in_inter ? 0 : group, ent.x, tid);
}

// ------------------------------------------------------------------------ inter-chunk
// LDS banking on gfx950 (measured with per-pattern bank-conflict counters): 64 banks of
// 4 bytes; a 16-byte write is served 8 lanes at a time (lanes 8i .. 8i+7, one aligned
// 128-byte window), an 8-byte write 16 lanes at a time (one 128-byte window), an 8-byte
// read -- the transposing ds_read_b64_tr_b16 included -- 32 lanes at a time (one
// 256-byte window); lanes of one such pass that hit the same bank at different addresses
// are served one after another. The tiles below are laid out so that the reads of every
// step, and the 16-byte writes, meet no conflict.
//
// K^ of the current chunk in LDS as a C x D matrix (one plane per operand part: bf16 hi
// and lo, or fp32), written by rows from the K side's A fragments and read by columns as
// the B operand of the state update, whose contraction runs over tokens. A row is D
// values in 16-byte groups; group g of row t is stored at position g ^ swz(t). With bf16
// planes (256-byte rows) swz(t) = 5 t mod 16: the 8 consecutive rows of a row-wise write
// (one group each) land in 8 distinct groups, and the 32 lanes of a column read (rows t0 ..
// t0 + 3 and t0 + 8 .. t0 + 11, ..., two 8-byte halves of one group each) in 32 distinct
// 8-byte slots.
template <int POL, int D, int C>
struct KTile {
  using F = typename Mma<POL>::Frag;
  static constexpr int KPL = Mma<POL>::KPL;
  static constexpr int ES = POL == kPolBF16X3 ? 2 : 4;  // bytes per element of a plane
  static constexpr int ROW = D * ES;
  static constexpr int GPR = ROW / 16;  // 16-byte groups per row
  static constexpr int PLANE = C * ROW;
  static constexpr int BYTES = POL == kPolBF16X3 ? 2 * PLANE : PLANE;
  __device__ __forceinline__ static int swz(int t) {
    if constexpr (POL == kPolBF16X3) return (5 * t) & (GPR - 1);
    return ((t & 7) ^ (((t >> 3) & 3) << 1)) & (GPR - 1);
  }
  __device__ __forceinline__ static int off(int t, int d) {
    return t * ROW + ((((d * ES) >> 4) ^ swz(t)) << 4) + ((d * ES) & 15);
  }
  // the A fragment holding row t, head-dim values d0 .. d0 + KPL - 1 (one 16-byte group)
  __device__ __forceinline__ static void put(char* base, int t, int d0, const F& f) {
    char* p = base + off(t, d0);
    if constexpr (POL == kPolBF16X3) {
      *reinterpret_cast<bf16x8*>(p) = f.hi;
      *reinterpret_cast<bf16x8*>(p + PLANE) = f.lo;
    } else {
      *reinterpret_cast<float4*>(p) = make_float4(f.v[0], f.v[1], f.v[2], f.v[3]);
    }
  }
  // The fragment of column d = d0 + l16 (d0 a multiple of 16), rows t0 .. t0 + KPL - 1,
  // for lane l16 of a 16-lane group (all 16 lanes of the group call it with the same d0
  // and t0). bf16 planes: gfx950's transposing LDS read (ds_read_b64_tr_b16) -- lane
  // s = 4 k + c of the group reads the 4 values of row k, columns 4 c .. 4 c + 3 of a 4 x 16
  // block, and lane j receives column j of the block, rows 0 .. 3 -- two per plane instead
  // of 8 single-value reads.
  __device__ __forceinline__ static F column16(const char* base, int d0, int t0, int l16) {
    if constexpr (POL == kPolBF16X3) {
      typedef short i16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      // (a chunk shorter than a k-step leaves groups of lanes past its last row; callers
      // discard their values, and the clamp keeps their reads inside the tile)
      if constexpr (C % Mma<POL>::KSTEP != 0) t0 = min(t0, C - 8);
      const int tr = t0 + (l16 >> 2), dc = d0 + 4 * (l16 & 3);
      const char* p0 = base + off(tr, dc);      // rows t0 .. t0 + 3
      const char* p1 = base + off(tr + 4, dc);  // rows t0 + 4 .. t0 + 7
      const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
      const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
      const i16x4 l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + PLANE));
      const i16x4 l1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1 + PLANE));
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 hv = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      const i16x8 lv = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
      F f;
      f.hi = __builtin_bit_cast(bf16x8, hv);
      f.lo = __builtin_bit_cast(bf16x8, lv);
      return f;
    } else {
      return column(base, d0 + l16, t0);
    }
  }
  // B fragment: column d, rows t0 .. t0 + KPL - 1
  __device__ __forceinline__ static F column(const char* base, int d, int t0) {
    F f;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const char* p = base + off(t0 + i, d);
      if constexpr (POL == kPolBF16X3) {
        f.hi[i] = *reinterpret_cast<const __bf16*>(p);
        f.lo[i] = *reinterpret_cast<const __bf16*>(p + PLANE);
      } else {
        f.v[i] = *reinterpret_cast<const float*>(p);
      }
    }
    return f;
  }
};

// A 16-row operand tile in LDS (the state slice, 16 x D, and R^T, U^T, Us^T, 16 x C),
// stored pre-split as Split<> does. bf16 planes: rows unpadded, 16-byte group g of row r
// at position g ^ (r mod NG) (NG groups per row), so that a fragment read (16 rows, one
// group column per 16 lanes) covers all banks once; a 4-value write is 8 bytes, half a
// group. fp32: rows padded by 4 values, as Split<> stores them.
template <int POL, int COLS>
struct RowTile {
  using M = Mma<POL>;
  using F = typename M::Frag;
  static constexpr bool kPlanes = POL == kPolBF16X3;
  static constexpr int LD = kPlanes ? COLS : COLS + 4;  // elements per row
  static constexpr int NG = COLS * 2 / 16;              // 16-byte groups per bf16 row
  static constexpr int PLANE = 16 * COLS * 2;           // bytes per bf16 plane
  static constexpr int BYTES = kPlanes ? 2 * PLANE : 16 * LD * 4;
  __device__ __forceinline__ static int off(int row, int col) {  // byte offset in a bf16 plane
    const int b = col * 2;
    return row * (COLS * 2) + ((((b >> 4) ^ row) & (NG - 1)) << 4) + (b & 15);
  }
  // the fragment of row `row`, columns col .. col + KPL - 1 (col a multiple of KPL)
  __device__ __forceinline__ static F load(const char* base, int row, int col) {
    if constexpr (kPlanes) {
      const char* p = base + off(row, col);
      F f;
      f.hi = *reinterpret_cast<const bf16x8*>(p);
      f.lo = *reinterpret_cast<const bf16x8*>(p + PLANE);
      return f;
    } else {
      return Split<POL>::load(base, 16, LD, row, col);
    }
  }
  // 4 consecutive values of row `row` from column col (a multiple of 4)
  __device__ __forceinline__ static void store4(char* base, int row, int col, const float* x) {
    if constexpr (kPlanes) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 h, l;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 t = static_cast<__bf16>(x[e]);
        h[e] = t;
        l[e] = static_cast<__bf16>(x[e] - static_cast<float>(t));
      }
      char* p = base + off(row, col);
      *reinterpret_cast<bf16x4*>(p) = h;
      *reinterpret_cast<bf16x4*>(p + PLANE) = l;
    } else {
      Split<POL>::store(base, 16, LD, row, col, x, 4);
    }
  }
};

// Everything one wave reads from global memory for one chunk; loaded one chunk ahead so
// the loads overlap the previous chunk's arithmetic. Waves 0-3 ("K side") hold K^ rows
// and T rows, waves 4-7 ("Q side") hold Q^ rows and P rows, of token tile wave % 4.
// x window of the fused v conv (see inter_chunk_kernel): positions a K-side lane reads per
// row block, its 4 output rows and the up to 3 before them
constexpr int kXWin = 7;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int POL, int D, int C, int NR, typename XT = float>
struct ChunkIn {
  using F = typename Mma<POL>::Frag;
  static constexpr int KSTEP = Mma<POL>::KSTEP;
  static constexpr int NV = D / KSTEP;                // k-steps over the head dim
  static constexpr int NK = (C + KSTEP - 1) / KSTEP;  // k-steps over the chunk's tokens
  F af[NV];     // K^ (or Q^) row of token 16*tt + l16
  F mf[NK];     // T (or P) row of token 16*tt + l16
  float vv[NR][4];  // v at the 4 output rows this lane holds in each of the workgroup's NR
                    // row blocks (K side; rows >= n masked at use)
  float eg[4];  // e^gam, beta and e^{gam_n - gam} at those rows
  float bt[4];
  float ed[4];
  float egn;    // e^{gam_n}, gam_n = gam of the chunk's last token
  int n;        // tokens in the chunk
  XT xw[NR][kXWin];  // fused v conv: the raw x (or conv-state) values of the lane's window
  u32x4 xt[NR];      // fused v conv, bf16 x: the lane's 16-byte piece of its wave's x tile
};

// What one launch of the inter-chunk kernel covers:
//   kModeWhole    : whole sequences, from the state in place to the final state, with outputs;
//   kModeTransfer : one segment's affine map: row blocks [0, d/16) run from identity rows
//                   with v = 0 and give M, the rest run from zero rows and give B; no outputs;
//   kModeSegment  : one segment's outputs, from its start state Z; the last segment of a
//                   sequence writes the final state.
constexpr int kModeWhole = 0;
constexpr int kModeTransfer = 1;
constexpr int kModeSegment = 2;

// NR: 16-row state blocks per workgroup. NR = 2 (whole sequences) serves two blocks of a
// head with one set of operand loads. A step is bound by the CU's memory pipe (each
// streams ~96 KiB of K^, Q^, T and P through it, at L2 latency), so where a launch has
// workgroups to spare, one two-block workgroup per CU that prefetches the next chunk moves
// half the operand bytes per state row of two one-block workgroups sharing the CU, and
// keeps its loads in flight across the step (on the ragged 8-sequence pack: 537 -> 357 us;
// two blocks without the prefetch lost to two one-block workgroups). Each block's
// arithmetic is the one-block kernel's, so the results are the same bits.
template <int POL, int D, int C, bool PF, int MODE, int NR = 1, int XV = 0>
__global__ __launch_bounds__(kInterThreads, (PF || NR > 1) ? 1 : 2) void inter_chunk_kernel(PrefillArgs a, Workspace w) {
  static_assert(NR == 1 || (NR == 2 && MODE == kModeWhole), "two blocks per workgroup: whole sequences only");
  static_assert(XV == 0 || (MODE == kModeWhole && PF && C == 64), "v convolved in the kernel: whole sequences, 64-token chunks");
  // fused v conv: XV = x dtype (1 bf16, 2 fp32) + 4 with SiLU (the activation chosen at
  // compile time, so that the conv computes no activation it then discards)
  using XT = typename std::conditional<(XV & 3) == 2, float, uint16_t>::type;
  constexpr bool kVAct = (XV & 4) != 0;
  using M = Mma<POL>;
  using SP = Split<POL>;
  using F = typename M::Frag;
  using In = ChunkIn<POL, D, C, NR, XT>;
  using FIO = FragIO<POL>;
  using KT = KTile<POL, D, C>;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP;
  constexpr int NBLK = D / kDVB;  // state-row blocks per head
  constexpr int NT = C / 16;      // token tiles per chunk
  constexpr int ST = D / 16;      // 16-column tiles of the state slice (one per wave)
  constexpr int NV = In::NV, NK = In::NK;
  using TS = RowTile<POL, D>;  // the state slice
  using TR = RowTile<POL, C>;  // R^T, U^T, Us^T
  static_assert(kDVB == 16, "16-row tiles");
  constexpr int S_BYTES = TS::BYTES;
  constexpr int R_BYTES = TR::BYTES;
  __shared__ __attribute__((aligned(16))) char lds[NR * (S_BYTES + 3 * R_BYTES) + KT::BYTES];
  char* Sl = lds;                     // state slices [NR][16][D]  B operand of K^S^T, Q^S^T
  char* Rt = lds + NR * S_BYTES;      // R^T          [NR][16][C]  B operand of T R
  char* Ut = Rt + NR * R_BYTES;       // U^T          [NR][16][C]  B operand of P U
  char* Us = Ut + NR * R_BYTES;       // (e^{gam_n-gam} U)^T       A operand of the update
  char* Kl = Us + NR * R_BYTES;       // K^           [C][D]       B operand of the update
  __shared__ __attribute__((aligned(16))) float Fl[2][3 * C];  // (prefetching form) e^gam, beta, e^{gam_n-gam} of two chunks
  // fused v conv with bf16 x: each K-side wave's x tile, positions 16 tt - 3 .. 16 tt + 15
  // of its token tile (rows) by the 16 channels of each row block (32 bytes a row)
  constexpr bool kXTile = (XV & 3) == 1;
  constexpr int kXPos = 19;
  __shared__ __attribute__((aligned(16))) uint16_t Xl[kXTile ? 4 : 1][NR][kXTile ? kXPos * 16 : 8];

  const RecurArgs& r = a.r;
  constexpr int RB = MODE == kModeTransfer ? 2 * NBLK : NBLK / NR;  // workgroups per head
  const int per_unit = RB * r.hv;
  const int L = blockIdx.x;
  const int zi = L / per_unit;
  const int rem = L % per_unit;
  // workgroups are dealt round-robin to the 8 XCDs: give the slices of one head
  // consecutive virtual ids on one XCD so they share that XCD's L2
  const int vid = (per_unit % 8 == 0) ? (rem % 8) * (per_unit / 8) + rem / 8 : rem;
  const int j = vid / RB, rb = vid % RB;
  int s, seg = 0, c_begin = 0, c_seg_end = 0;
  bool last_seg = true;
  if constexpr (MODE == kModeWhole) {
    s = w.order[zi];
  } else {
    if (zi >= *w.n_segs) return;
    const int4 e = w.seg_table[zi];
    s = e.x;
    seg = zi;
    c_begin = e.y;
    c_seg_end = e.z;
    last_seg = e.w != 0;
    if (MODE == kModeTransfer && last_seg) return;  // (the last segment's map is never used)
  }
  const bool mrow = MODE == kModeTransfer && rb < NBLK;  // a row block of M (else of B, or the state)
  const int blk = MODE == kModeTransfer && !mrow ? rb - NBLK : rb * NR;  // first 16-row block
  const int start = a.cu_seqlens[s];
  const int len = a.cu_seqlens[s + 1] - start;
  if (len <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int kl = KPL * lg;
  const bool qside = wave >= 4;
  const int tt = wave & 3;            // token tile

  // The fused entry point's v conv (XV = 1: bf16 x, 2: fp32 x), in place of reading v:
  // K-side lane (l16, lg) of token tile tt convolves channel l16 of each of the
  // workgroup's row blocks for its 4 output rows 16 tt + 4 lg + rr, from a window of the
  // x rows (or, before the sequence, conv-state rows) at positions 16 tt + 4 lg - (K-1) + i,
  // i < K + 3, loaded two chunks ahead; the per-channel arithmetic is the conv kernels'
  // (bias, then one fused multiply-add per tap, oldest row first, then the activation), so
  // v has the bits the v conv kernel would have written. The workgroup owns the conv
  // state of these channels and commits it at the end.
  typedef __attribute__((address_space(1))) const XT GXT;
  typedef __attribute__((address_space(1))) XT GXTw;
  const int kw = a.conv.width;
  const int64_t xs = a.conv.x_stride, cst = a.conv.channels;
  const int vch0 = 2 * r.hk * D + j * D + blk * kDVB + l16;  // channel of block q: vch0 + 16 q
  GXT* xv = nullptr;
  GXTw* cs = nullptr;
  if constexpr (XV != 0) {
    xv = (GXT*)static_cast<const XT*>(a.conv.x);
    cs = (GXTw*)reinterpret_cast<XT*>(a.conv.state_ptrs[s]);
  }
  auto xval = [](XT v) {
    if constexpr ((XV & 3) == 1) return __uint_as_float(static_cast<uint32_t>(v) << 16);
    else return static_cast<float>(v);
  };
  // new conv-state row i = z row len + i, z = [old conv state (K-1 rows) | the sequence's x],
  // by lanes lg = i of K-side wave 0 (the only wave that reads old rows, in its first
  // window). With len < K-1 a lane reads an old row another lane writes: per block that is
  // one load instruction of all the lanes, waited for, then one store, so every read lands
  // first.
  auto commit_v = [&]() {
    if constexpr (XV != 0) {
      if (!qside && tt == 0 && lg < kw - 1) {
        const int rz = len + lg;
#pragma unroll
        for (int q = 0; q < NR; ++q) {
          const int ch = vch0 + q * kDVB;
          const XT val = rz < kw - 1 ? cs[static_cast<int64_t>(rz) * cst + ch]
                                     : xv[static_cast<int64_t>(start + rz - (kw - 1)) * xs + ch];
          cs[static_cast<int64_t>(lg) * cst + ch] = val;
        }
      }
    }
  };
  const uint64_t sptr = r.state_ptrs[s];
  if (sptr == 0) {
    commit_v();
    return;
  }
  const int h = j / (r.hv / r.hk);
  const float vscale = mrow ? 0.f : 1.f;  // M's rows see v = 0
  // (In transfer mode the Q-side waves still load and compute, and only skip the o
  // store: one code shape for all modes keeps the registers within two workgroups per
  // CU; skipping their work made the compiler need 161.)
  constexpr bool kOut = MODE != kModeTransfer;  // outputs
  const size_t mat = static_cast<size_t>(D) * D;
  float* Sg = reinterpret_cast<float*>(sptr) + (static_cast<int64_t>(j) * D + blk * kDVB) * D;
  // (both are always true at C = 64, D = 128; writing them so lets the compiler see
  // straight-line loads, which keeps its wait counts exact and the prefetch alive)
  const bool active = NT >= 4 || tt < NT;
  const bool has_tile = ST >= 8 || wave < ST;  // this wave updates state tile `wave`
  constexpr bool kFullK = C % KSTEP == 0;      // every lane's k-slice of a chunk row is in range
  const int nch = (len + C - 1) / C;
  const int c_end = MODE == kModeWhole ? nch : c_seg_end;
  const int cbase = w.chunk_off[s];

  // Wave w's state tile is columns [16 w, 16 w + 16) of the slice; lane (l16, lg) holds
  // row l16, columns 16 w + 4 lg .. + 3 (the update is computed transposed, so that these
  // are 4 consecutive values: one 16-byte global and one 8- or 16-byte LDS access).
  const int scol = wave * 16 + 4 * lg;
  f32x4 sacc[NR];
  if (has_tile) {
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      if constexpr (MODE == kModeWhole) {
        sacc[q] = *reinterpret_cast<const f32x4*>(Sg + (q * kDVB + l16) * D + scol);
      } else if constexpr (MODE == kModeSegment) {
        sacc[q] = *reinterpret_cast<const f32x4*>(
            w.zs + (static_cast<size_t>(seg) * r.hv + j) * mat + static_cast<size_t>(blk * kDVB + l16) * D + scol);
      } else {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sacc[q][rr] = (mrow && blk * kDVB + l16 == scol + rr) ? 1.f : 0.f;
      }
      float sv[4] = {sacc[q][0], sacc[q][1], sacc[q][2], sacc[q][3]};
      TS::store4(Sl + q * S_BYTES, l16, scol, sv);
    }
  }

  // The operand loads of one chunk, in three groups so that the prefetching variant can
  // issue them at different points of the previous step.
  auto chunk_ptrs = [&](int c, const char*& kq, const char*& tp, const float*& gb) {
    const int64_t gc = cbase + c;
    // every operand fragment is one contiguous KiB per plane (fragment order, zero-padded)
    kq = w.kq + (gc * r.hk + h) * w.kq_stride;
    tp = w.tp + (gc * r.hv + j) * w.tp_stride;
    gb = reinterpret_cast<const float*>(tp + 2 * static_cast<size_t>(NT) * NK * FIO::BYTES);
  };
  // K^ (or Q^) rows of this wave's token tile: the A operand of phase 1
  auto load_a = [&](int c, In& in) {
    const char *kq, *tp;
    const float* gb;
    chunk_ptrs(c, kq, tp, gb);
    if (active) {
      const char* arows = kq + (qside ? static_cast<size_t>(NT) * NV * FIO::BYTES : 0);
#pragma unroll
      for (int v = 0; v < NV; ++v) in.af[v] = FIO::load(arows + static_cast<size_t>(tt * NV + v) * FIO::BYTES, lane);
    }
  };
  // T (or P) rows, the decay factors, beta and v (used by the K side only; with_v is a
  // constant at every call, so no load sits under a branch)
  auto load_m = [&](int c, In& in, bool with_v) {
    const char *kq, *tp;
    const float* gb;
    chunk_ptrs(c, kq, tp, gb);
    const int t0 = start + c * C;
    in.n = min(C, len - c * C);
    if constexpr (!PF) in.egn = gb[C - 1];
    if (active) {
      const char* mrows = tp + (qside ? static_cast<size_t>(NT) * NK * FIO::BYTES : 0);
      // (fragments wholly above the diagonal are not in the workspace, and their products
      // are skipped; tt is uniform over the wave)
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        if (kk * KSTEP < tt * 16 + 16)
          in.mf[kk] = FIO::load(mrows + static_cast<size_t>(tt * NK + kk) * FIO::BYTES, lane);
      // the factors of this lane's 4 output rows are 4 consecutive floats of each array;
      // the Q side uses e^gam only
      // (the prefetching form takes the factors from LDS instead: see Fl)
      if constexpr (!PF) {
        const float4 g4 = *reinterpret_cast<const float4*>(gb + tt * 16 + 4 * lg);
        in.eg[0] = g4.x; in.eg[1] = g4.y; in.eg[2] = g4.z; in.eg[3] = g4.w;
        if (!qside) {
          const float4 b4 = *reinterpret_cast<const float4*>(gb + C + tt * 16 + 4 * lg);
          in.bt[0] = b4.x; in.bt[1] = b4.y; in.bt[2] = b4.z; in.bt[3] = b4.w;
          const float4 d4 = *reinterpret_cast<const float4*>(gb + 2 * C + tt * 16 + 4 * lg);
          in.ed[0] = d4.x; in.ed[1] = d4.y; in.ed[2] = d4.z; in.ed[3] = d4.w;
        }
      }
      if (with_v) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int t = tt * 16 + 4 * lg + rr;
          // a valid row of this sequence, read unconditionally; rows past the chunk's end
          // are masked where the value is used (using a load in the step that issues it
          // would wait for every load before it, the prefetch included)
          const int tc = min(t, in.n - 1);
#pragma unroll
          for (int q = 0; q < NR; ++q)
            in.vv[q][rr] = vscale * r.v[static_cast<int64_t>(t0 + tc) * r.v_stride + j * D + (blk + q) * kDVB + l16];
        }
      }
    }
  };
  auto load = [&](int c, In& in, bool with_v) {
    load_a(c, in);
    load_m(c, in, with_v);
  };
  float cw[NR][4], cb[NR];  // fused v conv: taps and bias of the lane's channels
  if constexpr (XV != 0) {
    GXT* wt = (GXT*)static_cast<const XT*>(a.conv.w);
    GXT* bs = (GXT*)static_cast<const XT*>(a.conv.b);
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int ch = vch0 + q * kDVB;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) cw[q][jj] = jj < kw ? xval(wt[static_cast<int64_t>(ch) * kw + jj]) : 0.f;
      cb[q] = a.conv.b != nullptr ? xval(bs[ch]) : 0.f;
    }
  }
  // the x window of chunk c (positions past the sequence's end repeat its last row; the
  // rows they would feed are masked where v is used)
  auto load_x = [&](int c, In& in) {
    if constexpr (kXTile) {
      // one 16-byte piece per lane: position p = lane / 2 of the tile, channels 8 (lane % 2)
      // .. + 7 of each block (lanes past the tile repeat its last piece; positions past the
      // sequence's end repeat its last row, before its start come from the conv state)
      const int pl = min(lane, 2 * kXPos - 1);
      const int P = min(c * C + tt * 16 - 3 + (pl >> 1), len - 1);
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        const int ch = vch0 - l16 + q * kDVB + 8 * (pl & 1);
        GXT* src = P >= 0 ? xv + static_cast<int64_t>(start + P) * xs + ch
                          : cs + static_cast<int64_t>(max(P, 1 - kw) + kw - 1) * cst + ch;
        in.xt[q] = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(src);
      }
    } else if constexpr (XV != 0) {
      const int pbase = c * C + tt * 16 + 4 * lg - (kw - 1);
      if (c > 0 && xs <= 0x7FFFFFFF) {
        // (past the first chunk every position is in the sequence: one base row and 32-bit
        // row indices; the same loads in the same order as the general form below)
        GXT* xb = xv + static_cast<int64_t>(start) * xs + vch0;
#pragma unroll
        for (int i = 0; i < kXWin; ++i) {
          const uint32_t p = min(pbase + i, len - 1);
#pragma unroll
          for (int q = 0; q < NR; ++q) in.xw[q][i] = xb[static_cast<uint64_t>(p) * static_cast<uint32_t>(xs) + q * kDVB];
        }
      } else {
#pragma unroll
        for (int i = 0; i < kXWin; ++i) {
          const int p = min(pbase + i, len - 1);
#pragma unroll
          for (int q = 0; q < NR; ++q) {
            const int ch = vch0 + q * kDVB;
            GXT* src = p >= 0 ? xv + static_cast<int64_t>(start + p) * xs + ch
                              : cs + static_cast<int64_t>(p + kw - 1) * cst + ch;
            in.xw[q][i] = *src;
          }
        }
      }
    }
  };
  // v at this lane's 4 rows of chunk c, from the window
  auto conv_v = [&](In& in) {
    if constexpr (kXTile) {
      // the wave's tile into LDS, then each lane's window of its channel from there: the
      // LDS wait and a compiler barrier put the reads after every lane's write (a memory
      // fence here would also wait for the next chunk's operand loads, still in flight, and
      // measured 20 us slower at L = 4096). One 16-byte load per block and lane replaces 7
      // two-byte ones, of the ~140 vector loads a step issues.
      if (lane < 2 * kXPos) {
#pragma unroll
        for (int q = 0; q < NR; ++q) *reinterpret_cast<u32x4*>(&Xl[tt][q][8 * lane]) = in.xt[q];
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // (lgkmcnt(0): the tile's writes have landed)
      asm volatile("" ::: "memory");
      const int p0 = 4 * lg + 4 - kw;  // tile position of the lane's window start
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        float xwin[kXWin];
#pragma unroll
        for (int i = 0; i < kXWin; ++i) xwin[i] = bf16_to_f32(Xl[tt][q][min(p0 + i, kXPos - 1) * 16 + l16]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float acc = cb[q];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (jj < kw) acc = fmaf(cw[q][jj], xwin[rr + jj], acc);
          if constexpr (kVAct) acc = gdn::silu(acc);
          in.vv[q][rr] = vscale * acc;
        }
      }
    } else if constexpr (XV != 0) {
#pragma unroll
      for (int q = 0; q < NR; ++q) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float acc = cb[q];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (jj < kw) acc = fmaf(cw[q][jj], xval(in.xw[q][rr + jj]), acc);
          if constexpr (kVAct) acc = gdn::silu(acc);
          in.vv[q][rr] = vscale * acc;
        }
      }
    }
  };

  // phase 1: X = K^ S^T (K side; then R = diag(beta) (V - diag(e^gam) X) into LDS and the
  // K^ rows into the K^ tile) or Y = Q^ S^T (Q side; returns e^gam Y)
  auto phase1 = [&](const In& in, f32x4 (&oacc)[NR]) {
    if (!qside) {
      // K^ rows of this token tile into LDS for the update (read after two barriers)
#pragma unroll
      for (int v = 0; v < NV; ++v) KT::put(Kl, tt * 16 + l16, v * KSTEP + kl, in.af[v]);
    }
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      f32x4 a3[3];
      zero3(a3);
#pragma unroll
      for (int v = 0; v < NV; ++v) M::mma3(a3, in.af[v], TS::load(Sl + q * S_BYTES, l16, kl + v * KSTEP));
      const f32x4 acc = total(a3);
      if (!qside) {
        float rv[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float vt = (tt * 16 + 4 * lg + rr < in.n) ? in.vv[q][rr] : 0.f;
          rv[rr] = in.bt[rr] * (vt - in.eg[rr] * acc[rr]);
        }
        TR::store4(Rt + q * R_BYTES, l16, tt * 16 + 4 * lg, rv);
      } else {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) oacc[q][rr] = in.eg[rr] * acc[rr];
      }
    }
  };
  // phase 2 (K side): U = T R, T lower triangular; U^T and (e^{gam_n - gam} U)^T into LDS
  auto phase2 = [&](const In& in) {
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      f32x4 u3[3];
      zero3(u3);
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        if (kk * KSTEP < tt * 16 + 16) {
          const F rf =
              (kFullK || kk * KSTEP + kl < C) ? TR::load(Rt + q * R_BYTES, l16, kk * KSTEP + kl) : SP::zero();
          M::mma3(u3, kk * KSTEP + kl <= tt * 16 + l16 ? in.mf[kk] : SP::zero(), rf);
        }
      }
      const f32x4 uacc = total(u3);
      float ut[4], us[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        ut[rr] = uacc[rr];
        us[rr] = in.ed[rr] * uacc[rr];
      }
      TR::store4(Ut + q * R_BYTES, l16, tt * 16 + 4 * lg, ut);
      TR::store4(Us + q * R_BYTES, l16, tt * 16 + 4 * lg, us);
    }
  };
  // rows t < n of this wave's token tile of O for chunk c
  // (element (token, j, column) of o is at token * hv * D + j * D + column; the lane's
  // column of block q at token start is obase + 16 q, and a token's offset from it is
  // formed from a 32-bit token index)
  const int64_t obase = (static_cast<int64_t>(start) * r.hv + j) * D + blk * kDVB + l16;
  const uint32_t orow = static_cast<uint32_t>(r.hv * D);
  auto store_o = [&](int c, int n, const f32x4 (&o)[NR]) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int t = tt * 16 + 4 * lg + rr;
      if (kOut && t < n) {
        const int64_t e = obase + static_cast<int64_t>(static_cast<uint64_t>(static_cast<uint32_t>(c * C + t)) * orow);
#pragma unroll
        for (int q = 0; q < NR; ++q) {
          if (r.o_bf16)
            static_cast<uint16_t*>(r.o)[e + q * kDVB] = f32_to_bf16_rne(o[q][rr]);
          else
            static_cast<float*>(r.o)[e + q * kDVB] = o[q][rr];
        }
      }
    }
  };
  // phase 3, Q side: O = e^gam Y + P U
  auto phase3_out = [&](const In& in, f32x4 (&oacc)[NR]) {
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      f32x4 o3[3];
      zero3(o3);
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        if (kk * KSTEP < tt * 16 + 16) {
          const F uf =
              (kFullK || kk * KSTEP + kl < C) ? TR::load(Ut + q * R_BYTES, l16, kk * KSTEP + kl) : SP::zero();
          M::mma3(o3, kk * KSTEP + kl <= tt * 16 + l16 ? in.mf[kk] : SP::zero(), uf);
        }
      }
      oacc[q] += total(o3);
    }
  };
  // phase 3, state tile `wave`: S <- e^{gam_n} S + Us^T K^, computed as its transpose
  // K^T Us (A operand: columns of K^, B operand: rows of Us)
  auto phase3_state = [&](const In& in) {
    const float egn = in.egn;
    f32x4 s3[NR][3];
#pragma unroll
    for (int q = 0; q < NR; ++q) zero3(s3[q]);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const bool live = kFullK || kk * KSTEP + kl < C;
      const F kc = live ? KT::column16(Kl, wave * 16, kk * KSTEP + kl, l16) : SP::zero();
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        const F ub = live ? TR::load(Us + q * R_BYTES, l16, kk * KSTEP + kl) : SP::zero();
        M::mma3(s3[q], kc, ub);
      }
    }
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const f32x4 upd = total(s3[q]);
      float sv[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sv[rr] = fmaf(sacc[q][rr], egn, upd[rr]);
      sacc[q] = f32x4{sv[0], sv[1], sv[2], sv[3]};
      TS::store4(Sl + q * S_BYTES, l16, scol, sv);
    }
  };

  if constexpr (PF) {
    // Two operand buffers, one chunk ahead. The next chunk's loads are spread over the
    // step so that the 8 waves do not all queue theirs at the CU's load unit at once (a
    // burst stalls the issuing waves for longer than the loads take): K-side waves issue
    // the A rows at the top of the step and the rest after the second barrier; Q-side
    // waves, idle while the K side computes U, issue all of theirs after the first. The
    // two sides run separate loops with the same barriers, so that each side's loads are
    // straight-line code (loads under a branch inside one loop made the compiler wait for
    // the whole prefetch). Each step starts by waiting for all of the wave's outstanding
    // vector memory operations (its operands, issued one step earlier); the Q side then
    // stores the previous chunk's outputs, so that no store is in flight when a later
    // wait would otherwise have to include it (with loads and stores both outstanding the
    // compiler can only wait for everything). The prefetch index is clamped rather than
    // guarded (the last chunk is simply read twice).
    // The decay factors of a chunk (3 C floats, contiguous in the workspace) are loaded by
    // the Q side with one 16-byte load per lane, two chunks ahead, and written into Fl by
    // its token-tile-0 wave at the top of the step before their chunk's; every wave then
    // reads its own from Fl at the top of that chunk's step. (Each lane loading its 4
    // tokens' factors itself took 16 of a step's ~140 vector load instructions, whose issue
    // is what the step's loads wait on; this takes 4. Buffer (c + 1) % 2 is rewritten at the
    // top of step c, after the barriers of step c - 1, at whose top chunk c - 1's factors
    // were last read from it.)
    constexpr int kFL = 3 * C / 4;  // 16-byte pieces of a chunk's factors
    auto load_fac = [&](int c) {
      const char *kq, *tp;
      const float* gb;
      chunk_ptrs(c, kq, tp, gb);
      return *reinterpret_cast<const float4*>(gb + 4 * min(lane, kFL - 1));
    };
    auto put_fac = [&](int c, const float4& f) {
      if (tt == 0 && lane < kFL) *reinterpret_cast<float4*>(&Fl[c & 1][4 * lane]) = f;
    };
    auto get_fac = [&](int c, In& in) {
      const float* f = Fl[c & 1];
      const float4 g4 = *reinterpret_cast<const float4*>(f + tt * 16 + 4 * lg);
      in.eg[0] = g4.x; in.eg[1] = g4.y; in.eg[2] = g4.z; in.eg[3] = g4.w;
      if (!qside) {
        const float4 b4 = *reinterpret_cast<const float4*>(f + C + tt * 16 + 4 * lg);
        in.bt[0] = b4.x; in.bt[1] = b4.y; in.bt[2] = b4.z; in.bt[3] = b4.w;
        const float4 d4 = *reinterpret_cast<const float4*>(f + 2 * C + tt * 16 + 4 * lg);
        in.ed[0] = d4.x; in.ed[1] = d4.y; in.ed[2] = d4.z; in.ed[3] = d4.w;
      }
      in.egn = f[C - 1];
    };
    float4 fpre = make_float4(0.f, 0.f, 0.f, 0.f);
    if (qside) {
      const float4 f0 = load_fac(c_begin);
      wait_vmem();
      put_fac(c_begin, f0);
      fpre = load_fac(min(c_begin + 1, c_end - 1));
    }
    In in0, in1;
    load(c_begin, in0, !qside && XV == 0);
    if (!qside) {
      load_x(c_begin, in0);
      load_x(min(c_begin + 1, c_end - 1), in1);
      conv_v(in0);
    }
    __syncthreads();  // Sl filled
    // (with the fused v conv: v of chunk c is formed from its window first, and the wait
    // leaves the window of chunk c + 1, the loads issued last, in flight; the window of
    // chunk c + 2 goes into this buffer's slot once its operands are loaded)
    auto step_k = [&](int c, In& in, In& nxt, int cn) {
      if constexpr (XV != 0) {
        wait_vmem_leaving<(kXTile ? 1 : kXWin) * NR>();
      } else {
        wait_vmem();
      }
      get_fac(c, in);
      load_a(cn, nxt);
      f32x4 unused[NR];
      if (active) phase1(in, unused);
      __syncthreads();
      if (active) phase2(in);
      conv_v(nxt);  // (v of the next chunk, while the Q side still issues its loads)
      __syncthreads();
      load_m(cn, nxt, XV == 0);
      load_x(min(c + 2, c_end - 1), in);
      if (has_tile) phase3_state(in);
      __syncthreads();
    };
    f32x4 oprev[NR];  // outputs of the previous chunk, stored one step late
    int nprev = 0;    // (0: nothing to store)
    auto step_q = [&](int c, In& in, In& nxt, int cn) {
      wait_vmem();
      put_fac(c + 1, fpre);  // (chunk c + 1's factors, loaded during the previous step)
      get_fac(c, in);
      store_o(c - 1, nprev, oprev);
      f32x4 oacc[NR];
#pragma unroll
      for (int q = 0; q < NR; ++q) oacc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (active) phase1(in, oacc);
      __syncthreads();
      load(cn, nxt, false);
      fpre = load_fac(min(c + 2, c_end - 1));
      __syncthreads();
      if (active) phase3_out(in, oacc);
      if (has_tile) phase3_state(in);
      __syncthreads();
#pragma unroll
      for (int q = 0; q < NR; ++q) oprev[q] = oacc[q];
      nprev = in.n;
    };
    if (!qside) {
      for (int c = c_begin; c < c_end; c += 2) {
        step_k(c, in0, in1, min(c + 1, c_end - 1));
        if (c + 1 >= c_end) break;
        step_k(c + 1, in1, in0, min(c + 2, c_end - 1));
      }
    } else {
      for (int c = c_begin; c < c_end; c += 2) {
        step_q(c, in0, in1, min(c + 1, c_end - 1));
        if (c + 1 >= c_end) break;
        step_q(c + 1, in1, in0, min(c + 2, c_end - 1));
      }
      store_o(c_end - 1, nprev, oprev);
    }
  } else {
    // One operand buffer, loaded at the top of each step: half the registers, so two
    // workgroups share a CU and each one's load latency is covered by the other's work.
    In in0;
    __syncthreads();  // Sl filled
    for (int c = c_begin; c < c_end; ++c) {
      load(c, in0, true);  // (the Q side loads v too: fewer registers than a branch)
      f32x4 oacc[NR];
#pragma unroll
      for (int q = 0; q < NR; ++q) oacc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (active) phase1(in0, oacc);
      __syncthreads();
      if (active && !qside) phase2(in0);
      __syncthreads();
      if (active && qside) {
        phase3_out(in0, oacc);
        store_o(c, in0.n, oacc);
      }
      if (has_tile) phase3_state(in0);
      __syncthreads();
    }
  }

  if (has_tile) {
    if constexpr (MODE == kModeTransfer) {
      if (mrow) {
        // M^T[n][i] for row i = blk*16 + l16 and columns n = scol + rr of M
        float* mt = w.mt + (static_cast<size_t>(seg) * r.hv + j) * mat;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) mt[static_cast<size_t>(scol + rr) * D + blk * kDVB + l16] = sacc[0][rr];
      } else {
        float* bt = w.bt + (static_cast<size_t>(seg) * r.hv + j) * mat + static_cast<size_t>(blk * kDVB) * D;
        *reinterpret_cast<f32x4*>(bt + l16 * D + scol) = sacc[0];
      }
    } else if (last_seg) {
#pragma unroll
      for (int q = 0; q < NR; ++q) *reinterpret_cast<f32x4*>(Sg + (q * kDVB + l16) * D + scol) = sacc[q];
    }
  }
  commit_v();
}

// Start states of the segments of the chunk-parallel form: Z_0 = the state in place
// (copied, so that the segment launch never reads memory it also writes), then
// Z_{g+1} = Z_g M_g + B_g. One workgroup per (sequence, v-head, 16 state rows); wave w
// computes columns [16 w, 16 w + 16) of the row slice, with Z in LDS as the A operand
// and rows of M^T as the B operand. M_g and B_g do not depend on Z, so they are loaded
// ahead of use, and Z alternates between two LDS buffers (one barrier a step).
template <int POL, int D>
struct ScanIn {
  static constexpr int NV = D / Mma<POL>::KSTEP;
  float m[NV][Mma<POL>::KPL];  // row n of M^T, this lane's k-slices
  float b[4];                  // B at this lane's 4 output rows
};

template <int POL, int D>
__global__ __launch_bounds__(kInterThreads) void segment_scan_kernel(PrefillArgs a, Workspace w) {
  using M = Mma<POL>;
  using SP = Split<POL>;
  using In = ScanIn<POL, D>;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP;
  constexpr int NBLK = D / kDVB, ST = D / 16, NV = In::NV;
  constexpr int PADE = POL == kPolBF16X3 ? 8 : 4;
  constexpr int SLD = D + PADE;
  constexpr int ZB = kDVB * SLD * 4;
  __shared__ __attribute__((aligned(16))) char Sl[2 * ZB];
  const RecurArgs& r = a.r;
  const int per_seq = NBLK * r.hv;
  const int s = blockIdx.x / per_seq, rem = blockIdx.x % per_seq;
  const int j = rem / NBLK, blk = rem % NBLK;
  if (a.cu_seqlens[s + 1] - a.cu_seqlens[s] <= 0) return;
  const uint64_t sptr = r.state_ptrs[s];
  if (sptr == 0) return;
  const int g0 = w.seg_off[s], ns = w.seg_off[s + 1] - g0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int kl = KPL * lg;
  const bool has_tile = ST >= 8 || wave < ST;
  const int col = wave * 16 + l16;
  const size_t mat = static_cast<size_t>(D) * D;
  const size_t rows = static_cast<size_t>(blk * kDVB) * D;  // offset of the row slice
  const float* S0 = reinterpret_cast<const float*>(sptr) + static_cast<size_t>(j) * mat + rows;
  float* zs = w.zs + (static_cast<size_t>(g0) * r.hv + j) * mat + rows;  // Z_0's slice
  const size_t zstep = static_cast<size_t>(r.hv) * mat;                  // to the next segment

  auto load = [&](int g, In& in) {
    const size_t base = (static_cast<size_t>(g0 + g) * r.hv + j) * mat;
    const float* mrow = w.mt + base + static_cast<size_t>(col) * D;  // row n = col of M^T
#pragma unroll
    for (int v = 0; v < NV; ++v) load_k<KPL>(mrow + kl + v * KSTEP, in.m[v]);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) in.b[rr] = w.bt[base + rows + (4 * lg + rr) * D + col];
  };
  // Z_{g+1} = Z_g M_g + B_g from buffer `cur` of Sl into the other one and into zs
  auto step = [&](int g, const In& in, int cur) {
    const char* zin = Sl + cur * ZB;
    char* zout = Sl + (cur ^ 1) * ZB;
    f32x4 a3[3];
    zero3(a3);
#pragma unroll
    for (int v = 0; v < NV; ++v) M::mma3(a3, SP::load(zin, kDVB, SLD, l16, kl + v * KSTEP), M::frag(in.m[v]));
    const f32x4 prod = total(a3);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float z = in.b[rr] + prod[rr];
      SP::store1(zout, kDVB, SLD, 4 * lg + rr, col, z);
      zs[static_cast<size_t>(g + 1) * zstep + (4 * lg + rr) * D + col] = z;
    }
  };

  if (has_tile) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float v = S0[(4 * lg + rr) * D + col];
      SP::store1(Sl, kDVB, SLD, 4 * lg + rr, col, v);
      zs[(4 * lg + rr) * D + col] = v;
    }
  }
  // M_g and B_g come from memory written by the previous launch (about 2 us away), so
  // they are loaded three steps ahead, into four rotating register buffers; prefetch
  // indices are clamped, not guarded (the last step's operands may be read again).
  const int nsteps = ns - 1;
  In b0, b1, b2, b3;
  if (has_tile && nsteps > 0) {
    load(0, b0);
    load(min(1, nsteps - 1), b1);
    load(min(2, nsteps - 1), b2);
  }
  __syncthreads();
  for (int g = 0; g < nsteps; g += 4) {
    if (has_tile) {
      load(min(g + 3, nsteps - 1), b3);
      step(g, b0, 0);
    }
    __syncthreads();
    if (g + 1 >= nsteps) break;
    if (has_tile) {
      load(min(g + 4, nsteps - 1), b0);
      step(g + 1, b1, 1);
    }
    __syncthreads();
    if (g + 2 >= nsteps) break;
    if (has_tile) {
      load(min(g + 5, nsteps - 1), b1);
      step(g + 2, b2, 0);
    }
    __syncthreads();
    if (g + 3 >= nsteps) break;
    if (has_tile) {
      load(min(g + 6, nsteps - 1), b2);
      step(g + 3, b3, 1);
    }
    __syncthreads();
  }
}

// Whole sequences: NR 16-row blocks per workgroup, prefetching; XV: the fused v conv (0: none;
// else the x dtype, 1 bf16 or 2 fp32, plus 4 with SiLU)
template <int POL, int D, int C, int NR, int XV>
void launch_whole(const PrefillArgs& a, const Workspace& w, unsigned workgroups, hipStream_t s) {
  inter_chunk_kernel<POL, D, C, true, kModeWhole, NR, XV><<<workgroups, kInterThreads, 0, s>>>(a, w);
}

template <int POL, int D, int C>
hipError_t launch_chunked(const PrefillArgs& a, const Workspace& w, hipStream_t s) {
  const size_t mc = max_chunks_of(C, a.num_seqs, a.total_tokens);
  intra_chunk_kernel<POL, D, C><<<dim3(static_cast<unsigned>(mc), a.r.hk), kThreads, 0, s>>>(a, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int NBLK = D / kDVB;
  if (w.segmented) {
    // chunk-parallel form: segment maps, then the scan, then every segment's outputs
    const size_t ns = max_segments_of(C, a.num_seqs, a.total_tokens);
    inter_chunk_kernel<POL, D, C, false, kModeTransfer>
        <<<static_cast<unsigned>(ns * a.r.hv * 2 * NBLK), kInterThreads, 0, s>>>(a, w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    segment_scan_kernel<POL, D><<<static_cast<unsigned>(a.num_seqs * a.r.hv * NBLK), kInterThreads, 0, s>>>(a, w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    inter_chunk_kernel<POL, D, C, false, kModeSegment>
        <<<static_cast<unsigned>(ns * a.r.hv * NBLK), kInterThreads, 0, s>>>(a, w);
    return hipGetLastError();
  }
  const unsigned blocks = static_cast<unsigned>(NBLK * a.r.hv * a.num_seqs);
  const bool two = blocks >= 2 * kInterPrefetchMaxCUs;  // two 16-row blocks per workgroup (NBLK is even)
  if constexpr (C == 64) {
    if (a.v_in_inter) {
      auto go = [&](auto xv) {
        constexpr int XV = decltype(xv)::value;
        if (two) launch_whole<POL, D, C, 2, XV>(a, w, blocks / 2, s);
        else launch_whole<POL, D, C, 1, XV>(a, w, blocks, s);
      };
      if (a.conv.bf16) {
        if (a.conv.silu) go(std::integral_constant<int, 5>());
        else go(std::integral_constant<int, 1>());
      } else {
        if (a.conv.silu) go(std::integral_constant<int, 6>());
        else go(std::integral_constant<int, 2>());
      }
      return hipGetLastError();
    }
  }
  if (two) launch_whole<POL, D, C, 2, 0>(a, w, blocks / 2, s);
  else launch_whole<POL, D, C, 1, 0>(a, w, blocks, s);
  return hipGetLastError();
}

template <int POL, int D>
hipError_t by_chunk(const PrefillArgs& a, const Workspace& w, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_chunked<POL, D, 16>(a, w, s);
    case 32: return launch_chunked<POL, D, 32>(a, w, s);
    default: return launch_chunked<POL, D, 64>(a, w, s);
  }
}

template <int POL>
hipError_t by_dim(const PrefillArgs& a, const Workspace& w, hipStream_t s) {
  switch (a.r.d) {
    case 32: return by_chunk<POL, 32>(a, w, s);
    case 64: return by_chunk<POL, 64>(a, w, s);
    default: return by_chunk<POL, 128>(a, w, s);
  }
}

}  // namespace

size_t prefill_workspace_bytes(int32_t hk, int32_t hv, int32_t d, int32_t chunk, int32_t num_seqs,
                               int32_t total_tokens, int32_t form) {
  return workspace_bytes(hk, hv, d, chunk, num_seqs, total_tokens, form);
}

hipError_t launch_prefill(const PrefillArgs& args, hipStream_t s) {
  if (args.num_seqs == 0 || args.total_tokens == 0) return hipSuccess;
  const Workspace w = carve(args.workspace, args.r.hk, args.r.hv, args.r.d, args.chunk, args.num_seqs,
                            args.total_tokens, args.form);
  PrefillArgs a = args;
  hipError_t e;
  if (a.conv.x != nullptr) {
    // fused entry point: whole sequences in 64-token chunks convolve v inside the
    // inter-chunk kernel; otherwise the v channels' conv runs first, into r.v
    a.v_in_inter = (!w.segmented && a.chunk == 64) ? 1 : 0;
    if (!a.v_in_inter) {
      e = launch_conv_prefill_only(a.vconv, s);
      if (e != hipSuccess) return e;
    }
  } else {
    a.v_in_inter = 0;
  }
  // whole sequences, at most 64: the intra-chunk kernel finds its chunks from cu_seqlens
  a.table_free = (!w.segmented && a.num_seqs <= 64) ? 1 : 0;
  if (!a.table_free) {
    chunk_table_kernel<<<1, kMetaThreads, 0, s>>>(a.cu_seqlens, a.num_seqs, a.chunk, w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return a.mma == kPolFP32 ? by_dim<kPolFP32>(a, w, s) : by_dim<kPolBF16X3>(a, w, s);
}

}  // namespace gdn
