// Batched single-token decode of the gated delta rule, gfx950.
//
// For slot i and v-head j (k-head h = j / (Hv/Hk)), with k^ = k/sqrt(|k|^2+eps),
// q^ = scale * q/sqrt(|q|^2+eps), alpha = exp(g), and S the d_v x d_k state:
//     S_new = alpha S (I - beta k^ k^T) + beta v k^T   and   o = S_new q^.
// ("System Design" (project_6), "GDN Kernel Dispatch Detail", decode branch: decay of
// the temporal state with the delta write, then the query against the state;
// aprender #5279, "Phase plan", phase P5: the slot index on the launch grid and one
// 64-bit state address per slot in a device array.)
//
// Row r of the update only needs row r of S:
//     a_r = S_r . k^,  p_r = S_r . q^,  u_r = beta (v_r - alpha a_r)
//     S_r <- alpha S_r + u_r k^,        o_r = alpha p_r + u_r (k^ . q^)
// so the state is streamed once from HBM and written once, rows in any order.
//
// Work unit = one wave over P passes of RPP rows of one (slot, v-head). D/16 lanes
// share a row; lane c of a row group holds floats [4c + 4*LPR*u, +4), u = 0..3, so
// every load instruction of a wave covers RPP whole rows (RPP * D * 4 = 4 KiB
// contiguous). Units are dealt to waves in (slot, head, row) order, four waves per
// workgroup, so the grid sweeps each 2 MiB slot state front to back.
//
// What the memory system wants here (measured on MI355X at 30 layers x 64 slots):
//  * small units (one 4 KiB pass per wave at large m) beat long-lived waves that hold
//    16 KiB of state: reads and writes of many short waves interleave like a plain
//    streaming copy;
//  * state loads and stores go through the global (not flat) address space and carry
//    the nontemporal hint; the slot pointer, g and beta are wave-uniform scalar loads;
//  * every load of a unit is issued before any arithmetic, and nothing waits on a
//    store (v is read up front).
// The two row dots are reduced over the row's lanes with a fixed DPP butterfly, so the
// bits of a slot's result depend neither on m, nor on the unit size, nor on which
// other slots are in the call.

#include "conv_taps.h"
#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

typedef __attribute__((address_space(1))) f32x4 gf32x4;
typedef __attribute__((address_space(1))) float gfloat;
typedef __attribute__((address_space(1))) const float cgfloat;
typedef __attribute__((address_space(4))) const uint64_t cu64;
typedef __attribute__((address_space(4))) const float cfloat;
typedef __attribute__((address_space(1))) uint16_t gu16;
// (Generic -> global/constant pointer conversions are address-space casts, which C++
// spells only as C-style casts.)

constexpr int kDecodeWaves = 4;  // waves per workgroup

// Workgroups are dealt round-robin to MI355X's 8 XCDs, each with its own L2. With a
// slot's workgroups along grid.x (a multiple of 8 of them), workgroup x runs on XCD x % 8;
// renumbering them so that XCD r takes the consecutive block [r n/8, (r+1) n/8) puts the
// workgroups of one head -- which read the same k and q and write neighbouring bytes --
// on one XCD, sharing its L2.
__device__ __forceinline__ int xcd_block() {
  const int n = gridDim.x;
  const int b = blockIdx.x;
  return (n % 8 == 0) ? (b % 8) * (n / 8) + b / 8 : b;
}

// element `off` of o, in o's dtype: OB 0 fp32, 1 bf16, 2 as the o_bf16 flag says
template <int OB>
__device__ __forceinline__ void* o_row(const RecurArgs& a, int64_t off) {
  const bool b16 = OB == 1 || (OB == 2 && a.o_bf16);
  return b16 ? static_cast<void*>(static_cast<uint16_t*>(a.o) + off) : static_cast<void*>(static_cast<float*>(a.o) + off);
}

template <int D, int P>
struct DecodeCfg {
  static constexpr int LPR = D / 16;          // lanes per row (16 floats per lane)
  static constexpr int RPP = kWave / LPR;     // rows per pass
  static constexpr int ROWS = RPP * P;        // rows per unit
  static constexpr int NPART = D / ROWS;      // units per (slot, head)
  static_assert(NPART * ROWS == D, "units must tile the head");
};

// The arithmetic of one unit once its loads are in registers. The lane holds 16 columns
// of the raw k and q (unnormalised); with rk = 1/sqrt(|k|^2 + eps) and rq = scale/sqrt(
// |q|^2 + eps), k^ = rk k and q^ = rq q enter only through dot products and one scaled
// fma, so the vectors are never rescaled:
//     a_r = rk (S_r . k),  p_r = rq (S_r . q),  u_r = beta (v_r - alpha a_r),
//     S_r <- alpha S_r + (u_r rk) k,           o_r = alpha p_r + u_r (k^ . q^),
// with k^ . q^ = rk rq (k . q). 1/sqrt is the hardware reciprocal square root (about one
// ulp). Every decode kernel runs this code, so their bits agree.
// OB: how o is stored -- 0 fp32, 1 bf16 (rounded to nearest even), 2 as the o_bf16 flag says.
template <int D, int P, int OB>
__device__ __forceinline__ void decode_rows(const f32x4 (&s)[P][4], const f32x4 (&kv)[4], const f32x4 (&qv)[4],
                                            const float (&vr)[P], float gval, float beta, float eps, float scale,
                                            bool qk_norm, gf32x4* S, void* orow, bool o_bf16, int row0, int c) {
  using Cfg = DecodeCfg<D, P>;
  constexpr int LPR = Cfg::LPR, RPP = Cfg::RPP;
  // |k|^2, |q|^2 and k . q over the row's lanes
  float kk = 0.f, qq = 0.f, kqr = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kk = fmaf(kv[e].x, kv[e].x, kk); kk = fmaf(kv[e].y, kv[e].y, kk);
    kk = fmaf(kv[e].z, kv[e].z, kk); kk = fmaf(kv[e].w, kv[e].w, kk);
    qq = fmaf(qv[e].x, qv[e].x, qq); qq = fmaf(qv[e].y, qv[e].y, qq);
    qq = fmaf(qv[e].z, qv[e].z, qq); qq = fmaf(qv[e].w, qv[e].w, qq);
    kqr = fmaf(kv[e].x, qv[e].x, kqr); kqr = fmaf(kv[e].y, qv[e].y, kqr);
    kqr = fmaf(kv[e].z, qv[e].z, kqr); kqr = fmaf(kv[e].w, qv[e].w, kqr);
  }
  kk = group_sum<LPR>(kk);
  qq = group_sum<LPR>(qq);
  kqr = group_sum<LPR>(kqr);
  const float rk = qk_norm ? __builtin_amdgcn_rsqf(kk + eps) : 1.0f;
  const float rq = qk_norm ? scale * __builtin_amdgcn_rsqf(qq + eps) : scale;
  const float kq = kqr * (rk * rq);
  const float alpha = expf(gval);

#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int r = row0 + p * RPP;
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sk = fmaf(s[p][e].x, kv[e].x, sk); sk = fmaf(s[p][e].y, kv[e].y, sk);
      sk = fmaf(s[p][e].z, kv[e].z, sk); sk = fmaf(s[p][e].w, kv[e].w, sk);
      sq = fmaf(s[p][e].x, qv[e].x, sq); sq = fmaf(s[p][e].y, qv[e].y, sq);
      sq = fmaf(s[p][e].z, qv[e].z, sq); sq = fmaf(s[p][e].w, qv[e].w, sq);
    }
    sk = group_sum<LPR>(sk) * rk;
    sq = group_sum<LPR>(sq) * rq;
    const float ur = beta * (vr[p] - alpha * sk);
    const float urk = ur * rk;
    gf32x4* rowp = S + static_cast<int64_t>(r) * (D / 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f32x4 n;
      n.x = fmaf(urk, kv[e].x, alpha * s[p][e].x);
      n.y = fmaf(urk, kv[e].y, alpha * s[p][e].y);
      n.z = fmaf(urk, kv[e].z, alpha * s[p][e].z);
      n.w = fmaf(urk, kv[e].w, alpha * s[p][e].w);
      __builtin_nontemporal_store(n, rowp + c + LPR * e);
    }
    if (c == 0) {
      const float ov = fmaf(ur, kq, alpha * sq);
      if (OB == 1 || (OB == 2 && o_bf16))
        ((gu16*)orow)[r] = f32_to_bf16_rne(ov);
      else
        ((gfloat*)orow)[r] = ov;
    }
  }
}


// Grid: (units of a slot / 4, m); the slot is blockIdx.y, so the only runtime division
// a wave makes before its first load is the k-head of its v-head.
template <int D, int P, bool SCHED_FENCE, int OB>
__global__ __launch_bounds__(kDecodeWaves* kWave) void decode_kernel(RecurArgs a) {
  using Cfg = DecodeCfg<D, P>;
  constexpr int LPR = Cfg::LPR, RPP = Cfg::RPP, NPART = Cfg::NPART;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int us = xcd_block() * kDecodeWaves + w;  // unit within the slot
  if (us >= a.hv * NPART) return;
  const int part = us % NPART;
  const int j = us / NPART;
  const int i = blockIdx.y;
  const uint64_t sp = ((cu64*)a.state_ptrs)[i];
  if (sp == 0) return;  // inactive slot
  const int h = j / a.group;
  const int c = lane % LPR;   // column group inside the row
  const int rl = lane / LPR;  // row inside a pass
  const int row0 = part * Cfg::ROWS + rl;

  gf32x4* S = (gf32x4*)(reinterpret_cast<float*>(sp) + static_cast<int64_t>(j) * D * D);

  // every load of the unit first: state rows, k, q, v, g, beta
  f32x4 s[P][4];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      s[p][e] = __builtin_nontemporal_load(S + static_cast<int64_t>(row0 + p * RPP) * (D / 4) + c + LPR * e);
  const gf32x4* kp = (const gf32x4*)(a.k + static_cast<int64_t>(i) * a.k_stride + h * D);
  const gf32x4* qp = (const gf32x4*)(a.q + static_cast<int64_t>(i) * a.q_stride + h * D);
  f32x4 kv[4], qv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kv[e] = kp[c + LPR * e];
    qv[e] = qp[c + LPR * e];
  }
  const cgfloat* vrow = (const cgfloat*)(a.v + static_cast<int64_t>(i) * a.v_stride + static_cast<int64_t>(j) * D);
  float vr[P];
#pragma unroll
  for (int p = 0; p < P; ++p) vr[p] = vrow[row0 + p * RPP];
  const int64_t gi = static_cast<int64_t>(i) * a.hv + j;
  const float gval = ((cfloat*)a.g)[gi];
  const float beta = ((cfloat*)a.beta)[gi];
  if constexpr (SCHED_FENCE) __builtin_amdgcn_sched_barrier(0);

  decode_rows<D, P, OB>(s, kv, qv, vr, gval, beta, a.eps, a.scale, a.qk_norm != 0, S, o_row<OB>(a, gi * D), OB == 1, row0, c);
}

template <int D, int P, bool F>
hipError_t launch_units(const RecurArgs& a, int32_t m, hipStream_t s) {
  const int units = a.hv * DecodeCfg<D, P>::NPART;  // per slot
  const dim3 grid(static_cast<unsigned>((units + kDecodeWaves - 1) / kDecodeWaves), static_cast<unsigned>(m));
  if (a.o_bf16)
    decode_kernel<D, P, F, 1><<<grid, kDecodeWaves * kWave, 0, s>>>(a);
  else
    decode_kernel<D, P, F, 0><<<grid, kDecodeWaves * kWave, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

// Unit size by batch: one pass per wave once the call has thousands of (slot, head)
// pairs (m * Hv >= 1024), two passes below that, where fewer, longer waves hide the
// launch ramp better. Either choice gives the same bits.
hipError_t launch_decode(const RecurArgs& a, int32_t m, hipStream_t s) {
  if (m == 0) return hipSuccess;
  const bool big = static_cast<int64_t>(m) * a.hv >= 1024;
  switch (a.d) {
    case 32: return launch_units<32, 1, false>(a, m, s);
    case 64: return big ? launch_units<64, 1, false>(a, m, s) : launch_units<64, 2, true>(a, m, s);
    default: return big ? launch_units<128, 1, false>(a, m, s) : launch_units<128, 2, true>(a, m, s);
  }
}

namespace {
// ---------------------------------------------------------------- fused conv + decode
// One launch for the whole decode step of a layer: the depthwise conv of the token's q,
// k and v channels (against the slot's conv state), the conv-state commit, and the
// decode above, with the conv output kept in LDS. Two forms: in place (below) and
// streaming (further down), for when the new conv states go to other buffers.
//
// In place. One workgroup per (slot i, k-head h) holds everything that reads k-head h's q and k:
// its 2d q/k conv channels, and the G = hv/hk v-heads j = hG .. hG + G - 1 that share it,
// each with its d v channels and d state rows. Every conv-state value of the slot is then
// read by exactly one thread of one workgroup, and that thread writes the shifted rows
// back itself once its reads have returned (the values it stores are the values it
// loaded): no other workgroup ever reads them, so the commit needs no ordering across
// workgroups -- no counters and no workspace.
//
// The group's G d state rows are cut into blocks of ROWS rows (P passes of RPP rows, as a
// decode_kernel unit), dealt to the waves in order, so the waves sweep the slot's G
// consecutive head states front to back. Threads convolve 4 channels each (the q/k
// channels, then the v channels) with the conv kernels' per-channel arithmetic
// (conv4_raw) into LDS; one barrier that orders LDS only (state loads stay in flight
// across it); then every wave takes k, q and its rows' v from LDS and runs decode_rows,
// the code of decode_kernel, so o, the state and the conv state come out bit-identical to
// gdn_conv_update + gdn_decode_batched. (The price of the large workgroups: at m = 64 one
// of them fits a CU at a time, and each of a CU's rounds starts with a full memory round
// trip with nothing else in flight -- 53.9 us per launch against 47.5 us streaming.)
template <int D>
struct FusedCfg {
  static constexpr int P = D == 128 ? 2 : 1;   // passes per block
  using DC = DecodeCfg<D, P>;
  static constexpr int ROWS = DC::ROWS;        // state rows per block: 16 (d = 64, 128) or 32 (d = 32)
  static constexpr int MAXW = 16;              // waves per workgroup at most
  static constexpr int CV = 4;                 // channels per conv thread
  // waves of a workgroup for G v-heads per k-head, and blocks per wave
  __host__ static int waves(int G) { return (G * D / ROWS) < MAXW ? G * D / ROWS : MAXW; }
  __host__ static int iters(int G) { return (G * D / ROWS + waves(G) - 1) / waves(G); }
};

// The convolving waves load their conv inputs before their first state rows, so the conv
// waits only for its own (mostly cached) inputs.
template <typename T, int K, int D, bool SILU>
__global__ __launch_bounds__(FusedCfg<D>::MAXW * kWave) void fused_decode_kernel(FusedArgs f, int32_t nit) {
  using FC = FusedCfg<D>;
  using DC = typename FC::DC;
  using V4 = Vec4<T>;
  constexpr int P = FC::P, LPR = DC::LPR, RPP = DC::RPP, ROWS = FC::ROWS, V = FC::CV;
  typedef __attribute__((address_space(1))) T GT;
  extern __shared__ __attribute__((aligned(16))) float fused_lds[];  // conv output: q, k (2d), v of the group (G d)
  const RecurArgs& a = f.r;
  const int G = a.group;
  const int i = blockIdx.y;
  const int h = blockIdx.x;
  const uint64_t sp = ((cu64*)a.state_ptrs)[i];
  const uint64_t cp = ((cu64*)f.conv_ptrs)[i];
  if (sp == 0 || cp == 0) return;  // inactive slot (the whole workgroup)
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int nt = blockDim.x;
  const int nw = nt / kWave;
  const int c = lane % LPR;   // column group inside a row
  const int rl = lane / LPR;  // row inside a pass
  const int C = f.channels;
  const int NCG = (2 + G) * D / V;  // channel groups: q, k, then v of the group's v-heads
  GT* cs = (GT*)reinterpret_cast<T*>(cp);

  // channel group g: its first channel of x, the taps and the conv state (its LDS offset is g V)
  auto channel_of = [&](int g) {
    const int e = g * V;
    return e < D ? h * D + e : e < 2 * D ? a.hk * D + h * D + (e - D) : 2 * a.hk * D + h * G * D + (e - 2 * D);
  };
  typename V4::Raw xr, sr[K - 1], wr[K], br;
  auto load_conv = [&](int ch0) {
#pragma unroll
    for (int t = 0; t < K - 1; ++t) sr[t] = V4::load_raw_g(cs + static_cast<int64_t>(t) * C + ch0);
    xr = V4::load_raw(static_cast<const T*>(f.x) + static_cast<int64_t>(i) * f.x_stride + ch0);
#pragma unroll
    for (int t = 0; t < K; ++t) wr[t] = V4::load_raw(static_cast<const T*>(f.w) + static_cast<int64_t>(ch0) * K + t * V);
    // with no bias, taps stand in for the load and are never used
    br = V4::load_raw(static_cast<const T*>(f.b ? f.b : f.w) + ch0);
  };
  // convolve channel group g (loaded), put it in LDS and commit its new conv-state rows
  // (old rows 1 .. K-2, then x): this thread is the only reader of those values
  auto conv_commit = [&](int g, int ch0) {
    float out[V];
    conv4_raw<T, K>(wr, br, f.b != nullptr, sr, xr, SILU, out);
    *reinterpret_cast<f32x4*>(&fused_lds[g * V]) = f32x4{out[0], out[1], out[2], out[3]};
#pragma unroll
    for (int t = 0; t < K - 2; ++t) V4::store_raw_g(cs + static_cast<int64_t>(t) * C + ch0, sr[t + 1]);
    V4::store_raw_g(cs + static_cast<int64_t>(K - 2) * C + ch0, xr);
  };

  // block b of the group's rows: v-head h G + b ROWS / d, rows (b ROWS) % d + rl + p RPP
  f32x4 s[P][4];
  auto state_of = [&](int b) {
    const int jj = (b * ROWS) / D;
    return (gf32x4*)(reinterpret_cast<float*>(sp) + static_cast<int64_t>(h * G + jj) * D * D);
  };
  auto load_block = [&](int b) {
    gf32x4* S = state_of(b);
    const int row0 = (b * ROWS) % D + rl;
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s[p][e] = __builtin_nontemporal_load(S + static_cast<int64_t>(row0 + p * RPP) * (D / 4) + c + LPR * e);
  };

  const bool conv_wave = w * kWave < NCG;
  const int g0 = tid < NCG ? tid : NCG - 1;  // (lanes past the last group repeat it and drop the result)
  const int ch00 = channel_of(g0);
  const bool first_block = w * ROWS < G * D;
  if (conv_wave) load_conv(ch00);
  if (first_block) load_block(w);
  if (conv_wave) {
    if (tid < NCG) conv_commit(tid, ch00);
    // more channel groups than threads (many v-heads per k-head): the rest in turn
    for (int g = tid + nt; g < NCG; g += nt) {
      const int ch0 = channel_of(g);
      load_conv(ch0);
      conv_commit(g, ch0);
    }
  }
  // A barrier that orders LDS only: the state loads stay in flight across it, where
  // __syncthreads() would wait for all of them.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  for (int it = 0; it < nit; ++it) {
    const int b = it * nw + w;
    if (b * ROWS >= G * D) break;
    if (it > 0) load_block(b);
    const int jj = (b * ROWS) / D;
    const int j = h * G + jj;
    const int64_t gi = static_cast<int64_t>(i) * a.hv + j;
    const float gval = ((cfloat*)a.g)[gi];
    const float beta = ((cfloat*)a.beta)[gi];
    f32x4 kv[4], qv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[e] = *reinterpret_cast<const f32x4*>(&fused_lds[4 * (c + LPR * e)]);
      kv[e] = *reinterpret_cast<const f32x4*>(&fused_lds[D + 4 * (c + LPR * e)]);
    }
    const int row0 = (b * ROWS) % D + rl;
    float vr[P];
#pragma unroll
    for (int p = 0; p < P; ++p) vr[p] = fused_lds[2 * D + jj * D + row0 + p * RPP];
    decode_rows<D, P, 2>(s, kv, qv, vr, gval, beta, a.eps, a.scale, a.qk_norm != 0, state_of(b), o_row<2>(a, gi * D),
                         a.o_bf16 != 0, row0, c);
  }
}

// ------------------------------------------------------------- fused, streaming form
// When the new conv states go to other buffers than the old ones are read from, no
// workgroup's writes can reach another's reads, so a workgroup need not cover a whole
// k-head. This form keeps decode_kernel's units (one wave = P passes of RPP rows of one
// (slot, v-head), dealt in (slot, head, row) order), NW = min(4, units per head) waves to
// a workgroup, all on one (slot, v-head). The workgroup's threads convolve the k-head's 2d
// q and k channels between them, one channel each, and every wave the v channels of its
// own rows; the values meet in LDS behind one barrier that orders LDS only (the state
// loads stay in flight across it). Each new conv-state row is written once: a v channel by
// the thread that convolved it, the q/k channels by the workgroup holding the first rows of
// the (slot, k-head)'s first v-head.
//
// One channel of the conv with the operations of ConvTaps::apply and conv4_raw, in their
// order (acc = b; acc = fma(w_j, z_j, acc), j = 0 .. K-1; then the activation), so all
// give the same bits. z[0 .. K-2] are the preceding rows (oldest first), cur the token.
template <typename T, int K, bool SILU>
__device__ __forceinline__ float conv1(const float (&w)[K], float b, const float (&z)[K - 1], float cur) {
  float acc = b;
#pragma unroll
  for (int j = 0; j < K - 1; ++j) acc = fmaf(w[j], z[j], acc);
  acc = fmaf(w[K - 1], cur, acc);
  if constexpr (SILU) acc = gdn::silu(acc);
  return acc;
}

template <typename T>
__device__ __forceinline__ float to_f32(T v) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(v);
  else return v;
}

template <typename T, int K, int D, int P, bool SILU>
__global__ __launch_bounds__(kDecodeWaves* kWave) void fused_stream_kernel(FusedArgs f) {
  using Cfg = DecodeCfg<D, P>;
  constexpr int LPR = Cfg::LPR, RPP = Cfg::RPP, NPART = Cfg::NPART, ROWS = Cfg::ROWS;
  constexpr int NW = NPART < kDecodeWaves ? NPART : kDecodeWaves;  // waves per workgroup
  static_assert(NPART % NW == 0 && 2 * D <= NW * kWave && ROWS <= kWave, "workgroup shape");
  typedef __attribute__((address_space(1))) T GT;
  typedef __attribute__((address_space(1))) const T CGT;
  __shared__ __attribute__((aligned(16))) float qk_l[2 * D];  // q, k of the k-head
  __shared__ float v_l[NW][ROWS];                            // v at each wave's rows
  const RecurArgs& a = f.r;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int us = xcd_block() * NW + w;  // unit within the slot (NW divides NPART: whole workgroups)
  const int part = us % NPART;
  const int j = us / NPART;
  const int i = blockIdx.y;
  const uint64_t sp = ((cu64*)a.state_ptrs)[i];
  const uint64_t cin = ((cu64*)f.conv_ptrs)[i];
  const uint64_t cout = ((cu64*)f.conv_out_ptrs)[i];
  if (sp == 0 || cin == 0 || cout == 0) return;  // inactive slot (the whole workgroup)
  const int G = a.group;
  const int h = j / G;
  const int c = lane % LPR;
  const int rl = lane / LPR;
  const int row0 = part * ROWS + rl;
  const int C = f.channels;
  CGT* csin = (CGT*)reinterpret_cast<const T*>(cin);
  GT* csout = (GT*)reinterpret_cast<T*>(cout);
  const T* x = static_cast<const T*>(f.x) + static_cast<int64_t>(i) * f.x_stride;
  const T* wt = static_cast<const T*>(f.w);
  const T* bs = static_cast<const T*>(f.b ? f.b : f.w);  // (taps stand in when there is no bias)
  const bool has_b = f.b != nullptr;

  // conv inputs first (mostly cached: the conv then waits only for them while the state
  // streams in). Thread t < 2d: q/k channel t of the k-head; lane l < ROWS: the v channel
  // of the wave's row l. Threads without a channel load channel 0's and drop the result.
  const bool has_qk = tid < 2 * D;
  const int e = has_qk ? tid : 0;
  const int chq = e < D ? h * D + e : a.hk * D + h * D + (e - D);
  const bool has_v = lane < ROWS;
  const int chv = 2 * a.hk * D + j * D + part * ROWS + (has_v ? lane : 0);
  T qz[K - 1], qx, qb, vz[K - 1], vx, vb;
  float qw[K], vw[K];
#pragma unroll
  for (int t = 0; t < K - 1; ++t) {
    qz[t] = csin[static_cast<int64_t>(t) * C + chq];
    vz[t] = csin[static_cast<int64_t>(t) * C + chv];
  }
  qx = x[chq];
  vx = x[chv];
#pragma unroll
  for (int t = 0; t < K; ++t) {
    qw[t] = to_f32<T>(wt[static_cast<int64_t>(chq) * K + t]);
    vw[t] = to_f32<T>(wt[static_cast<int64_t>(chv) * K + t]);
  }
  qb = bs[chq];
  vb = bs[chv];
  gf32x4* S = (gf32x4*)(reinterpret_cast<float*>(sp) + static_cast<int64_t>(j) * D * D);
  f32x4 s[P][4];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      s[p][q] = __builtin_nontemporal_load(S + static_cast<int64_t>(row0 + p * RPP) * (D / 4) + c + LPR * q);
  const int64_t gi = static_cast<int64_t>(i) * a.hv + j;
  const float gval = ((cfloat*)a.g)[gi];
  const float beta = ((cfloat*)a.beta)[gi];

  {
    float zq[K - 1], zv[K - 1];
#pragma unroll
    for (int t = 0; t < K - 1; ++t) {
      zq[t] = to_f32<T>(qz[t]);
      zv[t] = to_f32<T>(vz[t]);
    }
    const float oq = conv1<T, K, SILU>(qw, has_b ? to_f32<T>(qb) : 0.f, zq, to_f32<T>(qx));
    const float ov = conv1<T, K, SILU>(vw, has_b ? to_f32<T>(vb) : 0.f, zv, to_f32<T>(vx));
    if (has_qk) qk_l[tid] = oq;
    if (has_v) v_l[w][lane] = ov;
  }
  if constexpr (NW > 1) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  } else {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }
  f32x4 kv[4], qv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    qv[q] = *reinterpret_cast<const f32x4*>(&qk_l[4 * (c + LPR * q)]);
    kv[q] = *reinterpret_cast<const f32x4*>(&qk_l[D + 4 * (c + LPR * q)]);
  }
  float vr[P];
#pragma unroll
  for (int p = 0; p < P; ++p) vr[p] = v_l[w][rl + p * RPP];
  decode_rows<D, P, 2>(s, kv, qv, vr, gval, beta, a.eps, a.scale, a.qk_norm != 0, S, o_row<2>(a, gi * D),
                       a.o_bf16 != 0, row0, c);

  // the new conv-state rows (old rows 1 .. K-2, then x)
  if (has_v) {
#pragma unroll
    for (int t = 0; t < K - 2; ++t) csout[static_cast<int64_t>(t) * C + chv] = vz[t + 1];
    csout[static_cast<int64_t>(K - 2) * C + chv] = vx;
  }
  if ((j % G) == 0 && part < NW && has_qk) {
#pragma unroll
    for (int t = 0; t < K - 2; ++t) csout[static_cast<int64_t>(t) * C + chq] = qz[t + 1];
    csout[static_cast<int64_t>(K - 2) * C + chq] = qx;
  }
}

template <typename T, int K, int D, int P>
hipError_t launch_stream_p(const FusedArgs& f, int32_t m, hipStream_t s) {
  using Cfg = DecodeCfg<D, P>;
  constexpr int NW = Cfg::NPART < kDecodeWaves ? Cfg::NPART : kDecodeWaves;
  const dim3 blocks(static_cast<unsigned>(f.r.hv * Cfg::NPART / NW), static_cast<unsigned>(m));
  if (f.silu)
    fused_stream_kernel<T, K, D, P, true><<<blocks, NW * kWave, 0, s>>>(f);
  else
    fused_stream_kernel<T, K, D, P, false><<<blocks, NW * kWave, 0, s>>>(f);
  return hipGetLastError();
}

// unit size as launch_decode (d = 32: one pass; d = 64: one pass of 16 rows, so that a
// head's rows fill a four-wave workgroup)
template <typename T, int K, int D>
hipError_t launch_stream_d(const FusedArgs& f, int32_t m, hipStream_t s) {
  if constexpr (D == 128) {
    if (static_cast<int64_t>(m) * f.r.hv >= 1024) return launch_stream_p<T, K, D, 1>(f, m, s);
    return launch_stream_p<T, K, D, 2>(f, m, s);
  } else {
    return launch_stream_p<T, K, D, 1>(f, m, s);
  }
}

template <typename T, int K, int D>
hipError_t launch_fused_d(const FusedArgs& f, int32_t m, hipStream_t s) {
  if (f.conv_out_ptrs != f.conv_ptrs) return launch_stream_d<T, K, D>(f, m, s);
  using FC = FusedCfg<D>;
  const int G = f.r.group;
  const dim3 blocks(static_cast<unsigned>(f.r.hk), static_cast<unsigned>(m));
  const unsigned threads = static_cast<unsigned>(FC::waves(G) * kWave);
  const size_t lds = static_cast<size_t>(2 + G) * D * sizeof(float);
  if (f.silu)
    fused_decode_kernel<T, K, D, true><<<blocks, threads, lds, s>>>(f, FC::iters(G));
  else
    fused_decode_kernel<T, K, D, false><<<blocks, threads, lds, s>>>(f, FC::iters(G));
  return hipGetLastError();
}

template <typename T, int K>
hipError_t launch_fused_k(const FusedArgs& f, int32_t m, hipStream_t s) {
  switch (f.r.d) {
    case 32: return launch_fused_d<T, K, 32>(f, m, s);
    case 64: return launch_fused_d<T, K, 64>(f, m, s);
    default: return launch_fused_d<T, K, 128>(f, m, s);
  }
}

template <typename T>
hipError_t launch_fused_t(const FusedArgs& f, int32_t m, hipStream_t s) {
  switch (f.width) {
    case 2: return launch_fused_k<T, 2>(f, m, s);
    case 3: return launch_fused_k<T, 3>(f, m, s);
    default: return launch_fused_k<T, 4>(f, m, s);
  }
}
}  // namespace

hipError_t launch_decode_fused(const FusedArgs& f, int32_t m, hipStream_t s) {
  if (m == 0) return hipSuccess;
  return f.bf16 ? launch_fused_t<uint16_t>(f, m, s) : launch_fused_t<float>(f, m, s);
}

namespace {
__global__ void slot_pointers_kernel(uint64_t base, int64_t slot_bytes, int32_t pool_slots, const int32_t* idx,
                                     int32_t m, uint64_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m) return;
  const int32_t s = idx[i];
  out[i] = (s >= 0 && s < pool_slots) ? base + static_cast<uint64_t>(s) * static_cast<uint64_t>(slot_bytes) : 0ull;
}
}  // namespace

// Slot copy: blockIdx.y = slot pair, each workgroup streams 16 KiB (256 threads x 4 x 16 B)
// of the slot's bytes with nontemporal 16-byte loads and stores.
namespace {
constexpr int kCopyThreads = 256;
constexpr int kCopyVecs = 4;  // 16-byte vectors per thread
__global__ __launch_bounds__(kCopyThreads) void slot_copy_kernel(const uint64_t* src, const uint64_t* dst,
                                                                 int64_t vecs) {
  const int i = blockIdx.y;
  const uint64_t sp = ((cu64*)src)[i];
  const uint64_t dp = ((cu64*)dst)[i];
  if (sp == 0 || dp == 0) return;
  const gf32x4* a = (const gf32x4*)reinterpret_cast<const float*>(sp);
  gf32x4* b = (gf32x4*)reinterpret_cast<float*>(dp);
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyThreads * kCopyVecs + threadIdx.x;
  f32x4 v[kCopyVecs];
#pragma unroll
  for (int e = 0; e < kCopyVecs; ++e) {
    const int64_t k = base + e * kCopyThreads;
    if (k < vecs) v[e] = __builtin_nontemporal_load(a + k);
  }
#pragma unroll
  for (int e = 0; e < kCopyVecs; ++e) {
    const int64_t k = base + e * kCopyThreads;
    if (k < vecs) __builtin_nontemporal_store(v[e], b + k);
  }
}
}  // namespace

hipError_t launch_slot_copy(const uint64_t* src, const uint64_t* dst, int64_t bytes, int32_t n, hipStream_t s) {
  if (n == 0 || bytes == 0) return hipSuccess;
  const int64_t vecs = bytes / 16;
  const int64_t per_block = static_cast<int64_t>(kCopyThreads) * kCopyVecs;
  const dim3 grid(static_cast<unsigned>((vecs + per_block - 1) / per_block), static_cast<unsigned>(n));
  slot_copy_kernel<<<grid, kCopyThreads, 0, s>>>(src, dst, vecs);
  return hipGetLastError();
}

hipError_t launch_slot_pointers(uint64_t base, int64_t slot_bytes, int32_t pool_slots, const int32_t* idx,
                                int32_t m, uint64_t* out, hipStream_t s) {
  if (m == 0) return hipSuccess;
  slot_pointers_kernel<<<(m + 255) / 256, 256, 0, s>>>(base, slot_bytes, pool_slots, idx, m, out);
  return hipGetLastError();
}

}  // namespace gdn
