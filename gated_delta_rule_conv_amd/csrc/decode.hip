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

// The arithmetic of one unit once its loads are in registers: normalise k and q (the
// lane holds 16 columns of each), then for each of the P row passes the two row dots,
// the delta-rule update of the rows and their outputs. Both decode kernels call this, so
// the fused kernel's bits equal the separate conv + decode launches.
// OB: how o is stored -- 0 fp32, 1 bf16 (rounded to nearest even), 2 as the o_bf16 flag says.
template <int D, int P, int OB>
__device__ __forceinline__ void decode_rows(const f32x4 (&s)[P][4], f32x4 (&kv)[4], f32x4 (&qv)[4], const float (&vr)[P],
                                            float gval, float beta, float eps, float scale, bool qk_norm, gf32x4* S,
                                            void* orow, bool o_bf16, int row0, int c) {
  using Cfg = DecodeCfg<D, P>;
  constexpr int LPR = Cfg::LPR, RPP = Cfg::RPP;
  // k^ and q^ at this lane's 16 columns, and k^ . q^
  float kk = 0.f, qq = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kk = fmaf(kv[e].x, kv[e].x, kk); kk = fmaf(kv[e].y, kv[e].y, kk);
    kk = fmaf(kv[e].z, kv[e].z, kk); kk = fmaf(kv[e].w, kv[e].w, kk);
    qq = fmaf(qv[e].x, qv[e].x, qq); qq = fmaf(qv[e].y, qv[e].y, qq);
    qq = fmaf(qv[e].z, qv[e].z, qq); qq = fmaf(qv[e].w, qv[e].w, qq);
  }
  kk = group_sum<LPR>(kk);
  qq = group_sum<LPR>(qq);
  const float rk = qk_norm ? 1.0f / sqrtf(kk + eps) : 1.0f;
  const float rq = qk_norm ? scale / sqrtf(qq + eps) : scale;
  float kq = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kv[e].x *= rk; kv[e].y *= rk; kv[e].z *= rk; kv[e].w *= rk;
    qv[e].x *= rq; qv[e].y *= rq; qv[e].z *= rq; qv[e].w *= rq;
    kq = fmaf(kv[e].x, qv[e].x, kq); kq = fmaf(kv[e].y, qv[e].y, kq);
    kq = fmaf(kv[e].z, qv[e].z, kq); kq = fmaf(kv[e].w, qv[e].w, kq);
  }
  kq = group_sum<LPR>(kq);
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
    sk = group_sum<LPR>(sk);
    sq = group_sum<LPR>(sq);
    const float ur = beta * (vr[p] - alpha * sk);
    gf32x4* rowp = S + static_cast<int64_t>(r) * (D / 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f32x4 n;
      n.x = fmaf(ur, kv[e].x, alpha * s[p][e].x);
      n.y = fmaf(ur, kv[e].y, alpha * s[p][e].y);
      n.z = fmaf(ur, kv[e].z, alpha * s[p][e].z);
      n.w = fmaf(ur, kv[e].w, alpha * s[p][e].w);
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


template <int D, int P, bool SCHED_FENCE, int OB>
__global__ __launch_bounds__(kDecodeWaves* kWave) void decode_kernel(RecurArgs a, int32_t total_units) {
  using Cfg = DecodeCfg<D, P>;
  constexpr int LPR = Cfg::LPR, RPP = Cfg::RPP, NPART = Cfg::NPART;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int u = blockIdx.x * kDecodeWaves + w;
  if (u >= total_units) return;
  const int part = u % NPART;
  const int j = (u / NPART) % a.hv;
  const int i = (u / NPART) / a.hv;
  const uint64_t sp = ((cu64*)a.state_ptrs)[i];
  if (sp == 0) return;  // inactive slot
  const int h = j / (a.hv / a.hk);
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
  const int64_t units = static_cast<int64_t>(m) * a.hv * DecodeCfg<D, P>::NPART;
  const unsigned blocks = static_cast<unsigned>((units + kDecodeWaves - 1) / kDecodeWaves);
  if (a.o_bf16)
    decode_kernel<D, P, F, 1><<<blocks, kDecodeWaves * kWave, 0, s>>>(a, static_cast<int32_t>(units));
  else
    decode_kernel<D, P, F, 0><<<blocks, kDecodeWaves * kWave, 0, s>>>(a, static_cast<int32_t>(units));
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
// One launch for the whole decode step of a layer: the depthwise conv of the token's
// q, k and v channels (against the slot's conv state), the conv state commit, and the
// decode above. A workgroup is WPB units of one (slot, v-head), i.e. VR consecutive
// state rows. Threads first convolve 4 channels each -- the 2d q/k channels of the
// head's k-head (wave 0) and then the VR v channels of the workgroup's rows -- into LDS
// with the conv kernels' arithmetic (conv4_raw). In one-pass units and short launches
// the conv inputs are loaded before the state rows, so the conv waits only for its own
// (mostly cached) inputs while the state is still streaming in; otherwise after them
// (see CONV_FIRST). The waves then take k, q and v from LDS and run decode_rows
// unchanged.
//
// Conv state commit. The v channels of a workgroup's rows are read by that workgroup
// alone, so their lanes write the shifted state right after reading it. The q/k
// channels of k-head h are read by every workgroup of the (hv/hk) v-heads sharing it;
// each of those workgroups adds one to counters[slot][h] once all its reads have
// returned, and the one that brings it to the total writes the q/k conv state (from
// the rows it keeps in LDS) and resets the counter to zero for the next call.
template <int D, int P>
struct FusedCfg {
  static constexpr int NPART = DecodeCfg<D, P>::NPART;
  static constexpr int WPB = NPART < kDecodeWaves ? NPART : kDecodeWaves;  // waves per workgroup
  static constexpr int BPH = NPART / WPB;                                 // workgroups per (slot, v-head)
  static constexpr int NT = WPB * kWave;
  static constexpr int VR = WPB * DecodeCfg<D, P>::ROWS;                  // state rows per workgroup
  static constexpr int CV = 4;                                            // channels per conv thread
  static constexpr int GQK = 2 * D / CV;                                  // q/k channel groups
  static constexpr int GV = VR / CV;                                      // v channel groups
  static constexpr int NCG = GQK + GV;
  static constexpr int NCW = (NCG + kWave - 1) / kWave;                   // waves that convolve
  static_assert(GQK <= kWave, "the q/k groups are wave 0's");
  static_assert(NCG <= NT, "one channel group per thread");
  // One-pass units with bf16 inputs are held to 72 VGPRs, at least 7 waves per SIMD
  // (they take 64: 8 waves); fp32 inputs need more registers for the raw conv inputs.
  template <typename T>
  static constexpr int min_blocks() { return (P == 1 && sizeof(T) == 2 && WPB == 4) ? 7 : 1; }
};

template <typename T, int K, int D, int P, bool SCHED_FENCE, bool CONV_FIRST>
__global__ __launch_bounds__((FusedCfg<D, P>::NT), (FusedCfg<D, P>::template min_blocks<T>())) void fused_decode_kernel(FusedArgs f) {
  using Cfg = DecodeCfg<D, P>;
  using FC = FusedCfg<D, P>;
  using V4 = Vec4<T>;
  constexpr int LPR = Cfg::LPR, RPP = Cfg::RPP, ROWS = Cfg::ROWS;
  constexpr int WPB = FC::WPB, BPH = FC::BPH, VR = FC::VR, GQK = FC::GQK, GV = FC::GV, NCG = FC::NCG;
  constexpr int V = FC::CV;
  typedef __attribute__((address_space(1))) T GT;
  __shared__ __attribute__((aligned(16))) float yqk[2 * D];  // q then k of the k-head
  __shared__ __attribute__((aligned(16))) float yv[VR];
  __shared__ typename V4::Raw qk_rows[K - 1][GQK];  // new q/k conv-state rows
  const RecurArgs& a = f.r;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int bh = blockIdx.x % BPH;
  const int j = (blockIdx.x / BPH) % a.hv;
  const int i = (blockIdx.x / BPH) / a.hv;
  const uint64_t sp = ((cu64*)a.state_ptrs)[i];
  const uint64_t cp = ((cu64*)f.conv_ptrs)[i];
  if (sp == 0 || cp == 0) return;  // inactive slot (the whole workgroup)
  const int h = j / (a.hv / a.hk);
  const int part = bh * WPB + w;
  const int c = lane % LPR;
  const int rl = lane / LPR;
  const int row0 = part * ROWS + rl;
  gf32x4* S = (gf32x4*)(reinterpret_cast<float*>(sp) + static_cast<int64_t>(j) * D * D);
  GT* cs = (GT*)reinterpret_cast<T*>(cp);
  const int C = f.channels;

  // Thread t < NCG takes channel group t (q/k groups, then v groups); other threads that
  // load repeat a v group and drop the result. Everything is in flight before anything
  // waits. CONV_FIRST: the conv inputs are loaded before the state rows, so the conv
  // waits only for its own (mostly cached) inputs -- best where the launch is short and
  // latency-bound; with two passes per wave every wave then loads conv inputs (loads
  // under a branch made the compiler copy their results at its end, which waits for them
  // before the state loads can issue). Otherwise the state rows go first and only the
  // convolving waves load conv inputs, which issues fewer loads where the launch fills
  // the chip.
  const bool conv_wave = w < FC::NCW;
  const int grp = tid < NCG ? tid : GQK + (tid - NCG) % GV;
  const bool is_qk = grp < GQK;
  const int ch0 = is_qk ? (grp * V < D ? h * D + grp * V : a.hk * D + h * D + (grp * V - D))
                        : 2 * a.hk * D + j * D + bh * VR + (grp - GQK) * V;
  typename V4::Raw xr, sr[K - 1], wr[K], br;
  auto load_conv = [&]() {
#pragma unroll
    for (int t = 0; t < K - 1; ++t) sr[t] = V4::load_raw_g(cs + static_cast<int64_t>(t) * C + ch0);
    xr = V4::load_raw(static_cast<const T*>(f.x) + static_cast<int64_t>(i) * f.x_stride + ch0);
#pragma unroll
    for (int t = 0; t < K; ++t) wr[t] = V4::load_raw(static_cast<const T*>(f.w) + static_cast<int64_t>(ch0) * K + t * V);
    // with no bias, taps stand in for the load and are never used
    br = V4::load_raw(static_cast<const T*>(f.b ? f.b : f.w) + ch0);
  };
  f32x4 s[P][4];
  auto load_state = [&]() {
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s[p][e] = __builtin_nontemporal_load(S + static_cast<int64_t>(row0 + p * RPP) * (D / 4) + c + LPR * e);
  };
  if constexpr (!CONV_FIRST) {
    load_state();
    if (conv_wave) load_conv();
  } else {
    if (conv_wave || P > 1) load_conv();
    load_state();
  }
  const int64_t gi = static_cast<int64_t>(i) * a.hv + j;
  const float gval = ((cfloat*)a.g)[gi];
  const float beta = ((cfloat*)a.beta)[gi];
  if constexpr (SCHED_FENCE) __builtin_amdgcn_sched_barrier(0);

  // Only wave 0 reads q/k conv state. Once its reads have returned (their values are
  // consumed here) it counts this workgroup in, with a relaxed atomic: no later write
  // can reach a read that is done, and the commit needs nothing from the other
  // workgroups but the count itself. (Acquire or release at device scope would write
  // back and invalidate this XCD's L2.) The count comes back while the waves compute.
  int32_t* ctr = f.counters + static_cast<int64_t>(i) * a.hk + h;
  int before = 0;
  if (conv_wave) {
    float out[V];
    conv4_raw<T, K>(wr, br, f.b != nullptr, sr, xr, f.silu != 0, out);
    if (tid < NCG) {
      float* dst = is_qk ? &yqk[grp * V] : &yv[(grp - GQK) * V];
      *reinterpret_cast<f32x4*>(dst) = f32x4{out[0], out[1], out[2], out[3]};
      // new conv-state rows = old rows 1 .. K-2, then x
      if (!is_qk) {
        // v channels: this thread is their only reader, so they are written now
#pragma unroll
        for (int t = 0; t < K - 2; ++t) V4::store_raw_g(cs + static_cast<int64_t>(t) * C + ch0, sr[t + 1]);
        V4::store_raw_g(cs + static_cast<int64_t>(K - 2) * C + ch0, xr);
      } else {
        // q/k channels: kept in LDS for the commit, in case this workgroup is the last
#pragma unroll
        for (int t = 0; t < K - 2; ++t) qk_rows[t][grp] = sr[t + 1];
        qk_rows[K - 2][grp] = xr;
      }
    }
    if (tid == 0) before = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // A barrier that orders LDS only: the waves' state loads (and wave 0's count) stay in
  // flight across it, where __syncthreads() would wait for all of them.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  f32x4 kv[4], qv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    qv[e] = *reinterpret_cast<const f32x4*>(&yqk[4 * (c + LPR * e)]);
    kv[e] = *reinterpret_cast<const f32x4*>(&yqk[D + 4 * (c + LPR * e)]);
  }
  float vr[P];
#pragma unroll
  for (int p = 0; p < P; ++p) vr[p] = yv[w * ROWS + rl + p * RPP];
  decode_rows<D, P, 2>(s, kv, qv, vr, gval, beta, a.eps, a.scale, a.qk_norm != 0, S, o_row<2>(a, gi * D), a.o_bf16 != 0, row0, c);

  // the last workgroup of (slot, k-head) writes the q/k conv state (wave 0, from the
  // rows it put in LDS itself) and leaves the counter at zero
  if (w == 0 && __builtin_amdgcn_readfirstlane(before) == (a.hv / a.hk) * BPH - 1) {
    if (lane < GQK) {
#pragma unroll
      for (int t = 0; t < K - 1; ++t) V4::store_raw_g(cs + static_cast<int64_t>(t) * C + ch0, qk_rows[t][lane]);
    }
    if (lane == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename T, int K, int D, int P, bool F, bool CF>
hipError_t launch_fused_units(const FusedArgs& f, int32_t m, hipStream_t s) {
  using FC = FusedCfg<D, P>;
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(m) * f.r.hv * FC::BPH);
  fused_decode_kernel<T, K, D, P, F, CF><<<blocks, FC::NT, 0, s>>>(f);
  return hipGetLastError();
}

template <typename T, int K>
hipError_t launch_fused_k(const FusedArgs& f, int32_t m, hipStream_t s) {
  // unit size as launch_decode; below m * Hv = 256 (a launch of a few hundred
  // workgroups) the two-pass units load the conv inputs first
  const int64_t mh = static_cast<int64_t>(m) * f.r.hv;
  switch (f.r.d) {
    case 32: return launch_fused_units<T, K, 32, 1, false, true>(f, m, s);
    case 64:
      if (mh >= 1024) return launch_fused_units<T, K, 64, 1, false, true>(f, m, s);
      return mh >= 256 ? launch_fused_units<T, K, 64, 2, true, false>(f, m, s)
                       : launch_fused_units<T, K, 64, 2, true, true>(f, m, s);
    default:
      if (mh >= 1024) return launch_fused_units<T, K, 128, 1, false, true>(f, m, s);
      return mh >= 256 ? launch_fused_units<T, K, 128, 2, true, false>(f, m, s)
                       : launch_fused_units<T, K, 128, 2, true, true>(f, m, s);
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

// Same unit-size rule as launch_decode.
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
