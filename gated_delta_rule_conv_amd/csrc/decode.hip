// Batched single-token decode of the gated delta rule, gfx950.
//
// For slot i and v-head j (k-head h = j / (Hv/Hk)), with k^ = k/sqrt(|k|^2+eps),
// q^ = scale * q/sqrt(|q|^2+eps), alpha = exp(g), and S the d_v x d_k state:
//     S_new = alpha S (I - beta k^ k^T) + beta v k^T   and   o = S_new q^.
// ("System Design" (project_6), "GDN Kernel Dispatch Detail", decode branch: decay of
// the temporal state with the delta write, then the query against the state;
// aprender #5279, "Phase plan", P5: the slot index on the grid and a device u64[m]
// array of per-slot state pointers.)
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

#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

typedef __attribute__((address_space(1))) f32x4 gf32x4;
typedef __attribute__((address_space(1))) float gfloat;
typedef __attribute__((address_space(1))) const float cgfloat;
typedef __attribute__((address_space(4))) const uint64_t cu64;
typedef __attribute__((address_space(4))) const float cfloat;
// (Generic -> global/constant pointer conversions are address-space casts, which C++
// spells only as C-style casts.)

constexpr int kDecodeWaves = 4;  // waves per workgroup

template <int D, int P>
struct DecodeCfg {
  static constexpr int LPR = D / 16;          // lanes per row (16 floats per lane)
  static constexpr int RPP = kWave / LPR;     // rows per pass
  static constexpr int ROWS = RPP * P;        // rows per unit
  static constexpr int NPART = D / ROWS;      // units per (slot, head)
  static_assert(NPART * ROWS == D, "units must tile the head");
};

template <int D, int P, bool SCHED_FENCE>
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
  const float rk = 1.0f / sqrtf(kk + a.eps);
  const float rq = a.scale / sqrtf(qq + a.eps);
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
  gfloat* orow = (gfloat*)(a.o + gi * D);

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
    if (c == 0) orow[r] = fmaf(ur, kq, alpha * sq);
  }
}

template <int D, int P, bool F>
hipError_t launch_units(const RecurArgs& a, int32_t m, hipStream_t s) {
  const int64_t units = static_cast<int64_t>(m) * a.hv * DecodeCfg<D, P>::NPART;
  const unsigned blocks = static_cast<unsigned>((units + kDecodeWaves - 1) / kDecodeWaves);
  decode_kernel<D, P, F><<<blocks, kDecodeWaves * kWave, 0, s>>>(a, static_cast<int32_t>(units));
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
