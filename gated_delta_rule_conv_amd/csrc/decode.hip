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
// Mapping (d = 128): a block is one (slot, v-head) = 64 KiB of state, 4 waves x 32 rows.
// Eight lanes share a row; lane c of the eight holds floats [4c + 32u, 4c + 32u + 4),
// u = 0..3, so each load instruction of a wave covers 8 rows x 128 contiguous bytes.
// Each lane issues its 16 float4 loads before any arithmetic. The two row dots are
// reduced over the eight lanes with a fixed DPP butterfly, so the bits of a slot's
// result do not depend on m, on the grid, or on which other slots are in the call.

#include "device_common.h"
#include "launch.h"

namespace gdn {
namespace {

template <int D>
struct DecodeCfg {
  static constexpr int kLanesPerRow = D / 16;          // 16 floats per lane per row
  static constexpr int kRowsPerPass = kWave / kLanesPerRow;
  static constexpr int kPasses = (D * D / 4096) > 0 ? (D * D / 4096) : 1;
  static constexpr int kRowsPerWave = kRowsPerPass * kPasses;
  static constexpr int kWaves = D / kRowsPerWave;
  static constexpr int kThreads = kWaves * kWave;
  static_assert(kWaves * kRowsPerWave == D, "rows must tile the head");
};

template <int D>
__global__ __launch_bounds__(DecodeCfg<D>::kThreads) void decode_kernel(RecurArgs a) {
  using Cfg = DecodeCfg<D>;
  constexpr int LPR = Cfg::kLanesPerRow;
  constexpr int P = Cfg::kPasses;
  const int j = blockIdx.x;  // v-head
  const int i = blockIdx.y;  // slot
  const uint64_t sp = a.state_ptrs[i];
  if (sp == 0) return;  // inactive slot
  const int h = j / (a.hv / a.hk);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c = lane % LPR;           // column group inside the row
  const int rlocal = lane / LPR;      // row inside a pass

  float* S = reinterpret_cast<float*>(sp) + static_cast<int64_t>(j) * D * D;
  const int row0 = wave * Cfg::kRowsPerWave + rlocal;

  // state rows: issue every load first
  f32x4 s[P][4];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const f32x4* rowp = reinterpret_cast<const f32x4*>(S + static_cast<int64_t>(row0 + p * Cfg::kRowsPerPass) * D);
#pragma unroll
    for (int u = 0; u < 4; ++u) s[p][u] = __builtin_nontemporal_load(rowp + c + LPR * u);
  }

  // k^ and q^ at this lane's 16 columns
  const float4* kp = reinterpret_cast<const float4*>(a.k + static_cast<int64_t>(i) * a.k_stride + h * D);
  const float4* qp = reinterpret_cast<const float4*>(a.q + static_cast<int64_t>(i) * a.q_stride + h * D);
  float4 kv[4], qv[4];
  float kk = 0.f, qq = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    kv[u] = kp[c + LPR * u];
    qv[u] = qp[c + LPR * u];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    kk = fmaf(kv[u].x, kv[u].x, kk); kk = fmaf(kv[u].y, kv[u].y, kk);
    kk = fmaf(kv[u].z, kv[u].z, kk); kk = fmaf(kv[u].w, kv[u].w, kk);
    qq = fmaf(qv[u].x, qv[u].x, qq); qq = fmaf(qv[u].y, qv[u].y, qq);
    qq = fmaf(qv[u].z, qv[u].z, qq); qq = fmaf(qv[u].w, qv[u].w, qq);
  }
  kk = group_sum<LPR>(kk);
  qq = group_sum<LPR>(qq);
  const float rk = 1.0f / sqrtf(kk + a.eps);
  const float rq = a.scale / sqrtf(qq + a.eps);
  float kq = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    kv[u].x *= rk; kv[u].y *= rk; kv[u].z *= rk; kv[u].w *= rk;
    qv[u].x *= rq; qv[u].y *= rq; qv[u].z *= rq; qv[u].w *= rq;
    kq = fmaf(kv[u].x, qv[u].x, kq); kq = fmaf(kv[u].y, qv[u].y, kq);
    kq = fmaf(kv[u].z, qv[u].z, kq); kq = fmaf(kv[u].w, qv[u].w, kq);
  }
  kq = group_sum<LPR>(kq);

  const int64_t gi = static_cast<int64_t>(i) * a.hv + j;
  const float alpha = expf(a.g[gi]);
  const float beta = a.beta[gi];
  const float* vrow = a.v + static_cast<int64_t>(i) * a.v_stride + static_cast<int64_t>(j) * D;
  float* orow = a.o + gi * D;

#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int r = row0 + p * Cfg::kRowsPerPass;
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sk = fmaf(s[p][u].x, kv[u].x, sk); sk = fmaf(s[p][u].y, kv[u].y, sk);
      sk = fmaf(s[p][u].z, kv[u].z, sk); sk = fmaf(s[p][u].w, kv[u].w, sk);
      sq = fmaf(s[p][u].x, qv[u].x, sq); sq = fmaf(s[p][u].y, qv[u].y, sq);
      sq = fmaf(s[p][u].z, qv[u].z, sq); sq = fmaf(s[p][u].w, qv[u].w, sq);
    }
    sk = group_sum<LPR>(sk);
    sq = group_sum<LPR>(sq);
    const float ur = beta * (vrow[r] - alpha * sk);
    f32x4* rowp = reinterpret_cast<f32x4*>(S + static_cast<int64_t>(r) * D);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4 n;
      n.x = fmaf(ur, kv[u].x, alpha * s[p][u].x);
      n.y = fmaf(ur, kv[u].y, alpha * s[p][u].y);
      n.z = fmaf(ur, kv[u].z, alpha * s[p][u].z);
      n.w = fmaf(ur, kv[u].w, alpha * s[p][u].w);
      __builtin_nontemporal_store(n, rowp + c + LPR * u);
    }
    if (c == 0) orow[r] = fmaf(ur, kq, alpha * sq);
  }
}

}  // namespace

hipError_t launch_decode(const RecurArgs& a, int32_t m, hipStream_t s) {
  if (m == 0) return hipSuccess;
  dim3 grid(a.hv, m);
  switch (a.d) {
    case 32: decode_kernel<32><<<grid, DecodeCfg<32>::kThreads, 0, s>>>(a); break;
    case 64: decode_kernel<64><<<grid, DecodeCfg<64>::kThreads, 0, s>>>(a); break;
    default: decode_kernel<128><<<grid, DecodeCfg<128>::kThreads, 0, s>>>(a); break;
  }
  return hipGetLastError();
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

hipError_t launch_slot_pointers(uint64_t base, int64_t slot_bytes, int32_t pool_slots, const int32_t* idx,
                                int32_t m, uint64_t* out, hipStream_t s) {
  if (m == 0) return hipSuccess;
  slot_pointers_kernel<<<(m + 255) / 256, 256, 0, s>>>(base, slot_bytes, pool_slots, idx, m, out);
  return hipGetLastError();
}

}  // namespace gdn
