// In-place streaming pass over a device buffer: the memory access pattern of the decode
// kernel's state pass (a wave reads 4 KiB contiguous with nontemporal 16-byte loads and
// writes it back the same way, four waves to a workgroup) with no arithmetic, for
// measuring the practical HBM rate.

#include <hip/hip_runtime.h>

#include "../../include/gdn_probe.h"
#include "device_common.h"

namespace gdn {
namespace {

constexpr int kProbeWaves = 4;
constexpr int kProbeVecs = 4;  // 16-byte vectors per lane

__global__ __launch_bounds__(kProbeWaves* kWave) void hbm_probe_kernel(f32x4* buf, uint32_t salt) {
  typedef __attribute__((address_space(1))) f32x4 G4;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kProbeWaves + threadIdx.x / kWave;
  G4* p = (G4*)buf + wave * (kWave * kProbeVecs) + (threadIdx.x & (kWave - 1));
  f32x4 v[kProbeVecs];
#pragma unroll
  for (int e = 0; e < kProbeVecs; ++e) v[e] = __builtin_nontemporal_load(p + kWave * e);
#pragma unroll
  for (int e = 0; e < kProbeVecs; ++e) {
    u32x4 u = __builtin_bit_cast(u32x4, v[e]);
    u ^= salt;
    __builtin_nontemporal_store(__builtin_bit_cast(f32x4, u), p + kWave * e);
  }
}

}  // namespace
}  // namespace gdn

extern "C" gdn_status gdn_hbm_probe(void* buf, size_t bytes, uint32_t salt, void* stream) {
  constexpr size_t kBlockBytes = static_cast<size_t>(gdn::kProbeWaves) * gdn::kWave * gdn::kProbeVecs * 16;
  if (!buf) return GDN_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) || bytes % kBlockBytes) return GDN_ERR_ALIGN;
  if (bytes == 0) return GDN_OK;
  const size_t blocks = bytes / kBlockBytes;
  if (blocks > 0x7fffffffu) return GDN_ERR_ALIGN;
  gdn::hbm_probe_kernel<<<static_cast<unsigned>(blocks), gdn::kProbeWaves * gdn::kWave, 0,
                          static_cast<hipStream_t>(stream)>>>(static_cast<gdn::f32x4*>(buf), salt);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}
