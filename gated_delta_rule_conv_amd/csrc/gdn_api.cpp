// C-ABI entry points of libgdn: host-side argument checks, then kernel launches.
// Every check is O(1) on host values; no device memory is read from the host and
// nothing is launched when a check fails.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/gdn.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gdn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return GDN_OK;
  return fail(GDN_ERR_HIP, "%s: HIP error %d (%s)", what, static_cast<int>(e), hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every entry point that takes dims.
gdn_status check_dims(const gdn_dims* d, const char* fn) {
  if (!d) return fail(GDN_ERR_NULL, "%s: dims is NULL", fn);
  if (d->struct_size != static_cast<int32_t>(sizeof(gdn_dims)))
    return fail(GDN_ERR_SHAPE, "%s: dims->struct_size is %d, expected %d", fn, d->struct_size,
                static_cast<int>(sizeof(gdn_dims)));
  if (d->num_k_heads < 1 || d->num_v_heads < 1)
    return fail(GDN_ERR_SHAPE, "%s: head counts must be >= 1 (Hk=%d, Hv=%d)", fn, d->num_k_heads, d->num_v_heads);
  if (d->num_v_heads % d->num_k_heads != 0)
    return fail(GDN_ERR_SHAPE, "%s: num_v_heads (%d) must be a multiple of num_k_heads (%d)", fn, d->num_v_heads,
                d->num_k_heads);
  if (d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128)
    return fail(GDN_ERR_UNSUPPORTED, "%s: head_dim %d not built (32, 64, 128)", fn, d->head_dim);
  if (d->conv_width < 2 || d->conv_width > 4)
    return fail(GDN_ERR_UNSUPPORTED, "%s: conv_width %d not built (2, 3, 4)", fn, d->conv_width);
  if (d->chunk_size != 16 && d->chunk_size != 32 && d->chunk_size != 64)
    return fail(GDN_ERR_UNSUPPORTED, "%s: chunk_size %d not built (16, 32, 64)", fn, d->chunk_size);
  if (d->activation != GDN_ACT_NONE && d->activation != GDN_ACT_SILU)
    return fail(GDN_ERR_DTYPE, "%s: unknown activation %d", fn, d->activation);
  if (d->in_dtype != GDN_F32 && d->in_dtype != GDN_BF16)
    return fail(GDN_ERR_DTYPE, "%s: unknown in_dtype %d", fn, d->in_dtype);
  if (d->mma != GDN_MMA_AUTO && d->mma != GDN_MMA_FP32 && d->mma != GDN_MMA_BF16X3)
    return fail(GDN_ERR_DTYPE, "%s: unknown mma policy %d", fn, d->mma);
  if (d->prefill_form != GDN_PREFILL_AUTO && d->prefill_form != GDN_PREFILL_WHOLE &&
      d->prefill_form != GDN_PREFILL_SEGMENTS)
    return fail(GDN_ERR_DTYPE, "%s: unknown prefill_form %d", fn, d->prefill_form);
  if (d->out_dtype != GDN_F32 && d->out_dtype != GDN_BF16)
    return fail(GDN_ERR_DTYPE, "%s: unknown out_dtype %d", fn, d->out_dtype);
  if (d->qk_l2norm_off != 0 && d->qk_l2norm_off != 1)
    return fail(GDN_ERR_DTYPE, "%s: qk_l2norm_off must be 0 or 1 (got %d)", fn, d->qk_l2norm_off);
  if (!(d->l2_eps >= 0.0f) || !(d->l2_eps < 1e30f))
    return fail(GDN_ERR_SHAPE, "%s: l2_eps must be finite and >= 0", fn);
  if (!(d->scale == d->scale) || d->scale > 1e30f || d->scale < -1e30f || d->scale == 0.0f)
    return fail(GDN_ERR_SHAPE, "%s: scale must be finite and nonzero (1.0 = no scaling)", fn);
  const int64_t C = static_cast<int64_t>(d->head_dim) * (2 * d->num_k_heads + d->num_v_heads);
  if (C > (1 << 24)) return fail(GDN_ERR_SHAPE, "%s: channel count %lld too large", fn, static_cast<long long>(C));
  return GDN_OK;
}

int64_t channels(const gdn_dims* d) {
  return static_cast<int64_t>(d->head_dim) * (2 * d->num_k_heads + d->num_v_heads);
}

// q/k/v of the recurrence entry points.
gdn_status check_qkv(const gdn_dims* d, const char* fn, const float* q, int64_t qs, const float* k, int64_t ks,
                     const float* v, int64_t vs, const float* g, const float* beta, const void* o, int32_t rows) {
  if (!q || !k || !v || !g || !beta || !o) return fail(GDN_ERR_NULL, "%s: q, k, v, g, beta and o are required", fn);
  const int64_t qk_w = static_cast<int64_t>(d->num_k_heads) * d->head_dim;
  const int64_t v_w = static_cast<int64_t>(d->num_v_heads) * d->head_dim;
  if (rows > 1 && (qs < qk_w || ks < qk_w || vs < v_w))
    return fail(GDN_ERR_SHAPE, "%s: row strides (q %lld, k %lld, v %lld) below row widths (%lld, %lld)", fn,
                static_cast<long long>(qs), static_cast<long long>(ks), static_cast<long long>(vs),
                static_cast<long long>(qk_w), static_cast<long long>(v_w));
  if (qs < 0 || ks < 0 || vs < 0) return fail(GDN_ERR_SHAPE, "%s: negative stride", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (qs % 4) || (ks % 4) || (vs % 4))
    return fail(GDN_ERR_ALIGN, "%s: q, k, v must be 16-byte aligned with strides a multiple of 4 elements", fn);
  return GDN_OK;
}

// the fused prefill's workspace: the chunked prefill's, then the v part of the conv output
size_t fused_prefill_bytes(const gdn_dims* d, int32_t num_seqs, int32_t total_tokens) {
  const size_t pre = gdn::prefill_workspace_bytes(d->num_k_heads, d->num_v_heads, d->head_dim, d->chunk_size,
                                                  num_seqs, total_tokens, d->prefill_form);
  const size_t yv = static_cast<size_t>(total_tokens) * d->num_v_heads * d->head_dim * sizeof(float);
  return pre + ((yv + 255) & ~static_cast<size_t>(255));
}

int resolve_mma(const gdn_dims* d) {
  if (d->mma != GDN_MMA_AUTO) return d->mma;
  return d->in_dtype == GDN_F32 ? GDN_MMA_FP32 : GDN_MMA_BF16X3;
}

// gdn_prefill_fused's checks and launches, for it and for gdn_prefill_fused_static
// (whose workspace is the library's own device array); fn names the caller in errors.
// launch = false: the host checks only (the workspace pointer is then never used).
gdn_status prefill_fused_impl(const char* fn, const gdn_dims* dims, const void* x, int64_t x_stride,
                              const void* conv_w, const void* conv_b, const float* g, const float* beta, void* o,
                              const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                              const uint64_t* state_ptrs, const uint64_t* conv_state_ptrs, void* workspace,
                              size_t workspace_bytes, void* stream, bool launch = true) {
  if (gdn_status st = check_dims(dims, fn)) return st;
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_ERR_SHAPE, "%s: negative count", fn);
  if (num_seqs == 0) {
    if (total_tokens != 0) return fail(GDN_ERR_SHAPE, "%s: tokens without sequences", fn);
    return GDN_OK;
  }
  if (!cu_seqlens || !state_ptrs || !conv_state_ptrs)
    return fail(GDN_ERR_NULL, "%s: cu_seqlens, state_ptrs and conv_state_ptrs are required", fn);
  const int64_t C = channels(dims);
  const int64_t esz = dims->in_dtype == GDN_BF16 ? 2 : 4;
  const int64_t qk = 2 * static_cast<int64_t>(dims->num_k_heads) * dims->head_dim;  // q | k channels
  const int64_t vw = static_cast<int64_t>(dims->num_v_heads) * dims->head_dim;
  if (total_tokens > 0) {
    if (!x || !conv_w || !g || !beta || !o)
      return fail(GDN_ERR_NULL, "%s: x, conv_w, g, beta and o are required", fn);
    if (x_stride < 0) return fail(GDN_ERR_SHAPE, "%s: negative stride", fn);
    if (total_tokens > 1 && x_stride < C)
      return fail(GDN_ERR_SHAPE, "%s: x row stride %lld below the channel count %lld", fn,
                  static_cast<long long>(x_stride), static_cast<long long>(C));
    if (!aligned16(x) || !aligned16(conv_w) || (conv_b && !aligned16(conv_b)) || (x_stride * esz) % 16)
      return fail(GDN_ERR_ALIGN, "%s: x, conv_w, conv_b must be 16-byte aligned and x_stride a multiple of 16 bytes",
                  fn);
  }
  const size_t pre = gdn::prefill_workspace_bytes(dims->num_k_heads, dims->num_v_heads, dims->head_dim,
                                                  dims->chunk_size, num_seqs, total_tokens, dims->prefill_form);
  const size_t need = fused_prefill_bytes(dims, num_seqs, total_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given%s", fn, need, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(GDN_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  if (total_tokens == 0 || !launch) return GDN_OK;  // (zero-length sequences only: nothing changes)
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* yv = reinterpret_cast<float*>(static_cast<char*>(workspace) + pre);  // v part of the conv output
  const int K = dims->conv_width;
  const bool silu = dims->activation == GDN_ACT_SILU, bf16 = dims->in_dtype == GDN_BF16;
  const char* xb = static_cast<const char*>(x);
  const char* wb = static_cast<const char*>(conv_w);
  const char* bb = static_cast<const char*>(conv_b);
  // the v channels' conv into the workspace (run by launch_prefill where the inter-chunk
  // kernel does not convolve v itself); the conv states are committed inside the prefill
  gdn::ConvArgs cv{xb + qk * esz, x_stride, yv, vw, wb + qk * K * esz, bb ? bb + qk * esz : nullptr, cu_seqlens,
                   conv_state_ptrs, num_seqs, total_tokens, static_cast<int32_t>(vw), K, silu, bf16, C,
                   static_cast<int32_t>(qk)};
  // the chunked prefill, the q/k conv inside its intra-chunk kernel
  gdn::PrefillArgs a{};
  a.r = gdn::RecurArgs{nullptr, 0, nullptr, 0, yv, vw, g, beta, o, state_ptrs, dims->num_k_heads,
                       dims->num_v_heads, dims->head_dim, dims->l2_eps, dims->scale,
                       dims->out_dtype == GDN_BF16, dims->qk_l2norm_off == 0,
                       dims->num_v_heads / dims->num_k_heads};
  a.conv = gdn::ConvIn{x, x_stride, conv_w, conv_b, conv_state_ptrs, static_cast<int32_t>(C), K, silu, bf16};
  a.vconv = cv;
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.chunk = dims->chunk_size;
  a.form = dims->prefill_form;
  a.mma = resolve_mma(dims);
  a.workspace = workspace;
  // (the conv states are committed by the last readers of their old rows: the q/k
  // channels by the intra-chunk kernel's chunk-0 workgroups, the v channels by the
  // inter-chunk kernel where it convolves v, else by the intra-chunk kernel too)
  return hip_status(gdn::launch_prefill(a, s), fn);
}

// The workspace of gdn_prefill_fused_static: a file-scope device array, one per GPU the
// library runs on, held until the process ends (64 MiB: the workspace of about 1280 tokens
// of a 16 q/k-head, 32 v-head, d = 128 layer, 48 KiB per token). Its device address on
// each GPU is looked up once, with that GPU current, and kept; host code never uses the
// array's own name as an address. Every call on a GPU uses the same array, so calls on one
// GPU must not overlap in time (one stream, or streams ordered by events); the prefill
// reads nothing from its workspace that it has not written in the same call, so nothing
// needs clearing between calls.
constexpr size_t kStaticScratchBytes = GDN_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the scratch array's device address on the GPU that `stream` runs on
gdn_status static_scratch(hipStream_t stream, const char* fn, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(GDN_ERR_HIP, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_status(e, fn);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, fn);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_status(e, fn);
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u))
      return fail(GDN_ERR_HIP, "%s: static scratch address %p unusable", fn, p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_last_error(void) { return g_last_error.c_str(); }

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

gdn_status gdn_dims_init(gdn_dims* dims, int32_t num_k_heads, int32_t num_v_heads, int32_t head_dim) {
  if (!dims) return fail(GDN_ERR_NULL, "gdn_dims_init: dims is NULL");
  gdn_dims d{};
  d.struct_size = static_cast<int32_t>(sizeof(gdn_dims));
  d.num_k_heads = num_k_heads;
  d.num_v_heads = num_v_heads;
  d.head_dim = head_dim;
  d.conv_width = 4;
  d.chunk_size = 64;
  d.activation = GDN_ACT_NONE;
  d.in_dtype = GDN_F32;
  d.mma = GDN_MMA_AUTO;
  d.l2_eps = 1e-6f;
  d.scale = 1.0f;
  d.prefill_form = GDN_PREFILL_AUTO;
  d.out_dtype = GDN_F32;
  d.qk_l2norm_off = 0;
  *dims = d;
  return GDN_OK;
}

gdn_status gdn_conv_update(const gdn_dims* dims, const void* x, int64_t x_stride, float* y, int64_t y_stride,
                           const void* conv_w, const void* conv_b, const int32_t* cu_seqlens,
                           const uint64_t* conv_state_ptrs, int32_t n, int32_t total_tokens, void* stream) {
  const char* fn = "gdn_conv_update";
  if (gdn_status st = check_dims(dims, fn)) return st;
  if (n < 0 || total_tokens < 0) return fail(GDN_ERR_SHAPE, "%s: negative n or total_tokens", fn);
  const bool decode = cu_seqlens == nullptr;
  if (decode && total_tokens != n)
    return fail(GDN_ERR_SHAPE, "%s: decode mode (cu_seqlens NULL) needs total_tokens == n (%d vs %d)", fn,
                total_tokens, n);
  if (!decode && n == 0 && total_tokens != 0)
    return fail(GDN_ERR_SHAPE, "%s: tokens without sequences", fn);
  if (total_tokens == 0 && n == 0) return GDN_OK;
  if (!x || !y || !conv_w || !conv_state_ptrs)
    return fail(GDN_ERR_NULL, "%s: x, y, conv_w and conv_state_ptrs are required", fn);
  const int64_t C = channels(dims);
  const int64_t esz = dims->in_dtype == GDN_BF16 ? 2 : 4;
  if (total_tokens > 1 && (x_stride < C || y_stride < C))
    return fail(GDN_ERR_SHAPE, "%s: row strides (x %lld, y %lld) below channel count %lld", fn,
                static_cast<long long>(x_stride), static_cast<long long>(y_stride), static_cast<long long>(C));
  if (x_stride < 0 || y_stride < 0) return fail(GDN_ERR_SHAPE, "%s: negative stride", fn);
  if (!aligned16(x) || !aligned16(y) || !aligned16(conv_w) || (conv_b && !aligned16(conv_b)) ||
      (x_stride * esz) % 16 || (y_stride * 4) % 16)
    return fail(GDN_ERR_ALIGN, "%s: x, y, conv_w, conv_b must be 16-byte aligned and row strides multiples of 16 bytes",
                fn);
  gdn::ConvArgs a{x, x_stride, y, y_stride, conv_w, conv_b, cu_seqlens, conv_state_ptrs, n, total_tokens,
                  static_cast<int32_t>(C), dims->conv_width, dims->activation == GDN_ACT_SILU,
                  dims->in_dtype == GDN_BF16, C, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(decode ? gdn::launch_conv_decode(a, s) : gdn::launch_conv_prefill(a, s), fn);
}

gdn_status gdn_prefill_workspace_size(const gdn_dims* dims, int32_t num_seqs, int32_t total_tokens, size_t* bytes) {
  const char* fn = "gdn_prefill_workspace_size";
  if (gdn_status st = check_dims(dims, fn)) return st;
  if (!bytes) return fail(GDN_ERR_NULL, "%s: bytes is NULL", fn);
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_ERR_SHAPE, "%s: negative count", fn);
  *bytes = gdn::prefill_workspace_bytes(dims->num_k_heads, dims->num_v_heads, dims->head_dim, dims->chunk_size, num_seqs,
                                      total_tokens, dims->prefill_form);
  return GDN_OK;
}

gdn_status gdn_prefill_chunked(const gdn_dims* dims, const float* q, int64_t q_stride, const float* k,
                               int64_t k_stride, const float* v, int64_t v_stride, const float* g,
                               const float* beta, void* o, const int32_t* cu_seqlens, int32_t num_seqs,
                               int32_t total_tokens, const uint64_t* state_ptrs, void* workspace,
                               size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_prefill_chunked";
  if (gdn_status st = check_dims(dims, fn)) return st;
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_ERR_SHAPE, "%s: negative count", fn);
  if (num_seqs == 0) {
    if (total_tokens != 0) return fail(GDN_ERR_SHAPE, "%s: tokens without sequences", fn);
    return GDN_OK;
  }
  if (!cu_seqlens || !state_ptrs) return fail(GDN_ERR_NULL, "%s: cu_seqlens and state_ptrs are required", fn);
  if (total_tokens > 0) {
    if (gdn_status st = check_qkv(dims, fn, q, q_stride, k, k_stride, v, v_stride, g, beta, o, total_tokens))
      return st;
  }
  const size_t need =
      gdn::prefill_workspace_bytes(dims->num_k_heads, dims->num_v_heads, dims->head_dim, dims->chunk_size, num_seqs,
                                      total_tokens, dims->prefill_form);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given%s", fn, need, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(GDN_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  gdn::PrefillArgs a{};
  a.r = gdn::RecurArgs{q, q_stride, k, k_stride, v, v_stride, g, beta, o, state_ptrs, dims->num_k_heads,
                       dims->num_v_heads, dims->head_dim, dims->l2_eps, dims->scale,
                       dims->out_dtype == GDN_BF16, dims->qk_l2norm_off == 0,
                       dims->num_v_heads / dims->num_k_heads};
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.chunk = dims->chunk_size;
  a.form = dims->prefill_form;
  a.mma = resolve_mma(dims);
  a.workspace = workspace;
  return hip_status(gdn::launch_prefill(a, static_cast<hipStream_t>(stream)), fn);
}

gdn_status gdn_prefill_fused_workspace_size(const gdn_dims* dims, int32_t num_seqs, int32_t total_tokens,
                                            size_t* bytes) {
  const char* fn = "gdn_prefill_fused_workspace_size";
  if (gdn_status st = check_dims(dims, fn)) return st;
  if (!bytes) return fail(GDN_ERR_NULL, "%s: bytes is NULL", fn);
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_ERR_SHAPE, "%s: negative count", fn);
  *bytes = fused_prefill_bytes(dims, num_seqs, total_tokens);
  return GDN_OK;
}

gdn_status gdn_prefill_fused(const gdn_dims* dims, const void* x, int64_t x_stride, const void* conv_w,
                             const void* conv_b, const float* g, const float* beta, void* o,
                             const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                             const uint64_t* state_ptrs, const uint64_t* conv_state_ptrs, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return prefill_fused_impl("gdn_prefill_fused", dims, x, x_stride, conv_w, conv_b, g, beta, o, cu_seqlens, num_seqs,
                            total_tokens, state_ptrs, conv_state_ptrs, workspace, workspace_bytes, stream);
}

gdn_status gdn_prefill_fused_static(const gdn_dims* dims, const void* x, int64_t x_stride, const void* conv_w,
                                    const void* conv_b, const float* g, const float* beta, void* o,
                                    const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                                    const uint64_t* state_ptrs, const uint64_t* conv_state_ptrs, void* stream) {
  const char* fn = "gdn_prefill_fused_static";
  if (gdn_status st = check_dims(dims, fn)) return st;
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_ERR_SHAPE, "%s: negative count", fn);
  if (num_seqs == 0) {
    if (total_tokens != 0) return fail(GDN_ERR_SHAPE, "%s: tokens without sequences", fn);
    return GDN_OK;
  }
  const size_t need = fused_prefill_bytes(dims, num_seqs, total_tokens);
  if (need > kStaticScratchBytes)
    return fail(GDN_ERR_WORKSPACE,
                "%s: %d sequences of %d tokens need %zu bytes of workspace, above the library's static %zu "
                "(split the batch, or pass a workspace to gdn_prefill_fused)",
                fn, num_seqs, total_tokens, need, kStaticScratchBytes);
  // every host check first (a stand-in for the array's address: 256-byte aligned, never used)
  void* ws = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  if (gdn_status st = prefill_fused_impl(fn, dims, x, x_stride, conv_w, conv_b, g, beta, o, cu_seqlens, num_seqs,
                                         total_tokens, state_ptrs, conv_state_ptrs, ws, kStaticScratchBytes, stream,
                                         false))
    return st;
  if (total_tokens == 0) return GDN_OK;
  if (gdn_status st = static_scratch(static_cast<hipStream_t>(stream), fn, &ws)) return st;
  return prefill_fused_impl(fn, dims, x, x_stride, conv_w, conv_b, g, beta, o, cu_seqlens, num_seqs, total_tokens,
                            state_ptrs, conv_state_ptrs, ws, kStaticScratchBytes, stream);
}

gdn_status gdn_decode_batched(const gdn_dims* dims, const float* q, int64_t q_stride, const float* k,
                              int64_t k_stride, const float* v, int64_t v_stride, const float* g,
                              const float* beta, void* o, const uint64_t* state_ptrs, int32_t m, void* stream) {
  const char* fn = "gdn_decode_batched";
  if (gdn_status st = check_dims(dims, fn)) return st;
  if (m < 0) return fail(GDN_ERR_SHAPE, "%s: negative m", fn);
  if (m == 0) return GDN_OK;
  if (m > 65535) return fail(GDN_ERR_SHAPE, "%s: m = %d above the grid limit 65535", fn, m);
  if (!state_ptrs) return fail(GDN_ERR_NULL, "%s: state_ptrs is required", fn);
  if (gdn_status st = check_qkv(dims, fn, q, q_stride, k, k_stride, v, v_stride, g, beta, o, m)) return st;
  gdn::RecurArgs a{q, q_stride, k, k_stride, v, v_stride, g, beta, o, state_ptrs, dims->num_k_heads,
                   dims->num_v_heads, dims->head_dim, dims->l2_eps, dims->scale,
                       dims->out_dtype == GDN_BF16, dims->qk_l2norm_off == 0,
                       dims->num_v_heads / dims->num_k_heads};
  return hip_status(gdn::launch_decode(a, m, static_cast<hipStream_t>(stream)), fn);
}

gdn_status gdn_decode_fused(const gdn_dims* dims, const void* x, int64_t x_stride, const void* conv_w,
                            const void* conv_b, const float* g, const float* beta, void* o,
                            const uint64_t* state_ptrs, const uint64_t* conv_state_ptrs,
                            const uint64_t* conv_state_out_ptrs, int32_t m, void* stream) {
  const char* fn = "gdn_decode_fused";
  if (gdn_status st = check_dims(dims, fn)) return st;
  if (m < 0) return fail(GDN_ERR_SHAPE, "%s: negative m", fn);
  if (m == 0) return GDN_OK;
  if (!x || !conv_w || !g || !beta || !o || !state_ptrs || !conv_state_ptrs)
    return fail(GDN_ERR_NULL, "%s: x, conv_w, g, beta, o, state_ptrs and conv_state_ptrs are required", fn);
  const int64_t C = channels(dims);
  const int64_t esz = dims->in_dtype == GDN_BF16 ? 2 : 4;
  if (x_stride < 0 || (m > 1 && x_stride < C))
    return fail(GDN_ERR_SHAPE, "%s: x row stride %lld below channel count %lld", fn, static_cast<long long>(x_stride),
                static_cast<long long>(C));
  if (!aligned16(x) || !aligned16(conv_w) || (conv_b && !aligned16(conv_b)) || (x_stride * esz) % 16)
    return fail(GDN_ERR_ALIGN, "%s: x, conv_w, conv_b must be 16-byte aligned and x_stride a multiple of 16 bytes", fn);
  // one workgroup per (slot, k-head) keeps the conv output of the k-head and its v-heads in LDS
  const int64_t group = dims->num_v_heads / dims->num_k_heads;
  if ((2 + group) * dims->head_dim * 4 > 65536)
    return fail(GDN_ERR_UNSUPPORTED, "%s: %lld v-heads per k-head at head_dim %d exceed one workgroup's LDS", fn,
                static_cast<long long>(group), dims->head_dim);
  if (m > 65535) return fail(GDN_ERR_SHAPE, "%s: m = %d above the grid limit 65535", fn, m);
  gdn::FusedArgs f{};
  f.r = gdn::RecurArgs{nullptr, 0, nullptr, 0, nullptr, 0, g, beta, o, state_ptrs, dims->num_k_heads,
                       dims->num_v_heads, dims->head_dim, dims->l2_eps, dims->scale,
                       dims->out_dtype == GDN_BF16, dims->qk_l2norm_off == 0,
                       dims->num_v_heads / dims->num_k_heads};
  f.x = x;
  f.x_stride = x_stride;
  f.w = conv_w;
  f.b = conv_b;
  f.conv_ptrs = conv_state_ptrs;
  f.conv_out_ptrs = conv_state_out_ptrs ? conv_state_out_ptrs : conv_state_ptrs;
  f.channels = static_cast<int32_t>(C);
  f.width = dims->conv_width;
  f.silu = dims->activation == GDN_ACT_SILU;
  f.bf16 = dims->in_dtype == GDN_BF16;
  return hip_status(gdn::launch_decode_fused(f, m, static_cast<hipStream_t>(stream)), fn);
}

gdn_status gdn_slot_copy(const gdn_dims* dims, const uint64_t* src_state_ptrs, const uint64_t* dst_state_ptrs,
                         const uint64_t* src_conv_ptrs, const uint64_t* dst_conv_ptrs, int32_t n, void* stream) {
  const char* fn = "gdn_slot_copy";
  if (gdn_status st = check_dims(dims, fn)) return st;
  if (n < 0) return fail(GDN_ERR_SHAPE, "%s: negative n", fn);
  if ((src_state_ptrs == nullptr) != (dst_state_ptrs == nullptr) ||
      (src_conv_ptrs == nullptr) != (dst_conv_ptrs == nullptr))
    return fail(GDN_ERR_NULL, "%s: source and destination pointer arrays come in pairs (both or neither)", fn);
  if (n == 0) return GDN_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t d = dims->head_dim;
  const int64_t channels = d * (2 * static_cast<int64_t>(dims->num_k_heads) + dims->num_v_heads);
  if (src_state_ptrs) {
    const int64_t bytes = static_cast<int64_t>(dims->num_v_heads) * d * d * 4;
    if (gdn_status st = hip_status(gdn::launch_slot_copy(src_state_ptrs, dst_state_ptrs, bytes, n, s), fn)) return st;
  }
  if (src_conv_ptrs) {
    const int64_t elt = dims->in_dtype == GDN_BF16 ? 2 : 4;
    const int64_t bytes = (dims->conv_width - 1) * channels * elt;
    if (gdn_status st = hip_status(gdn::launch_slot_copy(src_conv_ptrs, dst_conv_ptrs, bytes, n, s), fn)) return st;
  }
  return GDN_OK;
}

gdn_status gdn_slot_pointers(uint64_t pool_base, int64_t slot_bytes, int32_t pool_slots, const int32_t* slot_idx,
                             int32_t m, uint64_t* out_ptrs, void* stream) {
  const char* fn = "gdn_slot_pointers";
  if (m < 0 || pool_slots < 0 || slot_bytes <= 0) return fail(GDN_ERR_SHAPE, "%s: bad m, pool_slots or slot_bytes", fn);
  if (m == 0) return GDN_OK;
  if (!pool_base || !slot_idx || !out_ptrs) return fail(GDN_ERR_NULL, "%s: pool_base, slot_idx, out_ptrs required", fn);
  if ((pool_base & 15u) || (slot_bytes & 15))
    return fail(GDN_ERR_ALIGN, "%s: pool_base and slot_bytes must be multiples of 16", fn);
  return hip_status(
      gdn::launch_slot_pointers(pool_base, slot_bytes, pool_slots, slot_idx, m, out_ptrs, static_cast<hipStream_t>(stream)),
      fn);
}

}  // extern "C"
