// Internal launcher interface between the C-ABI layer (gdn_api.cpp) and the kernels.
// Launchers assume their arguments were validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct ConvArgs {
  const void* x;
  int64_t x_stride;
  float* y;
  int64_t y_stride;
  const void* w;
  const void* b;  // nullable
  const int32_t* cu_seqlens;  // nullable (decode mode)
  const uint64_t* state_ptrs;
  int32_t n;
  int32_t total_tokens;
  int32_t channels;
  int32_t width;  // K
  int32_t silu;
  int32_t bf16;  // in_dtype == BF16
  // prefill mode: conv state row r of a slot, channel c (of the `channels` processed) is
  // element r * state_stride + state_off + c (all channels: channels, 0)
  int64_t state_stride;
  int32_t state_off;
};

hipError_t launch_conv_prefill(const ConvArgs& a, hipStream_t s);  // conv, then the conv-state commit
hipError_t launch_conv_prefill_only(const ConvArgs& a, hipStream_t s);
hipError_t launch_conv_decode(const ConvArgs& a, hipStream_t s);

struct RecurArgs {
  const float* q;
  int64_t q_stride;
  const float* k;
  int64_t k_stride;
  const float* v;
  int64_t v_stride;
  const float* g;
  const float* beta;
  void* o;  // fp32, or bf16 when o_bf16
  const uint64_t* state_ptrs;
  int32_t hk;
  int32_t hv;
  int32_t d;
  float eps;
  float scale;
  int32_t o_bf16;   // o holds the fp32 results rounded to bf16 (nearest even)
  int32_t qk_norm;  // q and k L2-normalised (else used as given; q still times scale)
  int32_t group;    // hv / hk: v-heads per k-head
};

hipError_t launch_decode(const RecurArgs& a, int32_t m, hipStream_t s);

// Conv + decode in one launch (r.q, r.k, r.v unused).
struct FusedArgs {
  RecurArgs r;
  const void* x;
  int64_t x_stride;
  const void* w;
  const void* b;  // nullable
  const uint64_t* conv_ptrs;      // old conv state per slot (read)
  const uint64_t* conv_out_ptrs;  // new conv state per slot: conv_ptrs itself (in place) or other buffers
  int32_t channels;
  int32_t width;
  int32_t silu;
  int32_t bf16;
};

hipError_t launch_decode_fused(const FusedArgs& f, int32_t m, hipStream_t s);

// The depthwise conv of the q and k channels, computed inside the prefill (fused entry
// point); x == nullptr: q and k are read from RecurArgs instead.
struct ConvIn {
  const void* x;
  int64_t x_stride;
  const void* w;
  const void* b;                 // nullable
  const uint64_t* state_ptrs;    // per sequence, [K-1][channels] in the input dtype
  int32_t channels;              // all channels (2 Hk + Hv) d: the row length of a conv state
  int32_t width;
  int32_t silu;
  int32_t bf16;
};

struct PrefillArgs {
  RecurArgs r;
  ConvIn conv;
  // Fused entry point only (conv.x != nullptr): the conv of the v channels into r.v, which
  // launch_prefill runs as a kernel of its own unless the inter-chunk kernel convolves v
  // itself (whole sequences, 64-token chunks).
  ConvArgs vconv;
  int32_t v_in_inter;  // set by launch_prefill
  int32_t table_free;  // set by launch_prefill: no chunk-table launch (the intra-chunk kernel finds its chunks)
  const int32_t* cu_seqlens;
  int32_t num_seqs;
  int32_t total_tokens;
  int32_t chunk;
  int32_t mma;  // 1 = fp32, 2 = bf16x3 (resolved)
  int32_t form;  // gdn_prefill_form
  void* workspace;
};

size_t prefill_workspace_bytes(int32_t hk, int32_t hv, int32_t d, int32_t chunk, int32_t num_seqs,
                               int32_t total_tokens, int32_t form);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

hipError_t launch_slot_copy(const uint64_t* src, const uint64_t* dst, int64_t bytes, int32_t n, hipStream_t s);

hipError_t launch_slot_pointers(uint64_t base, int64_t slot_bytes, int32_t pool_slots, const int32_t* idx,
                                int32_t m, uint64_t* out, hipStream_t s);

}  // namespace gdn
