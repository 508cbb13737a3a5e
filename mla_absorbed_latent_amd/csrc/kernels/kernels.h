// kernels.h -- launcher interfaces of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_attn.h"

namespace mla {

hipError_t launch_append(int cache_dtype, void* pool, int64_t num_pages, const uint16_t* c_kv,
                         const uint16_t* k_pe, const int64_t* slots, int n, hipStream_t stream);

hipError_t launch_absorb_q(int num_heads, const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_uk,
                           uint16_t* q_abs, int batch, hipStream_t stream);

// One launch for a bf16 cache (append work-groups after the absorb grid);
// launch_append then launch_absorb_q for the other formats.
hipError_t launch_append_absorb(int cache_dtype, void* pool, int64_t num_pages, const uint16_t* c_kv,
                                const uint16_t* k_pe, const int64_t* slots, int n_new, int num_heads,
                                const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_uk, uint16_t* q_abs,
                                int batch, hipStream_t stream);

hipError_t launch_combine(int num_heads, const uint16_t* o_part, const float* lse_part, const int32_t* split_offsets,
                          float* o_lat, float* lse, int batch, hipStream_t stream);

hipError_t launch_out_proj(int num_heads, const float* o_lat, const uint16_t* w_uv, uint16_t* out,
                           float* out_f32, int batch, hipStream_t stream);

hipError_t launch_combine_out_proj(int num_heads, const uint16_t* o_part, const float* lse_part,
                                  const int32_t* split_offsets, const uint16_t* w_uv, uint16_t* out, float* out_f32,
                                  float* o_lat, float* lse, int batch, hipStream_t stream);
hipError_t launch_wo_proj(int in_features, const float* x, const uint16_t* w_o, int hidden, uint16_t* y,
                          int batch, hipStream_t stream);

hipError_t launch_layer_front(int num_heads, const uint16_t* x, int hidden, const uint16_t* w_q, const uint16_t* w_dkv,
                              const int32_t* positions, float rms_eps, float rope_base, float* workspace,
                              uint16_t* q_nope, uint16_t* q_pe, uint16_t* c_kv, uint16_t* k_pe, int n_tokens,
                              hipStream_t stream);

// launch_layer_front, and each token's row written into its cache slot in the
// format cache_dtype by the same launch (the per-channel INT8 format runs its
// usual two append launches after the front instead).
hipError_t launch_layer_front_append(int num_heads, const uint16_t* x, int hidden, const uint16_t* w_q,
                                     const uint16_t* w_dkv, const int32_t* positions, float rms_eps, float rope_base,
                                     float* workspace, uint16_t* q_nope, uint16_t* q_pe, uint16_t* c_kv,
                                     uint16_t* k_pe, int cache_dtype, void* pool, int64_t num_pages,
                                     const int64_t* slots, int n_tokens, hipStream_t stream);

// launch_layer_front with the fp32 projections in the library's per-device
// scratch (kFrontScratchBytes) instead of a caller workspace; allocates nothing.
constexpr size_t kFrontScratchBytes = size_t(16) << 20;
hipError_t launch_layer_front_noalloc(int num_heads, const uint16_t* x, int hidden, const uint16_t* w_q,
                                      const uint16_t* w_dkv, const int32_t* positions, float rms_eps,
                                      float rope_base, uint16_t* q_nope, uint16_t* q_pe, uint16_t* c_kv,
                                      uint16_t* k_pe, int n_tokens, hipStream_t stream);

hipError_t launch_out_residual(int num_heads, const uint16_t* attn_out, const uint16_t* w_o, int hidden,
                               const uint16_t* x_in, uint16_t* x_out, float* workspace, int n_tokens,
                               hipStream_t stream);

// Workspace of launch_prefill_attn: K_nope [H][Lp][128] and V^T [H][128][Lp]
// fp16, Lp = seq_len rounded up to 64.
int64_t prefill_padded_len(int seq_len);
hipError_t launch_prefill_attn(int num_heads, float softmax_scale, const uint16_t* q_nope, const uint16_t* q_pe,
                               int n_queries, const uint16_t* c_kv, const uint16_t* k_pe, int seq_len,
                               const uint16_t* w_uk, const uint16_t* w_uv, void* workspace, uint16_t* out,
                               float* lse, hipStream_t stream);

}  // namespace mla
