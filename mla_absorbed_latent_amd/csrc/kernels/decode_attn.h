// decode_attn.h -- launcher interface of the split-KV decode kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../../include/mla.h"

namespace mla {

struct DecodeArgs {
  const uint16_t* q_abs;        // [batch][H][576] fp16
  const uint8_t* pool;          // num_pages pages
  int64_t num_pages;
  const int32_t* block_table;   // [batch][max_pages]
  int32_t max_pages;
  const int32_t* seq_lens;      // [batch]
  const mla_work_item* items;   // [n_items]
  int32_t n_items;
  uint16_t* o_part;             // [rows][H][512] fp16
  float* lse_part;              // [rows][H]
  int32_t batch;
  float scale_log2;             // softmax_scale * log2(e)
};

hipError_t launch_decode_attn(const DecodeArgs& a, int num_heads, int cache_dtype, hipStream_t stream);

}  // namespace mla
