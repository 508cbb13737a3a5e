// api.cpp -- the C ABI declared in include/mla.h: argument validation, the
// gfx950 check, and dispatch to the kernels.  Validation happens entirely on
// the host before any HIP call, so a rejected call has no side effects.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../../include/mla.h"
#include "../kernels/kernels.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch_state[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mla_status hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int32_t>(e);
  return MLA_ERR_HIP;
}

// Checks that the current device is gfx950 (cached per device).
mla_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? MLA_OK : MLA_ERR_UNSUPPORTED;
}

mla_status launched(hipError_t e) { return e == hipSuccess ? MLA_OK : hip_fail(e); }

// Widest block-table row mla_decode_attn accepts: 2^24 pages (2^30 tokens), so
// that every token index a kernel forms, look-ahead tiles included, stays below
// 2^31.
constexpr int32_t kMaxPagesPerSeq = 1 << 24;

}  // namespace

extern "C" {

mla_status mla_config_check(const mla_config* cfg) {
  if (cfg == nullptr) return MLA_ERR_NULL;
  if (cfg->num_heads != 16 && cfg->num_heads != 128) return MLA_ERR_SHAPE;
  if (cfg->qk_nope_dim != 128 || cfg->kv_lora_rank != 512 || cfg->rope_dim != 64 || cfg->v_head_dim != 128 ||
      cfg->block_size != 64)
    return MLA_ERR_SHAPE;
  if (cfg->cache_dtype < MLA_CACHE_BF16 || cfg->cache_dtype > MLA_CACHE_INT8_CHAN) return MLA_ERR_VALUE;
  if (!(cfg->softmax_scale > 0.f) || !std::isfinite(cfg->softmax_scale)) return MLA_ERR_VALUE;
  return MLA_OK;
}

size_t mla_cache_bytes_per_token(const mla_config* cfg) {
  if (mla_config_check(cfg) != MLA_OK) return 0;
  switch (cfg->cache_dtype) {
    case MLA_CACHE_BF16: return 576 * 2;                       // latent + RoPE key, bf16
    case MLA_CACHE_INT8: return 576 + 16 * 4 + 8 * 4;          // codes + latent scales + key scales
    case MLA_CACHE_INT4: return 256 + 64 + 16 * 4 + 16 * 4 + 8 * 4;   // nibbles + key codes + scales + zeros + key scales
    case MLA_CACHE_INT4_SYM: return 256 + 64 + 16 * 4 + 8 * 4;          // nibbles + key codes + scales + key scales
    case MLA_CACHE_INT4_SYM_K4: return 256 + 32 + 16 * 4 + 8 * 4;       // nibbles + key nibbles + scales + key scales
    case MLA_CACHE_INT8_CHAN: return 512 + 64 + 512 * 4 / 32 + 8 * 4;   // codes + key codes + block scales / 32 + key scales
    default: return 576 + 4 + 8 * 4;                           // codes + the token's latent scale + key scales
  }
}

size_t mla_cache_page_bytes(const mla_config* cfg) {
  if (mla_config_check(cfg) != MLA_OK) return 0;
  // the per-channel block format also holds the open block's bf16 rows (overflow [32][512 B])
  if (cfg->cache_dtype == MLA_CACHE_INT8_CHAN) return 64 * (512 + 64 + 8 * 4) + 2 * 512 * 4 + 32 * 512;
  return 64 * mla_cache_bytes_per_token(cfg);
}

size_t mla_decode_workspace_bytes(const mla_config* cfg, int32_t n_items) {
  if (mla_config_check(cfg) != MLA_OK || n_items < 0) return 0;
  return (size_t)n_items * cfg->num_heads * (512 * sizeof(uint16_t) + sizeof(float));
}

mla_status mla_cache_append(const mla_config* cfg, void* pool, int64_t num_pages, const uint16_t* c_kv,
                            const uint16_t* k_pe, const int64_t* slot_mapping, int32_t n_tokens,
                            hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (n_tokens < 0 || num_pages < 0) return MLA_ERR_VALUE;
  if (n_tokens == 0) return MLA_OK;
  if (!pool || !c_kv || !k_pe || !slot_mapping) return MLA_ERR_NULL;
  if (!aligned16(pool) || !aligned16(c_kv) || !aligned16(k_pe) || !aligned16(slot_mapping)) return MLA_ERR_ALIGN;
  if ((s = check_device()) != MLA_OK) return s;
  return launched(mla::launch_append(cfg->cache_dtype, pool, num_pages, c_kv, k_pe, slot_mapping, n_tokens, stream));
}

mla_status mla_absorb_q(const mla_config* cfg, const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_uk,
                        uint16_t* q_abs, int32_t batch, hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (batch < 0) return MLA_ERR_VALUE;
  if (batch == 0) return MLA_OK;
  if (!q_nope || !q_pe || !w_uk || !q_abs) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(w_uk) || !aligned16(q_abs)) return MLA_ERR_ALIGN;
  if ((s = check_device()) != MLA_OK) return s;
  return launched(mla::launch_absorb_q(cfg->num_heads, q_nope, q_pe, w_uk, q_abs, batch, stream));
}

mla_status mla_append_absorb_q(const mla_config* cfg, void* pool, int64_t num_pages, const uint16_t* c_kv,
                               const uint16_t* k_pe, const int64_t* slot_mapping, int32_t n_tokens,
                               const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_uk, uint16_t* q_abs,
                               int32_t batch, hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (n_tokens < 0 || num_pages < 0 || batch < 0) return MLA_ERR_VALUE;
  if (n_tokens > 0) {
    if (!pool || !c_kv || !k_pe || !slot_mapping) return MLA_ERR_NULL;
    if (!aligned16(pool) || !aligned16(c_kv) || !aligned16(k_pe) || !aligned16(slot_mapping)) return MLA_ERR_ALIGN;
  }
  if (batch > 0) {
    if (!q_nope || !q_pe || !w_uk || !q_abs) return MLA_ERR_NULL;
    if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(w_uk) || !aligned16(q_abs)) return MLA_ERR_ALIGN;
  }
  if (n_tokens == 0 && batch == 0) return MLA_OK;
  if ((s = check_device()) != MLA_OK) return s;
  return launched(mla::launch_append_absorb(cfg->cache_dtype, pool, num_pages, c_kv, k_pe, slot_mapping, n_tokens,
                                            cfg->num_heads, q_nope, q_pe, w_uk, q_abs, batch, stream));
}

mla_status mla_decode_attn(const mla_config* cfg, const uint16_t* q_abs, const void* pool, int64_t num_pages,
                           const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                           const mla_work_item* items, int32_t n_items, uint16_t* o_part, float* lse_part,
                           int32_t batch, hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (n_items < 0 || batch < 0 || num_pages < 0 || max_pages_per_seq < 0) return MLA_ERR_VALUE;
  if (max_pages_per_seq > kMaxPagesPerSeq) return MLA_ERR_VALUE;
  if (n_items == 0) return MLA_OK;
  if (!q_abs || !pool || !block_table || !seq_lens || !items || !o_part || !lse_part) return MLA_ERR_NULL;
  if (!aligned16(q_abs) || !aligned16(pool) || !aligned16(block_table) || !aligned16(seq_lens) ||
      !aligned16(items) || !aligned16(o_part) || !aligned16(lse_part))
    return MLA_ERR_ALIGN;
  if ((s = check_device()) != MLA_OK) return s;
  mla::DecodeArgs a;
  a.q_abs = q_abs;
  a.pool = static_cast<const uint8_t*>(pool);
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_pages = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.items = items;
  a.n_items = n_items;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.batch = batch;
  a.scale_log2 = cfg->softmax_scale * 1.4426950408889634f;
  return launched(mla::launch_decode_attn(a, cfg->num_heads, cfg->cache_dtype, stream));
}

mla_status mla_decode_combine(const mla_config* cfg, const uint16_t* o_part, const float* lse_part,
                              const int32_t* split_offsets, float* o_lat, float* lse, int32_t batch,
                              hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (batch < 0) return MLA_ERR_VALUE;
  if (batch == 0) return MLA_OK;
  if (!o_part || !lse_part || !split_offsets || !o_lat) return MLA_ERR_NULL;
  if (!aligned16(o_part) || !aligned16(lse_part) || !aligned16(split_offsets) || !aligned16(o_lat) ||
      (lse && !aligned16(lse)))
    return MLA_ERR_ALIGN;
  if ((s = check_device()) != MLA_OK) return s;
  return launched(mla::launch_combine(cfg->num_heads, o_part, lse_part, split_offsets, o_lat, lse, batch, stream));
}

mla_status mla_out_proj(const mla_config* cfg, const float* o_lat, const uint16_t* w_uv, uint16_t* out,
                        const uint16_t* w_o, int32_t hidden, uint16_t* y, float* out_f32, int32_t batch,
                        hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (batch < 0) return MLA_ERR_VALUE;
  if (w_o != nullptr && hidden <= 0) return MLA_ERR_VALUE;
  if (batch == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  if (w_o != nullptr && (!y || !out_f32)) return MLA_ERR_NULL;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  if (w_o != nullptr && (!aligned16(w_o) || !aligned16(y) || !aligned16(out_f32))) return MLA_ERR_ALIGN;
  if ((s = check_device()) != MLA_OK) return s;
  hipError_t e = mla::launch_out_proj(cfg->num_heads, o_lat, w_uv, out, w_o ? out_f32 : nullptr, batch, stream);
  if (e != hipSuccess) return hip_fail(e);
  if (w_o != nullptr)
    return launched(mla::launch_wo_proj(cfg->num_heads * 128, out_f32, w_o, hidden, y, batch, stream));
  return MLA_OK;
}

mla_status mla_decode_combine_out_proj(const mla_config* cfg, const uint16_t* o_part, const float* lse_part,
                                       const int32_t* split_offsets, const uint16_t* w_uv, uint16_t* out,
                                       float* o_lat, float* lse, const uint16_t* w_o, int32_t hidden, uint16_t* y,
                                       float* out_f32, int32_t batch, hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (batch < 0) return MLA_ERR_VALUE;
  if (w_o != nullptr && hidden <= 0) return MLA_ERR_VALUE;
  if (batch == 0) return MLA_OK;
  if (!o_part || !lse_part || !split_offsets || !w_uv || !out) return MLA_ERR_NULL;
  if (w_o != nullptr && (!y || !out_f32)) return MLA_ERR_NULL;
  if (!aligned16(o_part) || !aligned16(lse_part) || !aligned16(split_offsets) || !aligned16(w_uv) ||
      !aligned16(out) || (o_lat && !aligned16(o_lat)) || (lse && !aligned16(lse)))
    return MLA_ERR_ALIGN;
  if (w_o != nullptr && (!aligned16(w_o) || !aligned16(y) || !aligned16(out_f32))) return MLA_ERR_ALIGN;
  if ((s = check_device()) != MLA_OK) return s;
  hipError_t e = mla::launch_combine_out_proj(cfg->num_heads, o_part, lse_part, split_offsets, w_uv, out,
                                              w_o ? out_f32 : nullptr, o_lat, lse, batch, stream);
  if (e != hipSuccess) return hip_fail(e);
  if (w_o != nullptr)
    return launched(mla::launch_wo_proj(cfg->num_heads * 128, out_f32, w_o, hidden, y, batch, stream));
  return MLA_OK;
}

size_t mla_layer_front_workspace_bytes(const mla_config* cfg, int32_t n_tokens) {
  if (mla_config_check(cfg) != MLA_OK || n_tokens < 0) return 0;
  return (size_t)n_tokens * (size_t)(576 + cfg->num_heads * 192) * sizeof(float);
}

mla_status mla_layer_front(const mla_config* cfg, const uint16_t* x, int32_t hidden, const uint16_t* w_q,
                           const uint16_t* w_dkv, const int32_t* positions, float rms_eps, float rope_base,
                           float* workspace, size_t workspace_bytes, uint16_t* q_nope, uint16_t* q_pe,
                           uint16_t* c_kv, uint16_t* k_pe, int32_t n_tokens, hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (n_tokens < 0 || hidden <= 0 || hidden % 8 != 0) return MLA_ERR_VALUE;
  if (!(rms_eps > 0.f) || !std::isfinite(rms_eps) || !(rope_base > 1.f) || !std::isfinite(rope_base))
    return MLA_ERR_VALUE;
  if (n_tokens == 0) return MLA_OK;
  if (!x || !w_q || !w_dkv || !positions || !workspace || !q_nope || !q_pe || !c_kv || !k_pe) return MLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_dkv) || !aligned16(positions) || !aligned16(workspace) ||
      !aligned16(q_nope) || !aligned16(q_pe) || !aligned16(c_kv) || !aligned16(k_pe))
    return MLA_ERR_ALIGN;
  if (workspace_bytes < mla_layer_front_workspace_bytes(cfg, n_tokens)) return MLA_ERR_WORKSPACE;
  if ((s = check_device()) != MLA_OK) return s;
  return launched(mla::launch_layer_front(cfg->num_heads, x, hidden, w_q, w_dkv, positions, rms_eps, rope_base,
                                          workspace, q_nope, q_pe, c_kv, k_pe, n_tokens, stream));
}

mla_status mla_layer_front_append(const mla_config* cfg, const uint16_t* x, int32_t hidden, const uint16_t* w_q,
                                  const uint16_t* w_dkv, const int32_t* positions, float rms_eps, float rope_base,
                                  float* workspace, size_t workspace_bytes, uint16_t* q_nope, uint16_t* q_pe,
                                  uint16_t* c_kv, uint16_t* k_pe, void* pool, int64_t num_pages,
                                  const int64_t* slot_mapping, int32_t n_tokens, hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (n_tokens < 0 || num_pages < 0 || hidden <= 0 || hidden % 8 != 0) return MLA_ERR_VALUE;
  if (!(rms_eps > 0.f) || !std::isfinite(rms_eps) || !(rope_base > 1.f) || !std::isfinite(rope_base))
    return MLA_ERR_VALUE;
  if (n_tokens == 0) return MLA_OK;
  if (!x || !w_q || !w_dkv || !positions || !workspace || !q_nope || !q_pe || !c_kv || !k_pe || !pool ||
      !slot_mapping)
    return MLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_dkv) || !aligned16(positions) || !aligned16(workspace) ||
      !aligned16(q_nope) || !aligned16(q_pe) || !aligned16(c_kv) || !aligned16(k_pe) || !aligned16(pool) ||
      !aligned16(slot_mapping))
    return MLA_ERR_ALIGN;
  if (workspace_bytes < mla_layer_front_workspace_bytes(cfg, n_tokens)) return MLA_ERR_WORKSPACE;
  if ((s = check_device()) != MLA_OK) return s;
  return launched(mla::launch_layer_front_append(cfg->num_heads, x, hidden, w_q, w_dkv, positions, rms_eps, rope_base,
                                                 workspace, q_nope, q_pe, c_kv, k_pe, cfg->cache_dtype, pool,
                                                 num_pages, slot_mapping, n_tokens, stream));
}

mla_status mla_layer_front_noalloc(const mla_config* cfg, const uint16_t* x, int32_t hidden, const uint16_t* w_q,
                                   const uint16_t* w_dkv, const int32_t* positions, float rms_eps, float rope_base,
                                   uint16_t* q_nope, uint16_t* q_pe, uint16_t* c_kv, uint16_t* k_pe,
                                   int32_t n_tokens, hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (n_tokens < 0 || hidden <= 0 || hidden % 8 != 0) return MLA_ERR_VALUE;
  if (!(rms_eps > 0.f) || !std::isfinite(rms_eps) || !(rope_base > 1.f) || !std::isfinite(rope_base))
    return MLA_ERR_VALUE;
  if (n_tokens == 0) return MLA_OK;
  if (!x || !w_q || !w_dkv || !positions || !q_nope || !q_pe || !c_kv || !k_pe) return MLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_dkv) || !aligned16(positions) || !aligned16(q_nope) ||
      !aligned16(q_pe) || !aligned16(c_kv) || !aligned16(k_pe))
    return MLA_ERR_ALIGN;
  if (mla_layer_front_workspace_bytes(cfg, n_tokens) > mla::kFrontScratchBytes) return MLA_ERR_WORKSPACE;
  if ((s = check_device()) != MLA_OK) return s;
  return launched(mla::launch_layer_front_noalloc(cfg->num_heads, x, hidden, w_q, w_dkv, positions, rms_eps,
                                                  rope_base, q_nope, q_pe, c_kv, k_pe, n_tokens, stream));
}

mla_status mla_out_residual(const mla_config* cfg, const uint16_t* attn_out, const uint16_t* w_o, int32_t hidden,
                            const uint16_t* x_in, uint16_t* x_out, float* workspace, size_t workspace_bytes,
                            int32_t n_tokens, hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (n_tokens < 0 || hidden <= 0) return MLA_ERR_VALUE;
  if (n_tokens == 0) return MLA_OK;
  if (!attn_out || !w_o || !x_in || !x_out || !workspace) return MLA_ERR_NULL;
  if (!aligned16(attn_out) || !aligned16(w_o) || !aligned16(workspace)) return MLA_ERR_ALIGN;
  if (workspace_bytes < (size_t)n_tokens * (size_t)hidden * sizeof(float)) return MLA_ERR_WORKSPACE;
  if ((s = check_device()) != MLA_OK) return s;
  return launched(mla::launch_out_residual(cfg->num_heads, attn_out, w_o, hidden, x_in, x_out, workspace, n_tokens,
                                           stream));
}

size_t mla_prefill_workspace_bytes(const mla_config* cfg, int32_t seq_len) {
  if (mla_config_check(cfg) != MLA_OK || seq_len < 0) return 0;
  return (size_t)cfg->num_heads * (size_t)mla::prefill_padded_len(seq_len) * 512u;
}

mla_status mla_prefill_attn(const mla_config* cfg, const uint16_t* q_nope, const uint16_t* q_pe, int32_t n_queries,
                            const uint16_t* c_kv, const uint16_t* k_pe, int32_t seq_len, const uint16_t* w_uk,
                            const uint16_t* w_uv, void* workspace, size_t workspace_bytes, uint16_t* out,
                            float* lse, hipStream_t stream) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (n_queries < 0 || seq_len < 0 || n_queries > seq_len || seq_len > (1 << 23)) return MLA_ERR_VALUE;
  if (n_queries == 0) return MLA_OK;
  if (!q_nope || !q_pe || !c_kv || !k_pe || !w_uk || !w_uv || !workspace || !out) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(c_kv) || !aligned16(k_pe) || !aligned16(w_uk) ||
      !aligned16(w_uv) || !aligned16(workspace) || !aligned16(out) || (lse && !aligned16(lse)))
    return MLA_ERR_ALIGN;
  if (workspace_bytes < mla_prefill_workspace_bytes(cfg, seq_len)) return MLA_ERR_WORKSPACE;
  if ((s = check_device()) != MLA_OK) return s;
  return launched(mla::launch_prefill_attn(cfg->num_heads, cfg->softmax_scale, q_nope, q_pe, n_queries, c_kv, k_pe,
                                           seq_len, w_uk, w_uv, workspace, out, lse, stream));
}

const char* mla_status_string(mla_status st) {
  switch (st) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "unsupported shape (num_heads must be 16 or 128; widths 128/512/64/128; block 64)";
    case MLA_ERR_VALUE: return "argument out of range";
    case MLA_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "caller buffer too small";
    case MLA_ERR_UNSUPPORTED: return "current device is not gfx950";
    case MLA_ERR_HIP: return "HIP call or kernel launch failed";
  }
  return "unknown status";
}

int32_t mla_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
