// KV planner: the caches of a whole layer stack laid out in one arena
// (page "Spark-X2.5 架构（4B / 1.7B）", §6 KV table: per token and layer,
// K and V of every KV head in bf16; full layers keep every token, sliding
// layers at most the window; §2: one full layer after every three sliding
// ones). Host arithmetic only.
#include <stdint.h>

#include "hattn.h"

namespace {

constexpr uint64_t kBlockAlign = 256;
constexpr int32_t kHeadDim = 256;
constexpr int32_t kMaxTokens = 1 << 30;

uint64_t align_up(uint64_t x) { return (x + kBlockAlign - 1) / kBlockAlign * kBlockAlign; }

// Bytes of one K (or V) block: [batch][num_kv_heads][capacity][256] bf16.
uint64_t block_bytes(int32_t batch, int32_t num_kv_heads, int32_t capacity) {
  return (uint64_t)batch * (uint64_t)num_kv_heads * (uint64_t)capacity * kHeadDim * 2u;
}

}  // namespace

extern "C" {

int hattn_kv_plan(int32_t n_layers, const int32_t* layer_types, int32_t num_kv_heads,
                  int32_t batch, int32_t max_tokens, int32_t window, hattn_kv_layer_plan* plan,
                  uint64_t* arena_bytes) {
  if (!plan || !arena_bytes) return HATTN_ERR_NULL;
  if (n_layers < 1 || batch < 1 || num_kv_heads < 1 || max_tokens < 1 || max_tokens > kMaxTokens)
    return HATTN_ERR_SHAPE;
  if (window < 1) return HATTN_ERR_WINDOW;
  if (layer_types) {
    for (int32_t i = 0; i < n_layers; ++i)
      if (layer_types[i] != HATTN_LAYER_SLIDING && layer_types[i] != HATTN_LAYER_FULL) return HATTN_ERR_SHAPE;
  }
  uint64_t at = 0;
  for (int32_t i = 0; i < n_layers; ++i) {
    hattn_kv_layer_plan e{};
    e.layer_type = layer_types ? layer_types[i] : (i % 4 == 3 ? HATTN_LAYER_FULL : HATTN_LAYER_SLIDING);
    if (e.layer_type == HATTN_LAYER_SLIDING && max_tokens > window) {
      e.kind = HATTN_KV_RING;
      e.capacity = window;
    } else {
      e.kind = HATTN_KV_LINEAR;
      e.capacity = max_tokens;
    }
    e.num_kv_heads = num_kv_heads;
    e.batch = batch;
    const uint64_t blk = block_bytes(batch, num_kv_heads, e.capacity);
    e.k_offset = at;
    at = align_up(at + blk);
    e.v_offset = at;
    at = align_up(at + blk);
    e.bytes = 2 * blk;
    plan[i] = e;
  }
  *arena_bytes = at;
  return HATTN_OK;
}

int hattn_kv_cache_at(const hattn_kv_layer_plan* layer, void* arena, hattn_kv_cache* out) {
  if (!layer || !arena || !out) return HATTN_ERR_NULL;
  if ((uintptr_t)arena % kBlockAlign) return HATTN_ERR_ALIGN;
  const hattn_kv_layer_plan& e = *layer;
  if (e.batch < 1 || e.num_kv_heads < 1 || e.capacity < 1) return HATTN_ERR_SHAPE;
  if (e.kind != HATTN_KV_RING && e.kind != HATTN_KV_LINEAR) return HATTN_ERR_SHAPE;
  const uint64_t blk = block_bytes(e.batch, e.num_kv_heads, e.capacity);
  if (e.bytes != 2 * blk || e.k_offset % kBlockAlign || e.v_offset % kBlockAlign ||
      (e.v_offset < e.k_offset + blk && e.k_offset < e.v_offset + blk))
    return HATTN_ERR_SHAPE;
  hattn_kv_cache c{};
  c.k = (char*)arena + e.k_offset;
  c.v = (char*)arena + e.v_offset;
  c.kind = e.kind;
  c.batch = e.batch;
  c.capacity = e.capacity;
  *out = c;
  return HATTN_OK;
}

}  // extern "C"
