// C entry points: argument validation, planning and launches. Every check
// runs on the host before anything is enqueued.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "hattn.h"
#include "hattn_internal.h"

using namespace hattn;

static_assert(sizeof(hattn_layer_desc) == 40, "hattn_layer_desc layout is part of the ABI");
static_assert(sizeof(hattn_kv_cache) == 48, "hattn_kv_cache layout is part of the ABI");

namespace {

constexpr int kHeadDimSupported = 256;
constexpr int kGroupSupported = 4;
constexpr int kMaxPos = 1 << 30;
constexpr int kDecodeTargetBlocks = 1024;  // 4 rounds of one workgroup per CU
constexpr long long kMaxDecodeSplits = 2048;  // the merge kernel's limit

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Rotated channel count, or -1 when head_dim * fraction is not a positive
// even integer no larger than head_dim.
int rotary_channels(double fraction, int head_dim) {
  if (!(fraction > 0.0) || !(fraction <= 1.0)) return -1;
  const double r = fraction * head_dim;
  const double ri = floor(r + 0.5);
  if (fabs(r - ri) > 1e-9 || ri < 2 || ri > head_dim) return -1;
  const int n = (int)ri;
  return (n % 2) ? -1 : n;
}

int check_desc(const hattn_layer_desc* d) {
  if (!d) return HATTN_ERR_NULL;
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0) return HATTN_ERR_SHAPE;
  if (d->num_q_heads % d->num_kv_heads) return HATTN_ERR_SHAPE;
  if (d->head_dim != kHeadDimSupported) return HATTN_ERR_UNSUPPORTED;
  if (d->num_q_heads / d->num_kv_heads != kGroupSupported) return HATTN_ERR_UNSUPPORTED;
  if (d->gate_act != HATTN_GATE_SIGMOID && d->gate_act != HATTN_GATE_SILU) return HATTN_ERR_UNSUPPORTED;
  if (!(d->rope_theta > 0.0) || !isfinite(d->rope_theta)) return HATTN_ERR_ROPE;
  const int r = rotary_channels(d->rotary_fraction, d->head_dim);
  if (r < 0) return HATTN_ERR_ROPE;
  if (r % 16) return HATTN_ERR_UNSUPPORTED;  // the kernels rotate 8-channel fragments in pairs
  if (d->layer_type == HATTN_LAYER_SLIDING) {
    if (d->window < 1) return HATTN_ERR_WINDOW;
  } else if (d->layer_type == HATTN_LAYER_FULL) {
    if (d->window > 0) return HATTN_ERR_WINDOW;
  } else {
    return HATTN_ERR_SHAPE;
  }
  return HATTN_OK;
}

// The cache's kind, batch, capacity and paging against the layer (no
// pointer checks: the workspace-size queries take a described cache).
int check_cache_shape(const hattn_layer_desc* d, const hattn_kv_cache* c, int batch) {
  if (!c) return HATTN_ERR_NULL;
  if (c->batch != batch || c->capacity < 1) return HATTN_ERR_CACHE;
  if (c->kind == HATTN_KV_RING) {
    if (d->layer_type != HATTN_LAYER_SLIDING || c->capacity != d->window) return HATTN_ERR_CACHE;
  } else if (c->kind == HATTN_KV_PAGED) {
    // full layers only; pages of whole 64-row tiles; one table row per sequence
    if (d->layer_type != HATTN_LAYER_FULL) return HATTN_ERR_CACHE;
    if (c->page_size < kMinPageSize || c->page_size % kMinPageSize || c->capacity % c->page_size)
      return HATTN_ERR_CACHE;
    if (c->capacity / c->page_size > kMaxPagesPerSeq || c->num_pages < 1) return HATTN_ERR_CACHE;
  } else if (c->kind != HATTN_KV_LINEAR) {
    return HATTN_ERR_CACHE;
  }
  return HATTN_OK;
}

// check_cache_shape plus the cache's pointers.
int check_cache(const hattn_layer_desc* d, const hattn_kv_cache* c, int batch) {
  const int st = check_cache_shape(d, c, batch);
  if (st != HATTN_OK) return st;
  if (!c->k || !c->v) return HATTN_ERR_NULL;
  if (!aligned16(c->k) || !aligned16(c->v)) return HATTN_ERR_ALIGN;
  if (c->kind == HATTN_KV_PAGED) {
    if (!c->block_table) return HATTN_ERR_NULL;
    if ((uintptr_t)c->block_table & 3u) return HATTN_ERR_ALIGN;
  }
  return HATTN_OK;
}

// The kernels' view of a paged cache (table == nullptr otherwise).
PagedKv paged_view(const hattn_kv_cache* c) {
  PagedKv p{};
  if (c->kind == HATTN_KV_PAGED) {
    p.table = c->block_table;
    p.page_size = c->page_size;
    p.pages_per_seq = c->capacity / c->page_size;
    p.num_pages = c->num_pages;
  }
  return p;
}

hattn_status from_hip(hipError_t e) { return e == hipSuccess ? HATTN_OK : HATTN_ERR_LAUNCH; }

// inv_freq_i = theta^(-2i/r), i < r/2, in fp64 (page §4 RoPE table: theta
// and the rotated-channel count r per layer type).
void fill_inv_freq(double theta, int r, double* out) {
  for (int i = 0; i < r / 2; ++i) out[i] = pow(theta, -2.0 * (double)i / (double)r);
}

// ---------------------------------------------------------------- profiling
struct EventPair {
  hipEvent_t start, stop;
};
bool g_profile = false;
std::vector<EventPair> g_recorded[2];
std::vector<EventPair> g_free;

// Records the start event of a profiled section; returns the event that
// closes it (null when profiling is off).
hipEvent_t profile_begin(int kind, hipStream_t s) {
  if (!g_profile) return nullptr;
  EventPair p{};
  if (!g_free.empty()) {
    p = g_free.back();
    g_free.pop_back();
  } else if (hipEventCreate(&p.start) != hipSuccess || hipEventCreate(&p.stop) != hipSuccess) {
    return nullptr;
  }
  if (hipEventRecord(p.start, s) != hipSuccess) {
    g_free.push_back(p);
    return nullptr;
  }
  g_recorded[kind].push_back(p);
  return p.stop;
}

void profile_end(hipEvent_t stop, hipStream_t s) {
  if (stop) (void)hipEventRecord(stop, s);
}

struct PrefillLayout {
  size_t table_bytes;   // cos/sin of the new tokens' angles
  size_t stage_bytes;   // per K or V staging buffer (ring caches only)
  int stage_rows;
  size_t total;
};

// total_tokens: packed new tokens of all sequences; max_len: the longest
// sequence's new tokens.
PrefillLayout prefill_layout(const hattn_layer_desc* d, const hattn_kv_cache* c, int B,
                             long long total_tokens, int max_len) {
  PrefillLayout L{};
  const int r = rotary_channels(d->rotary_fraction, d->head_dim);
  L.table_bytes = align_up((size_t)total_tokens * (r / 2) * 8, 256);
  if (c->kind == HATTN_KV_RING) {
    L.stage_rows = (d->window - 1) + max_len;
    L.stage_bytes = align_up((size_t)B * d->num_kv_heads * L.stage_rows * d->head_dim * 2, 256);
  }
  L.total = L.table_bytes + 2 * L.stage_bytes;
  return L;
}

// Longest visible key range of a decode query at a position <= max_pos.
long long decode_span(const hattn_layer_desc* d, const hattn_kv_cache* c, long long max_pos) {
  if (c->kind == HATTN_KV_RING) return std::min<long long>(max_pos + 1, c->capacity);
  if (d->window > 0) return std::min<long long>(max_pos + 1, d->window);
  return max_pos + 1;
}

struct DecodePlan {
  int nsplit;
  int split_keys;
};

// With at least this many (sequence, KV head) pairs, each pair gets one
// workgroup over its whole key range (one per CU, no split merge).
constexpr long long kDecodeWidePairs = 256;

// Otherwise split the key range so that the grid holds about
// kDecodeTargetBlocks workgroups, in multiples of 128 keys.
DecodePlan decode_plan(const hattn_layer_desc* d, const hattn_kv_cache* c, int B, long long span) {
  const long long base = (long long)B * d->num_kv_heads;
  if (base >= kDecodeWidePairs) return DecodePlan{1, (int)((span + 127) / 128 * 128)};
  long long want = (kDecodeTargetBlocks + base - 1) / base;
  long long most = (span + 127) / 128;
  long long n = std::max<long long>(1, std::min({want, most, (long long)kMaxDecodeSplits}));
  long long keys = (span + n - 1) / n;
  keys = (keys + 127) / 128 * 128;
  n = (span + keys - 1) / keys;
  return DecodePlan{(int)n, (int)keys};
}

// The most splits decode_plan gives for any visible span up to `span`: its
// split count is at most min(target, ceil(span / 128), limit), a bound that
// grows with span (the count itself need not: rounding the keys per split
// up to 128 can lower it at a larger span).
long long decode_max_splits(const hattn_layer_desc* d, int B, long long span) {
  const long long base = (long long)B * d->num_kv_heads;
  if (base >= kDecodeWidePairs) return 1;
  const long long want = (kDecodeTargetBlocks + base - 1) / base;
  return std::max<long long>(1, std::min({want, (span + 127) / 128, (long long)kMaxDecodeSplits}));
}

// Bytes of the split partials (o, then (m, l)) for n splits.
size_t decode_partials_bytes(const hattn_layer_desc* d, int B, long long n) {
  const size_t parts = (size_t)B * d->num_q_heads * (size_t)n;
  return align_up(parts * d->head_dim * 4, 256) + align_up(parts * 2 * 4, 256);
}

// Checks shared by both prefill entry points (before any sequence data).
int prefill_common_checks(const hattn_layer_desc* desc, const hattn_kv_cache* cache, int32_t batch,
                          const int32_t* start_pos) {
  int st = check_desc(desc);
  if (st != HATTN_OK) return st;
  if (batch <= 0) return HATTN_ERR_SHAPE;
  if (batch > kMaxPrefillBatch) return HATTN_ERR_UNSUPPORTED;
  st = check_cache(desc, cache, batch);
  if (st != HATTN_OK) return st;
  if (!start_pos) return HATTN_ERR_NULL;
  return HATTN_OK;
}

}  // namespace

namespace hattn {

int validate_layer_cache(const hattn_layer_desc* desc, const hattn_kv_cache* cache, int batch, bool pointers) {
  const int st = check_desc(desc);
  if (st != HATTN_OK) return st;
  if (batch <= 0) return HATTN_ERR_SHAPE;
  return pointers ? check_cache(desc, cache, batch) : check_cache_shape(desc, cache, batch);
}

size_t prefill_workspace_bytes(const hattn_layer_desc* desc, const hattn_kv_cache* cache, int batch,
                               long long total_tokens, int max_len) {
  return prefill_layout(desc, cache, batch, total_tokens, max_len).total;
}

size_t decode_workspace_bytes(const hattn_layer_desc* desc, const hattn_kv_cache* cache, int batch) {
  return hattn_decode_workspace_size(desc, cache, batch);
}

// One prefill call over packed new tokens: sequence b's tokens are rows
// tok0[b] .. tok0[b] + len[b] - 1 of q/k/v/gate/out, at positions
// start_pos[b] + 0 .. len[b] - 1.
// Token rows of q, k/v and gate are q_stride, kv_stride and gate_stride
// elements apart (dense: Hq * 256, Hkv * 256, Hq).
constexpr long long kMaxQStride = 1LL << 24;  // 65,536 query heads of 256 channels

int prefill_packed(const hattn_layer_desc* desc, const void* q, const void* k, const void* v,
                   const void* gate, int32_t batch, const int* tok0, const int* len, long long total,
                   const int32_t* start_pos, const hattn_kv_cache* cache, void* out, void* workspace,
                   size_t workspace_bytes, hipStream_t stream, long long q_stride, long long kv_stride,
                   long long gate_stride) {
  const int st = prefill_common_checks(desc, cache, batch, start_pos);
  if (st != HATTN_OK) return st;
  if (!tok0 || !len) return HATTN_ERR_NULL;
  const bool ring = cache->kind == HATTN_KV_RING;
  int max_len = 0;
  for (int b = 0; b < batch; ++b) {
    const long long s0 = start_pos[b];
    if (len[b] < 0) return HATTN_ERR_SHAPE;
    if (s0 < 0 || s0 + len[b] > kMaxPos) return HATTN_ERR_POSITION;
    if (!ring && s0 + len[b] > cache->capacity) return HATTN_ERR_CAPACITY;
    max_len = std::max(max_len, len[b]);
  }
  if (total == 0) return HATTN_OK;
  if (!q || !k || !v || !gate || !out) return HATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || ((uintptr_t)gate & 1u))
    return HATTN_ERR_ALIGN;
  // The attention kernel addresses a (sequence, KV head) slab of key rows
  // with 32-bit byte offsets (512 B per row).
  // (A paged cache is addressed per page.)
  const long long key_rows = ring ? (long long)desc->window - 1 + max_len : (long long)cache->capacity;
  if (cache->kind != HATTN_KV_PAGED && key_rows > kMaxPrefillKeyRows) return HATTN_ERR_UNSUPPORTED;
  // A query block's 32 rows are read with 32-bit byte offsets from its first
  // row (q_stride elements apart).
  if (q_stride > kMaxQStride) return HATTN_ERR_UNSUPPORTED;
  // one-dimensional grids: (query blocks x sequences x KV heads) workgroups
  if ((long long)((max_len + kPrefillBlockQ - 1) / kPrefillBlockQ) * batch * desc->num_kv_heads > INT32_MAX)
    return HATTN_ERR_UNSUPPORTED;
  const PrefillLayout L = prefill_layout(desc, cache, batch, total, max_len);
  if (!workspace || workspace_bytes < L.total) return HATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return HATTN_ERR_ALIGN;

  const int Hq = desc->num_q_heads, Hkv = desc->num_kv_heads;
  const int r = rotary_channels(desc->rotary_fraction, desc->head_dim);
  char* ws = (char*)workspace;
  float2* table = (float2*)ws;
  uint16_t* stage_k = ring ? (uint16_t*)(ws + L.table_bytes) : nullptr;
  uint16_t* stage_v = ring ? (uint16_t*)(ws + L.table_bytes + L.stage_bytes) : nullptr;
  const int w = desc->window;

  // 1. a ring's visible history -> staging rows 0 .. hist-1
  RingCopyArgs rc{};
  if (ring) {
    rc.ring_k = (uint16_t*)cache->k;
    rc.ring_v = (uint16_t*)cache->v;
    rc.stage_k = stage_k;
    rc.stage_v = stage_v;
    rc.B = batch;
    rc.Hkv = Hkv;
    rc.cap = cache->capacity;
    rc.stage_rows = L.stage_rows;
    for (int b = 0; b < batch; ++b) {
      // a sequence without new tokens needs no history
      const int hist = len[b] > 0 ? std::min(start_pos[b], w - 1) : 0;
      rc.count[b] = hist;
      rc.first_pos[b] = start_pos[b] - hist;
      rc.stage_row0[b] = 0;
    }
    hipError_t e = launch_ring_to_stage(rc, stream);
    if (e != hipSuccess) return HATTN_ERR_LAUNCH;
  }

  // 2. cos/sin table of the new positions; rotated K and V -> cache slots
  //    (linear) or staging rows and the ring's slots (ring)
  PrefillPrepArgs ra{};
  ra.k = (const uint16_t*)k;
  ra.v = (const uint16_t*)v;
  ra.kv_stride = kv_stride;
  ra.table = table;
  ra.dst_k = ring ? stage_k : (uint16_t*)cache->k;
  ra.dst_v = ring ? stage_v : (uint16_t*)cache->v;
  ra.B = batch;
  ra.max_len = max_len;
  ra.Hkv = Hkv;
  ra.dst_rows = ring ? L.stage_rows : cache->capacity;
  ra.paged = paged_view(cache);
  ra.r = r;
  // a ring keeps each sequence's last min(len, capacity) new tokens; the
  // prep kernel writes them to their slots (the history they replace is
  // already staged)
  ra.ring_k = ring ? (uint16_t*)cache->k : nullptr;
  ra.ring_v = ring ? (uint16_t*)cache->v : nullptr;
  ra.ring_cap = cache->capacity;
  fill_inv_freq(desc->rope_theta, r, ra.inv_freq);
  PrefillAttnArgs aa{};
  for (int b = 0; b < batch; ++b) {
    const int hist = ring ? std::min(start_pos[b], w - 1) : 0;
    ra.start[b] = start_pos[b];
    ra.dst_row0[b] = ring ? hist : start_pos[b];
    ra.tok0[b] = tok0[b];
    ra.len[b] = len[b];
    aa.start[b] = start_pos[b];
    aa.key_pos0[b] = ring ? start_pos[b] - hist : 0;
    aa.n_keys[b] = ring ? hist + len[b] : start_pos[b] + len[b];
    aa.tok0[b] = tok0[b];
    aa.len[b] = len[b];
  }
  hipError_t e = launch_prefill_prep(ra, stream);
  if (e != hipSuccess) return HATTN_ERR_LAUNCH;

  // 3. attention over the linear key rows (queries rotated in the kernel)
  aa.q = (const uint16_t*)q;
  aa.q_stride = q_stride;
  aa.gate_stride = gate_stride;
  aa.table = table;
  aa.kc = ring ? stage_k : (const uint16_t*)cache->k;
  aa.vc = ring ? stage_v : (const uint16_t*)cache->v;
  aa.gate = (const uint16_t*)gate;
  aa.out = (uint16_t*)out;
  aa.B = batch;
  aa.Hq = Hq;
  aa.Hkv = Hkv;
  aa.rows = ring ? L.stage_rows : cache->capacity;
  aa.paged = paged_view(cache);
  aa.window = desc->layer_type == HATTN_LAYER_SLIDING ? w : 0;
  aa.r = r;
  aa.gate_act = desc->gate_act;
  aa.q_tiles = (max_len + kPrefillBlockQ - 1) / kPrefillBlockQ;
  if (g_profile && prefill_clock_acc(&aa.clock_acc) != hipSuccess) aa.clock_acc = nullptr;
  hipEvent_t prof = profile_begin(HATTN_PROFILE_PREFILL, stream);
  e = launch_prefill_attn(aa, stream);
  profile_end(prof, stream);
  if (e != hipSuccess) return HATTN_ERR_LAUNCH;

  return HATTN_OK;
}

// hattn_decode with sequence rows of q, k/v and gate q_stride, kv_stride and
// gate_stride elements apart (dense: Hq * 256, Hkv * 256, Hq).
int decode_strided(const hattn_layer_desc* desc, const void* q, const void* k, const void* v,
                   const void* gate, int32_t batch, const int32_t* pos, int32_t max_pos,
                   const hattn_kv_cache* cache, void* out, void* workspace, size_t workspace_bytes,
                   hipStream_t stream, long long q_stride, long long kv_stride, long long gate_stride,
                   bool static_scratch) {
  int st = check_desc(desc);
  if (st != HATTN_OK) return st;
  if (batch <= 0) return HATTN_ERR_SHAPE;
  st = check_cache(desc, cache, batch);
  if (st != HATTN_OK) return st;
  if (!q || !k || !v || !gate || !pos || !out) return HATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || ((uintptr_t)gate & 1u) ||
      ((uintptr_t)pos & 3u))
    return HATTN_ERR_ALIGN;
  if (max_pos < 0 || max_pos >= kMaxPos) return HATTN_ERR_POSITION;
  if (cache->kind != HATTN_KV_RING && max_pos >= cache->capacity) return HATTN_ERR_CAPACITY;
  const long long span = decode_span(desc, cache, max_pos);
  const DecodePlan p = decode_plan(desc, cache, batch, span);
  // one-dimensional grids: (sequences x KV heads x splits) and (sequences x
  // heads x 4 channel quarters)
  if ((long long)batch * desc->num_kv_heads * p.nsplit > INT32_MAX ||
      (long long)batch * desc->num_q_heads * 4 > INT32_MAX)
    return HATTN_ERR_UNSUPPORTED;
  const size_t parts = (size_t)batch * desc->num_q_heads * p.nsplit;
  const size_t o_bytes = align_up(parts * desc->head_dim * 4, 256);
  const size_t need = p.nsplit == 1 ? 0 : decode_partials_bytes(desc, batch, p.nsplit);
  if (static_scratch) {
    // the library's own array: its size bounds the plan, its address is
    // looked up (no allocation) once the arguments are known to be valid
    if (need > workspace_bytes) return HATTN_ERR_WORKSPACE;
    if (need > 0 && decode_static_scratch(&workspace) != hipSuccess) return HATTN_ERR_LAUNCH;
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return HATTN_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return HATTN_ERR_ALIGN;

  DecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.gate = (const uint16_t*)gate;
  a.q_stride = q_stride;
  a.kv_stride = kv_stride;
  a.gate_stride = gate_stride;
  a.pos = pos;
  a.kc = (uint16_t*)cache->k;
  a.vc = (uint16_t*)cache->v;
  a.out = (uint16_t*)out;
  a.part_o = need ? (float*)workspace : nullptr;
  a.part_ml = need ? (float*)((char*)workspace + o_bytes) : nullptr;
  a.B = batch;
  a.Hq = desc->num_q_heads;
  a.Hkv = desc->num_kv_heads;
  a.cap = cache->capacity;
  a.ring = cache->kind == HATTN_KV_RING;
  a.paged = paged_view(cache);
  a.window = desc->layer_type == HATTN_LAYER_SLIDING ? desc->window : 0;
  a.max_pos = max_pos;
  a.r = rotary_channels(desc->rotary_fraction, desc->head_dim);
  a.gate_act = desc->gate_act;
  fill_inv_freq(desc->rope_theta, a.r, a.inv_freq);
  a.nsplit = p.nsplit;
  a.split_keys = p.split_keys;
  hipEvent_t prof = profile_begin(HATTN_PROFILE_DECODE, stream);
  const hipError_t e = launch_decode(a, stream);
  profile_end(prof, stream);
  return from_hip(e);
}

}  // namespace hattn

extern "C" {

const char* hattn_status_string(int status) {
  switch (status) {
    case HATTN_OK: return "ok";
    case HATTN_ERR_NULL: return "null pointer";
    case HATTN_ERR_SHAPE: return "invalid or inconsistent size";
    case HATTN_ERR_UNSUPPORTED: return "unsupported head_dim or GQA group size";
    case HATTN_ERR_ROPE: return "invalid RoPE theta or rotary fraction";
    case HATTN_ERR_WINDOW: return "window does not match the layer type";
    case HATTN_ERR_CACHE: return "cache kind, capacity or batch does not fit the layer";
    case HATTN_ERR_CAPACITY: return "positions exceed the linear cache capacity";
    case HATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case HATTN_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case HATTN_ERR_LAUNCH: return "HIP launch failed";
    case HATTN_ERR_POSITION: return "position out of range";
    default: return "unknown status";
  }
}

int hattn_layer_defaults(int32_t layer_type, int32_t num_q_heads, int32_t num_kv_heads,
                         hattn_layer_desc* out) {
  if (!out) return HATTN_ERR_NULL;
  hattn_layer_desc d{};
  d.layer_type = layer_type;
  d.num_q_heads = num_q_heads;
  d.num_kv_heads = num_kv_heads;
  d.head_dim = kHeadDimSupported;
  if (layer_type == HATTN_LAYER_SLIDING) {
    d.window = 512;
    d.rope_theta = 1.0e4;
    d.rotary_fraction = 1.0;
  } else if (layer_type == HATTN_LAYER_FULL) {
    d.window = 0;
    d.rope_theta = 5.0e6;
    d.rotary_fraction = 0.25;
  } else {
    return HATTN_ERR_SHAPE;
  }
  const int st = check_desc(&d);
  if (st != HATTN_OK) return st;
  *out = d;
  return HATTN_OK;
}

int hattn_rope_apply(void* x, int32_t n_tok, int32_t n_heads, int32_t head_dim, const int32_t* pos,
                     double theta, double rotary_fraction, hipStream_t stream) {
  if (n_tok < 0 || n_heads <= 0 || head_dim <= 0 || head_dim % 2) return HATTN_ERR_SHAPE;
  if (head_dim > 512) return HATTN_ERR_UNSUPPORTED;
  if (!(theta > 0.0) || !isfinite(theta)) return HATTN_ERR_ROPE;
  const int r = rotary_channels(rotary_fraction, head_dim);
  if (r < 0) return HATTN_ERR_ROPE;
  if (n_tok == 0) return HATTN_OK;
  if (!x || !pos) return HATTN_ERR_NULL;
  if (((uintptr_t)x & 1u) || ((uintptr_t)pos & 3u)) return HATTN_ERR_ALIGN;
  RopeApplyArgs a{};
  a.x = (uint16_t*)x;
  a.pos = pos;
  a.n_tok = n_tok;
  a.n_heads = n_heads;
  a.head_dim = head_dim;
  a.r = r;
  fill_inv_freq(theta, r, a.inv_freq);
  return from_hip(launch_rope_apply(a, stream));
}

size_t hattn_prefill_workspace_size(const hattn_layer_desc* desc, const hattn_kv_cache* cache,
                                    int32_t batch, int32_t seq_len) {
  if (check_desc(desc) != HATTN_OK || batch <= 0 || seq_len < 0 || check_cache_shape(desc, cache, batch) != HATTN_OK)
    return 0;
  return prefill_layout(desc, cache, batch, (long long)batch * seq_len, seq_len).total;
}

size_t hattn_prefill_varlen_workspace_size(const hattn_layer_desc* desc, const hattn_kv_cache* cache,
                                           int32_t batch, const int32_t* cu_seqlens) {
  if (check_desc(desc) != HATTN_OK || batch <= 0 || check_cache_shape(desc, cache, batch) != HATTN_OK ||
      !cu_seqlens || cu_seqlens[0] != 0)
    return 0;
  int max_len = 0;
  for (int b = 0; b < batch; ++b) {
    const long long n = (long long)cu_seqlens[b + 1] - cu_seqlens[b];
    if (n < 0) return 0;
    max_len = std::max<int>(max_len, (int)n);
  }
  return prefill_layout(desc, cache, batch, cu_seqlens[batch], max_len).total;
}

int hattn_prefill(const hattn_layer_desc* desc, const void* q, const void* k, const void* v,
                  const void* gate, int32_t batch, int32_t seq_len, const int32_t* start_pos,
                  const hattn_kv_cache* cache, void* out, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  int st = check_desc(desc);
  if (st != HATTN_OK) return st;
  if (batch <= 0 || seq_len < 0) return HATTN_ERR_SHAPE;
  st = prefill_common_checks(desc, cache, batch, start_pos);
  if (st != HATTN_OK) return st;
  if ((long long)batch * seq_len > INT32_MAX) return HATTN_ERR_UNSUPPORTED;
  int tok0[kMaxPrefillBatch], len[kMaxPrefillBatch];
  for (int b = 0; b < batch; ++b) {
    tok0[b] = b * seq_len;
    len[b] = seq_len;
  }
  return prefill_packed(desc, q, k, v, gate, batch, tok0, len, (long long)batch * seq_len, start_pos,
                        cache, out, workspace, workspace_bytes, stream, (long long)desc->num_q_heads * kHeadDimSupported,
                        (long long)desc->num_kv_heads * kHeadDimSupported, desc->num_q_heads);
}

int hattn_prefill_varlen(const hattn_layer_desc* desc, const void* q, const void* k, const void* v,
                         const void* gate, int32_t batch, const int32_t* cu_seqlens,
                         const int32_t* start_pos, const hattn_kv_cache* cache, void* out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = prefill_common_checks(desc, cache, batch, start_pos);
  if (st != HATTN_OK) return st;
  if (!cu_seqlens) return HATTN_ERR_NULL;
  if (cu_seqlens[0] != 0) return HATTN_ERR_SHAPE;
  int tok0[kMaxPrefillBatch], len[kMaxPrefillBatch];
  for (int b = 0; b < batch; ++b) {
    if (cu_seqlens[b + 1] < cu_seqlens[b]) return HATTN_ERR_SHAPE;
    tok0[b] = cu_seqlens[b];
    len[b] = cu_seqlens[b + 1] - cu_seqlens[b];
  }
  return prefill_packed(desc, q, k, v, gate, batch, tok0, len, cu_seqlens[batch], start_pos, cache, out,
                        workspace, workspace_bytes, stream, (long long)desc->num_q_heads * kHeadDimSupported,
                        (long long)desc->num_kv_heads * kHeadDimSupported, desc->num_q_heads);
}

size_t hattn_decode_workspace_size(const hattn_layer_desc* desc, const hattn_kv_cache* cache,
                                   int32_t batch) {
  if (check_desc(desc) != HATTN_OK || batch <= 0 || check_cache_shape(desc, cache, batch) != HATTN_OK) return 0;
  const long long span = cache->kind == HATTN_KV_RING
                             ? cache->capacity
                             : decode_span(desc, cache, (long long)cache->capacity - 1);
  const long long n = decode_max_splits(desc, batch, span);
  if (n == 1) return 256;  // no partials needed; keep a non-zero size
  return decode_partials_bytes(desc, batch, n);
}

int hattn_decode(const hattn_layer_desc* desc, const void* q, const void* k, const void* v,
                 const void* gate, int32_t batch, const int32_t* pos, int32_t max_pos,
                 const hattn_kv_cache* cache, void* out, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  const int st = check_desc(desc);
  if (st != HATTN_OK) return st;
  return decode_strided(desc, q, k, v, gate, batch, pos, max_pos, cache, out, workspace, workspace_bytes,
                        stream, (long long)desc->num_q_heads * kHeadDimSupported,
                        (long long)desc->num_kv_heads * kHeadDimSupported, desc->num_q_heads);
}

int hattn_decode_static(const hattn_layer_desc* desc, const void* q, const void* k, const void* v,
                        const void* gate, int32_t batch, const int32_t* pos, int32_t max_pos,
                        const hattn_kv_cache* cache, void* out, hipStream_t stream) {
  const int st = check_desc(desc);
  if (st != HATTN_OK) return st;
  return decode_strided(desc, q, k, v, gate, batch, pos, max_pos, cache, out, nullptr,
                        HATTN_DECODE_STATIC_SCRATCH_BYTES, stream, (long long)desc->num_q_heads * kHeadDimSupported,
                        (long long)desc->num_kv_heads * kHeadDimSupported, desc->num_q_heads,
                        /*static_scratch=*/true);
}

int hattn_profile_enable(int enable) {
  g_profile = enable != 0;
  if (g_profile) {  // start the current GPU's clock sums from zero
    unsigned long long* acc = nullptr;
    if (prefill_clock_acc(&acc) != hipSuccess || hipMemset(acc, 0, 2 * sizeof(unsigned long long)) != hipSuccess)
      return HATTN_ERR_LAUNCH;
  }
  return HATTN_OK;
}

int hattn_profile_read_clock(double* shader_ghz) {
  if (!shader_ghz) return HATTN_ERR_NULL;
  *shader_ghz = 0.0;
  unsigned long long* acc = nullptr;
  unsigned long long h[2] = {0, 0};
  int dev = 0, khz = 0;
  if (prefill_clock_acc(&acc) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(h, acc, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemset(acc, 0, sizeof(h)) != hipSuccess || hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return HATTN_ERR_LAUNCH;
  // shader ticks per real-time tick, times the real-time counter's rate
  if (h[1] > 0 && khz > 0) *shader_ghz = (double)h[0] / (double)h[1] * (double)khz * 1e-6;
  return HATTN_OK;
}

int hattn_profile_read(int kind, int64_t* count, double* total_ms) {
  if (kind != HATTN_PROFILE_PREFILL && kind != HATTN_PROFILE_DECODE) return HATTN_ERR_SHAPE;
  if (!count || !total_ms) return HATTN_ERR_NULL;
  double sum = 0.0;
  int64_t n = 0;
  int st = HATTN_OK;
  for (EventPair& p : g_recorded[kind]) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
      st = HATTN_ERR_LAUNCH;
    } else {
      sum += ms;
      ++n;
    }
    g_free.push_back(p);
  }
  g_recorded[kind].clear();
  *count = n;
  *total_ms = sum;
  return st;
}

int hattn_debug_read_probe(const void* buf, size_t bytes, int32_t blocks, uint32_t* sink, hipStream_t stream) {
  if (blocks < 1 || bytes % 16) return HATTN_ERR_SHAPE;
  if (bytes == 0) return HATTN_OK;
  if (!buf || !sink) return HATTN_ERR_NULL;
  if (!aligned16(buf) || ((uintptr_t)sink & 3u)) return HATTN_ERR_ALIGN;
  return from_hip(launch_read_probe(buf, bytes, blocks, sink, stream));
}

int hattn_debug_mfma_probe(int32_t blocks, int32_t iters, float* sink, hipStream_t stream) {
  if (blocks < 1 || iters < 1) return HATTN_ERR_SHAPE;
  if (!sink) return HATTN_ERR_NULL;
  if ((uintptr_t)sink & 3u) return HATTN_ERR_ALIGN;
  return from_hip(launch_mfma_probe(blocks, iters, sink, stream));
}

int hattn_debug_lds_probe(int32_t mode, int32_t blocks, int32_t iters, uint64_t* out, hipStream_t stream) {
  if (mode < 0 || mode > 2 || blocks < 1 || iters < 1) return HATTN_ERR_SHAPE;
  if (!out) return HATTN_ERR_NULL;
  if ((uintptr_t)out & 7u) return HATTN_ERR_ALIGN;
  return from_hip(launch_lds_probe(mode, blocks, iters, (unsigned long long*)out, stream));
}

int hattn_debug_index_probe(const hattn_layer_desc* desc, int32_t kv_kind, int32_t capacity,
                            int32_t q_pos0, int32_t n_q, uint8_t* mask, int32_t* key_pos,
                            int32_t* slot, hipStream_t stream) {
  const int st = check_desc(desc);
  if (st != HATTN_OK) return st;
  if (capacity < 1 || n_q < 0) return HATTN_ERR_SHAPE;
  if (kv_kind != HATTN_KV_RING && kv_kind != HATTN_KV_LINEAR) return HATTN_ERR_CACHE;
  if (kv_kind == HATTN_KV_RING && (desc->layer_type != HATTN_LAYER_SLIDING || capacity != desc->window))
    return HATTN_ERR_CACHE;
  if (q_pos0 < 0 || (long long)q_pos0 + n_q > kMaxPos) return HATTN_ERR_POSITION;
  if (n_q == 0) return HATTN_OK;
  if (!mask || !key_pos || !slot) return HATTN_ERR_NULL;
  ProbeArgs a{};
  a.mask = mask;
  a.key_pos = key_pos;
  a.slot = slot;
  a.ring = kv_kind == HATTN_KV_RING;
  a.cap = capacity;
  a.window = desc->layer_type == HATTN_LAYER_SLIDING ? desc->window : 0;
  a.q_pos0 = q_pos0;
  a.n_q = n_q;
  return from_hip(launch_index_probe(a, stream));
}

}  // extern "C"
