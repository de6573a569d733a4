/*
 * hattn.h - C ABI of the hybrid sliding-window / full causal GQA attention
 * core for MI355X (gfx950).
 *
 * The method (page "Spark-X2.5 架构（4B / 1.7B）"):
 *   - §2 混合注意力: every layer is either a sliding-window layer (window 512)
 *     or a full causal layer; three of every four layers slide.
 *   - §4 分层 RoPE, table: sliding layers rotate all 256 channels with
 *     theta = 1e4; full layers rotate only the first 64 channels
 *     (partial_rotary_factor 0.25) with theta = 5e6.
 *   - §3 逐头输出门控, Eq. 1: out = softmax(Q K^T / sqrt(d_head)) V, multiplied
 *     by sigmoid of one gate logit per (token, head) in fp32, stored as bf16.
 *     The same section notes that the model code also offers a silu gate
 *     activation (g * sigmoid(g)); the released checkpoints use sigmoid.
 *   - §1 config table: 16 query heads share 4 KV heads (8 / 2 for the 1.7B
 *     shape), head_dim 256, bf16.
 *   - §6 KV table: full layers keep every token, sliding layers only the last
 *     512 (page "Spark-X2.5-4B混合注意力架构原理…": the sliding cache keeps the
 *     512 most recent tokens and drops older ones).
 *
 * Conventions shared by every entry point
 *   - Tensors are caller-owned device memory (bf16 unless stated), dense,
 *     row-major in the layouts given below, 16-byte aligned.
 *   - The library allocates no device memory and keeps no state beyond the
 *     profiling events below, except that the attention-block entry points
 *     create one hipBLASLt handle per device on first use and cache their
 *     GEMM plans. Every call only enqueues work on `stream`
 *     (NULL = the default stream); results are valid after the stream
 *     synchronises.
 *   - Return value: HATTN_OK (0) or a negative hattn_status; arguments are
 *     validated on the host before anything is enqueued, so an error return
 *     leaves device memory untouched. hattn_status_string() names a code.
 *   - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 *     Only a group size of 4 and head_dim 256 are supported (both model
 *     shapes on the page); other values return HATTN_ERR_UNSUPPORTED.
 *   - Mask: a query at position p_q sees a key at position p_k iff
 *     p_k <= p_q and, with a window w > 0, p_q - p_k < w (itself plus the
 *     w - 1 previous tokens).
 *   - RoPE: r = head_dim * rotary_fraction rotated channels (a positive even
 *     integer); channel i < r/2 pairs with channel i + r/2 and turns by the
 *     angle p * theta^(-2i/r), formed in fp64; channels >= r pass through.
 *     Rotated values are rounded once to bf16 (round to nearest even).
 *   - Caches store the rotated key and the value as bf16, layout
 *     [batch][num_kv_heads][capacity][head_dim]. A linear cache keeps
 *     position p in slot p. A ring cache (sliding layers only) has
 *     capacity == window and keeps position p in slot p mod capacity. A
 *     paged cache (full layers only) keeps slot p in a page of a shared
 *     pool (hattn_kv_cache below).
 *   - Positions are int32 in [0, 2^30).
 *   - Calls that touch the same cache must be ordered on one stream.
 */
#ifndef HATTN_H
#define HATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HATTN_OK = 0,
  HATTN_ERR_NULL = -1,        /* a required pointer is NULL                     */
  HATTN_ERR_SHAPE = -2,       /* a size is <= 0 or inconsistent                 */
  HATTN_ERR_UNSUPPORTED = -3, /* head_dim != 256, group != 4, unknown gate_act  */
  HATTN_ERR_ROPE = -4,        /* theta <= 0 or head_dim*fraction not even int   */
  HATTN_ERR_WINDOW = -5,      /* sliding layer with window < 1, full with > 0   */
  HATTN_ERR_CACHE = -6,       /* cache kind/capacity/batch/paging does not fit  */
  HATTN_ERR_CAPACITY = -7,    /* a position does not fit the linear cache       */
  HATTN_ERR_WORKSPACE = -8,   /* workspace NULL or smaller than required        */
  HATTN_ERR_ALIGN = -9,       /* a tensor pointer is not 16-byte aligned        */
  HATTN_ERR_LAUNCH = -10,     /* the HIP runtime refused a launch               */
  HATTN_ERR_POSITION = -11    /* a host-side position is negative or too large  */
} hattn_status;

typedef enum { HATTN_LAYER_SLIDING = 0, HATTN_LAYER_FULL = 1 } hattn_layer_type;
/* Activation of the per-head output gate (page §3 逐头输出门控): sigmoid(g),
 * as in Eq. 1 and both released checkpoints, or silu(g) = g * sigmoid(g),
 * the alternative gate mode the model code supports. Evaluated in fp32. */
typedef enum { HATTN_GATE_SIGMOID = 0, HATTN_GATE_SILU = 1 } hattn_gate_act;
typedef enum { HATTN_KV_RING = 0, HATTN_KV_LINEAR = 1, HATTN_KV_PAGED = 2 } hattn_kv_kind;

/* Parameters of one attention layer (page §1 config table, §2, §4 table). */
typedef struct {
  int32_t layer_type;      /* hattn_layer_type                                  */
  int32_t window;          /* sliding: >= 1 (512 on the page); full: <= 0       */
  double rope_theta;       /* 1e4 sliding, 5e6 full                             */
  double rotary_fraction;  /* 1.0 sliding, 0.25 full                            */
  int32_t num_q_heads;     /* 16 (4B) or 8 (1.7B)                               */
  int32_t num_kv_heads;    /* 4 (4B) or 2 (1.7B)                                */
  int32_t head_dim;        /* 256                                               */
  int32_t gate_act;        /* hattn_gate_act; 0 (sigmoid) unless set            */
} hattn_layer_desc;

/* A caller-owned KV cache of one layer.
 *
 * Ring and linear caches: k, v are bf16 [batch][num_kv_heads][capacity][256].
 *
 * Paged caches (full layers only; the serving setting of page §6's closing
 * notes, where a 1M-token context's full-layer KV alone takes ~37 GB): k, v
 * are a pool of pages, bf16 [num_pages][num_kv_heads][page_size][256], and
 * block_table (DEVICE int32 [batch][capacity / page_size]) maps sequence
 * b's slot p (the token at position p, as in a linear cache) to row
 * p % page_size of page block_table[b][p / page_size]. page_size is a
 * multiple of 64 and capacity a multiple of page_size with at most 4096
 * pages per sequence. A table entry must name a pool page (0 .. num_pages-1)
 * for every page that holds a position a call reads or writes; the kernels
 * never touch memory outside the pool: an entry outside that range is
 * clamped into it for reads (the result is then unspecified) and its writes
 * are dropped. Pages may be shared between sequences only for positions
 * no call writes. */
typedef struct {
  void* k;           /* bf16 cache or page pool (layouts above)                 */
  void* v;           /* bf16, same layout                                       */
  int32_t kind;      /* hattn_kv_kind                                           */
  int32_t batch;     /* number of sequences                                     */
  int32_t capacity;  /* slots per (sequence, kv head); ring: == window          */
  int32_t page_size; /* paged: slots per page; otherwise ignored                */
  const int32_t* block_table; /* paged: device int32 [batch][capacity/page_size] */
  int32_t num_pages; /* paged: pages in the pool                                */
} hattn_kv_cache;

/* Fill *out with the page's parameters of a layer type (§2, §4 table) for
 * the given head counts, head_dim 256. */
int hattn_layer_defaults(int32_t layer_type, int32_t num_q_heads,
                         int32_t num_kv_heads, hattn_layer_desc* out);

/* RoPE in place (page §4 分层 RoPE, table and text).
 * x: bf16 [n_tok][n_heads][head_dim], device; pos: int32 [n_tok], device.
 * Rotates the first head_dim*rotary_fraction channels of every head of
 * token t by pos[t] as described above; the other channels are untouched. */
int hattn_rope_apply(void* x, int32_t n_tok, int32_t n_heads, int32_t head_dim,
                     const int32_t* pos, double theta, double rotary_fraction,
                     hipStream_t stream);

/* Bytes of device workspace hattn_prefill needs for this call shape. */
size_t hattn_prefill_workspace_size(const hattn_layer_desc* desc,
                                    const hattn_kv_cache* cache,
                                    int32_t batch, int32_t seq_len);

/* Prefill (page §2, §3 Eq. 1, §4): S new tokens per sequence at positions
 * start_pos[b] + 0 .. S-1, attending to the cache history plus themselves.
 *   q:    bf16 [B][S][num_q_heads][256]  (before RoPE)
 *   k, v: bf16 [B][S][num_kv_heads][256] (k before RoPE)
 *   gate: bf16 [B][S][num_q_heads] gate logits
 *   start_pos: int32 [B], HOST memory. A linear cache must hold positions
 *     0 .. start_pos[b]-1 and have capacity >= start_pos[b] + S. A ring
 *     cache must hold positions up to start_pos[b]-1 as ring slots.
 *   out:  bf16 [B][S][num_q_heads][256]; must not alias any input.
 * Cache slots outside the history may hold any bits, NaN included; they
 * never reach the result. The rotated keys and the values of the new tokens
 * are written to the cache (a ring keeps the last min(S, capacity) of
 * them). Limits, beyond which a call returns HATTN_ERR_UNSUPPORTED: B <=
 * 128; the key rows of one (sequence, KV head) -- a linear cache's
 * capacity, or window - 1 + S for a ring; paged caches are addressed page
 * by page and exempt -- at most 2^23; ceil(S / 32) * B * num_kv_heads
 * below 2^31; num_q_heads at most 65,536 (a query block's rows are read
 * with 32-bit byte offsets).
 * Numerics: keys are rotated in fp64 and cached as bf16 (one rounding);
 * the scores take the rotated queries as bf16 on full layers and as a bf16
 * high part plus a bf16 low part (~16 significant bits) on sliding layers;
 * products accumulate in fp32, probabilities enter P.V as bf16, and the
 * gated output is rounded once to bf16. */
int hattn_prefill(const hattn_layer_desc* desc, const void* q, const void* k,
                  const void* v, const void* gate, int32_t batch,
                  int32_t seq_len, const int32_t* start_pos,
                  const hattn_kv_cache* cache, void* out, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/* Ragged prefill: sequences with different numbers of new tokens in one
 * call (same page passages as hattn_prefill). New tokens are packed:
 *   cu_seqlens: int32 [B+1], HOST memory, cu_seqlens[0] = 0 and
 *     non-decreasing; sequence b's new tokens are packed rows
 *     cu_seqlens[b] .. cu_seqlens[b+1]-1 (none when equal).
 *   q: bf16 [T][num_q_heads][256], k, v: bf16 [T][num_kv_heads][256],
 *   gate: bf16 [T][num_q_heads], out: bf16 [T][num_q_heads][256], with
 *   T = cu_seqlens[B].
 *   start_pos, cache, workspace, stream: as for hattn_prefill; sequence b's
 *   token i sits at position start_pos[b] + i.
 * With every length equal to S this is hattn_prefill (the same layout, the
 * same kernels, the same bits). A sequence with no new tokens leaves its
 * cache untouched. Errors as for hattn_prefill; a decreasing or not
 * zero-based cu_seqlens is HATTN_ERR_SHAPE. */
size_t hattn_prefill_varlen_workspace_size(const hattn_layer_desc* desc,
                                           const hattn_kv_cache* cache,
                                           int32_t batch,
                                           const int32_t* cu_seqlens);
int hattn_prefill_varlen(const hattn_layer_desc* desc, const void* q,
                         const void* k, const void* v, const void* gate,
                         int32_t batch, const int32_t* cu_seqlens,
                         const int32_t* start_pos,
                         const hattn_kv_cache* cache, void* out,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Bytes of device workspace hattn_decode needs for a batch. */
size_t hattn_decode_workspace_size(const hattn_layer_desc* desc,
                                   const hattn_kv_cache* cache, int32_t batch);

/* Decode (page §2, §3 Eq. 1, §4; the explainer's per-step cache update): one
 * new token per sequence at position pos[b].
 *   q:    bf16 [B][num_q_heads][256], k, v: bf16 [B][num_kv_heads][256]
 *   gate: bf16 [B][num_q_heads]
 *   pos:  int32 [B], DEVICE memory; max_pos: a host upper bound of pos[]
 *     (checked against a linear or paged cache's capacity).
 *   out:  bf16 [B][num_q_heads][256]
 * The cache must hold positions 0 .. pos[b]-1 (slots outside the visible
 * range may hold any bits, NaN included; they never reach the result). The
 * new rotated key and value are written to their slot, and the attention
 * includes them. A pos[b] outside [0, max_pos] yields a NaN output row and
 * no cache write. The call holds no host synchronisation and reads the
 * positions on the device, so it can be captured in a HIP graph and
 * replayed with new positions. */
int hattn_decode(const hattn_layer_desc* desc, const void* q, const void* k,
                 const void* v, const void* gate, int32_t batch,
                 const int32_t* pos, int32_t max_pos,
                 const hattn_kv_cache* cache, void* out, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* Decode without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Arguments, results and errors are those of
 * hattn_decode; the split partials live instead in a library-owned device
 * array of HATTN_DECODE_STATIC_SCRATCH_BYTES per GPU, reserved when the
 * library is loaded and held until the process ends. Its device address is
 * looked up once per device, on the first call with that device current (a
 * symbol lookup, no allocation); the call itself makes no hipMalloc, hipFree
 * or other allocating call. A plan needing more than the array returns
 * HATTN_ERR_WORKSPACE (with a GQA group of 4 no plan does: at most
 * 4 x (1024 + 255) partial rows of 1,032 bytes). Every call on a GPU shares
 * that GPU's array and leaves its partials there; nothing in it needs to
 * start at zero. Calls that overlap on one GPU (concurrent streams, or
 * graphs replayed concurrently) race on the array: order them. */
#define HATTN_DECODE_STATIC_SCRATCH_BYTES (6u << 20)
int hattn_decode_static(const hattn_layer_desc* desc, const void* q,
                        const void* k, const void* v, const void* gate,
                        int32_t batch, const int32_t* pos, int32_t max_pos,
                        const hattn_kv_cache* cache, void* out,
                        hipStream_t stream);

/* ------------------------------------------------------------------------
 * The attention block around the core (page §2 figure 1, the decoder
 * layer's dataflow; §1 config table; §3; §5): with x the block input, the
 * fp32 residual stream (§5: the input embedding is taken to fp32 for the
 * backbone),
 *   h = RMSNorm(x)                     fp32, times the weight, cast to bf16
 *   [q | k | v | g] = h W_qkvg^T       q_k_v_proj and g_proj, bf16 outputs
 *   a = attention core(q, k, v, g)     as hattn_prefill_varlen / hattn_decode
 *   out = x + a W_o^T                  out_proj (bf16), then the residual add
 *                                      in fp32 (out stays fp32)
 * Linear layers have no bias (page §5: attention_bias false). The GEMMs are
 * bf16 in and out with fp32 accumulation: for at most 64 tokens (decode
 * batches) this library's weight-streaming kernel, whose out_proj
 * epilogue also does the residual add (same rounding: the bf16 projection
 * is added to the fp32 residual), otherwise hipBLASLt through one handle
 * per device, created on first use. The first hipBLASLt
 * call of a GEMM shape outside stream capture times a few candidates on its
 * own buffers and waits for them (once per shape and process); later calls,
 * and calls under capture, do not wait.
 */
typedef struct {
  const void* norm_weight;  /* bf16 [hidden]: the input RMSNorm's weight    */
  const void* qkvg_weight;  /* bf16 [(num_q_heads + 2 num_kv_heads) * 256 +
                               num_q_heads][hidden]: the q_k_v_proj rows (Q,
                               then K, then V; 6144 on the 4B shape) followed
                               by the g_proj rows (one per query head)       */
  const void* o_weight;     /* bf16 [hidden][num_q_heads * 256]: out_proj    */
  int32_t hidden;           /* 2560 (4B) or 2048 (1.7B); a multiple of 8     */
  float rms_eps;            /* the RMSNorm epsilon, > 0                      */
} hattn_block_weights;

/* Prefill of the block over a ragged batch, layouts as hattn_prefill_varlen:
 *   x:   fp32 [T][hidden] block inputs of the packed new tokens
 *   out: fp32 [T][hidden]; may be x (the residual stream updated in place)
 * The rotated keys and the values go to the cache as in hattn_prefill.
 * Errors: as hattn_prefill_varlen, plus HATTN_ERR_SHAPE for a hidden size
 * that is not a positive multiple of 8 or rms_eps <= 0, HATTN_ERR_NULL for
 * a missing weight, and HATTN_ERR_LAUNCH when hipBLASLt fails. */
size_t hattn_block_prefill_workspace_size(const hattn_layer_desc* desc,
                                          const hattn_block_weights* w,
                                          const hattn_kv_cache* cache,
                                          int32_t batch,
                                          const int32_t* cu_seqlens);
int hattn_block_prefill(const hattn_layer_desc* desc,
                        const hattn_block_weights* w, const void* x,
                        int32_t batch, const int32_t* cu_seqlens,
                        const int32_t* start_pos, const hattn_kv_cache* cache,
                        void* out, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* Decode of the block: x, out fp32 [B][hidden] (out may be x); pos,
 * max_pos and the cache as in hattn_decode. Errors as hattn_decode plus
 * those of hattn_block_prefill's weights. */
size_t hattn_block_decode_workspace_size(const hattn_layer_desc* desc,
                                         const hattn_block_weights* w,
                                         const hattn_kv_cache* cache,
                                         int32_t batch);
int hattn_block_decode(const hattn_layer_desc* desc,
                       const hattn_block_weights* w, const void* x,
                       int32_t batch, const int32_t* pos, int32_t max_pos,
                       const hattn_kv_cache* cache, void* out,
                       void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * KV planner (page §6 参数与 KV Cache 估算, KV table: K and V of every KV
 * head in bf16, 2 * num_kv_heads * 256 * 2 bytes per token and layer; full
 * layers keep every token, sliding layers at most the window; §2: layer i
 * (counting from 0) is a full layer iff i mod 4 == 3).
 *
 * hattn_kv_plan lays out the caches of a whole layer stack in one arena:
 *   layer_types: int32 [n_layers] hattn_layer_type, HOST memory, or NULL
 *     for the page's schedule (full iff i mod 4 == 3).
 *   batch: sequences; max_tokens: the largest context (positions
 *     0 .. max_tokens-1) any sequence will reach, 1 .. 2^30.
 *   window: the sliding layers' window (512 on the page), >= 1.
 *   plan: HOST array of n_layers entries, filled in.
 *   arena_bytes: receives the arena size the plan needs.
 * A full layer gets a linear cache of capacity max_tokens. A sliding layer
 * gets a ring of capacity == window when max_tokens > window, else a linear
 * cache of capacity max_tokens (the same visible set, no slot ever reused),
 * so its size is min(max_tokens, window) tokens, as on the page's table.
 * Every K and V block starts on a 256-byte boundary; blocks follow layer
 * order, K before V. Pure host arithmetic: nothing is allocated or enqueued.
 * Errors: HATTN_ERR_NULL (plan or arena_bytes NULL), HATTN_ERR_SHAPE
 * (n_layers, batch, num_kv_heads or max_tokens out of range, an unknown
 * layer type), HATTN_ERR_WINDOW (window < 1). */
typedef struct {
  int32_t layer_type;  /* hattn_layer_type                                    */
  int32_t kind;        /* hattn_kv_kind                                       */
  int32_t capacity;    /* slots per (sequence, kv head)                       */
  int32_t num_kv_heads;
  int32_t batch;       /* sequences                                           */
  int32_t reserved;    /* 0                                                   */
  uint64_t k_offset;   /* byte offset of the K block in the arena             */
  uint64_t v_offset;   /* byte offset of the V block                          */
  uint64_t bytes;      /* K + V bytes of the layer (padding excluded)         */
} hattn_kv_layer_plan;

int hattn_kv_plan(int32_t n_layers, const int32_t* layer_types,
                  int32_t num_kv_heads, int32_t batch, int32_t max_tokens,
                  int32_t window, hattn_kv_layer_plan* plan,
                  uint64_t* arena_bytes);

/* The cache descriptor of one planned layer inside an arena (device memory
 * of at least arena_bytes, 256-byte aligned, owned by the caller): k and v
 * point at arena + the layer's offsets. Errors: HATTN_ERR_NULL,
 * HATTN_ERR_ALIGN (arena not 256-byte aligned), HATTN_ERR_SHAPE (an
 * inconsistent plan entry). */
int hattn_kv_cache_at(const hattn_kv_layer_plan* layer, void* arena,
                      hattn_kv_cache* out);

/* Profiling hook for benchmarks. While enabled, every hattn_prefill records
 * a HIP event pair around its attention kernel (HATTN_PROFILE_PREFILL) and
 * every hattn_decode around its attention and merge kernels
 * (HATTN_PROFILE_DECODE), on the call's stream. hattn_profile_read waits for
 * the recorded events of one kind, returns how many pairs there were and
 * their summed elapsed milliseconds, and forgets them. Not thread-safe. */
typedef enum { HATTN_PROFILE_PREFILL = 0, HATTN_PROFILE_DECODE = 1 } hattn_profile_kind;
int hattn_profile_enable(int enable);
int hattn_profile_read(int kind, int64_t* count, double* total_ms);

/* The shader clock the prefill attention kernel ran at while profiling was
 * enabled: each workgroup of each profiled hattn_prefill adds its elapsed
 * shader clock ticks (s_memtime) and real-time counter ticks
 * (s_memrealtime) to two counters on the GPU; this returns their ratio times
 * the real-time counter's rate (hipDeviceAttributeWallClockRate), in GHz,
 * for the current device, and sets both counters back to zero
 * (hattn_profile_enable(1) zeroes them too). 0 when nothing was recorded.
 * Synchronises the device. Errors: HATTN_ERR_NULL, HATTN_ERR_LAUNCH. */
int hattn_profile_read_clock(double* shader_ghz);

/* Name of a status code (static string). */
const char* hattn_status_string(int status);

/* Test hook: the device index helpers the kernels use, evaluated on a grid.
 * For n_q queries at positions q_pos0 + i and n_keys key slots of a cache
 * of the given kind/capacity whose next position to write is q_pos0 + i
 * (decode view), writes
 *   mask[i][j] (uint8): 1 iff query i sees the key in slot j
 *   key_pos[i][j] (int32): position held by slot j (-1 if never written)
 *   slot[i] (int32): slot that query i's own token is written to.
 * All three outputs are device buffers. */
int hattn_debug_index_probe(const hattn_layer_desc* desc, int32_t kv_kind,
                            int32_t capacity, int32_t q_pos0, int32_t n_q,
                            uint8_t* mask, int32_t* key_pos, int32_t* slot,
                            hipStream_t stream);

/* Measurement probes (not on the attention path; used by the benchmark to
 * put the kernels' rates beside what the chip itself delivers).
 * hattn_debug_read_probe: streams `bytes` (a multiple of 16) of device
 *   memory with `blocks` 256-thread blocks, 16-byte loads, eight in flight
 *   per thread; sink: device uint32 [blocks], written only in a case random
 *   data never meets (it keeps the loads alive).
 * hattn_debug_mfma_probe: `blocks` blocks of four waves each run `iters`
 *   rounds of 8 independent bf16 MFMA 32x32x16 (262,144 flop per wave and
 *   round) on pseudo-random operands; sink: device float [blocks][4].
 * hattn_debug_lds_probe: `blocks` blocks of four waves (64 KiB of LDS, one
 *   per CU) each run `iters` rounds of LDS fragment reads as the prefill
 *   kernel issues them; mode 0: 8 ds_read_b128 per wave and round (32 KiB
 *   per block and round), mode 1: 8 ds_read_b64_tr_b16 (16 KiB), mode 2:
 *   64 bf16 MFMA 32x32x16 per wave and round with 32 b128 and 64 transposed
 *   reads among them (the prefill step without its softmax and tile loads).
 *   out: device uint64 [blocks][2]; out[2b] receives block b's elapsed
 *   shader clock ticks (s_memtime of its first wave), out[2b + 1] is written
 *   only in a case the data never meets.
 * Errors: HATTN_ERR_SHAPE, _NULL, _ALIGN as for the other entry points. */
int hattn_debug_read_probe(const void* buf, size_t bytes, int32_t blocks,
                           uint32_t* sink, hipStream_t stream);
int hattn_debug_mfma_probe(int32_t blocks, int32_t iters, float* sink,
                           hipStream_t stream);
int hattn_debug_lds_probe(int32_t mode, int32_t blocks, int32_t iters,
                          uint64_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HATTN_H */
