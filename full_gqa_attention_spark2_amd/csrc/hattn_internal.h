// Host-side plans and launch wrappers shared by the C-ABI layer and the
// kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace hattn {

constexpr int kMaxPrefillBatch = 128;
constexpr int kPrefillBlockQ = 32;   // query positions per prefill workgroup
constexpr long long kMaxPrefillKeyRows = 1LL << 23;  // key rows per (sequence, KV head) slab
constexpr int kMaxPagesPerSeq = 4096;  // block-table entries per sequence of a paged cache
constexpr int kMinPageSize = 64;       // a paged cache's page size is a multiple of this

// A paged cache as the kernels see it: pool [num_pages][Hkv][page_size][256],
// slot p of sequence b in page table[b * pages_per_seq + p / page_size].
// table == nullptr: not paged.
struct PagedKv {
  const int* table;
  int page_size;
  int pages_per_seq;
  int num_pages;
};

// Per new prefill token: cos/sin of its RoPE angles (fp32 table for the
// attention kernel's query rotation) and its rotated key and value, written
// as rows of dst (a cache or the staging buffer, [B][Hkv][rows][256]).
// New tokens are packed: sequence b's token i is row tok0[b] + i of k, v
// and the table, for i < len[b].
struct PrefillPrepArgs {
  const uint16_t* k;      // bf16 [T][Hkv][256], token rows kv_stride elements apart
  const uint16_t* v;
  long long kv_stride;    // Hkv * 256 when dense
  float2* table;          // [T][r/2] (cos, sin)
  uint16_t* dst_k;
  uint16_t* dst_v;
  int B, max_len, Hkv;
  int dst_rows;     // rows per (b, kv head) in dst (not paged)
  PagedKv paged;    // dst is a paged cache's pool (slot = position)
  int r;            // rotated channels
  uint16_t* ring_k; // ring cache that also receives each sequence's last
  uint16_t* ring_v; //   min(len, ring_cap) tokens (or null)
  int ring_cap;
  double inv_freq[128];
  int start[kMaxPrefillBatch];    // position of token 0 of sequence b
  int dst_row0[kMaxPrefillBatch]; // dst row of token 0 of sequence b
  int tok0[kMaxPrefillBatch];     // packed row of token 0 of sequence b
  int len[kMaxPrefillBatch];      // new tokens of sequence b
};

// Copies between a ring cache and the linear staging buffer.
struct RingCopyArgs {
  uint16_t* ring_k;
  uint16_t* ring_v;
  uint16_t* stage_k;
  uint16_t* stage_v;
  int B, Hkv, cap, stage_rows;
  int count[kMaxPrefillBatch];     // rows to copy for sequence b
  int first_pos[kMaxPrefillBatch]; // position of the first copied row
  int stage_row0[kMaxPrefillBatch];// staging row of the first copied row
};

// Queries are packed like the new tokens of PrefillPrepArgs.
struct PrefillAttnArgs {
  const uint16_t* q;      // bf16 [T][Hq][256], before RoPE; token rows q_stride apart
  long long q_stride;     // Hq * 256 when dense
  long long gate_stride;  // Hq when dense
  const float2* table;    // [T][r/2] cos/sin of the query positions
  const uint16_t* kc;     // bf16 [B][Hkv][rows][256], rotated keys (or a paged pool)
  const uint16_t* vc;
  PagedKv paged;          // key row j of sequence b is slot j of the paged cache
  const uint16_t* gate;   // bf16 [T][Hq]
  uint16_t* out;          // bf16 [T][Hq][256]
  int B, Hq, Hkv;
  int rows;               // rows per (b, kv head) in kc / vc
  int window;             // <= 0: unbounded
  int r;                  // rotated channels (multiple of 16)
  int q_tiles;            // ceil(max len / kPrefillBlockQ)
  int gate_act;           // 0 sigmoid, 1 silu
  int start[kMaxPrefillBatch];     // position of query 0
  int key_pos0[kMaxPrefillBatch];  // position held by key row 0
  int n_keys[kMaxPrefillBatch];    // valid key rows
  int tok0[kMaxPrefillBatch];      // packed row of query 0
  int len[kMaxPrefillBatch];       // queries of sequence b
  // When not null (profiling on): each workgroup adds its elapsed shader
  // clock ticks to [0] and real-time counter ticks to [1].
  unsigned long long* clock_acc;
};

struct DecodeArgs {
  const uint16_t* q;      // bf16 [B][Hq][256]
  const uint16_t* k;      // bf16 [B][Hkv][256]
  const uint16_t* v;
  long long q_stride;     // elements between sequences' rows of q (Hq * 256 when dense),
  long long kv_stride;    //   of k and v (Hkv * 256), and of gate (Hq)
  long long gate_stride;
  const uint16_t* gate;   // bf16 [B][Hq]
  const int* pos;         // int32 [B], device
  uint16_t* kc;           // cache [B][Hkv][cap][256] (or a paged pool)
  uint16_t* vc;
  PagedKv paged;
  uint16_t* out;          // bf16 [B][Hq][256]
  float* part_o;          // [B][Hq][nsplit][256]
  float* part_ml;         // [B][Hq][nsplit][2]
  int B, Hq, Hkv, cap, ring, window, max_pos;
  int r;
  int nsplit;
  int split_keys;         // keys per split, multiple of 128
  int gate_act;           // 0 sigmoid, 1 silu
  double inv_freq[128];
};

struct RopeApplyArgs {
  uint16_t* x;
  const int* pos;
  int n_tok, n_heads, head_dim, r;
  double inv_freq[256];
};

struct ProbeArgs {
  uint8_t* mask;
  int* key_pos;
  int* slot;
  int ring, cap, window, q_pos0, n_q;
};

// Input RMSNorm of the attention block: y[t] = bf16(w * x[t] / rms(x[t]))
// from the fp32 residual stream x.
struct RmsNormArgs {
  const float* x;     // fp32 [T][H]
  const uint16_t* w;  // bf16 [H]
  uint16_t* y;        // bf16 [T][H]
  int T, H;           // H a multiple of 8
  float eps;
};

// Skinny GEMM of the attention block's decode projections:
// d[T][N] = a[T][K] . w[N][K]^T, bf16, fp32 accumulation, T <= 64.
struct SkinnyGemmArgs {
  const uint16_t* w;  // [N][K]
  const uint16_t* a;  // [T] rows lda elements apart
  uint16_t* d;        // [T] rows ldd elements apart (unused when out is set)
  int N, K, T;
  long long lda, ldd;
  // Optional residual epilogue: out = x + bf16(D) in fp32, [T] rows ldd
  // elements apart (out may be x); d is not written then.
  const float* x;
  float* out;
};

// Kernel arguments travel by value; keep each struct within 4 KiB.
static_assert(sizeof(PrefillPrepArgs) <= 4096, "kernel argument size");
static_assert(sizeof(RingCopyArgs) <= 4096, "kernel argument size");
static_assert(sizeof(PrefillAttnArgs) <= 4096, "kernel argument size");
static_assert(sizeof(DecodeArgs) <= 4096, "kernel argument size");
static_assert(sizeof(RopeApplyArgs) <= 4096, "kernel argument size");

}  // namespace hattn

#include "hattn.h"

namespace hattn {

// The C-ABI prefill over packed new tokens (sequence b: rows tok0[b] ..
// tok0[b] + len[b] - 1) and decode, with token rows of q, k/v and gate
// q_stride, kv_stride and gate_stride elements apart. Validation as in the
// public entry points; return a hattn_status. With static_scratch, decode
// takes its split partials from the static array of hattn_decode_static
// (workspace_bytes is that array's size; workspace is ignored).
int prefill_packed(const hattn_layer_desc* desc, const void* q, const void* k, const void* v,
                   const void* gate, int32_t batch, const int* tok0, const int* len, long long total,
                   const int32_t* start_pos, const hattn_kv_cache* cache, void* out, void* workspace,
                   size_t workspace_bytes, hipStream_t stream, long long q_stride, long long kv_stride,
                   long long gate_stride);
int decode_strided(const hattn_layer_desc* desc, const void* q, const void* k, const void* v,
                   const void* gate, int32_t batch, const int32_t* pos, int32_t max_pos,
                   const hattn_kv_cache* cache, void* out, void* workspace, size_t workspace_bytes,
                   hipStream_t stream, long long q_stride, long long kv_stride, long long gate_stride,
                   bool static_scratch = false);
// The layer descriptor, a positive batch and the cache's kind, batch,
// capacity and paging, as the public entry points check them; with
// `pointers` also the cache's pointers. Returns a hattn_status.
int validate_layer_cache(const hattn_layer_desc* desc, const hattn_kv_cache* cache, int batch, bool pointers);
// Workspace bytes of prefill_packed / decode_strided.
size_t prefill_workspace_bytes(const hattn_layer_desc* desc, const hattn_kv_cache* cache, int batch,
                               long long total_tokens, int max_len);
size_t decode_workspace_bytes(const hattn_layer_desc* desc, const hattn_kv_cache* cache, int batch);

hipError_t launch_prefill_prep(const PrefillPrepArgs& a, hipStream_t s);
hipError_t launch_ring_to_stage(const RingCopyArgs& a, hipStream_t s);
hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t s);
// Device address of the current device's prefill clock accumulators (two
// unsigned 64-bit counters, see PrefillAttnArgs::clock_acc).
hipError_t prefill_clock_acc(unsigned long long** ptr);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// Device address of the current device's static decode scratch
// (HATTN_DECODE_STATIC_SCRATCH_BYTES), looked up on first use per device.
hipError_t decode_static_scratch(void** ptr);
hipError_t launch_rope_apply(const RopeApplyArgs& a, hipStream_t s);
hipError_t launch_index_probe(const ProbeArgs& a, hipStream_t s);
hipError_t launch_rms_norm(const RmsNormArgs& a, hipStream_t s);
// Whether the skinny GEMM takes a shape (T <= 64, K a multiple of 512, N,
// lda, ldd multiples of 8, 16-byte aligned pointers), and its launch.
bool skinny_gemm_fits(int N, int K, int T, long long lda, long long ldd, const void* w, const void* a,
                      const void* d);
hipError_t launch_skinny_gemm(const SkinnyGemmArgs& g, hipStream_t s);
hipError_t launch_read_probe(const void* buf, size_t bytes, int blocks, uint32_t* sink, hipStream_t s);
hipError_t launch_mfma_probe(int blocks, int iters, float* sink, hipStream_t s);
hipError_t launch_lds_probe(int mode, int blocks, int iters, unsigned long long* out, hipStream_t s);
hipError_t launch_residual_add(const float* x, const uint16_t* y, float* out, long long n, hipStream_t s);

}  // namespace hattn
