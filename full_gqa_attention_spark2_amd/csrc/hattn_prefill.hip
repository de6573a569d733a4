// Flash-style prefill attention for gfx950 (page "Spark-X2.5 架构（4B / 1.7B）",
// §3 Eq. 1: softmax(Q K^T / sqrt(256)) V times a per-head gate (sigmoid, or silu,
// the alternative the section mentions); §2:
// causal mask, plus the 512-token window on sliding layers; §4: the queries'
// partial RoPE).
//
// One workgroup = one (sequence, KV head, block of 32 query positions); its
// four waves are the four query heads of the GQA group, so every K/V tile
// staged in LDS feeds 4 x 32 query rows.
//
// Per 64-key tile and wave (bf16 MFMA 32x32x16, fp32 accumulate):
//   S^T[64 keys][32 q]  = K_tile . Q^T    (A = K from LDS, B = Q in registers)
//   online softmax per query column: one lane pair holds a query's 64 scores
//   O^T[256 d][32 q]   += V_tile^T . P^T  (A = V^T via ds_read_tr16_b64, B = P)
// The transposed orientation keeps a query's running max, sum and rescale
// factor in one lane.
//
// K and V tiles go from global memory straight into LDS by LDS DMA (buffer
// loads, 16 B per lane; each instruction fills one 1 KiB block from eight
// whole 128-byte lines) in a swizzled layout that keeps the MFMA fragment
// reads free of bank conflicts. Two K slots and two V slots form a pipeline:
// step t runs S(t+1) and P(t-1).V(t-1) on the matrix cores while the VALU
// computes the softmax of tile t, and K(t+2) and V(t) load meanwhile. Each
// wave issues its share of those loads at its own point of the matrix-core
// stream (wave w before element kLoadSpacing * w): the CU's load pipe takes
// the four shares one after another, so no wave waits behind the others'.
// The running max is only moved (and O rescaled) when a tile's max exceeds
// it by more than 2^8, so most tiles skip the rescale. On sliding-window
// layers the queries enter the scores as bf16 high + low parts (two S MFMAs
// per K fragment), for error margin.
#include <mutex>
#include <type_traits>

#include "hattn_device.h"
#include "hattn_internal.h"

// Clock accumulators of the profiling hook (sums of shader clock ticks and of
// real-time counter ticks over the profiled workgroups), one pair per GPU.
// Host code uses their device address from prefill_clock_acc(), never the
// symbol itself.
static __device__ unsigned long long clock_acc[2];

namespace hattn {

namespace {

constexpr int kBM = kPrefillBlockQ;              // query positions per workgroup
constexpr int kBN = 64;                          // keys per tile
constexpr int kTileBytes = kBN * kHeadDim * 2;   // 32 KiB: one K or V tile
constexpr float kScoreScale = kLog2e / 16.0f;    // 1/sqrt(256), in log2 units
constexpr float kRescaleSlack = 8.0f;            // log2 units

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4q __attribute__((ext_vector_type(4)));  // a buffer descriptor in scalar registers
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ s16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Buffer resource over one (sequence, KV head) slab of key rows (raw
// buffer, byte offsets, bounds = the slab size).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from the slab at byte offset voff + soff into LDS;
// lane l lands at lds + 16*l. (A buffer load rather than a global one: the
// compiler can then count LDS reads precisely around it instead of draining
// them.)
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}

// Larger of two scores. IEEE maximum (a NaN operand gives NaN, where fmaxf
// would return the other operand); the two agree on the finite and -inf
// values the softmax sees. It compiles to v_maximum3_f32 chains, while
// fmaxf on values the compiler cannot see into (the pinned scores) needs a
// canonicalising v_max per operand first.
__device__ __forceinline__ float max_f(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max and sum of a value over the lane pair (l, l ^ 32), by a VALU lane
// swap (no LDS traffic). After the swap of x with itself, lanes below 32
// hold (x[l], x[l + 32]) and the others (x[l - 32], x[l]): the pair in the
// same order on both lanes.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_u32(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Two floats to packed bf16 (low half first), rounded to nearest even by
// the hardware conversion (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)lo, (__bf16)hi});
}

__device__ __forceinline__ void unpack8(uint4 u, float* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Matrix-core streams of one tile step (see mma_stream in the kernel).
constexpr int kStreamS = 0;    // S^T only (first tile)
constexpr int kStreamSPv = 1;  // S^T of tile t+1 interleaved with P.V of tile t-1
constexpr int kStreamPv = 2;   // P.V only (last tile)
constexpr int stream_length(int mode) { return mode == kStreamSPv ? 64 : 32; }
constexpr int kRing = 4;  // fragment registers per operand kind
// LDS reads run this many stream elements ahead of their MFMA
constexpr int stream_ahead(int mode) { return mode == kStreamSPv ? 6 : 3; }
// A fragment register is rewritten by the read of the same-kind element
// kRing places later, so fewer than kRing same-kind reads may be ahead of
// an MFMA (in the mixed stream the kinds alternate).
static_assert(stream_ahead(kStreamS) < kRing && stream_ahead(kStreamPv) < kRing &&
                  stream_ahead(kStreamSPv) / 2 < kRing,
              "LDS read look-ahead overruns the fragment register ring");
// Stream elements between two waves' tile-load points. Every wave's point
// must fall inside the shortest stream that carries loads (the first step's).
constexpr int kLoadSpacing = 8;
static_assert(4 * kLoadSpacing <= stream_length(kStreamS), "a wave's tile loads would never be issued");
constexpr int stream_reads(int mode, int e) {  // LDS reads feeding element e
  return mode == kStreamS ? 1 : mode == kStreamPv ? 2 : ((e & 1) ? 2 : 1);
}

// f(integral_constant<int, I>) for I = B .. E-1, expanded at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Scheduling-group barriers for one stream, in issue order: the reads of
// the first `ahead` elements, then per element one MFMA, the reads of
// element e + ahead and up to kValu VALU / transcendental instructions (the
// softmax that runs beside the stream). Barriers only constrain the
// instructions that precede them in the same basic block.
// With split queries an S element is two MFMAs (the queries' high and low
// bf16 parts against the same K fragment).
constexpr int kSoftmaxValuPerMfma = 3;
constexpr int kSoftmaxValuPerMfmaEarly = 4;  // in the blocks between the load branches
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100, kSgValu = 0x002 | 0x400;
constexpr bool stream_is_s(int mode, int e) { return mode == kStreamS || (mode == kStreamSPv && (e & 1) == 0); }
template <int Mode, int E, int End, int Valu, bool kSplitQ>
__device__ __forceinline__ void issue_order_tail() {
  if constexpr (E < End) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, (kSplitQ && stream_is_s(Mode, E)) ? 2 : 1, 0);
    if constexpr (E + stream_ahead(Mode) < stream_length(Mode))
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, stream_reads(Mode, E + stream_ahead(Mode)), 0);
    if constexpr (Valu > 0) __builtin_amdgcn_sched_group_barrier(kSgValu, Valu, 0);
    issue_order_tail<Mode, E + 1, End, Valu, kSplitQ>();
  }
}
template <int Mode, int E, int Acc>
struct StreamHead {
  static constexpr int value = StreamHead<Mode, E - 1, Acc + stream_reads(Mode, E - 1)>::value;
};
template <int Mode, int Acc>
struct StreamHead<Mode, 0, Acc> {
  static constexpr int value = Acc;
};
template <int Mode, int Valu, bool kSplitQ>
__device__ __forceinline__ void issue_order() {
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, StreamHead<Mode, stream_ahead(Mode), 0>::value, 0);
  issue_order_tail<Mode, 0, stream_length(Mode), Valu, kSplitQ>();
}
// The same for the elements E .. E + kLoadSpacing - 1 alone: the basic block
// between two waves' tile-load branches (their reads ahead included).
template <int Mode, int E, int Valu, bool kSplitQ>
__device__ __forceinline__ void issue_order_block() {
  issue_order_tail<Mode, E, E + kLoadSpacing, Valu, kSplitQ>();
}

}  // namespace

// kPaged: key row j of sequence b is slot j of a paged cache (a full layer's
// positions 0 .. n_keys-1); its page indices for the workgroup's tiles are
// staged in LDS first, and every tile (64 rows, inside one page) is read
// through a buffer resource over its page.
// kSplitQ: each rotated query channel enters the scores as a bf16 high part
// plus a bf16 low part (x - hi, rounded), about 16 significant bits instead
// of 8, at the cost of a second S MFMA per K fragment (no extra LDS reads).
template <bool kPaged, bool kSplitQ>
__global__ __launch_bounds__(256, 1) void prefill_attn_kernel(PrefillAttnArgs a) {
  // Two K and two V tile slots (the swizzled block layout is described at
  // load_tile below). Four separate arrays (not one indexed array) so the
  // compiler can tell the slot being filled from the slot being read and
  // does not wait for the in-flight tile loads before reading the current
  // tile.
  __shared__ __attribute__((aligned(1024))) char k_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_lds1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds1[kTileBytes];
  __shared__ int page_of[kPaged ? kMaxPagesPerSeq : 1];  // pool page of logical page pg_lo + i

  // Longest query blocks first; then sequence, then KV head. In a ragged
  // batch the blocks past a shorter sequence's end leave at once.
  const int per_qt = a.B * a.Hkv;
  const int qt = a.q_tiles - 1 - (int)blockIdx.x / per_qt;
  const int r2 = (int)blockIdx.x % per_qt;
  const int b = r2 / a.Hkv;
  const int kvh = r2 % a.Hkv;
  const int len = a.len[b];
  if (qt * kBM >= len) return;
  // Profiling: the workgroup's start on the shader clock and on the
  // fixed-rate real-time counter, parked in LDS until its end.
  __shared__ unsigned long long clk_start[2];
  if (a.clock_acc && threadIdx.x == 0) {
    clk_start[0] = __builtin_amdgcn_s_memtime();
    clk_start[1] = __builtin_amdgcn_s_memrealtime();
  }
  const size_t tok0 = (size_t)a.tok0[b];  // packed row of the sequence's query 0

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = kvh * kGroup + wave;
  const int q0 = qt * kBM;
  const int nq = min(kBM, len - q0);
  const int pq_first = a.start[b] + q0;
  const int pq_last = pq_first + nq - 1;
  const int kp0 = a.key_pos0[b];
  const int nk = a.n_keys[b];
  const int lo_pos = a.window > 0 ? max(pq_first - a.window + 1, 0) : 0;
  const int row_lo = max(lo_pos - kp0, 0);
  const int row_hi = min(pq_last - kp0 + 1, nk);
  const int t_lo = row_lo / kBN;
  const int nt = (row_hi + kBN - 1) / kBN - t_lo;

  const size_t kv_off = kPaged ? 0 : ((size_t)b * a.Hkv + kvh) * (size_t)a.rows * kHeadDim;
  // the host limits a slab to 2^23 rows of 512 B
  const uint32_t slab_bytes = (uint32_t)min((uint64_t)a.rows * 512u, (uint64_t)0xffffffffu);
  const __amdgpu_buffer_rsrc_t krs = slab_rsrc(a.kc + kv_off, slab_bytes);
  const __amdgpu_buffer_rsrc_t vrs = slab_rsrc(a.vc + kv_off, slab_bytes);
  const int ps = kPaged ? a.paged.page_size : 1;
  const int pg_lo = kPaged ? t_lo * kBN / ps : 0;
  if constexpr (kPaged) {
    // the pages holding tiles t_lo .. t_lo + nt - 1 (at most the sequence's
    // table row); entries outside the pool are clamped into it
    const int n_pg = ((t_lo + nt) * kBN - 1) / ps - pg_lo + 1;
    const int* tb = a.paged.table + (size_t)b * a.paged.pages_per_seq + pg_lo;
    for (int i = threadIdx.x; i < n_pg; i += 256) page_of[i] = min(max(tb[i], 0), a.paged.num_pages - 1);
    __syncthreads();
  }

  // A K or V tile (64 key rows x 512 B) sits in LDS as 32 blocks of 1 KiB;
  // block 4g + c holds rows 8g .. 8g+7, bytes 128c .. 128c+127 of each row.
  // Inside a block, the 16-byte chunk k of row r is at position
  // 8r + (k ^ sigma(g, r)), with sigma = r ^ (g & 1) for K and (2r) & 7 for
  // V. Each load instruction fills one block from 8 whole 128-byte lines
  // (one row segment per 8 lanes), and the swizzle keeps the MFMA fragment
  // reads below free of bank conflicts. Each wave loads blocks 8w .. 8w+7.
  // Rows past the valid keys re-read the last valid key; their scores are
  // masked, so they contribute exactly zero.
  // With split queries the registers run short: the lane's row and chunk
  // are then recomputed from the lane id at each tile load (asm, so the
  // compiler neither hoists nor keeps them). Held across the tile loop they
  // are among the first values the register allocator spills, and a reload
  // from scratch inside the matrix-core stream stalls the wave on its memory
  // counter. The plain kernel has registers to spare and keeps them.
  auto load_lane = [&]() __attribute__((always_inline)) {
    uint32_t l = (uint32_t)lane;
    if constexpr (kSplitQ) asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
  };
  auto load_tile = [&](__amdgpu_buffer_rsrc_t rs, bool is_v, int t, char* slot) __attribute__((always_inline)) {
    const uint32_t ln = load_lane();
    const uint32_t r = ln >> 3, c = ln & 7;
    const uint32_t chunk0 = 16u * (is_v ? (c ^ ((2 * r) & 7)) : (c ^ r));
    const uint32_t chunk1 = 16u * (is_v ? (c ^ ((2 * r) & 7)) : (c ^ r ^ 1));
    char* dst = slot + wave * 8 * 1024;
    const int row0 = t * kBN + 16 * wave + (int)r;
    const int base_row = kPaged ? t * kBN / ps * ps : 0;  // first row of the tile's page
    const uint32_t off0 = (uint32_t)(min(row0, nk - 1) - base_row) * 512u + chunk0;
    const uint32_t off1 = (uint32_t)(min(row0 + 8, nk - 1) - base_row) * 512u + chunk1;
#pragma unroll
    for (int u = 0; u < 8; ++u) load_lds16(rs, u < 4 ? off0 : off1, 128 * (u & 3), dst + u * 1024);
  };
  // Buffer resource over the page that holds tile t (paged caches).
  auto page_rsrc = [&](const uint16_t* pool, int t) __attribute__((always_inline)) {
    const int pg = __builtin_amdgcn_readfirstlane(page_of[t * kBN / ps - pg_lo]);
    return slab_rsrc(pool + ((size_t)pg * a.Hkv + kvh) * (size_t)ps * kHeadDim, (uint32_t)ps * 512u);
  };
  auto load_k = [&](int t, char* slot) __attribute__((always_inline)) {
    load_tile(kPaged ? page_rsrc(a.kc, t) : krs, false, t, slot);
  };

  // The first K tiles, in flight during the query RoPE. (The fast query
  // path below requests the second one only once its queries, staged in
  // that tile's slot, have been read; V of the first tile is loaded by the
  // first step, ahead of its P.V in the second.)
  auto load_first_tiles = [&]() __attribute__((always_inline)) {
    load_k(t_lo, k_lds0);
    if (nt > 1) load_k(t_lo + 1, k_lds1);
  };

  // ---- queries: RoPE in fp32 from the cos/sin table, then bf16 fragments
  // (B operand of S^T): lane holds query lane % 32, channels
  // ks*16 + (lane / 32)*8 .. +7 for ks = 0..15.
  const int qrow = q0 + (lane & 31);
  const bool qvalid = qrow < len;
  // the gate logit, requested now and used in the epilogue
  const size_t orow = (tok0 + (qvalid ? qrow : len - 1)) * (size_t)a.gate_stride + h;
  const uint16_t gate_bits = a.gate[orow];
  bf16x8 qf[16];
  bf16x8 qlo[kSplitQ ? 16 : 1];
  const bool late_second_tile = a.r == 64 || a.r == 256;  // the fast query path below
  {
    const int qr = qvalid ? qrow : len - 1;
    const uint16_t* qp = a.q + (tok0 + qr) * (size_t)a.q_stride + (size_t)h * kHeadDim;
    const int half = a.r >> 1;
    const float2* tp = a.table + (tok0 + qr) * half;
    // With r a multiple of 32 (the pages' 64 and 256), the partner of
    // fragment ks (channels 16ks + 8(lane/32) ..) is fragment ks +- r/32 of
    // the same lane: every load is issued up front, in one round trip, and
    // the rotation runs on registers.
    auto rope_fast = [&](auto np) __attribute__((always_inline)) {
      constexpr int NP = decltype(np)::value;  // rotated fragment pairs (ks, ks + NP)
      // The cos/sin rows of the block's 32 queries (128 NP bytes each) are
      // the same for all four waves. They come into the free V slot v_lds1
      // by LDS DMA, whole 128-byte lines per instruction (NP instructions
      // per wave), instead of 4 NP loads per lane that each touch 32 rows.
      // Row i (query q0 + i, clamped like qr) keeps its 16-byte chunk c at
      // position c ^ (i & 7), which spreads the reads below over the banks.
      constexpr int kRowBytes = 128 * NP;
      {
        // a resource over the block's own rows (nq of them), so every offset
        // stays below 32 KiB whatever the sequence's length
        const __amdgpu_buffer_rsrc_t trs =
            slab_rsrc(a.table + (tok0 + q0) * (size_t)half, (uint32_t)nq * (uint32_t)kRowBytes);
#pragma unroll
        for (int u = 0; u < NP; ++u) {
          const uint32_t off = (uint32_t)(wave * NP + u) * 1024u + 16u * (uint32_t)lane;  // byte in the copy
          const int i = (int)(off / kRowBytes);
          const uint32_t pos = (off % kRowBytes) / 16u;
          const uint32_t src = (uint32_t)min(i, nq - 1) * kRowBytes + 16u * (pos ^ (uint32_t)(i & 7));
          load_lds16(trs, src, 0, v_lds1 + (wave * NP + u) * 1024);
        }
      }
      // The wave's 32 query rows (512 B of its head each) come the same way
      // into 16 KiB of the slots k_lds1 and v_lds0, which the second K tile
      // and the first V tile fill only after the queries have been read:
      // instruction u fills rows 2u, 2u + 1 from whole lines, instead of 16
      // loads per lane that each touch 32 rows. Row i keeps its 16-byte
      // chunk c at position c ^ (i & 31), so the 16 lanes of a fragment read
      // hit 16 different bank groups. Rows past the end repeat row nq - 1.
      // These copies are issued from inline asm (waited for below by count):
      // through the builtin, the compiler could not tell which slot the
      // selected pointer writes and waited for the K tile's copies too
      // before reading the queries.
      const char* qst = (wave < 2 ? k_lds1 : v_lds0) + (wave & 1) * 16384;
      {
        const uint16_t* qbase = a.q + (tok0 + q0) * (size_t)a.q_stride + (size_t)h * kHeadDim;
        const uint64_t qa = (uint64_t)(uintptr_t)qbase;
        const uint32_t qbytes = (uint32_t)(nq - 1) * (uint32_t)a.q_stride * 2u + 512u;
        const int d0 = __builtin_amdgcn_readfirstlane((int)(uint32_t)qa);
        const int d1 = __builtin_amdgcn_readfirstlane((int)((qa >> 32) & 0xffff));
        const int d2 = __builtin_amdgcn_readfirstlane((int)qbytes);
        const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_u32(qst));
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int i = 2 * u + (lane >> 5);
          const uint32_t c = (uint32_t)((lane & 31) ^ (i & 31));
          const uint32_t voff = (uint32_t)min(i, nq - 1) * (uint32_t)a.q_stride * 2u + 16u * c;
          asm volatile(
              "s_mov_b32 m0, %0\n\t"
              "s_nop 0\n\t"
              "buffer_load_dwordx4 %1, %2, 0 offen lds"
              :
              : "s"(m0 + 1024u * (uint32_t)u), "v"(voff), "s"(i32x4q{d0, d1, d2, 0x00020000})
              : "memory", "m0");
        }
      }
      asm volatile("" ::: "memory");  // issue order: table rows, queries, then the first K tile
      load_k(t_lo, k_lds0);
      // This wave's table rows and queries have landed once at most the
      // first tile's 8 loads are outstanding; after the barrier, every
      // wave's have. (A bare s_barrier: __syncthreads would also wait for
      // the tile.)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // The query reads are asm as well: the compiler, not seeing the copies
      // above, would otherwise still wait for the K tile's copy before them.
      uint4 raw[16];
      {
        const int i = lane & 31;
        const uint32_t qrow = lds_u32(qst) + (uint32_t)i * 512u;
        i32x4q rv[16];
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          const uint32_t ad = qrow + 16u * (uint32_t)((2 * ks + (lane >> 5)) ^ i);
          asm volatile("ds_read_b128 %0, %1" : "=v"(rv[ks]) : "v"(ad) : "memory");
        }
        // The wait names the 16 results as operands, so no use of them can
        // be scheduled ahead of it (the hardware does not hold a VALU read
        // of a register an LDS read is still filling).
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(rv[0]), "+v"(rv[1]), "+v"(rv[2]), "+v"(rv[3]), "+v"(rv[4]), "+v"(rv[5]), "+v"(rv[6]),
                       "+v"(rv[7])
                     :
                     : "memory");
        asm volatile(""
                     : "+v"(rv[8]), "+v"(rv[9]), "+v"(rv[10]), "+v"(rv[11]), "+v"(rv[12]), "+v"(rv[13]),
                       "+v"(rv[14]), "+v"(rv[15]));
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) raw[ks] = __builtin_bit_cast(uint4, rv[ks]);
      }
      uint4 cs[NP][4];  // (cos, sin) of table entries 16p + 8(lane/32) + 0..7
      {
        const int i = qr - q0;
#pragma unroll
        for (int pp = 0; pp < NP; ++pp)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            cs[pp][u] = *(const uint4*)(v_lds1 + i * kRowBytes + 16 * ((8 * pp + 4 * (lane >> 5) + u) ^ (i & 7)));
      }
      // Rows past the sequence's end hold the last row's queries (qr is
      // clamped): their columns repeat a column of the same wave, so they
      // change none of its decisions, and their outputs are not stored.
      auto put = [&](int ks, const float* x) __attribute__((always_inline)) {
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (__bf16)x[j];
        qf[ks] = v;
        if constexpr (kSplitQ) {
          bf16x8 lo;
#pragma unroll
          for (int j = 0; j < 8; ++j) lo[j] = (__bf16)(x[j] - (float)v[j]);
          qlo[ks] = lo;
        }
      };
      // each rotated pair (pp, pp + NP) is unpacked once
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        float xa[8], xb[8], ra[8], rb[8];
        unpack8(raw[pp], xa);
        unpack8(raw[pp + NP], xb);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint4 w = cs[pp][j >> 1];
          const float2 t = (j & 1) ? make_float2(__uint_as_float(w.z), __uint_as_float(w.w))
                                   : make_float2(__uint_as_float(w.x), __uint_as_float(w.y));
          // explicit fused multiply-adds: the rounding does not depend on
          // how the compiler would contract the expression
          ra[j] = __builtin_fmaf(xa[j], t.x, -(xb[j] * t.y));
          rb[j] = __builtin_fmaf(xb[j], t.x, xa[j] * t.y);
        }
        put(pp, ra);
        put(pp + NP, rb);
      }
      // channels past r pass through: their bf16 bits are the fragments
#pragma unroll
      for (int ks = 2 * NP; ks < 16; ++ks) {
        qf[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
        if constexpr (kSplitQ) qlo[ks] = bf16x8{};
      }
      // every wave has read its queries: the second K tile may replace them
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (nt > 1) load_k(t_lo + 1, k_lds1);
    };
    // Any other r (a multiple of 16): fragment by fragment, partners and
    // table entries loaded per fragment.
    auto rope_generic = [&]() __attribute__((always_inline)) {
      load_first_tiles();
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const int d0 = ks * 16 + (lane >> 5) * 8;
        float x[8];
        unpack8(*(const uint4*)(qp + d0), x);
        if (d0 < a.r) {
          const bool first = d0 < half;
          float xp[8];
          unpack8(*(const uint4*)(qp + (first ? d0 + half : d0 - half)), xp);
          const float2* cs = tp + (first ? d0 : d0 - half);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float2 t = cs[j];
            x[j] = first ? __builtin_fmaf(x[j], t.x, -(xp[j] * t.y)) : __builtin_fmaf(x[j], t.x, xp[j] * t.y);
          }
        }
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (__bf16)(qvalid ? x[j] : 0.f);
        qf[ks] = v;
        if constexpr (kSplitQ) {
          bf16x8 lo;
#pragma unroll
          for (int j = 0; j < 8; ++j) lo[j] = (__bf16)(qvalid ? x[j] - (float)v[j] : 0.f);
          qlo[ks] = lo;
        }
      }
    };
    if (a.r == 64) rope_fast(std::integral_constant<int, 2>{});
    else if (a.r == 256) rope_fast(std::integral_constant<int, 8>{});
    else rope_generic();
    // The fragments are only ever MFMA operands: keep them in the
    // accumulation registers, which leaves the VGPRs to the softmax.
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) asm volatile("" : "+a"(qf[ks]));
    if constexpr (kSplitQ) {
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) asm volatile("" : "+a"(qlo[ks]));
    }
  }

  auto need_mask = [&](int t) __attribute__((always_inline)) {
    const int row0 = t * kBN;
    return (kp0 + row0 + kBN - 1 > pq_first) || (a.window > 0 && kp0 + row0 <= pq_last - a.window) ||
           (row0 + kBN > nk);
  };

  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  float m_i = -1e30f;  // running max (log2 units) of this lane's query
  float l_i = 0.f;     // running sum

  // K fragment of S MFMA (k-step ks, key block h): lane l reads row
  // 32h + l%32, channels 16ks + 8(l/32) .. +7, at
  // k_addr[ks % 4] + 16384h + 1024(ks / 4).
  int k_addr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    k_addr[q] = ((lane & 31) >> 3) * 4096 + 128 * (lane & 7) +
                16 * ((2 * q + (lane >> 5)) ^ (lane & 7) ^ (((lane & 31) >> 3) & 1));
  // V^T fragments by transposed reads: in 16-lane group G, source lane
  // w + 4v fetches 8 B (channels 32db + 16(G%2) + 4w .. +3) of key
  // 16tt + 8j2 + 4(G/2) + v; output lane i then holds channel
  // 32db + 16(G%2) + i of those 4 keys, which are the key slots
  // 8(G/2) + 4j2 + 0..3 of the P^T fragment. Address:
  // v_addr[db % 2] + 8192tt + 4096j2 + 1024(db / 2).
  int v_addr[2];
  {
    const int G = lane >> 4, w = lane & 3, v = (lane >> 2) & 3;
#pragma unroll
    for (int e = 0; e < 2; ++e)
      v_addr[e] = 512 * (G >> 1) + 128 * v + 16 * ((4 * e + 2 * (G & 1) + (w >> 1)) ^ (2 * v)) + 8 * (w & 1);
  }
  // The V slots lie above 64 KiB of LDS, past the reach of a DS
  // instruction's 16-bit offset field, so the compiler built every
  // transposed read's address with its own v_or (64 per step). With the
  // slot's LDS address added to v_addr once, in registers it cannot see
  // into, the remaining constant fits the offset field. The reads still
  // index the slot array itself (slot + (va_abs - address of slot)), so the
  // compiler keeps telling them apart from the DMA into the other slot.
  uint32_t va_abs[2][2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      va_abs[sl][e] = (uint32_t)v_addr[e] + lds_u32(sl ? v_lds1 : v_lds0);
      asm volatile("" : "+v"(va_abs[sl][e]));
    }

  // Mask of tile t's scores. Register i of block kb holds key row
  // t*64 + kb*32 + 8*(i/4) + 4*(lane/32) + i%4 for query lane % 32.
  // Branch-free (key_visible's short-circuit tests compiled to a branch per
  // element): a key at distance d = pq - pk behind the query is visible iff
  // 0 <= d < window (any d >= 0 without a window) and its row is valid; one
  // unsigned compare covers both bounds, since a negative d turns into a
  // value of 2^31 or more. Key positions are never negative here (kp0 >= 0).
  const unsigned wlim = a.window > 0 ? (unsigned)a.window : 0x7fffffffu;
  auto mask_s = [&](int t, f32x16& s0, f32x16& s1) __attribute__((always_inline)) {
    const int pq = pq_first + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k0 = t * kBN + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      const int d0 = pq - (kp0 + k0);
      const bool ok0 = ((unsigned)d0 < wlim) & (k0 < nk);
      const bool ok1 = ((unsigned)(d0 - 32) < wlim) & (k0 + 32 < nk);
      s0[i] = ok0 ? s0[i] : -__builtin_inff();
      s1[i] = ok1 ? s1[i] : -__builtin_inff();
    }
  };

  // One stream of matrix-core work per tile: S^T of the next tile (32
  // MFMAs, K fragments from LDS) interleaved with P.V of the previous tile
  // (32 MFMAs, V^T fragments from LDS). With both, stream element e is an S
  // MFMA when e is even and a P.V MFMA when odd. The LDS fragments of
  // element e + ahead are read just before element e issues; the
  // scheduling-group barriers placed after the step's code (issue_order)
  // hold the compiler to that order, so every read has several MFMAs to land.
  auto mma_stream = [&](auto mode, const char* kslot, const char* vslot, f32x16& s0, f32x16& s1,
                        const bf16x8* p, auto&& before) __attribute__((always_inline)) {
    constexpr bool kS = decltype(mode)::value != kStreamPv;
    constexpr bool kP = decltype(mode)::value != kStreamS;
    constexpr int kN = stream_length(decltype(mode)::value);
    constexpr int kAhead = stream_ahead(decltype(mode)::value);
    bf16x8 kr[kRing];
    s16x8 vr[kRing];
    auto is_s = [](int e) constexpr { return kS && (!kP || (e & 1) == 0); };
    auto index = [](int e) constexpr { return (kS && kP) ? e >> 1 : e; };
    auto issue = [&](int e) __attribute__((always_inline)) {
      const int i = index(e);
      if (is_s(e)) {  // S MFMA i: k-step i/2, key block i%2
        const int ks = i >> 1;
        kr[i % kRing] = *(const bf16x8*)(kslot + k_addr[ks & 3] + (i & 1) * 16384 + (ks >> 2) * 1024);
      } else {        // P.V MFMA i = tt*8 + db
        const uint32_t vb = va_abs[vslot == v_lds1 ? 1 : 0][i & 1];
        const char* vp = vslot + (vb - lds_u32(vslot)) + (i >> 3) * 8192 + ((i & 7) >> 1) * 1024;
        const s16x4 lo = lds_read_tr(vp);
        const s16x4 hi = lds_read_tr(vp + 4096);
        vr[i % kRing] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    if (kS) {
      s0 = f32x16{};
      s1 = f32x16{};
    }
#pragma unroll
    for (int e = 0; e < kAhead; ++e) issue(e);
    // Expanded at compile time (the hook sees each element index as a
    // constant): a plain unrolled loop stops being unrolled once the hooks
    // carry the softmax parts.
    static_for<0, kN>([&](auto ec) __attribute__((always_inline)) {
      constexpr int e = decltype(ec)::value;
      before(ec);  // work placed ahead of element e (tile loads, softmax parts)
      if constexpr (e + kAhead < kN) issue(e + kAhead);
      constexpr int i = index(e);
      if constexpr (is_s(e)) {
        f32x16& sb = (i & 1) ? s1 : s0;
        sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[i % kRing], qf[i >> 1], sb, 0, 0, 0);
        if constexpr (kSplitQ)
          sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[i % kRing], qlo[i >> 1], sb, 0, 0, 0);
      } else {
        acc[i & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vr[i % kRing]), p[i >> 3],
                                                            acc[i & 7], 0, 0, 0);
      }
    });
  };

  // Softmax of one tile's scores into pb, in three parts that the step
  // spreads over its stream: the max (the running max moves only when the
  // tile's max exceeds it by more than 2^8; alpha is the factor O must be
  // rescaled by, 1 when the max did not move), the probabilities of score
  // registers i0 .. i1-1, and the sum. Reductions are balanced trees: short
  // dependency chains interleave with the matrix-core stream without
  // stalling it.
  struct SoftmaxPart {
    float m_use;
    bool rescale;
    float q16[16];
  };
  auto softmax_max = [&](const f32x16& s0, const f32x16& s1, SoftmaxPart& sp, float& alpha)
                         __attribute__((always_inline)) {
    float t16[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t16[i] = max_f(s0[i], s1[i]);
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) t16[i] = max_f(t16[i], t16[i + w]);
    const float mx = pair_max(t16[0]) * kScoreScale;
    const float m_new = max_f(m_i, mx);
    sp.rescale = __any(m_new > m_i + kRescaleSlack);
    sp.m_use = sp.rescale ? m_new : m_i;
    alpha = fast_exp2(m_i - sp.m_use);
  };
  // step tt of P^T covers keys 16tt .. +15; its key slot (lane/32)*8 + j
  // is register 8*(tt%2) + j of block tt/2
  auto softmax_exp = [&](const f32x16& s0, const f32x16& s1, bf16x8* pb, SoftmaxPart& sp, int i0, int i1)
                         __attribute__((always_inline)) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const float p0 = fast_exp2(fmaf(s0[i], kScoreScale, -sp.m_use));
      const float p1 = fast_exp2(fmaf(s1[i], kScoreScale, -sp.m_use));
      sp.q16[i] = p0 + p1;
      pb[i >> 3][i & 7] = (__bf16)p0;
      pb[2 + (i >> 3)][i & 7] = (__bf16)p1;
    }
  };
  auto softmax_sum = [&](SoftmaxPart& sp, float alpha) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) sp.q16[i] += sp.q16[i + w];
    l_i = l_i * alpha + sp.q16[0];   // per-lane partial; the lane pair is summed at the end
    m_i = sp.m_use;
  };
  // O *= alpha in place in the accumulation registers (read, multiply,
  // write back per element), so O never has to move to VGPRs.
  auto rescale_o = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float tmp;
        asm volatile(
            "v_accvgpr_read_b32 %1, %0\n\t"
            "v_mul_f32 %1, %1, %2\n\t"
            "v_accvgpr_write_b32 %0, %1"
            : "+a"(acc[db][i]), "=&v"(tmp)
            : "v"(alpha));
      }
  };

  // Iteration j (tile t = t_lo + j) overlaps three things: the softmax of
  // S(t) (VALU), S(t+1) = K(t+1) Q^T and P(t-1).V(t-1) (MFMA), and the loads
  // of K(t+2) and V(t). Tile j's K lives in k_lds[j % 2] and its V in
  // v_lds[j % 2]; the score and probability registers alternate the same
  // way, so every slot and register set is fixed at compile time.
  using ModeS = std::integral_constant<int, kStreamS>;
  using ModeSPv = std::integral_constant<int, kStreamSPv>;
  using ModePv = std::integral_constant<int, kStreamPv>;
  bool rescale_pending = false;
  float alpha_pending = 1.0f;
  f32x16 sA0, sA1, sB0, sB1;  // scores of even / odd tiles
  bf16x8 pA[4], pB[4];        // probabilities of even / odd tiles
  // The first K tile has landed once at most the second one's 8 loads are
  // outstanding: the fast query path requests that tile only at its end
  // (the other path requests both up front).
  if (late_second_tile && nt > 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else wait_loads();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  mma_stream(ModeS{}, k_lds0, v_lds0, sA0, sA1, pA, [](auto) {});
  issue_order<kStreamS, 0, kSplitQ>();
  if (need_mask(t_lo)) mask_s(t_lo, sA0, sA1);

  // One iteration; the first one has no P.V yet. On the last tile S(t+1)
  // is computed from a stale slot and discarded, which keeps the body free
  // of data-dependent branches between its MFMAs and its softmax (the only
  // branches are the uniform ones around each wave's tile loads).
  auto step = [&](auto mode, int j, const char* kn, const char* vp, char* kf, char* vf, f32x16& sc0,
                  f32x16& sc1, f32x16& sn0, f32x16& sn1, const bf16x8* pp,
                  bf16x8* pn) __attribute__((always_inline)) {
    constexpr int kMode = decltype(mode)::value;
    const int t = t_lo + j;
    wait_loads();
    __syncthreads();
    // Page lookups (paged caches) at the step's start; each wave's loads at
    // its own point of the stream. Without a K load (the last two steps)
    // the K lookup takes tile t, whose page is staged.
    const int tk = j + 2 < nt ? t + 2 : t;
    const __amdgpu_buffer_rsrc_t rk = kPaged ? page_rsrc(a.kc, tk) : krs;
    const __amdgpu_buffer_rsrc_t rv = kPaged ? page_rsrc(a.vc, t) : vrs;
    auto load_tiles = [&]() __attribute__((always_inline)) {
      if (j + 2 < nt) load_tile(rk, false, t + 2, kf);
      load_tile(rv, true, t, vf);
    };
    // O holds P.V up to tile t-2 plus (below) tile t-1, all relative to the
    // max before softmax(t-1); a max move found by softmax(t-1) is applied
    // here, before P(t-1).V(t-1) is added, so no branch on the max sits
    // inside the stream. In the first P.V step (j = 1) O is still zero while
    // the first softmax always moves the max off its start value: that
    // rescale would only multiply zeros (the running sum is rescaled inside
    // the softmax).
    if (rescale_pending && j > 1) rescale_o(alpha_pending);
    // The softmax of S(t) runs beside the stream. With split queries (twice
    // the S MFMAs) its max goes beside elements 0-7, the probabilities of
    // score registers 0-3 and 4-7 beside 8-15 and 16-23, the rest and the
    // sum beside the long last block; each part is pinned where it is placed
    // (ahead of the next load branch), so the compiler cannot sink it into
    // the next block. The plain kernel keeps the whole softmax in the last
    // block, which measured faster there.
    SoftmaxPart sp;
    mma_stream(mode, kn, vp, sn0, sn1, pp, [&](auto ec) __attribute__((always_inline)) {
        constexpr int e = decltype(ec)::value;
        if constexpr (!kSplitQ) {
        } else if constexpr (e == kLoadSpacing) {
          softmax_max(sc0, sc1, sp, alpha_pending);
          asm volatile("" : "+v"(sp.m_use), "+v"(alpha_pending));
          issue_order_block<kMode, 0, kSoftmaxValuPerMfmaEarly, kSplitQ>();
        } else if constexpr (e == 2 * kLoadSpacing || e == 3 * kLoadSpacing) {
          constexpr int i0 = e == 2 * kLoadSpacing ? 0 : 4;
          softmax_exp(sc0, sc1, pn, sp, i0, i0 + 4);
          asm volatile("" : "+v"(pn[0]), "+v"(pn[2]), "+v"(sp.q16[i0]), "+v"(sp.q16[i0 + 1]),
                       "+v"(sp.q16[i0 + 2]), "+v"(sp.q16[i0 + 3]));
          issue_order_block<kMode, e - kLoadSpacing, kSoftmaxValuPerMfmaEarly, kSplitQ>();
        }
        if constexpr (e % kLoadSpacing == 0 && e < 4 * kLoadSpacing) {
          if (wave == e / kLoadSpacing) load_tiles();
        }
    });
    if constexpr (!kSplitQ) {
      softmax_max(sc0, sc1, sp, alpha_pending);
      softmax_exp(sc0, sc1, pn, sp, 0, 8);
    }
    softmax_exp(sc0, sc1, pn, sp, 8, 16);
    softmax_sum(sp, alpha_pending);
    rescale_pending = sp.rescale;
    issue_order<kMode, kSoftmaxValuPerMfma, kSplitQ>();
    // The softmax's results are used here, ahead of the mask branch: nothing
    // below needs them before the next step, and without this use the
    // compiler may sink the whole softmax past that branch, out of the
    // matrix-core stream it is interleaved with.
    asm volatile("" : "+v"(pn[0]), "+v"(pn[1]), "+v"(pn[2]), "+v"(pn[3]), "+v"(alpha_pending), "+v"(l_i),
                 "+v"(m_i));
    // The next tile's scores are wanted in VGPRs at the step's end: without
    // this the compiler copies them out of the accumulation registers at the
    // start of the next step, 32 reads in a row ahead of its barrier, and
    // zeroes the accumulators with 32 writes per two steps.
    asm volatile("" : "+v"(sn0), "+v"(sn1));
    if (j + 1 < nt && need_mask(t + 1)) mask_s(t + 1, sn0, sn1);
  };
  // even j: S(t) in sA, P(t) -> pA, P(t-1) in pB; odd j: the other way round
  step(ModeS{}, 0, k_lds1, v_lds1, k_lds0, v_lds0, sA0, sA1, sB0, sB1, pB, pA);
  for (int j = 1; j < nt; j += 2) {
    step(ModeSPv{}, j, k_lds0, v_lds0, k_lds1, v_lds1, sB0, sB1, sA0, sA1, pA, pB);
    if (j + 1 < nt) step(ModeSPv{}, j + 1, k_lds1, v_lds1, k_lds0, v_lds0, sA0, sA1, sB0, sB1, pB, pA);
  }
  // P.V of the last tile (with a single tile, O is still zero: no rescale)
  wait_loads();
  __syncthreads();
  if (rescale_pending && nt > 1) rescale_o(alpha_pending);
  if ((nt - 1) & 1) {
    mma_stream(ModePv{}, k_lds0, v_lds1, sA0, sA1, pB, [](auto) {});
    issue_order<kStreamPv, 0, kSplitQ>();
  } else {
    mma_stream(ModePv{}, k_lds0, v_lds0, sA0, sA1, pA, [](auto) {});
    issue_order<kStreamPv, 0, kSplitQ>();
  }
  l_i = pair_sum(l_i);

  // ---- epilogue: divide by the softmax sum, gate in fp32, one bf16 store.
  // acc[db] register i holds channel db*32 + 8*(i/4) + 4*(lane/32) + i%4 of
  // query lane % 32. The rows go through LDS so that each store instruction
  // writes two whole 512-byte rows: wave w stages its 32 rows in 16 KiB of
  // the K slots, which no wave reads any more (the barrier before the last
  // P.V lies behind every S stream; the last P.V reads V slots only). Row r
  // keeps its 16-byte chunk c at position c ^ r, so neither the 8-byte
  // writes nor the 16-byte reads collide on banks.
  {
    const float g = bf16_bits_to_float(gate_bits);
    const float f = (1.0f / l_i) * gate_factor(g, a.gate_act);
    char* stage = (wave < 2 ? k_lds0 : k_lds1) + (wave & 1) * 16384;
    const int row = lane & 31;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w0 = pack_bf16x2(acc[db][4 * c + 0] * f, acc[db][4 * c + 1] * f);
        const uint32_t w1 = pack_bf16x2(acc[db][4 * c + 2] * f, acc[db][4 * c + 3] * f);
        *(uint2*)(stage + row * 512 + (((db * 4 + c) ^ row) << 4) + (lane >> 5) * 8) = make_uint2(w0, w1);
      }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = 2 * k + (lane >> 5);
      const uint4 v = *(const uint4*)(stage + r * 512 + (((lane & 31) ^ r) << 4));
      if (q0 + r < len)
        *(uint4*)(a.out + ((tok0 + q0 + r) * a.Hq + h) * kHeadDim + (lane & 31) * 8) = v;
    }
  }
  if (a.clock_acc && threadIdx.x == 0) {
    atomicAdd(&a.clock_acc[0], __builtin_amdgcn_s_memtime() - clk_start[0]);
    atomicAdd(&a.clock_acc[1], __builtin_amdgcn_s_memrealtime() - clk_start[1]);
  }
}

hipError_t prefill_clock_acc(unsigned long long** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static unsigned long long* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(clock_acc));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = (unsigned long long*)p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t s) {
  const int grid = a.q_tiles * a.B * a.Hkv;
  if (grid == 0) return hipSuccess;
  // Sliding-window layers take the split queries: bf16 queries alone leave
  // little of the error budget there. The choice is per layer type, not per
  // call, so a layer's results do not depend on how its prefill is chunked.
  // Full layers (and paged caches, which belong to them) run the plain
  // kernel.
  if (a.paged.table)
    hipLaunchKernelGGL((prefill_attn_kernel<true, false>), dim3(grid), dim3(256), 0, s, a);
  else if (a.window > 0)
    hipLaunchKernelGGL((prefill_attn_kernel<false, true>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_attn_kernel<false, false>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hattn
