// Split-K decode attention for gfx950 (page "Spark-X2.5 架构（4B / 1.7B）",
// §3 Eq. 1 and §4; the explainer page: each generated token reads the layer's
// KV cache, which on sliding layers is bounded to the last 512 tokens).
//
// One workgroup = one (sequence, KV head, split of the visible key range),
// four waves, one workgroup per CU. Decode is HBM-bound: every K/V byte of
// the split is read once and serves the 4 query heads of the GQA group.
// Each wave streams its own 16-key chunks (chunks w, w+4, ...) through a
// private two-slot LDS ring: the K and V rows of the next chunk are moved by
// LDS DMA (16 B per lane, whole 128-byte lines per instruction) while the
// current chunk is computed, so loads hold no registers. Per chunk:
//   S[16 keys][16 cols] = K . Qc   (bf16 MFMA 16x16x32; columns 0-3 hold the
//     bf16 high parts of the 4 rotated queries, columns 4-7 their low parts,
//     so scores see ~16 significant query bits)
//   O[16 rows][256]    += P . V    (bf16 MFMA 16x16x16; rows 0-3: bf16 high
//     parts of the 4 heads' probabilities, rows 4-7 their low parts; V read
//     transposed by ds_read_tr16_b64)
// The token's own inputs (q, new k and v, RoPE frequencies) are staged by
// LDS DMA too, and where the visible range starts at a fixed key (ring
// caches, unbounded windows) each wave's first chunk is requested before the
// position has arrived. The waves merge (m, l, o) in LDS; with several splits
// a second kernel merges the splits in a fixed order.
#include <mutex>

#include "hattn_device.h"
#include "hattn_internal.h"

// Split partials of hattn_decode_static: one array per GPU, reserved with the
// code object and kept until the process ends. Host code never passes the
// symbol itself to a kernel: decode_static_scratch() looks up its device
// address once per device.
static __device__ __align__(256) unsigned char scratch[HATTN_DECODE_STATIC_SCRATCH_BYTES];

namespace hattn {

namespace {

constexpr int kChunk = 16;                      // keys per wave iteration
constexpr int kChunkBytes = kChunk * kHeadDim * 2;  // 8 KiB of K (or of V)
constexpr int kWaves = 4;
constexpr float kScoreScale = kLog2e / 16.0f;   // 1/sqrt(256), in log2 units
constexpr float kRescaleSlack = 8.0f;           // log2 units


__device__ __forceinline__ s16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}
typedef int i32x4 __attribute__((ext_vector_type(4)));
// Buffer descriptor of a slab (raw buffer, byte offsets, range-checked).
__device__ __forceinline__ i32x4 slab_desc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffff), (int)bytes, 0x00020000};
}
// 16 bytes per lane from memory into LDS (lane l lands at lds + 16 l).
// Issued from inline asm so that the compiler does not make every later LDS
// read wait for it (it cannot tell which LDS bytes a DMA writes); the caller
// waits with s_waitcnt vmcnt, counting these loads. M0 needs one wait state
// after it is written; the compiler sets M0 itself before each of its own
// uses, so listing it as clobbered is only a statement of fact.
// The cached keys and values are read once per call: the loads carry the
// non-temporal cache policy (nt), which streams them past the caches (4 GiB
// of K/V: 709 -> 637 us per call).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4 rs, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
}
__device__ __forceinline__ void dma16_stream(i32x4 rs, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Sum / max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane groups),
// by VALU lane swaps.
__device__ __forceinline__ float group4_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace

// A chunk slot holds the chunk's K rows (8 KiB) then its V rows (8 KiB).
// Row r's 16-byte piece c (0..31) sits at (r/2)*1024 + ((r%2)*32 + (c ^ s(r)))*16
// with s(r) = r for K and 2r mod 16 for V: each DMA instruction fills one
// 1 KiB block (rows 2u, 2u+1) and the XOR keeps the MFMA operand reads free
// of bank conflicts.
// kPaged: the cache is paged (a full layer, visible keys 0 .. p); the page
// indices of the split's keys are staged in LDS once the position is known,
// and each chunk (16 keys, inside one page) is read through a buffer
// resource over its page.
template <bool kPaged>
__global__ __launch_bounds__(256, 1) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char ring0[kWaves][2 * kChunkBytes];   // 64 KiB
  __shared__ __attribute__((aligned(1024))) char ring1[kWaves][2 * kChunkBytes];   // 64 KiB
  __shared__ __attribute__((aligned(16))) uint16_t qcols[8][kHeadDim];           // 4 KiB
  __shared__ float red_m[kWaves][4];
  __shared__ float red_l[kWaves][4];
  __shared__ __attribute__((aligned(16))) uint16_t newrow[2][kHeadDim];          // new k^, v
  // Staging of the token's inputs (LDS DMA): q of the 4 heads, new k and v
  // (512 B each, the rest of each 1 KiB block is zero) and the RoPE
  // frequencies (128 doubles).
  __shared__ __attribute__((aligned(1024))) uint16_t q_stage[kGroup][kHeadDim];  // 2 KiB
  __shared__ __attribute__((aligned(1024))) uint16_t kv_stage[2][512];           // 2 KiB
  __shared__ __attribute__((aligned(1024))) double freq_stage[128];              // 1 KiB
  __shared__ int page_of[kPaged ? kMaxPagesPerSeq : 1];  // table entries of the split's pages

  const int sp = (int)blockIdx.x % a.nsplit;
  const int r2 = (int)blockIdx.x / a.nsplit;
  const int kvh = r2 % a.Hkv;
  const int b = r2 / a.Hkv;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);

  const int p = a.pos[b];   // scalar load, waited for below
  // The 4 heads' gate logits, requested now and used at the end.
  uint16_t gate_bits[kGroup];
#pragma unroll
  for (int hh = 0; hh < kGroup; ++hh)
    gate_bits[hh] = a.nsplit == 1 ? a.gate[(size_t)b * a.gate_stride + kvh * kGroup + hh] : 0;

  // ---- the token's inputs, one DMA instruction per wave
  {
    const uint16_t* src;
    uint32_t bytes, voff = 16u * lane;
    void* dst;
    if (wave < 2) {
      src = a.q + (size_t)b * a.q_stride + (size_t)kvh * kGroup * kHeadDim;
      bytes = kGroup * kHeadDim * 2;
      voff += 1024u * wave;
      dst = (char*)q_stage + 1024 * wave;
    } else if (wave == 2) {
      src = a.k + (size_t)b * a.kv_stride + (size_t)kvh * kHeadDim;
      bytes = kHeadDim * 2;
      dst = kv_stage[0];
    } else {
      src = a.v + (size_t)b * a.kv_stride + (size_t)kvh * kHeadDim;
      bytes = kHeadDim * 2;
      dst = kv_stage[1];
    }
    dma16(slab_desc(src, bytes), voff, __builtin_amdgcn_readfirstlane(lds_off(dst)));
  }
  if (wave == 0) {
    const char* kp = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
    dma16(slab_desc(kp + __builtin_offsetof(DecodeArgs, inv_freq), 128 * 8), 16u * lane,
          __builtin_amdgcn_readfirstlane(lds_off(freq_stage)));
  }

  const size_t kv_off = kPaged ? 0 : ((size_t)b * a.Hkv + kvh) * (size_t)a.cap * kHeadDim;
  const uint32_t slab_bytes = (uint32_t)min((uint64_t)a.cap * 512u, (uint64_t)0xffffffffu);
  const i32x4 krs = slab_desc(a.kc + kv_off, slab_bytes);
  const i32x4 vrs = slab_desc(a.vc + kv_off, slab_bytes);
  const int ps = kPaged ? a.paged.page_size : 1;
  int pg_lo = 0;  // logical page of page_of[0]

  // DMA of the 16 keys from key0 into a slot: instruction u moves rows 2u,
  // 2u+1 (lane l: row 2u + l/32, piece (l%32) ^ s(row)). Row indices are
  // clamped to last. With a paged cache the 16 rows lie in one page (key0 is
  // a multiple of 16, the page size of 64) and last is in it too.
  auto load_rows = [&](int key0, int last, char* dst) __attribute__((always_inline)) {
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_off(dst));
    i32x4 kr = krs, vr = vrs;
    int base_row = 0;
    if constexpr (kPaged) {
      const int lp = key0 / ps;
      const int pg = min(max(__builtin_amdgcn_readfirstlane(page_of[lp - pg_lo]), 0), a.paged.num_pages - 1);
      const size_t off = ((size_t)pg * a.Hkv + kvh) * (size_t)ps * kHeadDim;
      kr = slab_desc(a.kc + off, (uint32_t)ps * 512u);
      vr = slab_desc(a.vc + off, (uint32_t)ps * 512u);
      base_row = lp * ps;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = 2 * u + (lane >> 5);
      const uint32_t rowoff = (uint32_t)(min(key0 + row, last) - base_row) * 512u;
      dma16_stream(kr, rowoff + 16u * ((lane & 31) ^ row), l0 + u * 1024);
      dma16_stream(vr, rowoff + 16u * ((lane & 31) ^ ((2 * row) & 15)), l0 + kChunkBytes + u * 1024);
    }
  };

  // Where the start of the visible range does not depend on the position
  // (ring caches, unbounded windows), the first chunk is requested now,
  // before the position has arrived; rows past the end of the visible range
  // are fixed below. (Not for a paged cache: its pages are staged first.)
  const bool spec = !kPaged && (a.ring != 0 || a.window <= 0) && sp * a.split_keys + wave * kChunk < a.cap;
  const int spec_key0 = sp * a.split_keys + wave * kChunk;
  if (spec) {
    load_rows(spec_key0, a.cap - 1, ring0[wave]);
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");   // this wave's staging load
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __builtin_amdgcn_s_barrier();   // every wave's staging load has landed

  if (p < 0 || p > a.max_pos) {
    if (a.nsplit == 1) {
      for (int hh = 0; hh < kGroup; ++hh)
        a.out[((size_t)b * a.Hq + kvh * kGroup + hh) * kHeadDim + t] = 0x7fc0;  // NaN
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }
  int lo, hi;
  decode_key_range(p, a.ring, a.cap, a.window, &lo, &hi);
  const int k0 = lo + sp * a.split_keys;
  const int k1 = min(k0 + a.split_keys, hi);
  const int slot = cache_slot(p, a.ring, a.cap);
  const int nchunks = k1 > k0 ? (k1 - k0 + kChunk - 1) / kChunk : 0;
  if constexpr (kPaged) {
    // the table entries of the pages holding keys k0 .. k1 - 1 (at most
    // one table row); the caller's staging loads have all landed above
    pg_lo = k0 / ps;
    const int n_pg = k1 > k0 ? (k1 - 1) / ps - pg_lo + 1 : 0;
    const int* tb = a.paged.table + (size_t)b * a.paged.pages_per_seq + pg_lo;
    for (int i = t; i < n_pg; i += 256) page_of[i] = tb[i];
    __syncthreads();
  }

  // DMA of chunk c of this split into a slot; rows past the split end re-read
  // its last key (their scores are masked).
  auto load_chunk = [&](int c, char* dst) __attribute__((always_inline)) {
    load_rows(k0 + c * kChunk, k1 - 1, dst);
  };
  // The first chunk: requested above if it held only visible keys, else now
  // (a later DMA into the same slot lands after an earlier one).
  if (wave < nchunks && (!spec || spec_key0 + kChunk > k1)) load_chunk(wave, ring0[wave]);
  const bool own_slot = slot >= k0 && slot < k1;
  const int slot_chunk = own_slot ? (slot - k0) / kChunk : -1;

  // ---- RoPE of the 4 queries: cos/sin of the fp64-reduced angle, rotation
  // in fp32, split into bf16 high and low parts. The owner of the new slot
  // also writes the new key, rotated in fp64 and rounded once to bf16 like
  // every cached key, and the new value; the LDS copy of the chunk that holds
  // the slot is patched with both (the DMA may have read the slot before the
  // store).
  {
    const int d = t;
    const int half = a.r >> 1;
    const int dp = d < half ? d + half : d - half;  // rotation partner
    double c = 1.0, s = 0.0;
    if (d < a.r) rope_sincos(p, freq_stage[d < half ? d : d - half], &s, &c);
    const float cf = (float)c, sf = (float)s;
#pragma unroll
    for (int hh = 0; hh < kGroup; ++hh) {
      const float qx = bf16_bits_to_float(q_stage[hh][d]);
      const float qxp = bf16_bits_to_float(q_stage[hh][dp]);
      float y = qx;
      if (d < a.r) y = d < half ? fmaf(qx, cf, -qxp * sf) : fmaf(qx, cf, qxp * sf);
      const uint16_t yh = float_to_bf16_bits(y);
      qcols[hh][d] = yh;
      qcols[4 + hh][d] = float_to_bf16_bits(y - bf16_bits_to_float(yh));
    }
    if (own_slot) {
      const double kx = (double)bf16_bits_to_float(kv_stage[0][d]);
      const double kxp = (double)bf16_bits_to_float(kv_stage[0][dp]);
      double y = kx;
      if (d < a.r) y = d < half ? kx * c - kxp * s : kx * c + kxp * s;
      const uint16_t kh = double_to_bf16_bits(y);
      const uint16_t vn = kv_stage[1][d];
      if constexpr (kPaged) {
        const int pg = page_of[slot / ps - pg_lo];
        if ((unsigned)pg < (unsigned)a.paged.num_pages) {  // else the write is dropped
          const size_t o = (((size_t)pg * a.Hkv + kvh) * ps + slot % ps) * kHeadDim + d;
          a.kc[o] = kh;
          a.vc[o] = vn;
        }
      } else {
        a.kc[kv_off + (size_t)slot * kHeadDim + d] = kh;
        a.vc[kv_off + (size_t)slot * kHeadDim + d] = vn;
      }
      newrow[0][d] = kh;
      newrow[1][d] = vn;
    }
  }
  // LDS-only barrier: the chunk loads and the new row's global stores stay
  // in flight.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();

  const int col = lane & 15;   // MFMA column (S) / row (P) index of this lane
  const int grp = lane >> 4;   // 16-lane group
  bf16x8 qb[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    bf16x8 v = bf16x8{};
    if (col < 8) v = *(const bf16x8*)(&qcols[col][ks * 32 + grp * 8]);
    qb[ks] = v;
  }

  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{};
  float m_run = -1e30f;  // running max of head col (lanes with col < 4)
  float l_run = 0.f;     // this lane's share of the running sum

  // LDS read offsets inside a slot. S, k-step ks: lane reads K row col,
  // piece 4ks + grp. P.V, MFMA n (channels 16n..16n+15): source lane
  // (w + 4v) of group grp reads V row 4grp + v, piece 2n + w/2, byte 8(w%2).
  const int vr_row = 4 * grp + ((lane >> 2) & 3);
  const int vr_w = lane & 3;
  const int k_base = (col >> 1) * 1024 + (col & 1) * 512;
  const int v_base = kChunkBytes + (vr_row >> 1) * 1024 + (vr_row & 1) * 512 + 8 * (vr_w & 1);

  // The new token's rows in the LDS copy of its chunk: row slot - key0, and
  // when the slot is the last visible key, also the rows past the end that
  // re-read it (their probabilities are zero, but a value read before the
  // store may be any bits, and 0 * NaN would reach the output).
  auto patch_new_row = [&](char* sl, int key0) __attribute__((always_inline)) {
    const int pc = lane & 31;                            // 16-byte piece
    const bool is_v = lane >= 32;
    const uint4 val = *(const uint4*)&newrow[is_v ? 1 : 0][pc * 8];
    const int r_end = slot == k1 - 1 ? kChunk : slot - key0 + 1;
    for (int r = slot - key0; r < r_end; ++r) {
      const int sw = is_v ? ((2 * r) & 15) : r;
      *(uint4*)(sl + (is_v ? kChunkBytes : 0) + (r >> 1) * 1024 + ((r & 1) * 32 + (pc ^ sw)) * 16) = val;
    }
  };
  auto compute = [&](char* sl, int c) __attribute__((always_inline)) {
    const int key0 = k0 + c * kChunk;
    if (c == slot_chunk) patch_new_row(sl, key0);
    // S = K . Qc
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 kf = *(const bf16x8*)(sl + k_base + 16 * ((4 * ks + grp) ^ col));
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qb[ks], sacc, 0, 0, 0);
    }
    // Register i: key key0 + 4grp + i, column col. Add each high column's
    // low partner (column + 4), scale, mask.
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = sacc[i] + __shfl_xor(sacc[i], 4, 64);
      x[i] = (key0 + 4 * grp + i < k1) ? v * kScoreScale : -__builtin_inff();
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = group4_max(mx);
    // lazy rescale: the running max moves only when a score exceeds it by
    // more than 2^8 (per head; the decision is per wave)
    const float m_new = fmaxf(m_run, mx);
    const bool move = __any(col < 4 && m_new > m_run + kRescaleSlack);
    const float m_use = move ? m_new : m_run;
    const float alpha = fast_exp2(m_run - m_use);
    float pr[4], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = fast_exp2(x[i] - m_use);
      ps += pr[i];
    }
    l_run = l_run * alpha + ps;
    m_run = m_use;
    if (move) {
      float al[4];
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) al[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), hh));
#pragma unroll
      for (int blk = 0; blk < 16; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[blk][i] *= al[i];
    }
    // P as the A operand (row col, keys 4grp + j): rows 0-3 the bf16 high
    // parts, rows 4-7 the low parts of head col - 4 (from lane - 4).
    s16x4 pa;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pl = __shfl_xor(pr[j], 4, 64);
      const uint16_t ph = float_to_bf16_bits(pr[j]);
      uint16_t pv = 0;
      if (col < 4) pv = ph;
      else if (col < 8) pv = float_to_bf16_bits(pl - bf16_bits_to_float(float_to_bf16_bits(pl)));
      pa[j] = (short)pv;
    }
    // O += P . V
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const s16x4 vb = lds_read_tr(sl + v_base + 16 * ((2 * n + (vr_w >> 1)) ^ ((2 * vr_row) & 15)));
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, acc[n], 0, 0, 0);
    }
  };

  // Two-slot ring per wave: the wave's chunks alternate between its slots.
  // Before a chunk is computed, the next one is requested into the other
  // slot (whose reads have finished: lgkmcnt(0)); then all but that
  // request's 16 loads must have landed.
  for (int c = wave; c < nchunks; c += 2 * kWaves) {
    // slot 0 holds chunk c; start chunk c + 4 into slot 1
    const int c1 = c + kWaves;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (c1 < nchunks) {
      load_chunk(c1, ring1[wave]);
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");   // chunk c has landed
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    compute(ring0[wave], c);
    if (c1 >= nchunks) break;
    const int c2 = c1 + kWaves;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (c2 < nchunks) {
      load_chunk(c2, ring0[wave]);
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    compute(ring1[wave], c1);
  }

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // also an unused first chunk
  // ---- merge: lane groups 0 and 1 hold the high and low parts of the 4
  // heads' outputs (one float4 of heads per channel); the four lane groups
  // hold disjoint keys of each head's running sum.
  {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane16_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  __syncthreads();
  f32x4* om = (f32x4*)&ring0[0][0];  // [wave][high, low][channel] -> float4 over heads
  if (grp < 2) {
#pragma unroll
    for (int blk = 0; blk < 16; ++blk) om[(wave * 2 + grp) * kHeadDim + blk * 16 + col] = acc[blk];
  }
  if (lane < 4) {
    red_m[wave][lane] = m_run;
    red_l[wave][lane] = l_run;
  }
  __syncthreads();
  const int d = t;
  float M[kGroup], L[kGroup], O[kGroup];
#pragma unroll
  for (int hh = 0; hh < kGroup; ++hh) {
    M[hh] = red_m[0][hh];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M[hh] = fmaxf(M[hh], red_m[w][hh]);
    L[hh] = 0.f;
    O[hh] = 0.f;
  }
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const f32x4 hi = om[(w * 2) * kHeadDim + d];
    const f32x4 lo = om[(w * 2 + 1) * kHeadDim + d];
#pragma unroll
    for (int hh = 0; hh < kGroup; ++hh) {
      const float e = fast_exp2(red_m[w][hh] - M[hh]);
      L[hh] += e * red_l[w][hh];
      O[hh] += e * (hi[hh] + lo[hh]);
    }
  }
#pragma unroll
  for (int hh = 0; hh < kGroup; ++hh) {
    const int h = kvh * kGroup + hh;
    if (a.nsplit == 1) {
      const float g = bf16_bits_to_float(gate_bits[hh]);
      a.out[((size_t)b * a.Hq + h) * kHeadDim + d] = float_to_bf16_bits(O[hh] / L[hh] * gate_factor(g, a.gate_act));
    } else {
      const size_t pi = ((size_t)b * a.Hq + h) * a.nsplit + sp;
      a.part_o[pi * kHeadDim + d] = O[hh];
      if (d == 0) {
        a.part_ml[pi * 2 + 0] = M[hh];
        a.part_ml[pi * 2 + 1] = L[hh];
      }
    }
  }
}

// Merge of the split partials, gate, bf16 store. One block per (sequence,
// head, quarter of the channels), so even a single sequence spreads over
// 64 blocks: the block turns every split's (m, l) into a weight 2^(m_s - M)
// and the total L, then 16 thread groups each sum every 16th split for the
// block's 64 channels (8 loads in flight per thread) and combine in a fixed
// order, so the result does not depend on timing.
constexpr int kMergeThreads = 1024;
constexpr int kMaxSplits = 2048;
constexpr int kMergeChannels = 64;                          // channels per block
constexpr int kMergeGroups = kMergeThreads / kMergeChannels;  // split groups per block
constexpr int kMergeBlocksPerHead = kHeadDim / kMergeChannels;

__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[kMergeThreads / 64];
  __shared__ float part[kMergeGroups][kMergeChannels];
  const int bh = (int)blockIdx.x / kMergeBlocksPerHead;
  const int c0 = ((int)blockIdx.x % kMergeBlocksPerHead) * kMergeChannels;
  const int b = bh / a.Hq;
  const int h = bh % a.Hq;
  const int t = threadIdx.x;
  const int p = a.pos[b];
  uint16_t* o = a.out + ((size_t)b * a.Hq + h) * kHeadDim + c0;
  if (p < 0 || p > a.max_pos) {
    if (t < kMergeChannels) o[t] = 0x7fc0;
    return;
  }
  const size_t base = ((size_t)b * a.Hq + h) * a.nsplit;
  // M = max_s m_s
  float mx = -__builtin_inff();
  for (int s = t; s < a.nsplit; s += kMergeThreads) mx = fmaxf(mx, a.part_ml[(base + s) * 2]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  float M = red[0];
  for (int i = 1; i < kMergeThreads / 64; ++i) M = fmaxf(M, red[i]);
  __syncthreads();
  // weights and L = sum_s w_s l_s
  float ls = 0.f;
  for (int s = t; s < a.nsplit; s += kMergeThreads) {
    const float w = fast_exp2(a.part_ml[(base + s) * 2] - M);
    wgt[s] = w;
    ls += w * a.part_ml[(base + s) * 2 + 1];
  }
  for (int off = 32; off > 0; off >>= 1) ls += __shfl_xor(ls, off, 64);
  if ((t & 63) == 0) red[t >> 6] = ls;
  __syncthreads();
  float L = 0.f;
  for (int i = 0; i < kMergeThreads / 64; ++i) L += red[i];
  // O[d] = sum_s w_s o_s[d]; thread group g takes splits g, g + 16, ...
  const int g = t / kMergeChannels, dl = t % kMergeChannels;
  const float* po = a.part_o + base * kHeadDim + c0 + dl;
  float acc = 0.f;
  int s = g;
  for (; s + 7 * kMergeGroups < a.nsplit; s += 8 * kMergeGroups) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = po[(size_t)(s + kMergeGroups * u) * kHeadDim];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += wgt[s + kMergeGroups * u] * v[u];
  }
  for (; s < a.nsplit; s += kMergeGroups) acc += wgt[s] * po[(size_t)s * kHeadDim];
  part[g][dl] = acc;
  __syncthreads();
  if (g == 0) {
    float O = part[0][dl];
#pragma unroll
    for (int i = 1; i < kMergeGroups; ++i) O += part[i][dl];
    const float gl = bf16_bits_to_float(a.gate[(size_t)b * a.gate_stride + h]);
    o[dl] = float_to_bf16_bits(O / L * gate_factor(gl, a.gate_act));
  }
}

hipError_t decode_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int grid = a.B * a.Hkv * a.nsplit;
  if (grid == 0) return hipSuccess;
  if (a.paged.table)
    hipLaunchKernelGGL(decode_kernel<true>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(decode_kernel<false>, dim3(grid), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(a.B * a.Hq * kMergeBlocksPerHead), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hattn
