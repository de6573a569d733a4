// Flash-style prefill attention for gfx950 (page "Spark-X2.5 架构（4B / 1.7B）",
// §3 Eq. 1: softmax(Q K^T / sqrt(256)) V times a per-head sigmoid gate; §2:
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
// K and V tiles go from global memory straight into LDS (global_load_lds,
// 16 B per lane) in the order the MFMA reads them, so every LDS read is a
// contiguous, conflict-free 512 B per half-wave at "lane base + constant".
// Two K slots and two V slots form a pipeline: step t computes S(t) and
// issues P(t-1).V(t-1), so the softmax of tile t (VALU) runs while the
// matrix cores work on P.V of tile t-1, and tiles t+1 (K) and t (V) load
// meanwhile. The running max is only moved (and O rescaled) when a tile's max
// exceeds it by more than 2^8, so most tiles skip the rescale; the step body
// has no branch between its MFMAs and its softmax.
#include <type_traits>

#include "hattn_device.h"
#include "hattn_internal.h"

namespace hattn {

namespace {

constexpr int kBM = kPrefillBlockQ;              // query positions per workgroup
constexpr int kBN = 64;                          // keys per tile
constexpr int kTileBytes = kBN * kHeadDim * 2;   // 32 KiB: one K or V tile
constexpr float kScoreScale = kLog2e / 16.0f;    // 1/sqrt(256), in log2 units
constexpr float kRescaleSlack = 8.0f;            // log2 units

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ s16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// 16 bytes per lane from global memory to LDS; lane l lands at lds + 16*l.
__device__ __forceinline__ void load_lds16(const void* g, char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void unpack8(uint4 u, float* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

}  // namespace

__global__ __launch_bounds__(256, 1) void prefill_attn_kernel(PrefillAttnArgs a) {
  // K slot layout: block (ks, h) = channels (2*ks + h)*8 .. +7 of the 64 rows,
  // 16 B per row, at (2*ks + h) * 1 KiB. V slot layout: block (tt, db) at
  // (tt*8 + db) * 1 KiB holds keys 16*tt .. +15 x channels 32*db .. +31 as 64
  // units of 8 B; unit L = 16g + 4v + a of half j2 (512 B each) is key
  // 16tt + 8j2 + 4(g/2) + v, channels 32db + 16(g%2) + 4a .. +3.
  // Four separate arrays (not one indexed array) so the compiler can tell the
  // slot being filled from the slot being read and does not wait for the
  // in-flight tile loads before reading the current tile.
  __shared__ __attribute__((aligned(1024))) char k_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_lds1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds1[kTileBytes];

  // Longest query blocks first; then sequence, then KV head.
  const int per_qt = a.B * a.Hkv;
  const int qt = a.q_tiles - 1 - (int)blockIdx.x / per_qt;
  const int r2 = (int)blockIdx.x % per_qt;
  const int b = r2 / a.Hkv;
  const int kvh = r2 % a.Hkv;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = kvh * kGroup + wave;
  const int q0 = qt * kBM;
  const int nq = min(kBM, a.S - q0);
  const int pq_first = a.start[b] + q0;
  const int pq_last = pq_first + nq - 1;
  const int kp0 = a.key_pos0[b];
  const int nk = a.n_keys[b];
  const int lo_pos = a.window > 0 ? max(pq_first - a.window + 1, 0) : 0;
  const int row_lo = max(lo_pos - kp0, 0);
  const int row_hi = min(pq_last - kp0 + 1, nk);
  const int t_lo = row_lo / kBN;
  const int nt = (row_hi + kBN - 1) / kBN - t_lo;

  const size_t kv_off = ((size_t)b * a.Hkv + kvh) * (size_t)a.rows * kHeadDim;
  const char* kbase = (const char*)(a.kc + kv_off);
  const char* vbase = (const char*)(a.vc + kv_off);

  // Each wave stages 8 of the 32 K blocks and 8 of the 32 V blocks of a
  // tile. Rows past the valid keys re-read the last valid key; their scores
  // are masked, so they contribute exactly zero.
  const int v_lane_key = 8 * (lane >> 5) + 4 * ((lane >> 4) & 1) + ((lane >> 1) & 3);
  const int v_lane_col = 32 * ((lane >> 3) & 1) + 16 * (lane & 1);  // bytes
  auto load_k = [&](int t, char* slot) __attribute__((always_inline)) {
    char* dst = slot + wave * 8 * 1024;
    const uint32_t off = (uint32_t)min(t * kBN + lane, nk - 1) * 512u + (uint32_t)wave * 128u;
#pragma unroll
    for (int u = 0; u < 8; ++u) load_lds16(kbase + off + u * 16, dst + u * 1024);
  };
  auto load_v = [&](int t, char* slot) __attribute__((always_inline)) {
    char* dst = slot + wave * 8 * 1024;
    const uint32_t off = (uint32_t)min(t * kBN + 16 * wave + v_lane_key, nk - 1) * 512u + (uint32_t)v_lane_col;
#pragma unroll
    for (int db = 0; db < 8; ++db) load_lds16(vbase + off + db * 64, dst + db * 1024);
  };

  // Start the first tiles moving before the query prologue.
  load_k(t_lo, k_lds0);
  if (nt > 1) load_k(t_lo + 1, k_lds1);
  load_v(t_lo, v_lds0);

  // ---- queries: RoPE in fp32 from the cos/sin table, then bf16 fragments
  // (B operand of S^T): lane holds query lane % 32, channels
  // ks*16 + (lane / 32)*8 .. +7 for ks = 0..15.
  const int qrow = q0 + (lane & 31);
  const bool qvalid = qrow < a.S;
  bf16x8 qf[16];
  {
    const int qr = qvalid ? qrow : a.S - 1;
    const uint16_t* qp = a.q + (((size_t)b * a.S + qr) * a.Hq + h) * kHeadDim;
    const int half = a.r >> 1;
    const float2* tp = a.table + ((size_t)b * a.S + qr) * half;
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
          x[j] = first ? x[j] * t.x - xp[j] * t.y : x[j] * t.x + xp[j] * t.y;
        }
      }
      bf16x8 v;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (__bf16)(qvalid ? x[j] : 0.f);
      qf[ks] = v;
    }
    // The fragments are only ever MFMA operands: keep them in the
    // accumulation registers, which leaves the VGPRs to the softmax.
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) asm volatile("" : "+a"(qf[ks]));
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

  // V^T fragments: lane (16g + i) of a transposed read gets channel
  // 32db + 16(g%2) + i of keys 16tt + 8j2 + 4(g/2) + 0..3, which are the key
  // slots (g/2)*8 + 4*j2 + 0..3 of the P^T fragment.
  const int tr_off = lane * 8;
  // P.V with the V^T fragments read 3 MFMAs ahead of their use, so LDS
  // latency hides behind the matrix cores.
  auto pv = [&](const char* vslot, const bf16x8* p) __attribute__((always_inline)) {
    const char* vt = vslot + tr_off;
    constexpr int kAhead = 3;
    s16x4 vl[kAhead + 1], vh[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      vl[i] = lds_read_tr(vt + i * 1024);
      vh[i] = lds_read_tr(vt + i * 1024 + 512);
    }
#pragma unroll
    for (int n = 0; n < 32; ++n) {  // n = tt*8 + db
      if (n + kAhead < 32) {
        vl[(n + kAhead) % (kAhead + 1)] = lds_read_tr(vt + (n + kAhead) * 1024);
        vh[(n + kAhead) % (kAhead + 1)] = lds_read_tr(vt + (n + kAhead) * 1024 + 512);
      }
      const s16x8 both = __builtin_shufflevector(vl[n % (kAhead + 1)], vh[n % (kAhead + 1)], 0, 1, 2, 3, 4, 5, 6, 7);
      acc[n & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), p[n >> 3], acc[n & 7], 0, 0, 0);
    }
    // Keep O resident in the accumulation registers between tiles (the
    // register allocator otherwise parks it in VGPRs and copies it every
    // tile).
#pragma unroll
    for (int db = 0; db < 8; ++db) asm volatile("" : "+a"(acc[db]));
  };

  // Mask of tile t's scores. Register i of block kb holds key row
  // t*64 + kb*32 + 8*(i/4) + 4*(lane/32) + i%4 for query lane % 32.
  auto mask_s = [&](int t, f32x16& s0, f32x16& s1) __attribute__((always_inline)) {
    const int pq = pq_first + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k0 = t * kBN + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      const bool ok0 = k0 < nk && key_visible(pq, kp0 + k0, a.window);
      const bool ok1 = k0 + 32 < nk && key_visible(pq, kp0 + k0 + 32, a.window);
      s0[i] = ok0 ? s0[i] : -__builtin_inff();
      s1[i] = ok1 ? s1[i] : -__builtin_inff();
    }
  };
  // S^T with the K fragments read 3 k-steps ahead of their use.
  auto compute_s = [&](const char* kslot, f32x16& s0, f32x16& s1) __attribute__((always_inline)) {
    const char* base = kslot + (lane >> 5) * 1024 + (lane & 31) * 16;
    constexpr int kAhead = 3;
    bf16x8 fa[kAhead + 1], fb[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      fa[i] = *(const bf16x8*)(base + i * 2048);
      fb[i] = *(const bf16x8*)(base + i * 2048 + 512);
    }
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      if (ks + kAhead < 16) {
        fa[(ks + kAhead) % (kAhead + 1)] = *(const bf16x8*)(base + (ks + kAhead) * 2048);
        fb[(ks + kAhead) % (kAhead + 1)] = *(const bf16x8*)(base + (ks + kAhead) * 2048 + 512);
      }
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks % (kAhead + 1)], qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks % (kAhead + 1)], qf[ks], s1, 0, 0, 0);
    }
    // scores feed VALU code: produce them in VGPRs
    asm volatile("" : "+v"(s0), "+v"(s1));
  };
  // Softmax of one tile's scores into pb. The running max moves only when
  // the tile's max exceeds it by more than 2^8; returns the factor O must be
  // rescaled by (1 when the max did not move).
  auto softmax = [&](f32x16& s0, f32x16& s1, bf16x8* pb) __attribute__((always_inline)) {
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32)) * kScoreScale;
    const float m_new = fmaxf(m_i, mx);
    const bool rescale = __any(m_new > m_i + kRescaleSlack);
    const float m_use = rescale ? m_new : m_i;
    const float alpha = fast_exp2(m_i - m_use);
    // step tt of P^T covers keys 16tt .. +15; its key slot (lane/32)*8 + j
    // is register 8*(tt%2) + j of block tt/2
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p0 = fast_exp2(fmaf(s0[i], kScoreScale, -m_use));
      const float p1 = fast_exp2(fmaf(s1[i], kScoreScale, -m_use));
      rs += p0 + p1;
      pb[i >> 3][i & 7] = (__bf16)p0;
      pb[2 + (i >> 3)][i & 7] = (__bf16)p1;
    }
    rs += wave_shfl_xor(rs, 32);
    l_i = l_i * alpha + rs;
    m_i = m_use;
    return rescale ? alpha : 1.0f;
  };
  // O *= alpha in place in the accumulation registers (read, multiply,
  // write back per element), so O never has to move to VGPRs.
  auto rescale_o = [&](float alpha) __attribute__((always_inline)) {
    if (alpha != 1.0f) {
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
    }
  };

  // Iteration j (tile t = t_lo + j) overlaps three things: the softmax of
  // S(t) (VALU), S(t+1) = K(t+1) Q^T and P(t-1).V(t-1) (MFMA), and the loads
  // of K(t+2) and V(t). Tile j's K lives in k_lds[j % 2] and its V in
  // v_lds[j % 2]; the score and probability registers alternate the same
  // way, so every slot and register set is fixed at compile time.
  load_k(t_lo, k_lds0);
  if (nt > 1) load_k(t_lo + 1, k_lds1);
  f32x16 sA0, sA1, sB0, sB1;  // scores of even / odd tiles
  bf16x8 pA[4], pB[4];        // probabilities of even / odd tiles
  wait_loads();
  __syncthreads();
  compute_s(k_lds0, sA0, sA1);
  if (need_mask(t_lo)) mask_s(t_lo, sA0, sA1);

  // One iteration; kPv is false only for the first tile. On the last tile
  // S(t+1) is computed from a stale slot and discarded, which keeps the body
  // free of branches between its MFMAs and its softmax.
  auto step = [&](auto has_pv, int j, const char* kn, const char* vp, char* kf, char* vf, f32x16& sc0,
                  f32x16& sc1, f32x16& sn0, f32x16& sn1, const bf16x8* pp,
                  bf16x8* pn) __attribute__((always_inline)) {
    constexpr bool kPv = decltype(has_pv)::value;
    const int t = t_lo + j;
    wait_loads();
    __syncthreads();
    if (j + 2 < nt) load_k(t + 2, kf);
    load_v(t, vf);
    compute_s(kn, sn0, sn1);
    if (kPv) pv(vp, pp);
    const float alpha = softmax(sc0, sc1, pn);
    rescale_o(alpha);
    if (j + 1 < nt && need_mask(t + 1)) mask_s(t + 1, sn0, sn1);
  };
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  // even j: S(t) in sA, P(t) -> pA, P(t-1) in pB; odd j: the other way round
  step(F_{}, 0, k_lds1, v_lds1, k_lds0, v_lds0, sA0, sA1, sB0, sB1, pB, pA);
  for (int j = 1; j < nt; j += 2) {
    step(T_{}, j, k_lds0, v_lds0, k_lds1, v_lds1, sB0, sB1, sA0, sA1, pA, pB);
    if (j + 1 < nt) step(T_{}, j + 1, k_lds1, v_lds1, k_lds0, v_lds0, sA0, sA1, sB0, sB1, pB, pA);
  }
  // P.V of the last tile
  wait_loads();
  __syncthreads();
  if ((nt - 1) & 1) pv(v_lds1, pB);
  else pv(v_lds0, pA);

  // ---- epilogue: divide by the softmax sum, gate in fp32, one bf16 store.
  // acc[db] register i holds channel db*32 + 8*(i/4) + 4*(lane/32) + i%4.
  if (qvalid) {
    const size_t orow = ((size_t)b * a.S + qrow) * a.Hq + h;
    const float g = bf16_bits_to_float(a.gate[orow]);
    const float f = (1.0f / l_i) * (1.0f / (1.0f + expf(-g)));
    uint16_t* op = a.out + orow * kHeadDim + 4 * (lane >> 5);
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w0 = (uint32_t)float_to_bf16_bits(acc[db][4 * c + 0] * f) |
                            ((uint32_t)float_to_bf16_bits(acc[db][4 * c + 1] * f) << 16);
        const uint32_t w1 = (uint32_t)float_to_bf16_bits(acc[db][4 * c + 2] * f) |
                            ((uint32_t)float_to_bf16_bits(acc[db][4 * c + 3] * f) << 16);
        *(uint2*)(op + db * 32 + 8 * c) = make_uint2(w0, w1);
      }
  }
}

hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t s) {
  const int grid = a.q_tiles * a.B * a.Hkv;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hattn
