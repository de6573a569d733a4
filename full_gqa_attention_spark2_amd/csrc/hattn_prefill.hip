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
// Two K slots and two V slots form a pipeline: while tile t's softmax and
// P.V run, S for tile t+1 is computed and tiles t+1 (V) and t+2 (K) load.
// The running max is only moved (and O rescaled) when a tile's max exceeds it
// by more than 2^8, so most tiles skip the rescale.
#include "hattn_device.h"
#include "hattn_internal.h"

namespace hattn {

namespace {

constexpr int kBM = 32;                          // query positions per workgroup
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
  const int wave = threadIdx.x >> 6;
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
  const uint16_t* kbase = a.kc + kv_off;
  const uint16_t* vbase = a.vc + kv_off;

  // Each wave stages 8 of the 32 K blocks and 8 of the 32 V blocks of a
  // tile. Rows past the valid keys re-read the last valid key; their scores
  // are masked, so they contribute exactly zero.
  auto load_k = [&](int t, char* slot) {
    char* dst = slot + wave * 8 * 1024;
    const int row = min(t * kBN + lane, nk - 1);
    const uint16_t* src = kbase + (size_t)row * kHeadDim + wave * 64;
#pragma unroll
    for (int u = 0; u < 8; ++u) load_lds16(src + u * 8, dst + u * 1024);
  };
  auto load_v = [&](int t, char* slot) {
    char* dst = slot + wave * 8 * 1024;
    const int key = t * kBN + 16 * wave + 8 * (lane >> 5) + 4 * ((lane >> 4) & 1) + ((lane >> 1) & 3);
    const uint16_t* src = vbase + (size_t)min(key, nk - 1) * kHeadDim + 16 * ((lane >> 3) & 1) + 8 * (lane & 1);
#pragma unroll
    for (int db = 0; db < 8; ++db) load_lds16(src + db * 32, dst + db * 1024);
  };

  // Start the first tiles moving before the query prologue.
  load_k(t_lo, k_lds0);
  load_v(t_lo, v_lds0);
  if (nt > 1) load_k(t_lo + 1, k_lds1);

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
  }

  auto compute_s = [&](const char* kt, f32x16& s0, f32x16& s1) {
    const char* base = kt + (lane >> 5) * 1024 + (lane & 31) * 16;
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8 a0 = *(const bf16x8*)(base + ks * 2048);
      const bf16x8 a1 = *(const bf16x8*)(base + ks * 2048 + 512);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], s1, 0, 0, 0);
    }
  };
  auto need_mask = [&](int t) {
    const int row0 = t * kBN;
    return (kp0 + row0 + kBN - 1 > pq_first) || (a.window > 0 && kp0 + row0 <= pq_last - a.window) ||
           (row0 + kBN > nk);
  };
  // Register i of block kb holds key row t*64 + kb*32 + 8*(i/4) + 4*(lane/32)
  // + i%4 for query lane % 32.
  auto mask_s = [&](int t, f32x16& s0, f32x16& s1) {
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

  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  float m_i = -1e30f;  // running max (log2 units) of this lane's query
  float l_i = 0.f;     // running sum

  wait_loads();
  __syncthreads();
  f32x16 sc0, sc1;
  compute_s(k_lds0, sc0, sc1);
  if (need_mask(t_lo)) mask_s(t_lo, sc0, sc1);

  // V^T fragments: lane (16g + i) of a transposed read gets channel
  // 32db + 16(g%2) + i of keys 16tt + 8j2 + 4(g/2) + 0..3, which are the key
  // slots (g/2)*8 + 4*j2 + 0..3 the P^T fragment below uses.
  const int tr_off = lane * 8;

  // One pipeline step for tile t = t_lo + j. Slots: kn holds K(t+1), vc holds
  // V(t); K(t+2) goes to kf and V(t+1) to vf, the slots step j-1 read.
  auto step = [&](int j, const char* kn, const char* vc, char* kf, char* vf) {
    const int t = t_lo + j;
    wait_loads();
    __syncthreads();
    if (j + 1 < nt) load_v(t + 1, vf);
    if (j + 2 < nt) load_k(t + 2, kf);

    // ---- running max of tile t; rescale only when it grows by > 2^8
    float mx = fmaxf(sc0[0], sc1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(sc0[i], sc1[i]));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32)) * kScoreScale;
    const float m_new = fmaxf(m_i, mx);
    if (__any(m_new > m_i + kRescaleSlack)) {
      const float alpha = fast_exp2(m_i - m_new);
      l_i *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      m_i = m_new;
    }

    // ---- S for tile t+1 (on the last tile this reads a stale slot and is
    // discarded); independent of the softmax below, so the two interleave.
    f32x16 sn0, sn1;
    compute_s(kn, sn0, sn1);

    // ---- probabilities of tile t and P^T fragments: step tt covers keys
    // 16tt .. +15; key slot (lane/32)*8 + j of the step is register
    // 8*(tt%2) + j of block tt/2.
    float rs = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p0 = fast_exp2(fmaf(sc0[i], kScoreScale, -m_i));
      const float p1 = fast_exp2(fmaf(sc1[i], kScoreScale, -m_i));
      rs += p0 + p1;
      pb[i >> 3][i & 7] = (__bf16)p0;
      pb[2 + (i >> 3)][i & 7] = (__bf16)p1;
    }
    rs += wave_shfl_xor(rs, 32);
    l_i += rs;

    // ---- O^T += V^T P^T for tile t
    const char* vt = vc + tr_off;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const char* blk = vt + (tt * 8 + db) * 1024;
        const s16x4 lo = lds_read_tr(blk);
        const s16x4 hi = lds_read_tr(blk + 512);
        const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pb[tt], acc[db], 0, 0, 0);
      }

    if (j + 1 < nt && need_mask(t + 1)) mask_s(t + 1, sn0, sn1);
    sc0 = sn0;
    sc1 = sn1;
  };

  for (int j = 0; j < nt; j += 2) {
    step(j, k_lds1, v_lds0, k_lds0, v_lds1);
    if (j + 1 < nt) step(j + 1, k_lds0, v_lds1, k_lds1, v_lds0);
  }

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
