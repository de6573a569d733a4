// Flash-style prefill attention for gfx950 (page "Spark-X2.5 架构（4B / 1.7B）",
// §3 Eq. 1: softmax(Q K^T / sqrt(256)) V times a per-head sigmoid gate; §2:
// causal mask, plus the 512-token window on sliding layers).
//
// One workgroup = one (sequence, KV head, block of 32 query positions); its
// four waves are the four query heads of the GQA group, so every K/V tile
// staged in LDS feeds 4 x 32 query rows.
//
// Per 64-key tile and wave (bf16 MFMA 32x32x16, fp32 accumulate):
//   S^T[64 keys][32 q]  = K_tile . Q^T   (A = K from LDS, B = Q in registers)
//   online softmax per query column: one lane pair holds a query's 64 scores
//   O^T[256 d][32 q]   += V_tile^T . P^T (A = V^T via ds_read_tr16_b64, B = P)
// Keeping the transposed orientation puts a query's running max, sum and
// rescale factor in one lane, so the O rescale is a per-lane multiply.
// Tiles wholly outside the causal window are never visited; only tiles that
// straddle the diagonal, the window edge or the end of the keys are masked.
#include "hattn_device.h"
#include "hattn_internal.h"

namespace hattn {

namespace {

constexpr int kBM = 32;          // query positions per workgroup (per wave)
constexpr int kBN = 64;          // keys per tile
// Padded row pitches keep every LDS address "lane base + constant", so the
// unrolled reads use immediate offsets. K rows are 16 B apart in bank space:
// the 16 rows one b128 read phase touches at a fixed chunk hit 16 different
// bank groups. V rows are 64 B apart: the 4 rows x 64 B that one half-wave of
// a transposed read touches cover all 64 banks once.
constexpr int kKPitch = kHeadDim * 2 + 16;      // 528 B
constexpr int kVPitch = kHeadDim * 2 + 64;      // 576 B
constexpr int kKTileBytes = kBN * kKPitch;
constexpr int kVTileBytes = kBN * kVPitch;
constexpr int kStageBytes = kKTileBytes + kVTileBytes;  // 69 KiB
constexpr float kScoreScale = kLog2e / 16.0f;   // 1/sqrt(256), in log2 units

__device__ __forceinline__ int k_off(int row, int ch) { return row * kKPitch + (ch << 4); }
__device__ __forceinline__ int v_off(int row, int ch) { return row * kVPitch + (ch << 4); }

typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ s16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

}  // namespace

__global__ __launch_bounds__(256, 1) void prefill_attn_kernel(PrefillAttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];  // 138 KiB

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
  const int t_hi = (row_hi + kBN - 1) / kBN;

  const size_t kv_off = ((size_t)b * a.Hkv + kvh) * (size_t)a.rows * kHeadDim;
  const uint16_t* kbase = a.kc + kv_off;
  const uint16_t* vbase = a.vc + kv_off;

  // Q fragments (B operand of S^T): lane holds query (lane % 32), channels
  // ks*16 + (lane / 32)*8 .. +7 for ks = 0..15.
  const int qrow = q0 + (lane & 31);
  const bool qvalid = qrow < a.S;
  bf16x8 qf[16];
  {
    const uint16_t* qp = a.qhat + (((size_t)b * a.S + (qvalid ? qrow : 0)) * a.Hq + h) * kHeadDim + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      bf16x8 v = *(const bf16x8*)(qp + ks * 16);
      if (!qvalid) v = bf16x8{};
      qf[ks] = v;
    }
  }

  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  float m_i = -1e30f;  // running max (log2 units) of this lane's query
  float l_i = 0.f;     // running sum

  // Global -> register staging of one K and one V tile: 2048 16-byte chunks
  // each, 8 per thread; rows past the valid keys are zero-filled.
  uint4 kr[8], vr[8];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = threadIdx.x + 256 * u;
      const int row = c >> 5, ch = c & 31;
      const int krow = t * kBN + row;
      if (krow < nk) {
        kr[u] = *(const uint4*)(kbase + (size_t)krow * kHeadDim + ch * 8);
        vr[u] = *(const uint4*)(vbase + (size_t)krow * kHeadDim + ch * 8);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int stage) {
    char* ks = smem + stage * kStageBytes;
    char* vs = ks + kKTileBytes;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = threadIdx.x + 256 * u;
      const int row = c >> 5, ch = c & 31;
      *(uint4*)(ks + k_off(row, ch)) = kr[u];
      *(uint4*)(vs + v_off(row, ch)) = vr[u];
    }
  };

  if (t_lo < t_hi) {
    load_tile(t_lo);
    store_tile(0);
  }
  __syncthreads();

  // Lane-constant pieces of the transposed V read (see v_frag below).
  const int g16 = lane >> 4;         // 16-lane group
  const int i16 = lane & 15;
  const int tr_a = i16 & 3;          // which 4-channel slice this lane fetches
  const int tr_v = i16 >> 2;         // which key row of the 4 this lane fetches
  const int tr_h = g16 >> 1;

  for (int t = t_lo; t < t_hi; ++t) {
    const int stage = (t - t_lo) & 1;
    const bool has_next = t + 1 < t_hi;
    if (has_next) load_tile(t + 1);
    const char* Ks = smem + stage * kStageBytes;
    const char* Vs = Ks + kKTileBytes;

    // ---- S^T = K Q^T for keys t*64 .. +63
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const int ch = ks * 2 + (lane >> 5);
      const int r = lane & 31;
      const bf16x8 a0 = *(const bf16x8*)(Ks + k_off(r, ch));
      const bf16x8 a1 = *(const bf16x8*)(Ks + k_off(r + 32, ch));
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], s1, 0, 0, 0);
    }

    // ---- mask and online softmax. Register i of block kb holds key row
    // t*64 + kb*32 + 8*(i/4) + 4*(lane/32) + i%4 for query lane % 32.
    float x[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = s0[i] * kScoreScale;
      x[16 + i] = s1[i] * kScoreScale;
    }
    const int row0 = t * kBN;
    const bool need_mask = (kp0 + row0 + kBN - 1 > pq_first) ||
                           (a.window > 0 && kp0 + row0 <= pq_last - a.window) ||
                           (row0 + kBN > nk);
    if (need_mask) {
      const int pq = pq_first + (lane & 31);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int krow = row0 + (j >> 4) * 32 + 8 * ((j & 15) >> 2) + 4 * (lane >> 5) + (j & 3);
        if (!(krow < nk && key_visible(pq, kp0 + krow, a.window))) x[j] = -__builtin_inff();
      }
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) mx = fmaxf(mx, x[j]);
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float m_new = fmaxf(m_i, mx);
    const float alpha = fast_exp2(m_i - m_new);
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      x[j] = fast_exp2(x[j] - m_new);
      rs += x[j];
    }
    rs += wave_shfl_xor(rs, 32);
    l_i = l_i * alpha + rs;
    m_i = m_new;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;

    // ---- P^T as the B operand: step tt covers keys 16*tt .. +15; key slot
    // (lane/32)*8 + j of that step is register 8*(tt%2) + j of block tt/2.
    bf16x8 pb[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[tt][j] = (__bf16)x[(tt >> 1) * 16 + 8 * (tt & 1) + j];

    // ---- O^T += V^T P^T. A operand lane l holds V[key(slot)][d] for
    // d = db*32 + l%32 and key slots (l/32)*8 + j; slots 0..3 of a lane half
    // are keys 4*(l/32) + 0..3 and slots 4..7 are keys 8 + 4*(l/32) + 0..3 of
    // the step. ds_read_tr16_b64 gives lane i of a 16-lane group element
    // (i % 4) of the 8-byte rows fetched by lanes i/4 + 4v, v = 0..3, so lane
    // (a + 4v) fetches row (base + v), channels d0 + 4a .. +3.
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int rowA = tt * 16 + 4 * tr_h + tr_v;
      const int rowB = rowA + 8;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int col = db * 32 + (g16 & 1) * 16 + 4 * tr_a;
        const int ch = col >> 3, off = (col & 7) * 2;
        const s16x4 lo = lds_read_tr(Vs + v_off(rowA, ch) + off);
        const s16x4 hi = lds_read_tr(Vs + v_off(rowB, ch) + off);
        const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pb[tt], acc[db], 0, 0, 0);
      }
    }

    if (has_next) store_tile(stage ^ 1);
    __syncthreads();
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
