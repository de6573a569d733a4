// Split-K decode attention for gfx950 (page "Spark-X2.5 架构（4B / 1.7B）",
// §3 Eq. 1 and §4; the explainer page: each generated token reads the layer's
// KV cache, which on sliding layers is bounded to the last 512 tokens).
//
// One workgroup = one (sequence, KV head, split of the visible key range).
// Decode is HBM-bound: every K/V byte of the split is read once and serves
// the 4 query heads of the GQA group. Its four waves take 32-key chunks in
// turn; per chunk and wave:
//   S^T[16 keys][16 cols] = K . Qc   (bf16 MFMA 16x16x32, K straight from
//     HBM in A-operand layout; columns 0-3 hold the bf16 high parts of the 4
//     rotated queries, columns 4-7 their bf16 low parts, so the score is
//     computed with ~16 significant query bits)
//   O[16 rows][256]      += P . V     (rows 0-3: bf16 high parts of the 4
//     heads' probabilities, rows 4-7 their low parts; V goes through a
//     wave-private LDS buffer and comes back transposed by ds_read_tr16_b64)
// The spare MFMA rows and columns carry the low parts, so the extra
// precision costs no extra instructions. The waves merge (m, l, o) in LDS;
// with several splits a second kernel merges the splits in a fixed order.
#include "hattn_device.h"
#include "hattn_internal.h"

namespace hattn {

namespace {

constexpr int kChunk = 32;                      // keys per wave iteration
constexpr float kScoreScale = kLog2e / 16.0f;   // 1/sqrt(256), in log2 units

typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ s16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// V chunk in LDS with a 544 B row pitch: a transposed read touches 16 rows x
// 32 B at one column; rows 32 B apart in bank space put each half-wave's 8
// rows on distinct banks, and addresses stay "lane base + constant".
constexpr int kVPitch = kHeadDim * 2 + 32;
__device__ __forceinline__ int v_off(int row, int ch) { return row * kVPitch + (ch << 4); }

__device__ __forceinline__ float sigmoidf_(float g) { return 1.0f / (1.0f + expf(-g)); }

}  // namespace

template <int kWaves>
__global__ __launch_bounds__(kWaves * 64, 8 / kWaves) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char vbuf[kWaves][kChunk * kVPitch];   // 17 KiB per wave
  __shared__ __attribute__((aligned(16))) uint16_t qcols[8][kHeadDim];  // 4 KiB
  __shared__ float red_m[kWaves][4];
  __shared__ float red_l[kWaves][4];

  const int sp = (int)blockIdx.x % a.nsplit;
  const int r2 = (int)blockIdx.x / a.nsplit;
  const int kvh = r2 % a.Hkv;
  const int b = r2 / a.Hkv;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;

  const int p = a.pos[b];
  if (p < 0 || p > a.max_pos) {
    if (a.nsplit == 1 && t < kHeadDim) {
      for (int hh = 0; hh < kGroup; ++hh)
        a.out[((size_t)b * a.Hq + kvh * kGroup + hh) * kHeadDim + t] = 0x7fc0;  // NaN
    }
    return;
  }
  int lo, hi;
  decode_key_range(p, a.ring, a.cap, a.window, &lo, &hi);
  const int k0 = lo + sp * a.split_keys;
  const int k1 = min(k0 + a.split_keys, hi);
  const int slot = cache_slot(p, a.ring, a.cap);
  const size_t kv_off = ((size_t)b * a.Hkv + kvh) * (size_t)a.cap * kHeadDim;

  // ---- RoPE of the 4 queries: cos/sin of the fp64-reduced angle, rotation
  // in fp32, split into bf16 high and low parts (~16 significant bits, far
  // above what the scores need). The owner of the new slot also writes the
  // new key, rotated in fp64 and rounded once to bf16 like every cached key.
  if (t < kHeadDim) {
    const int d = t;
    const int half = a.r >> 1;
    double c = 1.0, s = 0.0;
    if (d < a.r) rope_sincos(p, a.inv_freq[d < half ? d : d - half], &s, &c);
    const float cf = (float)c, sf = (float)s;
    const int dp = d < half ? d + half : d - half;  // rotation partner
    auto rot32 = [&](const uint16_t* x) -> float {
      const float xd = bf16_bits_to_float(x[d]);
      if (d >= a.r) return xd;
      const float xp = bf16_bits_to_float(x[dp]);
      return d < half ? fmaf(xd, cf, -xp * sf) : fmaf(xd, cf, xp * sf);
    };
#pragma unroll
    for (int hh = 0; hh < kGroup; ++hh) {
      const float y = rot32(a.q + ((size_t)b * a.Hq + kvh * kGroup + hh) * kHeadDim);
      const uint16_t yh = float_to_bf16_bits(y);
      qcols[hh][d] = yh;
      qcols[4 + hh][d] = float_to_bf16_bits(y - bf16_bits_to_float(yh));
    }
    if (slot >= k0 && slot < k1) {
      const size_t nk_off = ((size_t)b * a.Hkv + kvh) * kHeadDim;
      const uint16_t* x = a.k + nk_off;
      const double xd = (double)bf16_bits_to_float(x[d]);
      double y = xd;
      if (d < a.r) {
        const double xp = (double)bf16_bits_to_float(x[dp]);
        y = d < half ? xd * c - xp * s : xd * c + xp * s;
      }
      a.kc[kv_off + (size_t)slot * kHeadDim + d] = double_to_bf16_bits(y);
      a.vc[kv_off + (size_t)slot * kHeadDim + d] = a.v[nk_off + d];
    }
  }
  // Workgroup-scope ordering is enough: the new row is read back only by
  // this workgroup, through the same CU. (A device-scope fence would write
  // back and invalidate the whole L2 of the XCD.)
  __syncthreads();

  const int col = lane & 15;   // MFMA column / row index of this lane
  const int grp = lane >> 4;   // 16-lane group
  bf16x8 qb[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    bf16x8 v = bf16x8{};
    if (col < 8) v = *(const bf16x8*)(&qcols[col][ks * 32 + grp * 8]);
    qb[ks] = v;
  }

  const uint16_t* kbase = a.kc + kv_off;
  const uint16_t* vbase = a.vc + kv_off;
  char* vb = vbuf[wave];
  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{};
  float m_run = -1e30f, l_run = 0.f;

  const int tr_a = col & 3, tr_v = col >> 2;
  const int nchunks = k1 > k0 ? (k1 - k0 + kChunk - 1) / kChunk : 0;
  for (int c = wave; c < nchunks; c += kWaves) {
    const int ck = k0 + c * kChunk;
    // K fragments: lane holds key ck + kb*16 + col, channels ks*32 + grp*8 ..
    // Keys past the split end re-read its last key and are masked below.
    bf16x8 kf[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(ck + kb * 16 + col, k1 - 1);
      const uint16_t* kp = kbase + (size_t)key * kHeadDim + grp * 8;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[kb][ks] = *(const bf16x8*)(kp + ks * 32);
    }
    uint4 vr[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int key = min(ck + u * 2 + (lane >> 5), k1 - 1);
      vr[u] = *(const uint4*)(vbase + (size_t)key * kHeadDim + (lane & 31) * 8);
    }

    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], qb[ks], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], qb[ks], sacc[1], 0, 0, 0);
    }
    // Register i of block kb: key ck + kb*16 + grp*4 + i, column col.
    float x[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sacc[kb][i];
        v += wave_shfl_xor(v, 4);  // high + low query parts
        const int key = ck + kb * 16 + grp * 4 + i;
        x[kb * 4 + i] = (col < 8 && key < k1) ? v * kScoreScale : -__builtin_inff();
      }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = fast_exp2(x[j] - m_new);
      ps += x[j];
    }
    ps += wave_shfl_xor(ps, 16);
    ps += wave_shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    // O rows grp*4 + i (i = head) of groups 0 and 1 scale by that head's alpha.
    float al[4];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) al[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), hh));
    if (al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f) {
#pragma unroll
      for (int blk = 0; blk < 16; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[blk][i] *= al[i];
    }

    // P as the A operand: lane holds row col, key slots grp*8 + j; slot j < 4
    // is key grp*4 + j (block 0), slot j >= 4 is key 16 + grp*4 + j - 4.
    bf16x8 pa;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint16_t ph = float_to_bf16_bits(x[j]);
      uint16_t pv = 0;
      if (col < 4) pv = ph;
      else if (col < 8) pv = float_to_bf16_bits(x[j] - bf16_bits_to_float(ph));
      pa[j] = __builtin_bit_cast(__bf16, pv);
    }

#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int row = u * 2 + (lane >> 5);
      *(uint4*)(vb + v_off(row, lane & 31)) = vr[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // B operand lane l: V[key(slot)][16*blk + col] for slots grp*8 + j; lane
    // (a + 4v) of a 16-lane group fetches row base + v, channels d0 + 4a ..
    const int rowA = 4 * grp + tr_v;
    const int rowB = 16 + rowA;
#pragma unroll
    for (int blk = 0; blk < 16; ++blk) {
      const int cc = blk * 16 + 4 * tr_a;
      const int ch = cc >> 3, off = (cc & 7) * 2;
      const s16x4 lo4 = lds_read_tr(vb + v_off(rowA, ch) + off);
      const s16x4 hi4 = lds_read_tr(vb + v_off(rowB, ch) + off);
      const s16x8 both = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, both), acc[blk], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge high and low rows (groups 0 and 1), then the waves.
#pragma unroll
  for (int blk = 0; blk < 16; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[blk][i] += wave_shfl_xor(acc[blk][i], 16);
  __syncthreads();
  float* om = (float*)&vbuf[0][0];  // [wave][head][256]
  if (grp == 0) {
#pragma unroll
    for (int blk = 0; blk < 16; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) om[(wave * 4 + i) * kHeadDim + blk * 16 + col] = acc[blk][i];
  }
  if (lane < 4) {
    red_m[wave][lane] = m_run;
    red_l[wave][lane] = l_run;
  }
  __syncthreads();
  if (t >= kHeadDim) return;
  const int d = t;
#pragma unroll
  for (int hh = 0; hh < kGroup; ++hh) {
    float M = red_m[0][hh];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_m[w][hh]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = fast_exp2(red_m[w][hh] - M);
      L += e * red_l[w][hh];
      O += e * om[(w * 4 + hh) * kHeadDim + d];
    }
    const int h = kvh * kGroup + hh;
    if (a.nsplit == 1) {
      const float g = bf16_bits_to_float(a.gate[(size_t)b * a.Hq + h]);
      a.out[((size_t)b * a.Hq + h) * kHeadDim + d] = float_to_bf16_bits(O / L * sigmoidf_(g));
    } else {
      const size_t pi = ((size_t)b * a.Hq + h) * a.nsplit + sp;
      a.part_o[pi * kHeadDim + d] = O;
      if (d == 0) {
        a.part_ml[pi * 2 + 0] = M;
        a.part_ml[pi * 2 + 1] = L;
      }
    }
  }
}

// Merge of the split partials, gate, bf16 store. One block per (sequence,
// head): the block first turns every split's (m, l) into a weight
// 2^(m_s - M) and the total L, then 4 thread groups each sum a quarter of the
// splits' partial outputs (8 loads in flight per thread) and combine in a
// fixed order, so the result does not depend on timing.
constexpr int kMergeThreads = 1024;
constexpr int kMaxSplits = 2048;

__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[kMergeThreads / 64];
  __shared__ float part[3][kHeadDim];
  const int b = (int)blockIdx.x / a.Hq;
  const int h = (int)blockIdx.x % a.Hq;
  const int t = threadIdx.x;
  const int p = a.pos[b];
  uint16_t* o = a.out + ((size_t)b * a.Hq + h) * kHeadDim;
  if (p < 0 || p > a.max_pos) {
    if (t < kHeadDim) o[t] = 0x7fc0;
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
  // O[d] = sum_s w_s o_s[d]; thread group g takes splits g, g+4, ...
  const int g = t >> 8, d = t & 255;
  float acc = 0.f;
  int s = g;
  for (; s + 28 < a.nsplit; s += 32) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = a.part_o[(base + s + 4 * u) * kHeadDim + d];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += wgt[s + 4 * u] * v[u];
  }
  for (; s < a.nsplit; s += 4) acc += wgt[s] * a.part_o[(base + s) * kHeadDim + d];
  if (g > 0) part[g - 1][d] = acc;
  __syncthreads();
  if (g == 0) {
    const float O = ((acc + part[0][d]) + part[1][d]) + part[2][d];
    const float gl = bf16_bits_to_float(a.gate[(size_t)b * a.Hq + h]);
    o[d] = float_to_bf16_bits(O / L * sigmoidf_(gl));
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int grid = a.B * a.Hkv * a.nsplit;
  if (grid == 0) return hipSuccess;
  if (a.waves == 8)
    hipLaunchKernelGGL(decode_kernel<8>, dim3(grid), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(decode_kernel<4>, dim3(grid), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(a.B * a.Hq), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hattn
