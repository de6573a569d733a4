// RoPE and cache-copy kernels (page "Spark-X2.5 架构（4B / 1.7B）", §4 分层 RoPE:
// per-layer-type theta and rotated-channel count; §6 / the explainer page:
// sliding layers keep the last 512 tokens).
//
// Angles are p * theta^(-2i/r) in fp64 and cos/sin are evaluated in fp64; the
// rotation of stored keys runs in fp64 and each rotated value is rounded once
// to bf16.
#include "hattn_device.h"
#include "hattn_internal.h"

namespace hattn {

// Rotated value of channel d of one head (x points at the head's 256-channel
// row): channel i < r/2 pairs with i + r/2.
__device__ __forceinline__ uint16_t rotate_channel(const uint16_t* x, int d, int half, int r,
                                                   const double* cs, const double* sn) {
  if (d >= r) return x[d];
  double a = (double)bf16_bits_to_float(x[d]);
  double y;
  if (d < half) {
    double b = (double)bf16_bits_to_float(x[d + half]);
    y = a * cs[d] - b * sn[d];
  } else {
    double b = (double)bf16_bits_to_float(x[d - half]);
    y = a * cs[d - half] + b * sn[d - half];
  }
  return double_to_bf16_bits(y);
}

// One block per (new token, sequence): the token's cos/sin table row, its
// rotated keys (fp64 rotation, one bf16 rounding) and its values.
__global__ __launch_bounds__(256) void prefill_prep_kernel(PrefillPrepArgs a) {
  __shared__ double cs[128];
  __shared__ double sn[128];
  const int i = blockIdx.x;
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int p = a.start[b] + i;
  const int half = a.r >> 1;
  if (t < half) {
    double s, c;
    rope_sincos(p, a.inv_freq[t], &s, &c);
    cs[t] = c;
    sn[t] = s;
    a.table[((size_t)b * a.S + i) * half + t] = make_float2((float)c, (float)s);
  }
  __syncthreads();
  const size_t kbase = ((size_t)b * a.S + i) * a.Hkv * kHeadDim;
  const int row = a.dst_row0[b] + i;
  for (int e = t; e < a.Hkv * kHeadDim; e += 256) {
    const int h = e >> 8, d = e & 255;
    const size_t o = (((size_t)b * a.Hkv + h) * a.dst_rows + row) * kHeadDim + d;
    a.dst_k[o] = rotate_channel(a.k + kbase + (size_t)h * kHeadDim, d, half, a.r, cs, sn);
  }
  for (int c = t; c < a.Hkv * 32; c += 256) {  // values: 16-byte chunks
    const int h = c >> 5, ch = c & 31;
    const size_t o = (((size_t)b * a.Hkv + h) * a.dst_rows + row) * kHeadDim;
    ((uint4*)(a.dst_v + o))[ch] = ((const uint4*)(a.v + kbase + (size_t)h * kHeadDim))[ch];
  }
}

// One block per (copied row, sequence): all KV heads, K and V, 16 B per lane.
template <bool kToStage>
__global__ __launch_bounds__(256) void ring_copy_kernel(RingCopyArgs a) {
  const int j = blockIdx.x;
  const int b = blockIdx.y;
  if (j >= a.count[b]) return;
  const int pos = a.first_pos[b] + j;
  const int slot = pos % a.cap;
  const int srow = a.stage_row0[b] + j;
  const int n16 = a.Hkv * 2 * (kHeadDim * 2 / 16);  // 16-byte chunks per row
  for (int c = threadIdx.x; c < n16; c += 256) {
    const int kv = c / (a.Hkv * 32);
    const int rem = c % (a.Hkv * 32);
    const int h = rem >> 5, ch = rem & 31;
    uint16_t* ring = kv ? a.ring_v : a.ring_k;
    uint16_t* stage = kv ? a.stage_v : a.stage_k;
    uint4* rp = (uint4*)(ring + (((size_t)b * a.Hkv + h) * a.cap + slot) * kHeadDim) + ch;
    uint4* sp = (uint4*)(stage + (((size_t)b * a.Hkv + h) * a.stage_rows + srow) * kHeadDim) + ch;
    if (kToStage) *sp = *rp; else *rp = *sp;
  }
}

__global__ __launch_bounds__(256) void rope_apply_kernel(RopeApplyArgs a) {
  __shared__ double cs[256];
  __shared__ double sn[256];
  const int tok = blockIdx.x;
  const int half = a.r >> 1;
  const int p = a.pos[tok];
  for (int i = threadIdx.x; i < half; i += 256) {
    double s, c;
    rope_sincos(p, a.inv_freq[i], &s, &c);
    cs[i] = c;
    sn[i] = s;
  }
  __syncthreads();
  uint16_t* x = a.x + (size_t)tok * a.n_heads * a.head_dim;
  for (int e = threadIdx.x; e < a.n_heads * half; e += 256) {
    const int h = e / half, i = e % half;
    uint16_t* row = x + (size_t)h * a.head_dim;
    double u = (double)bf16_bits_to_float(row[i]);
    double w = (double)bf16_bits_to_float(row[i + half]);
    row[i] = double_to_bf16_bits(u * cs[i] - w * sn[i]);
    row[i + half] = double_to_bf16_bits(w * cs[i] + u * sn[i]);
  }
}

__global__ __launch_bounds__(256) void index_probe_kernel(ProbeArgs a) {
  const int qi = blockIdx.x;
  const int p = a.q_pos0 + qi;
  if (threadIdx.x == 0) a.slot[qi] = cache_slot(p, a.ring, a.cap);
  for (int j = threadIdx.x; j < a.cap; j += 256) {
    const int kp = slot_position(j, p, a.ring, a.cap);
    a.key_pos[(size_t)qi * a.cap + j] = kp;
    a.mask[(size_t)qi * a.cap + j] = key_visible(p, kp, a.window) ? 1 : 0;
  }
}

hipError_t launch_prefill_prep(const PrefillPrepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(prefill_prep_kernel, dim3(a.S, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

static int max_count(const RingCopyArgs& a) {
  int m = 0;
  for (int b = 0; b < a.B; ++b) m = a.count[b] > m ? a.count[b] : m;
  return m;
}

hipError_t launch_ring_to_stage(const RingCopyArgs& a, hipStream_t s) {
  const int m = max_count(a);
  if (m == 0) return hipSuccess;
  hipLaunchKernelGGL(ring_copy_kernel<true>, dim3(m, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stage_to_ring(const RingCopyArgs& a, hipStream_t s) {
  const int m = max_count(a);
  if (m == 0) return hipSuccess;
  hipLaunchKernelGGL(ring_copy_kernel<false>, dim3(m, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rope_apply(const RopeApplyArgs& a, hipStream_t s) {
  if (a.n_tok == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_apply_kernel, dim3(a.n_tok), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_index_probe(const ProbeArgs& a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  hipLaunchKernelGGL(index_probe_kernel, dim3(a.n_q), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hattn
