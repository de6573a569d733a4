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

// One block per (new token, sequence): the token's cos/sin table row, its
// rotated keys (fp64 rotation, one bf16 rounding) and its values, written to
// the destination rows and, for a ring, when the token is among the last
// min(S, capacity), also to its ring slot. Each thread takes 16-byte chunks
// (8 channels of one head); the loads go out before the angles are
// evaluated.
constexpr int kPrepTokens = 1;
constexpr int kPrepThreads = 128;

__global__ __launch_bounds__(kPrepThreads) void prefill_prep_kernel(PrefillPrepArgs a) {
  __shared__ double cs[kPrepTokens][128];
  __shared__ double sn[kPrepTokens][128];
  const int i0 = blockIdx.x * kPrepTokens;
  const int b = blockIdx.y;
  const int len = a.len[b];
  if (i0 >= len) return;  // a shorter sequence of a ragged batch
  const int t = threadIdx.x;
  const int half = a.r >> 1;
  const int ntok = min(kPrepTokens, len - i0);
  const int nchunk = ntok * a.Hkv * 32;
  const size_t row0 = (size_t)a.tok0[b] + i0;  // packed row of the block's first token
  const int ring_from = len - min(len, a.ring_cap);

  // chunk c: token c / (32 Hkv), head (c / 32) % Hkv, channels 8(c % 32) .. +7
  auto src_off = [&](int c) {
    return (row0 + c / (a.Hkv * 32)) * (size_t)a.kv_stride + (size_t)((c >> 5) % a.Hkv) * kHeadDim;
  };
  auto partner = [&](int ch) {  // chunk holding the RoPE partners of chunk ch
    const int d0 = ch * 8;
    return d0 < a.r ? (d0 < half ? d0 + half : d0 - half) >> 3 : ch;
  };
  auto finish = [&](int c, uint4 kx, uint4 kp, uint4 vx) {
    const int tok = c / (a.Hkv * 32), h = (c >> 5) % a.Hkv, ch = c & 31;
    const int d0 = ch * 8;
    uint4 ko = kx;
    if (d0 < a.r) {
      const uint16_t* x = (const uint16_t*)&kx;
      const uint16_t* xp = (const uint16_t*)&kp;
      uint16_t* y = (uint16_t*)&ko;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = d0 + j;
        const double u = (double)bf16_bits_to_float(x[j]);
        const double w = (double)bf16_bits_to_float(xp[j]);
        y[j] = d < half ? double_to_bf16_bits(u * cs[tok][d] - w * sn[tok][d])
                        : double_to_bf16_bits(u * cs[tok][d - half] + w * sn[tok][d - half]);
      }
    }
    const int i = i0 + tok;
    if (a.paged.table) {  // slot = position, in the page the table names
      const int p = a.start[b] + i;
      const int ps = a.paged.page_size;
      const int pg = a.paged.table[(size_t)b * a.paged.pages_per_seq + p / ps];
      if ((unsigned)pg < (unsigned)a.paged.num_pages) {  // else the write is dropped
        const size_t o = (((size_t)pg * a.Hkv + h) * ps + p % ps) * kHeadDim;
        ((uint4*)(a.dst_k + o))[ch] = ko;
        ((uint4*)(a.dst_v + o))[ch] = vx;
      }
    } else {
      const size_t o = (((size_t)b * a.Hkv + h) * a.dst_rows + a.dst_row0[b] + i) * kHeadDim;
      ((uint4*)(a.dst_k + o))[ch] = ko;
      ((uint4*)(a.dst_v + o))[ch] = vx;
    }
    if (a.ring_k && i >= ring_from) {
      const int slot = (a.start[b] + i) % a.ring_cap;
      const size_t ro = (((size_t)b * a.Hkv + h) * a.ring_cap + slot) * kHeadDim;
      ((uint4*)(a.ring_k + ro))[ch] = ko;
      ((uint4*)(a.ring_v + ro))[ch] = vx;
    }
  };

  // first round of chunks: loads first
  uint4 kx[2], kp[2], vx[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = t + kPrepThreads * u;
    if (c < nchunk) {
      const size_t off = src_off(c);
      kx[u] = ((const uint4*)(a.k + off))[c & 31];
      kp[u] = ((const uint4*)(a.k + off))[partner(c & 31)];
      vx[u] = ((const uint4*)(a.v + off))[c & 31];
    }
  }
  for (int e = t; e < ntok * half; e += kPrepThreads) {
    const int tok = e / half, j = e % half;
    double s, c;
    rope_sincos(a.start[b] + i0 + tok, a.inv_freq[j], &s, &c);
    cs[tok][j] = c;
    sn[tok][j] = s;
    a.table[(row0 + tok) * half + j] = make_float2((float)c, (float)s);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = t + kPrepThreads * u;
    if (c < nchunk) finish(c, kx[u], kp[u], vx[u]);
  }
  for (int c = t + 2 * kPrepThreads; c < nchunk; c += kPrepThreads) {  // more than 8 KV heads
    const size_t off = src_off(c);
    finish(c, ((const uint4*)(a.k + off))[c & 31], ((const uint4*)(a.k + off))[partner(c & 31)],
           ((const uint4*)(a.v + off))[c & 31]);
  }
}

// A ring's visible history into the staging rows: one block per (copied
// row, sequence), all KV heads, K and V, 16 B per lane.
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
    *sp = *rp;
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
  hipLaunchKernelGGL(prefill_prep_kernel, dim3((a.max_len + kPrepTokens - 1) / kPrepTokens, a.B),
                     dim3(kPrepThreads), 0, s, a);
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
  hipLaunchKernelGGL(ring_copy_kernel, dim3(m, a.B), dim3(256), 0, s, a);
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
