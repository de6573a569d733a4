// Elementwise kernels of the attention block around the core (page
// "Spark-X2.5 架构（4B / 1.7B）", §2 figure 1 decoder-layer dataflow and §5:
// the input embedding is taken to fp32 for the backbone, so the residual
// stream x is fp32; the norm computes in fp32 and hands the projections the
// model dtype, bf16): the input RMSNorm and the residual add. Both are
// HBM-bound; each thread moves 8 values at a time.
#include <algorithm>

#include "hattn_device.h"
#include "hattn_internal.h"

namespace hattn {

namespace {

constexpr int kNormThreads = 256;

__device__ __forceinline__ void unpack8f(uint4 u, float* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void load8f32(const float* p, float* x) {
  const float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ uint4 pack8f(const float* x) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)float_to_bf16_bits(x[2 * i]) | ((uint32_t)float_to_bf16_bits(x[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

// One block per token: y = bf16(w * x / sqrt(mean(x^2) + eps)) from the
// fp32 residual stream x, computed in fp32 (page §5: the norm is computed in
// fp32, multiplied by the weight, and cast back to the model dtype). Rows of
// up to kNormHeld chunks per thread (hidden <= 8192) stay in registers, and
// their weights are loaded with them: one round trip to memory instead of
// two. Each thread sums its chunks in the same order either way.
constexpr int kNormHeld = 4;
__global__ __launch_bounds__(kNormThreads) void rms_norm_kernel(RmsNormArgs a) {
  __shared__ float part[kNormThreads / 64];
  const int t = threadIdx.x;
  const float* x = a.x + (size_t)blockIdx.x * a.H;
  uint4* y = (uint4*)(a.y + (size_t)blockIdx.x * a.H);
  const uint4* w = (const uint4*)a.w;
  const int n = a.H / 8;
  const bool held = n <= kNormHeld * kNormThreads;
  float v[kNormHeld][8];
  uint4 wv[kNormHeld];
  float ss = 0.f;
  if (held) {
#pragma unroll
    for (int i = 0; i < kNormHeld; ++i) {
      const int c = t + i * kNormThreads;
      if (c < n) {
        load8f32(x + 8 * c, v[i]);
        wv[i] = w[c];
      }
    }
#pragma unroll
    for (int i = 0; i < kNormHeld; ++i)
      if (t + i * kNormThreads < n) {
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(v[i][j], v[i][j], ss);
      }
  } else {
    for (int c = t; c < n; c += kNormThreads) {
      float u[8];
      load8f32(x + 8 * c, u);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(u[j], u[j], ss);
    }
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((t & 63) == 0) part[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kNormThreads / 64; ++i) tot += part[i];
  const float r = rsqrtf(tot / (float)a.H + a.eps);
  if (held) {
#pragma unroll
    for (int i = 0; i < kNormHeld; ++i) {
      const int c = t + i * kNormThreads;
      if (c < n) {
        float g[8];
        unpack8f(wv[i], g);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[i][j] = v[i][j] * r * g[j];
        y[c] = pack8f(v[i]);
      }
    }
  } else {
    for (int c = t; c < n; c += kNormThreads) {
      float u[8], g[8];
      load8f32(x + 8 * c, u);
      unpack8f(w[c], g);
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = u[j] * r * g[j];
      y[c] = pack8f(u);
    }
  }
}

// out = x + y in fp32 over n8 chunks of 8 values: the residual add of the
// block, the fp32 stream x plus the bf16 out_proj result y (out may be x).
__global__ __launch_bounds__(256) void residual_add_kernel(const float* x, const uint16_t* y, float* out,
                                                           long long n8) {
  for (long long c = (long long)blockIdx.x * 256 + threadIdx.x; c < n8; c += (long long)gridDim.x * 256) {
    float a[8], b[8];
    load8f32(x + 8 * c, a);
    unpack8f(((const uint4*)y)[c], b);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] += b[j];
    ((float4*)(out + 8 * c))[0] = make_float4(a[0], a[1], a[2], a[3]);
    ((float4*)(out + 8 * c))[1] = make_float4(a[4], a[5], a[6], a[7]);
  }
}

hipError_t launch_rms_norm(const RmsNormArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(rms_norm_kernel, dim3(a.T), dim3(kNormThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_residual_add(const float* x, const uint16_t* y, float* out, long long n, hipStream_t s) {
  const long long n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  const long long blocks = std::min<long long>((n8 + 255) / 256, 4096);
  hipLaunchKernelGGL(residual_add_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, y, out, n8);
  return hipGetLastError();
}

}  // namespace hattn
