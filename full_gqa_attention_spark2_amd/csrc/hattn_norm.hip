// Elementwise kernels of the attention block around the core (page
// "Spark-X2.5 架构（4B / 1.7B）", §2 figure 1 decoder-layer dataflow and §5
// norms): the input RMSNorm and the residual add. Both are HBM-bound; each
// thread moves 16-byte chunks (8 bf16 values).
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

__device__ __forceinline__ uint4 pack8f(const float* x) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)float_to_bf16_bits(x[2 * i]) | ((uint32_t)float_to_bf16_bits(x[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

// One block per token: y = bf16(w * x / sqrt(mean(x^2) + eps)), in fp32
// (page §5: the norm is computed in fp32, multiplied by the weight, and cast
// back to the model dtype).
__global__ __launch_bounds__(kNormThreads) void rms_norm_kernel(RmsNormArgs a) {
  __shared__ float part[kNormThreads / 64];
  const int t = threadIdx.x;
  const uint4* x = (const uint4*)(a.x + (size_t)blockIdx.x * a.H);
  uint4* y = (uint4*)(a.y + (size_t)blockIdx.x * a.H);
  const uint4* w = (const uint4*)a.w;
  const int n = a.H / 8;
  float ss = 0.f;
  for (int c = t; c < n; c += kNormThreads) {
    float v[8];
    unpack8f(x[c], v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((t & 63) == 0) part[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kNormThreads / 64; ++i) tot += part[i];
  const float r = rsqrtf(tot / (float)a.H + a.eps);
  for (int c = t; c < n; c += kNormThreads) {
    float v[8], g[8];
    unpack8f(x[c], v);
    unpack8f(w[c], g);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * r * g[j];
    y[c] = pack8f(v);
  }
}

// out = bf16(x + y) over n8 chunks of 8 values (the residual add of the
// block; out may be x).
__global__ __launch_bounds__(256) void residual_add_kernel(const uint16_t* x, const uint16_t* y, uint16_t* out,
                                                           long long n8) {
  for (long long c = (long long)blockIdx.x * 256 + threadIdx.x; c < n8; c += (long long)gridDim.x * 256) {
    float a[8], b[8];
    unpack8f(((const uint4*)x)[c], a);
    unpack8f(((const uint4*)y)[c], b);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] += b[j];
    ((uint4*)out)[c] = pack8f(a);
  }
}

hipError_t launch_rms_norm(const RmsNormArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(rms_norm_kernel, dim3(a.T), dim3(kNormThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_residual_add(const uint16_t* x, const uint16_t* y, uint16_t* out, long long n, hipStream_t s) {
  const long long n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  const long long blocks = std::min<long long>((n8 + 255) / 256, 4096);
  hipLaunchKernelGGL(residual_add_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, y, out, n8);
  return hipGetLastError();
}

}  // namespace hattn
