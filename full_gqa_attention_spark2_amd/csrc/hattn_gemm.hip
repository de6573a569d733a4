// Skinny GEMM for the attention block's decode projections (page
// "Spark-X2.5 架构（4B / 1.7B）", §2 figure 1: q_k_v_proj + g_proj before the
// attention, out_proj after it): D[T][N] = A[T][K] . W[N][K]^T with few
// tokens (T <= 64), bf16 in and out, fp32 accumulation.
//
// With 64 tokens each weight byte serves 64 multiply-adds, so the product
// is bound by streaming W once from HBM. One workgroup owns NB output
// columns (NB weight rows) for all tokens; its four waves split K into
// quarters. Each wave streams its quarter through a private ring of LDS
// slots by LDS DMA (16 B per lane, eight 128-byte row pieces per
// instruction): a slot holds a 64-k chunk of its NB weight rows and of the
// 64 token rows of A (A is shared by every workgroup and served by the L2),
// kSlots - 1 chunks stay in flight while one is computed, and the bf16 MFMA
// 16x16x32 reads its fragments back from LDS. The four partial sums meet in
// LDS (reusing the rings) and are added in a fixed order (wave 0 + 1 + 2 +
// 3), then rounded once to bf16. With a residual (out_proj), the epilogue
// also adds that bf16 value to the fp32 residual row and writes the fp32 sum.
#include "hattn_device.h"
#include "hattn_internal.h"

namespace hattn {

namespace {

constexpr int kGemmWaves = 4;
constexpr int kGemmTokens = 64;    // token rows per call (4 blocks of 16)
constexpr int kChunkK = 64;        // k per slot: 128 bytes of every row
constexpr int kSlots = 3;          // ring slots per wave

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor (raw, byte offsets, range-checked).
__device__ __forceinline__ i32x4 buf_desc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffff), (int)bytes, 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// 16 bytes per lane from memory into LDS (lane l lands at lds + 16 l).
// Issued from inline asm so that the compiler does not make every later LDS
// read wait for it (it cannot tell which LDS bytes a DMA writes); the kernel
// waits with s_waitcnt vmcnt, counting these loads. The descriptor (uniform
// by construction) is read from the first lane so that it sits in scalar
// registers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4 rs, uint32_t voff, uint32_t lds) {
  const i32x4 su = {__builtin_amdgcn_readfirstlane(rs[0]), __builtin_amdgcn_readfirstlane(rs[1]),
                    __builtin_amdgcn_readfirstlane(rs[2]), __builtin_amdgcn_readfirstlane(rs[3])};
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(su) : "memory", "m0");
}
#pragma clang diagnostic pop

// NB output columns per workgroup (16 or 32).
template <int NB>
__global__ __launch_bounds__(256, 1) void skinny_gemm_kernel(SkinnyGemmArgs g) {
  constexpr int NBLK = NB / 16;                          // 16-row weight fragments
  constexpr int kRowBytes = kChunkK * 2;                 // 128 B of a row per slot
  constexpr int kWBytes = NB * kRowBytes;
  constexpr int kSlotBytes = kWBytes + kGemmTokens * kRowBytes;
  constexpr int kDmaPerChunk = kSlotBytes / 1024;        // NB / 8 + 8
  constexpr int kRedBytes = kGemmWaves * kGemmTokens * (NB + 4) * 4;
  constexpr int kRingBytes = kGemmWaves * kSlots * kSlotBytes;
  __shared__ __attribute__((aligned(1024))) char lds[kRingBytes > kRedBytes ? kRingBytes : kRedBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * NB;
  const int kq = g.K / kGemmWaves;  // a multiple of kChunkK
  const int k0 = wave * kq;
  const int nchunks = kq / kChunkK;
  char* ring = lds + wave * kSlots * kSlotBytes;
  const uint32_t ring_addr = __builtin_amdgcn_readfirstlane(lds_addr(ring));

  // Chunk c of this wave: W rows n0 .. n0+NB-1 and A rows 0 .. 63, k in
  // k0 + 64c .. +63. DMA instruction u fills rows 8u .. 8u+7 of the slot
  // (W rows first, then A rows); lane l: row 8u + l/8, 16-byte piece p =
  // (l % 8) ^ (row % 8) of the row's 128 bytes, so piece q of a row sits at
  // LDS position q ^ (row % 8) and the fragment reads below spread over the
  // banks. Rows past N or T re-read the last valid row (results dropped).
  const i32x4 wrs = buf_desc(g.w, (uint32_t)((size_t)g.N * g.K * 2));
  const i32x4 ars = buf_desc(g.a, (uint32_t)min(((size_t)(g.T - 1) * g.lda + g.K) * 2, (size_t)0xffffffffu));
  auto issue = [&](int c, int slot) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)(k0 + c * kChunkK) * 2u;
#pragma unroll
    for (int u = 0; u < kDmaPerChunk; ++u) {
      const int row = 8 * u + (lane >> 3);
      const uint32_t piece = 16u * (uint32_t)((lane & 7) ^ (row & 7));
      if (u < NB / 8) {  // rows 8u .. 8u+7 are weight rows
        const uint32_t off = (uint32_t)((size_t)min(n0 + row, g.N - 1) * g.K * 2) + kb + piece;
        dma16(wrs, off, ring_addr + slot * kSlotBytes + u * 1024);
      } else {
        const uint32_t off = (uint32_t)((size_t)min(row - NB, g.T - 1) * g.lda * 2) + kb + piece;
        dma16(ars, off, ring_addr + slot * kSlotBytes + u * 1024);
      }
    }
  };

  f32x4 acc[NBLK][4];
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[nb][tb] = f32x4{};

  // Fragments of k-step s (0, 1) of a slot: lane reads row r = lane % 16 of
  // its 16-row block, piece 4s + lane / 16 (k 32s + 8 (lane / 16) .. +7).
  const int r16 = lane & 15, grp = lane >> 4;
  auto frag = [&](const char* sl, int row, int s) __attribute__((always_inline)) {
    return *(const bf16x8*)(sl + row * kRowBytes + 16 * ((4 * s + grp) ^ (row & 7)));
  };
  auto mma_chunk = [&](int slot) __attribute__((always_inline)) {
    const char* sl = ring + slot * kSlotBytes;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 wf[NBLK], af[4];
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb) wf[nb] = frag(sl, 16 * nb + r16, s);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) af[tb] = frag(sl + kWBytes, 16 * tb + r16, s);
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          acc[nb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nb], af[tb], acc[nb][tb], 0, 0, 0);
    }
  };

  // The ring: chunk c lives in slot c % kSlots. Iteration c refills the slot
  // of chunk c - 1 (every read of it has completed: lgkmcnt(0)) with chunk
  // c + kSlots - 1, then waits until at most the chunks issued after c are
  // in flight.
#pragma unroll
  for (int c = 0; c < kSlots - 1; ++c)
    if (c < nchunks) issue(c, c);
  for (int c = 0; c < nchunks; ++c) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int cn = c + kSlots - 1;
    if (cn < nchunks) issue(cn, cn % kSlots);
    const int after = min(nchunks - 1 - c, kSlots - 1);  // chunks issued after c
    if (after >= 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * kDmaPerChunk) : "memory");
    else if (after == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kDmaPerChunk) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    mma_chunk(c % kSlots);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();  // every wave is done with its ring: the LDS becomes `red`

  // acc[nb][tb] register i: column n0 + 16nb + 4(lane/16) + i, token 16tb + lane%16
  float (*red)[kGemmTokens][NB + 4] = (float (*)[kGemmTokens][NB + 4])lds;
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][tb * 16 + r16][nb * 16 + 4 * grp + i] = acc[nb][tb][i];
  __syncthreads();
  // thread: token t, 8 consecutive columns
  constexpr int kGroups = NB / 8;
  for (int e = threadIdx.x; e < kGemmTokens * kGroups; e += 256) {
    const int t = e / kGroups, c = (e % kGroups) * 8;
    if (t >= g.T || n0 + c >= g.N) continue;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      y[j] = ((red[0][t][c + j] + red[1][t][c + j]) + red[2][t][c + j]) + red[3][t][c + j];
    uint16_t yb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) yb[j] = float_to_bf16_bits(y[j]);
    if (g.out) {
      // each element is read and written by this thread alone: out may be x
      const size_t o = (size_t)t * g.ldd + n0 + c;
      const float4 x0 = *(const float4*)(g.x + o), x1 = *(const float4*)(g.x + o + 4);
      const float4 s0 = make_float4(x0.x + bf16_bits_to_float(yb[0]), x0.y + bf16_bits_to_float(yb[1]),
                                    x0.z + bf16_bits_to_float(yb[2]), x0.w + bf16_bits_to_float(yb[3]));
      const float4 s1 = make_float4(x1.x + bf16_bits_to_float(yb[4]), x1.y + bf16_bits_to_float(yb[5]),
                                    x1.z + bf16_bits_to_float(yb[6]), x1.w + bf16_bits_to_float(yb[7]));
      *(float4*)(g.out + o) = s0;
      *(float4*)(g.out + o + 4) = s1;
    } else {
      uint4 o;
      o.x = (uint32_t)yb[0] | ((uint32_t)yb[1] << 16);
      o.y = (uint32_t)yb[2] | ((uint32_t)yb[3] << 16);
      o.z = (uint32_t)yb[4] | ((uint32_t)yb[5] << 16);
      o.w = (uint32_t)yb[6] | ((uint32_t)yb[7] << 16);
      *(uint4*)(g.d + (size_t)t * g.ldd + n0 + c) = o;
    }
  }
}

}  // namespace

bool skinny_gemm_fits(int N, int K, int T, long long lda, long long ldd, const void* w, const void* a,
                      const void* d) {
  const uintptr_t al = (uintptr_t)w | (uintptr_t)a | (uintptr_t)d;
  return T >= 1 && T <= kGemmTokens && N >= 8 && N % 8 == 0 && K >= kGemmWaves * kChunkK &&
         K % (kGemmWaves * kChunkK) == 0 && (long long)N * K * 2 < (1LL << 32) &&
         ((long long)(T - 1) * lda + K) * 2 < (1LL << 32) && lda % 8 == 0 && ldd % 8 == 0 && lda >= K &&
         ldd >= N && (al & 15u) == 0;
}

hipError_t launch_skinny_gemm(const SkinnyGemmArgs& g, hipStream_t s) {
  // 32 columns per workgroup where that still gives at least 160
  // workgroups, else 16
  if ((g.N + 31) / 32 >= 160)
    hipLaunchKernelGGL(skinny_gemm_kernel<32>, dim3((g.N + 31) / 32), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(skinny_gemm_kernel<16>, dim3((g.N + 15) / 16), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace hattn
