// The attention block around the core (page "Spark-X2.5 架构（4B / 1.7B）",
// §2 figure 1: RMSNorm -> q_k_v_proj and g_proj -> RoPE and attention ->
// per-head gate -> out_proj -> + residual; §5: the residual stream is fp32).
// The two projections are plain GEMMs: hipBLASLt for many tokens, this
// library's weight-streaming kernel for a few (decode); the norm, the core
// and the residual add are this library's kernels.
#include <stdint.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include <hipblaslt/hipblaslt.h>

#include "hattn.h"
#include "hattn_internal.h"

using namespace hattn;

namespace {

constexpr size_t kGemmWorkspace = 32u << 20;  // hipBLASLt workspace per GEMM
constexpr int kGemmCandidates = 16;           // heuristic results considered
constexpr int kTunedCandidates = 8;           // of those, timed on the first call of a shape
constexpr int kMaxDevices = 64;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

std::mutex g_mu;
hipblasLtHandle_t g_handle[kMaxDevices];

hipblasLtHandle_t lt_handle() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_handle[dev] && hipblasLtCreate(&g_handle[dev]) != HIPBLAS_STATUS_SUCCESS) g_handle[dev] = nullptr;
  return g_handle[dev];
}

// One row-major GEMM, D[T][N] = A[T][K] W[N][K]^T, bf16 in and out, fp32
// accumulate. In hipBLASLt's column-major terms: D^T (N x T, ld ldd) =
// op_T(W^T: K x N, ld K) * A^T (K x T, ld lda).
struct GemmPlan {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulAlgo_t algo{};                       // the one in use
  hipblasLtMatmulAlgo_t cand[kGemmCandidates]{};      // heuristic candidates that fit the workspace
  int n_cand = 0;
  bool tuned = false;  // algo is the fastest candidate measured on this shape
  bool ok = false;
};
std::map<std::tuple<int, int, int, long long, long long, int>, GemmPlan> g_plans;

GemmPlan* gemm_plan(hipblasLtHandle_t h, int N, int K, int T, long long lda, long long ldd) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lock(g_mu);
  const auto key = std::make_tuple(N, K, T, lda, ldd, dev);
  auto it = g_plans.find(key);
  if (it != g_plans.end()) return it->second.ok ? &it->second : nullptr;
  GemmPlan p;
  bool ok = hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  ok = ok && hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, T, lda) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.ld, HIP_R_16BF, N, T, ldd) == HIPBLAS_STATUS_SUCCESS;
  if (ok) {
    hipblasLtMatmulPreference_t pref = nullptr;
    const uint64_t ws = kGemmWorkspace;
    ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof(ws)) ==
             HIPBLAS_STATUS_SUCCESS;
    // the best-ranked algorithm that fits the workspace (the ranking does not
    // always honour the workspace preference)
    hipblasLtMatmulHeuristicResult_t res[kGemmCandidates];
    int n = 0;
    ok = ok && hipblasLtMatmulAlgoGetHeuristic(h, p.op, p.la, p.lb, p.ld, p.ld, pref, kGemmCandidates, res, &n) ==
                   HIPBLAS_STATUS_SUCCESS;
    for (int i = 0; ok && i < n; ++i)
      if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= kGemmWorkspace)
        p.cand[p.n_cand++] = res[i].algo;
    ok = ok && p.n_cand > 0;
    if (ok) p.algo = p.cand[0];
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  }
  p.ok = ok;
  return (g_plans[key] = p).ok ? &g_plans[key] : nullptr;
}

// The first call of a shape outside stream capture times the first
// kTunedCandidates candidates on its own buffers (twice each, best of two)
// and keeps the fastest; the heuristic's ranking is often not the fastest
// order on this chip. Under capture the top candidate is used untimed.
void tune(hipblasLtHandle_t h, GemmPlan* p, const void* W, const void* A, void* D, void* ws, hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (p->tuned || p->n_cand < 2 || hipStreamIsCapturing(s, &cs) != hipSuccess ||
      cs != hipStreamCaptureStatusNone)
    return;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return;
  }
  const float alpha = 1.f, beta = 0.f;
  float best = 1e30f;
  for (int i = 0; i < p->n_cand && i < kTunedCandidates; ++i) {
    float t_i = 1e30f;
    for (int r = 0; r < 2; ++r) {
      float ms = 0.f;
      if (hipEventRecord(e0, s) != hipSuccess ||
          hipblasLtMatmul(h, p->op, &alpha, W, p->la, A, p->lb, &beta, D, p->ld, D, p->ld, &p->cand[i], ws,
                          kGemmWorkspace, s) != HIPBLAS_STATUS_SUCCESS ||
          hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
          hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
        break;
      t_i = std::min(t_i, ms);
    }
    if (t_i < best) {
      best = t_i;
      p->algo = p->cand[i];
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  p->tuned = true;
}

// D = A . W^T. With resid_out set and the weight-streaming kernel taken,
// the residual add is fused into its epilogue (resid_out = resid_x +
// bf16(D) in fp32, rows ldd apart; D is not written) and *fused is set.
int gemm(const void* W, int N, int K, const void* A, int T, long long lda, void* D, long long ldd, void* ws,
         hipStream_t s, const float* resid_x = nullptr, float* resid_out = nullptr, bool* fused = nullptr) {
  if (T == 0) return HATTN_OK;
  // a few tokens (decode): the weight-streaming kernel of this library
  if (skinny_gemm_fits(N, K, T, lda, ldd, W, A, D) &&
      (!resid_out || ((((uintptr_t)resid_x | (uintptr_t)resid_out) & 15u) == 0))) {
    SkinnyGemmArgs g{(const uint16_t*)W, (const uint16_t*)A, (uint16_t*)D, N, K, T, lda, ldd, resid_x, resid_out};
    if (fused) *fused = resid_out != nullptr;
    return launch_skinny_gemm(g, s) == hipSuccess ? HATTN_OK : HATTN_ERR_LAUNCH;
  }
  hipblasLtHandle_t h = lt_handle();
  if (!h) return HATTN_ERR_LAUNCH;
  GemmPlan* p = gemm_plan(h, N, K, T, lda, ldd);
  if (!p) return HATTN_ERR_LAUNCH;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    tune(h, p, W, A, D, ws, s);
  }
  const float alpha = 1.f, beta = 0.f;
  return hipblasLtMatmul(h, p->op, &alpha, W, p->la, A, p->lb, &beta, D, p->ld, D, p->ld, &p->algo, ws,
                         kGemmWorkspace, s) == HIPBLAS_STATUS_SUCCESS
             ? HATTN_OK
             : HATTN_ERR_LAUNCH;
}

int check_weights(const hattn_layer_desc* d, const hattn_block_weights* w) {
  if (!d || !w) return HATTN_ERR_NULL;
  if (!w->norm_weight || !w->qkvg_weight || !w->o_weight) return HATTN_ERR_NULL;
  if (w->hidden <= 0 || w->hidden % 8 || !(w->rms_eps > 0.f)) return HATTN_ERR_SHAPE;
  if (((uintptr_t)w->norm_weight | (uintptr_t)w->qkvg_weight | (uintptr_t)w->o_weight) & 15u) return HATTN_ERR_ALIGN;
  return HATTN_OK;
}

// Row stride of the fused q/k/v/g projection's output: its (Hq + 2 Hkv) * 256
// + Hq columns rounded up to a multiple of 8, so every row (and every q, k,
// v slice in it) starts 16-byte aligned, as the kernels' 16-byte loads of
// those rows require.
long long fused_row_stride(int Hq, int Hkv) {
  const long long n1 = (long long)(Hq + 2 * Hkv) * 256 + Hq;
  return (n1 + 7) / 8 * 8;
}

// Workspace of one block call over T tokens: h [T][hidden], the fused
// projection [T][N1], the core's output [T][Hq*256], the out_proj result
// [T][hidden], the GEMM workspace, then the core's own workspace.
struct BlockLayout {
  size_t h, qkvg, attn, y, gemm, core_off, total;
};
BlockLayout block_layout(const hattn_layer_desc* d, const hattn_block_weights* w, long long T, size_t core) {
  BlockLayout L{};
  const long long n1 = fused_row_stride(d->num_q_heads, d->num_kv_heads);
  L.h = 0;
  L.qkvg = L.h + align256((size_t)T * w->hidden * 2);
  L.attn = L.qkvg + align256((size_t)T * n1 * 2);
  L.y = L.attn + align256((size_t)T * d->num_q_heads * 256 * 2);
  L.gemm = L.y + align256((size_t)T * w->hidden * 2);
  L.core_off = L.gemm + kGemmWorkspace;
  L.total = L.core_off + core;
  return L;
}

// The shared block pipeline around `core` (a callable that runs the core on
// the projections); T tokens.
template <class Core>
int block_run(const hattn_layer_desc* desc, const hattn_block_weights* w, const void* x, long long T,
              void* out, char* ws, const BlockLayout& L, hipStream_t s, Core core) {
  const int Hq = desc->num_q_heads, Hkv = desc->num_kv_heads, H = w->hidden;
  const long long n1 = (long long)(Hq + 2 * Hkv) * 256 + Hq;  // fused projection outputs
  const long long ld1 = fused_row_stride(Hq, Hkv);             // their row stride
  uint16_t* h = (uint16_t*)(ws + L.h);
  uint16_t* qkvg = (uint16_t*)(ws + L.qkvg);
  uint16_t* attn = (uint16_t*)(ws + L.attn);
  uint16_t* y = (uint16_t*)(ws + L.y);
  RmsNormArgs na{};
  na.x = (const float*)x;
  na.w = (const uint16_t*)w->norm_weight;
  na.y = h;
  na.T = (int)T;
  na.H = H;
  na.eps = w->rms_eps;
  if (launch_rms_norm(na, s) != hipSuccess) return HATTN_ERR_LAUNCH;
  int st = gemm(w->qkvg_weight, (int)n1, H, h, (int)T, H, qkvg, ld1, ws + L.gemm, s);
  if (st != HATTN_OK) return st;
  st = core(qkvg, qkvg + (size_t)Hq * 256, qkvg + (size_t)(Hq + Hkv) * 256, qkvg + (size_t)(Hq + 2 * Hkv) * 256,
            ld1, attn);
  if (st != HATTN_OK) return st;
  bool fused = false;
  st = gemm(w->o_weight, H, Hq * 256, attn, (int)T, (long long)Hq * 256, y, H, ws + L.gemm, s, (const float*)x,
            (float*)out, &fused);
  if (st != HATTN_OK || fused) return st;
  return launch_residual_add((const float*)x, y, (float*)out, T * H, s) == hipSuccess ? HATTN_OK
                                                                                     : HATTN_ERR_LAUNCH;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

size_t hattn_block_prefill_workspace_size(const hattn_layer_desc* desc, const hattn_block_weights* w,
                                          const hattn_kv_cache* cache, int32_t batch, const int32_t* cu_seqlens) {
  if (check_weights(desc, w) != HATTN_OK || validate_layer_cache(desc, cache, batch, false) != HATTN_OK ||
      batch > kMaxPrefillBatch || !cu_seqlens || cu_seqlens[0] != 0)
    return 0;
  int max_len = 0;
  for (int b = 0; b < batch; ++b) {
    if (cu_seqlens[b + 1] < cu_seqlens[b]) return 0;
    max_len = std::max(max_len, cu_seqlens[b + 1] - cu_seqlens[b]);
  }
  const long long T = cu_seqlens[batch];
  return block_layout(desc, w, T, prefill_workspace_bytes(desc, cache, batch, T, max_len)).total;
}

int hattn_block_prefill(const hattn_layer_desc* desc, const hattn_block_weights* w, const void* x, int32_t batch,
                        const int32_t* cu_seqlens, const int32_t* start_pos, const hattn_kv_cache* cache,
                        void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_weights(desc, w);
  if (st != HATTN_OK) return st;
  st = validate_layer_cache(desc, cache, batch, true);
  if (st != HATTN_OK) return st;
  if (batch > kMaxPrefillBatch) return HATTN_ERR_UNSUPPORTED;
  if (!cu_seqlens || !start_pos) return HATTN_ERR_NULL;
  if (cu_seqlens[0] != 0) return HATTN_ERR_SHAPE;
  int tok0[kMaxPrefillBatch], len[kMaxPrefillBatch], max_len = 0;
  for (int b = 0; b < batch; ++b) {
    if (cu_seqlens[b + 1] < cu_seqlens[b]) return HATTN_ERR_SHAPE;
    tok0[b] = cu_seqlens[b];
    len[b] = cu_seqlens[b + 1] - cu_seqlens[b];
    max_len = std::max(max_len, len[b]);
  }
  const long long T = cu_seqlens[batch];
  if (T == 0) return HATTN_OK;
  if (!x || !out) return HATTN_ERR_NULL;
  if (!aligned16(x) || !aligned16(out) || !aligned16(workspace)) return HATTN_ERR_ALIGN;
  const size_t core_bytes = prefill_workspace_bytes(desc, cache, batch, T, max_len);
  const BlockLayout L = block_layout(desc, w, T, core_bytes);
  if (!workspace || workspace_bytes < L.total) return HATTN_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  return block_run(desc, w, x, T, out, ws, L, stream,
                   [&](const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g, long long ld,
                       uint16_t* attn) {
                     return prefill_packed(desc, q, k, v, g, batch, tok0, len, T, start_pos, cache, attn,
                                           ws + L.core_off, core_bytes, stream, ld, ld, ld);
                   });
}

size_t hattn_block_decode_workspace_size(const hattn_layer_desc* desc, const hattn_block_weights* w,
                                         const hattn_kv_cache* cache, int32_t batch) {
  if (check_weights(desc, w) != HATTN_OK || validate_layer_cache(desc, cache, batch, false) != HATTN_OK) return 0;
  return block_layout(desc, w, batch, decode_workspace_bytes(desc, cache, batch)).total;
}

int hattn_block_decode(const hattn_layer_desc* desc, const hattn_block_weights* w, const void* x, int32_t batch,
                       const int32_t* pos, int32_t max_pos, const hattn_kv_cache* cache, void* out, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  int st = check_weights(desc, w);
  if (st != HATTN_OK) return st;
  st = validate_layer_cache(desc, cache, batch, true);
  if (st != HATTN_OK) return st;
  if (!x || !out) return HATTN_ERR_NULL;
  if (!aligned16(x) || !aligned16(out) || !aligned16(workspace)) return HATTN_ERR_ALIGN;
  const size_t core_bytes = decode_workspace_bytes(desc, cache, batch);
  const BlockLayout L = block_layout(desc, w, batch, core_bytes);
  if (!workspace || workspace_bytes < L.total) return HATTN_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  return block_run(desc, w, x, batch, out, ws, L, stream,
                   [&](const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g, long long ld,
                       uint16_t* attn) {
                     return decode_strided(desc, q, k, v, g, batch, pos, max_pos, cache, attn, ws + L.core_off,
                                           core_bytes, stream, ld, ld, ld);
                   });
}

}  // extern "C"
