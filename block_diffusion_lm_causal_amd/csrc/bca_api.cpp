// C ABI of libbca.so: argument validation and kernel dispatch.
//
// Every check that needs only host-visible values runs before anything is
// enqueued, so an invalid call returns a status and leaves the stream alone.
// Nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/bca.h"
#include "bca_kernels.hpp"

namespace {

thread_local char g_last_error[512] = "";

bca_status_t fail(bca_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

bca_status_t hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return BCA_OK;
  return fail(BCA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxDecodeSplits = 256;
constexpr int kMaxGraphSteps = 4096;  // decode steps one captured graph may hold  // the combine kernel stages one weight per split and row

// Checks shared by the packed-segment entry points.
bca_status_t check_packed(const void* q, const void* k, const void* v, const void* o,
                          const void* lse, const int32_t* cu, int32_t nseq, int32_t max_seqlen,
                          int32_t total, int32_t hq, int32_t hkv, int32_t d, int32_t block_size,
                          float scale) {
  if (nseq < 0 || total < 0) return fail(BCA_ERR_SHAPE, "nseq (%d) and total (%d) must be >= 0", nseq, total);
  if (hq <= 0 || hkv <= 0) return fail(BCA_ERR_SHAPE, "hq (%d) and hkv (%d) must be > 0", hq, hkv);
  if (hq % hkv != 0) return fail(BCA_ERR_SHAPE, "hq (%d) must be a multiple of hkv (%d)", hq, hkv);
  if (d != 64 && d != 128) return fail(BCA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d);
  if (block_size < 1) return fail(BCA_ERR_SHAPE, "block_size must be >= 1 (got %d)", block_size);
  if (!std::isfinite(scale)) return fail(BCA_ERR_SHAPE, "scale must be finite");
  if (nseq == 0 || total == 0) return BCA_OK;
  if (max_seqlen < 1) return fail(BCA_ERR_SHAPE, "max_seqlen must be >= 1 when total > 0");
  if (!q || !k || !v || !o || !lse || !cu) return fail(BCA_ERR_NULL, "a required pointer is NULL");
  if ((long long)total * hq * d >= (1LL << 40)) return fail(BCA_ERR_SHAPE, "problem too large");
  return BCA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int32_t bca_abi_version(void) { return BCA_ABI_VERSION; }

const char* bca_status_string(int32_t status) {
  switch (status) {
    case BCA_OK: return "ok";
    case BCA_ERR_NULL: return "null pointer";
    case BCA_ERR_SHAPE: return "invalid shape";
    case BCA_ERR_DTYPE: return "unsupported dtype";
    case BCA_ERR_UNSUPPORTED: return "unsupported configuration";
    case BCA_ERR_WORKSPACE: return "workspace too small";
    case BCA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bca_last_error(void) { return g_last_error; }

}  // extern "C"

// Forward of every packed variant: per-segment copies (s_copies) or a table of
// copy groups (group_start / group_pe / group_copies), or neither.
static bca_status_t fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* cu_seqlens, const int32_t* s_copies,
                             const int32_t* group_start, const int32_t* group_pe,
                             const int32_t* group_copies, int32_t nseq, int32_t max_seqlen,
                             int32_t total, int32_t hq, int32_t hkv, int32_t d,
                             int32_t block_size, float scale, bca_dtype_t dtype, void* stream) {
  bca_status_t st = check_packed(q, k, v, o, lse, cu_seqlens, nseq, max_seqlen, total, hq, hkv,
                                 d, block_size, scale);
  if (st != BCA_OK) return st;
  if (dtype != BCA_BF16 && dtype != BCA_F32) return fail(BCA_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (nseq == 0 || total == 0) return BCA_OK;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(BCA_ERR_SHAPE, "q, k, v and o must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == BCA_BF16) {
    bca::FwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.cu_seqlens = cu_seqlens;
    a.s_copies = s_copies;
    a.group_start = group_start;
    a.group_pe = group_pe;
    a.group_copies = group_copies;
    a.nseq = nseq;
    a.total = total;
    a.hq = hq;
    a.hkv = hkv;
    a.d = d;
    a.block_size = block_size;
    a.hpw = bca::heads_per_wg(hq, hkv);
    a.scale_log2 = scale * kLog2e;
    return hip_status(bca::launch_fwd_bf16(a, max_seqlen, s), "forward launch");
  }
  bca::FwdF32Args a{};
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.v = static_cast<const float*>(v);
  a.o = static_cast<float*>(o);
  a.lse = lse;
  a.cu_seqlens = cu_seqlens;
  a.s_copies = s_copies;
  a.group_start = group_start;
  a.group_pe = group_pe;
  a.group_copies = group_copies;
  a.nseq = nseq;
  a.total = total;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.block_size = block_size;
  a.scale_log2 = scale * kLog2e;
  return hip_status(bca::launch_fwd_f32(a, max_seqlen, s), "forward launch");
}

extern "C" {

bca_status_t bca_staircase_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                               const int32_t* cu_seqlens, const int32_t* s_copies, int32_t nseq,
                               int32_t max_seqlen, int32_t total, int32_t hq, int32_t hkv,
                               int32_t d, int32_t block_size, float scale, bca_dtype_t dtype,
                               void* stream) {
  g_last_error[0] = '\0';
  return fwd_impl(q, k, v, o, lse, cu_seqlens, s_copies, nullptr, nullptr, nullptr, nseq,
                  max_seqlen, total, hq, hkv, d, block_size, scale, dtype, stream);
}

bca_status_t bca_staircase_groups_fwd(const void* q, const void* k, const void* v, void* o,
                                      float* lse, const int32_t* cu_seqlens,
                                      const int32_t* group_start, const int32_t* group_pe,
                                      const int32_t* group_copies, int32_t nseq,
                                      int32_t max_seqlen, int32_t total, int32_t hq, int32_t hkv,
                                      int32_t d, int32_t block_size, float scale,
                                      bca_dtype_t dtype, void* stream) {
  g_last_error[0] = '\0';
  if (nseq > 0 && total > 0 && (!group_start || !group_pe || !group_copies))
    return fail(BCA_ERR_NULL, "group_start, group_pe and group_copies are required");
  return fwd_impl(q, k, v, o, lse, cu_seqlens, nullptr, group_start, group_pe, group_copies,
                  nseq, max_seqlen, total, hq, hkv, d, block_size, scale, dtype, stream);
}

bca_status_t bca_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen, int32_t total,
                     int32_t hq, int32_t hkv, int32_t d, int32_t block_size, float scale,
                     bca_dtype_t dtype, void* stream) {
  return bca_staircase_fwd(q, k, v, o, lse, cu_seqlens, nullptr, nseq, max_seqlen, total, hq,
                           hkv, d, block_size, scale, dtype, stream);
}

size_t bca_staircase_bwd_workspace(int32_t total, int32_t hq, int32_t hkv, int32_t d) {
  if (total < 0 || hq <= 0 || hkv <= 0 || d <= 0) return 0;
  const size_t rows = (((size_t)hq * total * sizeof(float)) + 255) & ~(size_t)255;
  return 2 * rows;  // delta, then LSE * log2(e)
}

}  // extern "C"

static bca_status_t bwd_impl(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             const int32_t* cu_seqlens, const int32_t* s_copies,
                             const int32_t* group_start, const int32_t* group_pe,
                             const int32_t* group_copies, int32_t nseq, int32_t max_seqlen,
                             int32_t total, int32_t hq, int32_t hkv, int32_t d,
                             int32_t block_size, float scale, bca_dtype_t dtype, void* workspace,
                             size_t ws_bytes, void* stream) {
  bca_status_t st = check_packed(q, k, v, o, lse, cu_seqlens, nseq, max_seqlen, total, hq, hkv,
                                 d, block_size, scale);
  if (st != BCA_OK) return st;
  if (dtype != BCA_BF16) return fail(BCA_ERR_DTYPE, "the backward supports bf16 only");
  if (nseq == 0 || total == 0) return BCA_OK;
  if (!dout || !dq || !dk || !dv) return fail(BCA_ERR_NULL, "a required gradient pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(BCA_ERR_SHAPE, "tensors must be 16-byte aligned");
  const size_t need = bca_staircase_bwd_workspace(total, hq, hkv, d);
  if (!workspace || ws_bytes < need)
    return fail(BCA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (!aligned16(workspace)) return fail(BCA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  bca::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.delta = static_cast<float*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + need / 2);
  a.cu_seqlens = cu_seqlens;
  a.s_copies = s_copies;
  a.group_start = group_start;
  a.group_pe = group_pe;
  a.group_copies = group_copies;
  a.nseq = nseq;
  a.total = total;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.block_size = block_size;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  return hip_status(bca::launch_bwd_bf16(a, max_seqlen, static_cast<hipStream_t>(stream)),
                    "backward launch");
}

extern "C" {

bca_status_t bca_staircase_bwd(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               const int32_t* cu_seqlens, const int32_t* s_copies, int32_t nseq,
                               int32_t max_seqlen, int32_t total, int32_t hq, int32_t hkv,
                               int32_t d, int32_t block_size, float scale, bca_dtype_t dtype,
                               void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, s_copies, nullptr, nullptr,
                  nullptr, nseq, max_seqlen, total, hq, hkv, d, block_size, scale, dtype,
                  workspace, ws_bytes, stream);
}

bca_status_t bca_staircase_groups_bwd(const void* q, const void* k, const void* v,
                                      const void* o, const float* lse, const void* dout,
                                      void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
                                      const int32_t* group_start, const int32_t* group_pe,
                                      const int32_t* group_copies, int32_t nseq,
                                      int32_t max_seqlen, int32_t total, int32_t hq, int32_t hkv,
                                      int32_t d, int32_t block_size, float scale,
                                      bca_dtype_t dtype, void* workspace, size_t ws_bytes,
                                      void* stream) {
  g_last_error[0] = '\0';
  if (nseq > 0 && total > 0 && (!group_start || !group_pe || !group_copies))
    return fail(BCA_ERR_NULL, "group_start, group_pe and group_copies are required");
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, nullptr, group_start, group_pe,
                  group_copies, nseq, max_seqlen, total, hq, hkv, d, block_size, scale, dtype,
                  workspace, ws_bytes, stream);
}

// Split-KV plan of the decode step: the 64-key tiles are dealt evenly to
// the splits.  By default a split is one round of at most the 5 tiles a
// workgroup stages in LDS, with at least 8 splits of 2 or more tiles for a
// short cache, and no more workgroups than the 256 compute units while that
// allows (a longer split is processed in rounds).
static int decode_splits(int32_t q_len, int32_t kv_len, int32_t hq, int32_t hkv, int32_t req) {
  const int hpw = bca::heads_per_wg(hq, hkv);
  const int tok = 32 * (4 / hpw);
  const int ntok = (q_len + tok - 1) / tok;
  const int base_wgs = (hq / hpw) * ntok;
  const int tiles = (kv_len + 63) / 64;
  int ns;
  if (req > 0) {
    ns = req;
  } else {
    ns = (tiles + 4) / 5;
    if (ns < 8) ns = tiles / 2 < 8 ? tiles / 2 : 8;
    const int cap = base_wgs < 256 ? 256 / base_wgs : 1;
    if (ns > cap) ns = cap;
  }
  if (ns > tiles) ns = tiles;
  return ns < 1 ? 1 : ns;
}

size_t bca_decode_workspace(int32_t q_len, int32_t kv_len, int32_t hq, int32_t hkv, int32_t d,
                            int32_t num_splits) {
  if (q_len <= 0 || kv_len <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || (d != 64 && d != 128) ||
      num_splits < 0)
    return 0;
  const int ns = decode_splits(q_len, kv_len, hq, hkv, num_splits);
  if (ns <= 1) return 0;
  const size_t rows = (size_t)ns * hq * ((q_len + 31) / 32) * 32;
  const size_t po = (rows * d * sizeof(float) + 255) & ~(size_t)255;
  const size_t pl = (rows * sizeof(float) + 255) & ~(size_t)255;
  return po + pl;
}

}  // extern "C"

// Checks of a decode call and the kernel arguments it maps to (shared by the
// direct call and the captured loop).
static bca_status_t decode_args(const void* q, const void* k, const void* v, void* o, float* lse,
                                int32_t q_len, int32_t kv_len, int32_t hq, int32_t hkv, int32_t d,
                                float scale, bca_dtype_t dtype, int32_t num_splits,
                                void* workspace, size_t ws_bytes, bca::DecodeArgs* a) {
  if (q_len < 1 || kv_len < q_len)
    return fail(BCA_ERR_SHAPE, "need 1 <= q_len (%d) <= kv_len (%d)", q_len, kv_len);
  if (hq <= 0 || hkv <= 0 || hq % hkv)
    return fail(BCA_ERR_SHAPE, "hq (%d) must be a positive multiple of hkv (%d)", hq, hkv);
  if (d != 64 && d != 128) return fail(BCA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d);
  if (!std::isfinite(scale)) return fail(BCA_ERR_SHAPE, "scale must be finite");
  if (num_splits < 0 || num_splits > kMaxDecodeSplits)
    return fail(BCA_ERR_SHAPE, "num_splits must be in [0, %d]", kMaxDecodeSplits);
  if (dtype != BCA_BF16) return fail(BCA_ERR_DTYPE, "decode supports bf16 only");
  if (!q || !k || !v || !o || !lse) return fail(BCA_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(BCA_ERR_SHAPE, "q, k, v and o must be 16-byte aligned");
  const int ns = decode_splits(q_len, kv_len, hq, hkv, num_splits);
  const size_t need = bca_decode_workspace(q_len, kv_len, hq, hkv, d, num_splits);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(BCA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (need > 0 && !aligned16(workspace)) return fail(BCA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  a->q = static_cast<const uint16_t*>(q);
  a->k = static_cast<const uint16_t*>(k);
  a->v = static_cast<const uint16_t*>(v);
  a->o = static_cast<uint16_t*>(o);
  a->lse = lse;
  const size_t po =
      ((size_t)ns * hq * ((q_len + 31) / 32) * 32 * d * sizeof(float) + 255) & ~(size_t)255;
  a->part_o = ns > 1 ? static_cast<float*>(workspace) : nullptr;
  a->part_lse = ns > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + po) : nullptr;
  a->q_len = q_len;
  a->kv_len = kv_len;
  a->hq = hq;
  a->hkv = hkv;
  a->d = d;
  a->hpw = bca::heads_per_wg(hq, hkv);
  a->nsplit = ns;
  a->scale_log2 = scale * kLog2e;
  a->k8 = nullptr;
  a->v8 = nullptr;
  a->o_mul = 1.f;
  return BCA_OK;
}

struct bca_decode_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
  int32_t steps;
};

extern "C" {

bca_status_t bca_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                        int32_t q_len, int32_t kv_len, int32_t hq, int32_t hkv, int32_t d,
                        float scale, bca_dtype_t dtype, int32_t num_splits, void* workspace,
                        size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  bca::DecodeArgs a{};
  const bca_status_t st = decode_args(q, k, v, o, lse, q_len, kv_len, hq, hkv, d, scale, dtype,
                                      num_splits, workspace, ws_bytes, &a);
  if (st != BCA_OK) return st;
  return hip_status(bca::launch_decode_bf16(a, static_cast<hipStream_t>(stream)), "decode launch");
}

bca_status_t bca_decode_fp8(const void* q, const void* k8, const void* v8, float k_scale,
                            float v_scale, void* o, float* lse, int32_t q_len, int32_t kv_len,
                            int32_t hq, int32_t hkv, int32_t d, float scale, int32_t num_splits,
                            void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale <= 0.f || v_scale <= 0.f)
    return fail(BCA_ERR_SHAPE, "k_scale and v_scale must be finite and > 0");
  bca::DecodeArgs a{};
  const bca_status_t st = decode_args(q, k8, v8, o, lse, q_len, kv_len, hq, hkv, d, scale,
                                      BCA_BF16, num_splits, workspace, ws_bytes, &a);
  if (st != BCA_OK) return st;
  a.k8 = static_cast<const uint8_t*>(k8);
  a.v8 = static_cast<const uint8_t*>(v8);
  a.k = nullptr;
  a.v = nullptr;
  a.scale_log2 *= k_scale;
  a.o_mul = v_scale;
  return hip_status(bca::launch_decode_fp8(a, static_cast<hipStream_t>(stream)), "decode launch");
}

bca_status_t bca_decode_graph_create(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int32_t q_len, int32_t kv_len, int32_t hq,
                                     int32_t hkv, int32_t d, float scale, bca_dtype_t dtype,
                                     int32_t num_splits, void* workspace, size_t ws_bytes,
                                     int32_t steps, bca_decode_graph_t** graph) {
  g_last_error[0] = '\0';
  if (!graph) return fail(BCA_ERR_NULL, "graph handle pointer is NULL");
  *graph = nullptr;
  if (steps < 1 || steps > kMaxGraphSteps)
    return fail(BCA_ERR_SHAPE, "steps must be in [1, %d] (got %d)", kMaxGraphSteps, steps);
  bca::DecodeArgs a{};
  const bca_status_t st = decode_args(q, k, v, o, lse, q_len, kv_len, hq, hkv, d, scale, dtype,
                                      num_splits, workspace, ws_bytes, &a);
  if (st != BCA_OK) return st;
  hipStream_t s = nullptr;
  hipError_t err = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (err != hipSuccess) return hip_status(err, "capture stream");
  err = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (err != hipSuccess) {
    (void)hipStreamDestroy(s);
    return hip_status(err, "begin capture");
  }
  hipError_t launch_err = hipSuccess;
  for (int32_t i = 0; i < steps && launch_err == hipSuccess; ++i)
    launch_err = bca::launch_decode_bf16(a, s);
  hipGraph_t g = nullptr;
  err = hipStreamEndCapture(s, &g);
  (void)hipStreamDestroy(s);
  if (launch_err != hipSuccess || err != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return hip_status(launch_err != hipSuccess ? launch_err : err, "decode capture");
  }
  hipGraphExec_t exec = nullptr;
  err = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  if (err != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_status(err, "graph instantiate");
  }
  *graph = new bca_decode_graph{g, exec, steps};
  return BCA_OK;
}

bca_status_t bca_decode_graph_launch(bca_decode_graph_t* graph, void* stream) {
  g_last_error[0] = '\0';
  if (!graph) return fail(BCA_ERR_NULL, "graph handle is NULL");
  return hip_status(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)), "graph launch");
}

void bca_decode_graph_destroy(bca_decode_graph_t* graph) {
  if (!graph) return;
  (void)hipGraphExecDestroy(graph->exec);
  (void)hipGraphDestroy(graph->graph);
  delete graph;
}

}  // extern "C"
