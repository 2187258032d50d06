// C ABI of libbca.so: argument validation and kernel dispatch.
//
// Every check that needs only host-visible values runs before anything is
// enqueued, so an invalid call returns a status and leaves the stream alone.
// Nothing here allocates device memory, frees or synchronises -- except that
// with BCA_VALIDATE=1 in the environment the packed entry points copy their
// device tables (cu_seqlens, s_copies, the copy-group table) to the host,
// synchronising the stream, and check them before any launch.  With
// BCA_POISON=1 every workspace is filled with NaN words before the kernels
// that use it run, so that a read of a workspace word no kernel wrote shows.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

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
constexpr uint32_t kPoisonWord = 0x7FC07FC0u;  // a float32 NaN whose two halves are bf16 NaNs

// An environment switch is on when set to anything but "" or "0".  Read at
// every call, so a process may turn it on and off between calls.
bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && std::strcmp(v, "0") != 0;
}
constexpr int kMaxDecodeSplits = 256;
constexpr int kMaxGraphSteps = 4096;  // decode steps one captured graph may hold

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
  if (!std::isfinite(scale) || scale <= 0.f)
    return fail(BCA_ERR_SHAPE, "scale must be finite and > 0");
  if (nseq == 0 || total == 0) return BCA_OK;
  if (max_seqlen < 1) return fail(BCA_ERR_SHAPE, "max_seqlen must be >= 1 when total > 0");
  if (!q || !k || !v || !o || !lse || !cu) return fail(BCA_ERR_NULL, "a required pointer is NULL");
  if ((long long)total * hq * d >= (1LL << 40)) return fail(BCA_ERR_SHAPE, "problem too large");
  return BCA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename T>
hipError_t to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t s) {
  dst.assign(n, T{});
  if (n == 0) return hipSuccess;
  return hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, s);
}

// BCA_VALIDATE: the device tables of a packed call, checked on the host
// before anything is enqueued (this copies them and synchronises `s`).
//   cu_seqlens[0] = 0, non-decreasing, cu_seqlens[nseq] = total, every
//   length <= max_seqlen; per segment S >= 0 copies, P = L - S B >= 0 and,
//   with copies, P % B = 0; copy groups: group_start non-decreasing from 0,
//   each pe a multiple of B in [0, P], non-decreasing within the segment,
//   copies >= 0.
bca_status_t validate_tables_impl(const int32_t* cu, const int32_t* s_copies,
                                  const int32_t* gstart, const int32_t* gpe, const int32_t* gcp,
                                  int32_t nseq, int32_t max_seqlen, int32_t total, int32_t B,
                                  hipStream_t s) {
  std::vector<int32_t> hcu, hsc, hgs, hpe, hcp;
  hipError_t err = to_host(hcu, cu, (size_t)nseq + 1, s);
  if (err == hipSuccess && s_copies) err = to_host(hsc, s_copies, (size_t)nseq, s);
  if (err == hipSuccess && gstart) err = to_host(hgs, gstart, (size_t)nseq + 1, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return hip_status(err, "validation copy");
  if (hcu[0] != 0) return fail(BCA_ERR_SHAPE, "validation: cu_seqlens[0] = %d, not 0", hcu[0]);
  for (int32_t i = 0; i < nseq; ++i) {
    const long long L = (long long)hcu[i + 1] - hcu[i];
    if (L < 0) return fail(BCA_ERR_SHAPE, "validation: cu_seqlens decreases at segment %d", i);
    if (L > max_seqlen)
      return fail(BCA_ERR_SHAPE, "validation: segment %d has %lld tokens > max_seqlen %d", i, L,
                  max_seqlen);
  }
  if (hcu[nseq] != total)
    return fail(BCA_ERR_SHAPE, "validation: cu_seqlens[nseq] = %d, total = %d", hcu[nseq], total);
  if (gstart) {
    if (hgs[0] != 0) return fail(BCA_ERR_SHAPE, "validation: group_start[0] = %d, not 0", hgs[0]);
    for (int32_t i = 0; i < nseq; ++i)
      if (hgs[i + 1] < hgs[i])
        return fail(BCA_ERR_SHAPE, "validation: group_start decreases at segment %d", i);
    if (hgs[nseq] > (1 << 26))
      return fail(BCA_ERR_SHAPE, "validation: group_start[nseq] = %d groups", hgs[nseq]);
    err = to_host(hpe, gpe, (size_t)hgs[nseq], s);
    if (err == hipSuccess) err = to_host(hcp, gcp, (size_t)hgs[nseq], s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err != hipSuccess) return hip_status(err, "validation copy");
  }
  for (int32_t i = 0; i < nseq; ++i) {
    const long long L = (long long)hcu[i + 1] - hcu[i];
    long long S = 0;
    if (gstart) {
      for (int32_t g = hgs[i]; g < hgs[i + 1]; ++g) {
        if (hcp[g] < 0) return fail(BCA_ERR_SHAPE, "validation: group %d has %d copies", g, hcp[g]);
        S += hcp[g];
      }
    } else if (s_copies) {
      S = hsc[i];
      if (S < 0) return fail(BCA_ERR_SHAPE, "validation: segment %d has %lld copies", i, S);
    }
    const long long P = L - S * B;
    if (P < 0)
      return fail(BCA_ERR_SHAPE, "validation: segment %d: %lld copies of %d exceed %lld tokens",
                  i, S, B, L);
    if (S > 0 && P % B != 0)
      return fail(BCA_ERR_SHAPE, "validation: segment %d: prefix %lld is not a multiple of %d",
                  i, P, B);
    if (gstart) {
      long long prev = 0;
      for (int32_t g = hgs[i]; g < hgs[i + 1]; ++g) {
        const long long pe = hpe[g];
        if (pe % B != 0 || pe < 0 || pe > P || pe < prev)
          return fail(BCA_ERR_SHAPE,
                      "validation: group %d: prefix end %lld must be a multiple of B in [%lld, "
                      "%lld]",
                      g, pe, prev, P);
        prev = pe;
      }
    }
  }
  return BCA_OK;
}

// No exception crosses the C ABI: a failed host allocation of the copies
// becomes a status.
bca_status_t validate_tables(const int32_t* cu, const int32_t* s_copies, const int32_t* gstart,
                             const int32_t* gpe, const int32_t* gcp, int32_t nseq,
                             int32_t max_seqlen, int32_t total, int32_t B, hipStream_t s) {
  try {
    return validate_tables_impl(cu, s_copies, gstart, gpe, gcp, nseq, max_seqlen, total, B, s);
  } catch (const std::bad_alloc&) {
    return fail(BCA_ERR_HOST_MEMORY, "validation: no host memory for copies of %d segments",
                nseq);
  }
}

bca_status_t poison(void* p, size_t bytes, hipStream_t s) {
  return hip_status(bca::launch_fill_u32(p, bytes / 4, kPoisonWord, s), "poison fill");
}

}  // namespace

extern "C" {

int32_t bca_abi_version(void) { return BCA_ABI_VERSION; }

const char* bca_status_string(bca_status_t status) {
  switch (status) {
    case BCA_OK: return "ok";
    case BCA_ERR_NULL: return "null pointer";
    case BCA_ERR_SHAPE: return "invalid shape";
    case BCA_ERR_DTYPE: return "unsupported dtype";
    case BCA_ERR_UNSUPPORTED: return "unsupported configuration";
    case BCA_ERR_WORKSPACE: return "workspace too small";
    case BCA_ERR_HIP: return "HIP runtime error";
    case BCA_ERR_HOST_MEMORY: return "host memory exhausted";
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
  if (env_on("BCA_VALIDATE")) {
    st = validate_tables(cu_seqlens, s_copies, group_start, group_pe, group_copies, nseq,
                         max_seqlen, total, block_size, s);
    if (st != BCA_OK) return st;
  }
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
                             size_t ws_bytes, int32_t stage, void* stream) {
  if (stage < 0 || stage > 3) return fail(BCA_ERR_SHAPE, "stage must be 0, 1, 2 or 3 (got %d)", stage);
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (env_on("BCA_VALIDATE")) {
    st = validate_tables(cu_seqlens, s_copies, group_start, group_pe, group_copies, nseq,
                         max_seqlen, total, block_size, s);
    if (st != BCA_OK) return st;
  }
  // The row terms are written by stage 1; later stages only read them.
  if ((stage == 0 || stage == 1) && env_on("BCA_POISON")) {
    st = poison(workspace, need, s);
    if (st != BCA_OK) return st;
  }
  return hip_status(bca::launch_bwd_bf16(a, max_seqlen, stage, s), "backward launch");
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
                  workspace, ws_bytes, 0, stream);
}

bca_status_t bca_staircase_bwd_stage(int32_t stage, const void* q, const void* k, const void* v,
                                     const void* o, const float* lse, const void* dout, void* dq,
                                     void* dk, void* dv, const int32_t* cu_seqlens,
                                     const int32_t* s_copies, int32_t nseq, int32_t max_seqlen,
                                     int32_t total, int32_t hq, int32_t hkv, int32_t d,
                                     int32_t block_size, float scale, bca_dtype_t dtype,
                                     void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, s_copies, nullptr, nullptr,
                  nullptr, nseq, max_seqlen, total, hq, hkv, d, block_size, scale, dtype,
                  workspace, ws_bytes, stage, stream);
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
                  workspace, ws_bytes, 0, stream);
}

// Split-KV plan of the decode step: the 64-key tiles are dealt to the splits
// in turn.  By default: as few splits as give the smallest possible number of
// tiles per split while one workgroup per split and KV head fits the 256
// compute units.  Each CU streams its tiles at a fixed rate, so the kernel
// lasts as long as its longest split, and fewer splits mean fewer partial
// bytes to write and merge (129 tiles: 26 splits of at most 5 tiles, not 32
// splits of which one has 5).
static int decode_splits(int32_t q_len, int32_t kv_len, int32_t hq, int32_t hkv, int32_t req) {
  const int hpw = bca::heads_per_wg(hq, hkv);
  const int tok = 32 * (4 / hpw);
  const int ntok = (q_len + tok - 1) / tok;
  const int base_wgs = (hq / hpw) * ntok;
  const int tiles = (kv_len + 63) / 64;
  int ns = req;
  if (req <= 0) {
    const int ns_max = base_wgs < 256 ? 256 / base_wgs : 1;
    const int per_split = (tiles + ns_max - 1) / ns_max;  // fewest tiles the longest split can have
    ns = (tiles + per_split - 1) / per_split;
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
  const size_t po = (rows * d * sizeof(uint16_t) + 255) & ~(size_t)255;  // bf16 partial O
  const size_t pl = (rows * sizeof(float) + 255) & ~(size_t)255;          // float32 LSE
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
  if (!std::isfinite(scale) || scale <= 0.f)
    return fail(BCA_ERR_SHAPE, "scale must be finite and > 0");
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
      ((size_t)ns * hq * ((q_len + 31) / 32) * 32 * d * sizeof(uint16_t) + 255) & ~(size_t)255;
  a->part_o = ns > 1 ? static_cast<uint16_t*>(workspace) : nullptr;
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

// Enqueue a decode step: with BCA_POISON the partial buffers are NaN-filled
// first (only the kernels' own writes may reach the combine).
static hipError_t decode_enqueue(const bca::DecodeArgs& a, bool fp8, hipStream_t s) {
  if (a.nsplit > 1 && env_on("BCA_POISON")) {
    const size_t rows = (size_t)a.nsplit * a.hq * ((a.q_len + 31) / 32) * 32;
    hipError_t err = bca::launch_fill_u32(a.part_o, rows * a.d / 2, kPoisonWord, s);
    if (err == hipSuccess) err = bca::launch_fill_u32(a.part_lse, rows, kPoisonWord, s);
    if (err != hipSuccess) return err;
  }
  return fp8 ? bca::launch_decode_fp8(a, s) : bca::launch_decode_bf16(a, s);
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
  return hip_status(decode_enqueue(a, false, static_cast<hipStream_t>(stream)), "decode launch");
}

bca_status_t bca_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                int32_t q_len, int32_t kv_len, int32_t hq, int32_t hkv, int32_t d,
                                float scale, bca_dtype_t dtype, int32_t num_splits,
                                void* stream) {
  g_last_error[0] = '\0';
  const size_t need = bca_decode_workspace(q_len, kv_len, hq, hkv, d, num_splits);
  if (need > bca::kNoAllocScratchBytes)
    return fail(BCA_ERR_WORKSPACE,
                "this decode needs %zu bytes of scratch; the library holds %zu per device "
                "(fewer splits or a caller workspace with bca_decode)",
                need, bca::kNoAllocScratchBytes);
  // Every argument check first (with a stand-in for the scratch address, so
  // that a bad call never touches the HIP runtime), then the real address.
  bca::DecodeArgs a{};
  void* const stand_in = reinterpret_cast<void*>(uintptr_t(256));
  bca_status_t st = decode_args(q, k, v, o, lse, q_len, kv_len, hq, hkv, d, scale, dtype,
                                num_splits, need > 0 ? stand_in : nullptr, need, &a);
  if (st != BCA_OK) return st;
  if (need > 0) {
    void* scratch = nullptr;
    st = hip_status(bca::noalloc_scratch(&scratch), "scratch address");
    if (st != BCA_OK) return st;
    st = decode_args(q, k, v, o, lse, q_len, kv_len, hq, hkv, d, scale, dtype, num_splits,
                     scratch, need, &a);
    if (st != BCA_OK) return st;
  }
  return hip_status(decode_enqueue(a, false, static_cast<hipStream_t>(stream)), "decode launch");
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
  return hip_status(decode_enqueue(a, true, static_cast<hipStream_t>(stream)), "decode launch");
}

}  // extern "C"

// Record `steps` decode calls into a HIP graph through a private capture
// stream and instantiate it: step i uses a0 with q, o and lse advanced by i
// times the given element strides.
static bca_status_t capture_decode(const bca::DecodeArgs& a0, int32_t steps, size_t q_step,
                                   size_t o_step, size_t lse_step, bca_decode_graph_t** graph) {
  hipStream_t s = nullptr;
  hipError_t err = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (err != hipSuccess) return hip_status(err, "capture stream");
  err = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (err != hipSuccess) {
    (void)hipStreamDestroy(s);
    return hip_status(err, "begin capture");
  }
  hipError_t launch_err = hipSuccess;
  for (int32_t i = 0; i < steps && launch_err == hipSuccess; ++i) {
    bca::DecodeArgs a = a0;
    a.step = i;
    a.q += (size_t)i * q_step;
    a.o += (size_t)i * o_step;
    a.lse += (size_t)i * lse_step;
    launch_err = decode_enqueue(a, false, s);
  }
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
  *graph = new (std::nothrow) bca_decode_graph{g, exec, steps};
  if (!*graph) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(g);
    return fail(BCA_ERR_HOST_MEMORY, "no host memory for the graph handle");
  }
  return BCA_OK;
}

extern "C" {

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
  return capture_decode(a, steps, 0, 0, 0, graph);
}

bca_status_t bca_decode_loop_create(const void* q, const void* k, const void* v, void* o,
                                    float* lse, const int32_t* kv_len_dev,
                                    const int32_t* steps_dev, int32_t q_len,
                                    int32_t kv_capacity, int32_t hq, int32_t hkv, int32_t d,
                                    float scale, bca_dtype_t dtype, int32_t num_splits,
                                    void* workspace, size_t ws_bytes, int32_t steps,
                                    bca_decode_graph_t** graph) {
  g_last_error[0] = '\0';
  if (!graph) return fail(BCA_ERR_NULL, "graph handle pointer is NULL");
  *graph = nullptr;
  if (steps < 1 || steps > kMaxGraphSteps)
    return fail(BCA_ERR_SHAPE, "steps must be in [1, %d] (got %d)", kMaxGraphSteps, steps);
  if (!kv_len_dev) return fail(BCA_ERR_NULL, "kv_len_dev is NULL");
  if ((reinterpret_cast<uintptr_t>(kv_len_dev) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(steps_dev) & 3u) != 0)
    return fail(BCA_ERR_SHAPE, "kv_len_dev and steps_dev must be 4-byte aligned");
  bca::DecodeArgs a{};
  const bca_status_t st = decode_args(q, k, v, o, lse, q_len, kv_capacity, hq, hkv, d, scale,
                                      dtype, num_splits, workspace, ws_bytes, &a);
  if (st != BCA_OK) return st;
  if ((long long)steps * q_len * hq * d >= (1LL << 40))
    return fail(BCA_ERR_SHAPE, "problem too large");
  a.kv_len_dev = kv_len_dev;
  a.steps_dev = steps_dev;
  const size_t qo_step = (size_t)q_len * hq * d;
  return capture_decode(a, steps, qo_step, qo_step, (size_t)hq * q_len, graph);
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
