// Kernel argument blocks and host launchers of the bca library (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bca {

// Forward over packed segments (block-causal when s_copies is NULL).
struct FwdArgs {
  const uint16_t* q;  // [total, hq, d] bf16
  const uint16_t* k;  // [total, hkv, d]
  const uint16_t* v;
  uint16_t* o;        // [total, hq, d]
  float* lse;         // [hq, total]
  const int32_t* cu_seqlens;
  const int32_t* s_copies;      // may be NULL
  const int32_t* group_start;   // copy groups (NULL: s_copies rule), [nseq + 1]
  const int32_t* group_pe;      // prefix end per group
  const int32_t* group_copies;  // copies per group
  int nseq, total, hq, hkv, d, block_size;
  int hpw;            // query heads per workgroup (4, 2 or 1; divides hq / hkv)
  float scale_log2;   // scale * log2(e)
};

struct FwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const int32_t* cu_seqlens;
  const int32_t* s_copies;
  const int32_t* group_start;
  const int32_t* group_pe;
  const int32_t* group_copies;
  int nseq, total, hq, hkv, d, block_size;
  float scale_log2;
};

struct DecodeArgs {
  const uint16_t* q;  // [q_len, hq, d]
  const uint16_t* k;  // [kv_len, hkv, d] bf16 (decode_bf16_kernel)
  const uint16_t* v;
  const uint8_t* k8;  // [kv_len, hkv, d] fp8 E4M3 (decode_fp8_kernel)
  const uint8_t* v8;
  float o_mul;        // multiplies O (the V scale of an fp8 cache; 1 for bf16)
  uint16_t* o;        // [q_len, hq, d]
  float* lse;         // [hq, q_len]
  // Split partials (nsplit > 1), per (split, head, 32-token tile):
  // part_o   [nsplit, hq, ceil(q_len/32), 32 * d] bf16, normalised, in the MFMA
  //          accumulator order
  // part_lse [nsplit, hq, ceil(q_len/32), 32] float32
  uint16_t* part_o;
  float* part_lse;
  int q_len, kv_len, hq, hkv, d, hpw;
  // Device-resident cache length (NULL: kv_len).  When set, the kernels
  // attend to min(max(*kv_len_dev, q_len), kv_len) keys; kv_len is then the
  // capacity the grid and the partials were planned for.
  const int32_t* kv_len_dev;
  // Device-resident step count of a captured loop (NULL: every step runs):
  // the launches of step `step` return at once when step >= *steps_dev.
  const int32_t* steps_dev;
  int step;
  int nsplit;         // split s takes key tiles s, s + nsplit, ... < T, T = ceil(kv_len / 64)
  float scale_log2;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;       // [hq, total] float32 workspace: rowsum(dO * O)
  float* lse2;        // [hq, total] float32 workspace: LSE * log2(e)
  const int32_t* cu_seqlens;
  const int32_t* s_copies;
  const int32_t* group_start;
  const int32_t* group_pe;
  const int32_t* group_copies;
  int nseq, total, hq, hkv, d, block_size;
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
};

// Query rows of one wave are 32 consecutive tokens of one head; a workgroup
// of four waves covers hpw heads of one KV group.
inline int heads_per_wg(int hq, int hkv) {
  const int group = hq / hkv;
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int max_seqlen, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdF32Args& a, int max_seqlen, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t stream);
// Backward kernels: stage 0 = all three in order, 1 = row terms (delta and
// LSE * log2 e), 2 = dK/dV, 3 = dQ.
hipError_t launch_bwd_bf16(const BwdArgs& a, int max_seqlen, int stage, hipStream_t stream);

// Bytes of the per-device scratch array behind bca_decode_noalloc.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;

// Device address of the calling thread's current device's scratch array
// (fetched with hipGetSymbolAddress on the first call per device, then
// cached).  Allocates nothing.
hipError_t noalloc_scratch(void** ptr);

// p[0 .. nwords) = value (a grid-stride fill kernel).
hipError_t launch_fill_u32(void* p, size_t nwords, uint32_t value, hipStream_t stream);

}  // namespace bca
