// Device-side helpers shared by the bca kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running-max sentinel: finite so that exp2(sentinel - sentinel) = 1 and no
// inf - inf appears while a row has not yet met an admitted key.
constexpr float kNegBig = -1.0e30f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even pack of two floats into two bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 x = {lo, hi};
  bf16x2 y = __builtin_convertvector(x, bf16x2);
  return __builtin_bit_cast(uint32_t, y);
}

// LDS address-space pointer types for the direct-to-LDS and transposed-read builtins.
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ lds_void* as_lds(void* p) { return (lds_void*)(p); }

// Buffer resource over [base, base + nbytes): loads at or past nbytes return zero.
// Word 3 holds the data-format bits of a raw (untyped, stride 0) buffer on gfx9.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           0x00020000);
}

// 16 bytes per lane from buffer `r` at byte offset voffset into LDS at
// lds_base + 16 * lane (lanes write consecutive 16-byte slots).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                                  uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, as_lds(lds_base), 16, voffset, 0, 0, 0);
}

// Wait until this wave's outstanding vector-memory operations (including
// direct-to-LDS loads) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// if address-lane 4r + q points at element [row0 + r][col0 + 4q] of a
// row-major 16-bit matrix, lane c receives rows row0..row0+3 of column
// col0 + c.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// 16-byte chunk swizzle of a row-major tile with D/8 chunks per row: chunk c
// of row r is stored at chunk c ^ swz(r).  Chosen so that 16 consecutive rows
// read at one logical chunk, and 4 consecutive rows read at 4 consecutive
// chunks through the transposed read, both hit distinct LDS banks.
template <int D>
__device__ __forceinline__ int swz(int row) {
  return D == 128 ? 4 * (row & 3) + ((row >> 2) & 3) : 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

// x combined with the value of the lane 32 positions away (v_permlane32_swap:
// swaps the upper half-wave of one register with the lower of another).
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------
// Admitted keys of one query row.
//
// Block-causal attention ("On-Policy Residual Learning for Diffusion Language
// Models", thread page, highlight 3) and its staircase packed-replay variant
// (paper cards page, Figure 3 caption): in a segment of L tokens whose last
// S*B tokens are S copies of one B-token block and whose first P = L - S*B
// tokens are the clean prefix,
//   prefix row i < P   : keys [0, min(P, (floor(i/B) + 1) * B))
//   copy row, copy c   : keys [0, P)  and  [P + c*B, P + (c+1)*B)
// Positions are relative to the segment start.  With S = 0, P = L and the
// last (possibly partial) block stays bidirectional.
struct RowKeys {
  int e1;  // first interval is [0, e1)
  int s2;  // second interval is [s2, e2) (empty for prefix rows)
  int e2;
};

__device__ __forceinline__ RowKeys row_keys(int i, int P, int L, int B) {
  RowKeys r;
  if (i < P) {
    int e = (i / B + 1) * B;
    r.e1 = e < P ? e : P;
    r.s2 = 0;
    r.e2 = 0;
  } else {
    int c = (i - P) / B;
    int e = P + (c + 1) * B;
    r.e1 = P;
    r.s2 = P + c * B;
    r.e2 = e < L ? e : L;
  }
  return r;
}

__device__ __forceinline__ bool admitted(const RowKeys& r, int j) {
  return j < r.e1 || (j >= r.s2 && j < r.e2);
}

// The query rows that admit key j (0 <= j < L), which always form one
// interval [lo, hi): a prefix key of block floor(j/B) is seen by the prefix
// rows of that block and later ones and by every copy row; a key of copy c
// only by the rows of copy c.
struct KeyRows {
  int lo, hi;
};

__device__ __forceinline__ KeyRows key_rows(int j, int P, int L, int B) {
  KeyRows r;
  if (j < P) {
    r.lo = (j / B) * B;
    r.hi = L;
  } else {
    const int c = (j - P) / B;
    const int e = P + (c + 1) * B;
    r.lo = P + c * B;
    r.hi = e < L ? e : L;
  }
  return r;
}

// Key ranges a tile of query rows [q_first, q_last] (inclusive, all inside
// the segment) must visit: [0, r1e) and [r2s, r2e), merged when they touch.
struct TileKeys {
  int r1e;
  int r2s;
  int r2e;
};

__device__ __forceinline__ TileKeys tile_keys(int q_first, int q_last, int P, int L, int B) {
  TileKeys t;
  if (q_last < P) {
    int e = (q_last / B + 1) * B;
    t.r1e = e < P ? e : P;
    t.r2s = t.r2e = 0;
  } else {
    int c_first = q_first >= P ? (q_first - P) / B : 0;
    int c_last = (q_last - P) / B;
    t.r1e = P;
    t.r2s = P + c_first * B;
    t.r2e = P + (c_last + 1) * B;
    if (t.r2e > L) t.r2e = L;
  }
  if (t.r2e > t.r2s && t.r2s <= t.r1e) {  // contiguous: one range
    t.r1e = t.r2e > t.r1e ? t.r2e : t.r1e;
    t.r2s = t.r2e = 0;
  }
  return t;
}

}  // namespace bca
