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

// The same descriptor as four words, for inline assembly.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xffffu), (int)nbytes, 0x00020000};
}

// Direct-to-LDS loads written as inline assembly: from buffer `r` at
// voffset into LDS at byte address lds_addr + W * lane, W = 16 bytes
// (buffer_load_lds16_asm) or 4 bytes (buffer_load_lds4_asm).  The compiler
// does not know these write LDS, so it adds no wait for them before later
// LDS reads, and counts them in none of its own vmcnt waits (which can
// only grow stricter by it): the caller orders the data with explicit vmcnt
// waits and barriers.  M0 is written here and nowhere else in the kernels
// that use these (the compiler reserves it, so it is listed only for the
// reader).  The nops cover the write-to-use distances of the descriptor
// SGPRs (when the compiler builds them with a VALU op) and of M0.
// The descriptor and the LDS address are wave-uniform by construction; the
// compiler may still hold such a value in a VGPR (a uniform select lowered to
// v_cndmask), which an "s" operand cannot take, so every word goes through
// readfirstlane (free when the value already sits in an SGPR).
__device__ __forceinline__ i32x4 uniform_words(i32x4 r) {
  return i32x4{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
               __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}
__device__ __forceinline__ void buffer_load_lds16_asm(i32x4 r, uint32_t lds_addr,
                                                      uint32_t voffset) {
  r = uniform_words(r);
  lds_addr = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voffset), "s"(r)
      : "memory");
}
__device__ __forceinline__ void buffer_load_lds4_asm(i32x4 r, uint32_t lds_addr,
                                                     uint32_t voffset) {
  r = uniform_words(r);
  lds_addr = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voffset), "s"(r)
      : "memory");
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_void*)(p));
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

// Workgroup barrier that leaves direct-to-LDS loads in flight.  __syncthreads()
// would wait for them: its release fence waits for every earlier memory
// operation.  LDS reads issued before this barrier have returned (lgkmcnt),
// so a buffer may be overwritten after it; the memory clobber keeps the
// compiler from moving memory accesses across it.  Data of a direct load is
// visible to other waves only once its issuer has waited for it (vmcnt) and
// then passed a barrier.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The same, after this wave's direct-to-LDS loads have landed.  Written as one
// asm block so that the wait stays at the end of the phase.
__device__ __forceinline__ void wait_vmem_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
// Models", thread page, highlight 3) and its staircase packed-replay variants
// (paper cards page, Figure 3 caption; thread page, Insight 3).  A segment of
// L tokens is a clean prefix of P tokens followed by copies of B-token blocks,
// grouped: the copies of group g are noisy states of one block and see the
// clean keys [0, pe_g) (pe_g = that block's start; groups ordered by pe_g,
// non-decreasing) and, bidirectionally, their own B tokens.  The plain
// staircase is one group with pe = P; plain block-causal has no copies.
//   prefix row i < P       : keys [0, min(P, (floor(i/B) + 1) * B))
//   copy row of copy c     : keys [0, pe_g(c))  and  [P + c*B, P + (c+1)*B)
// Positions are relative to the segment start; copies are numbered from 0
// over the whole segment.  With no copies, P = L and the last (possibly
// partial) block stays bidirectional.
struct Stair {
  int P, L, B;
  int S;                   // copies in the segment
  const int32_t* gpe;      // group prefix ends (NULL: one group with pe = P)
  const int32_t* gcp;      // copies per group
  int ng;                  // groups
};

// The segment's rule from the packed metadata: per-segment copy counts
// (s_copies, one group with pe = P) or a group table (group_start [nseq+1]
// indexing group_pe / group_copies).
__device__ __forceinline__ Stair make_stair(int seg, int L, int B, const int32_t* s_copies,
                                            const int32_t* group_start, const int32_t* group_pe,
                                            const int32_t* group_copies) {
  Stair st;
  st.L = L;
  st.B = B;
  st.gpe = nullptr;
  st.gcp = nullptr;
  st.ng = 0;
  int S = 0;
  if (group_start) {
    const int g0 = group_start[seg], g1 = group_start[seg + 1];
    st.gpe = group_pe + g0;
    st.gcp = group_copies + g0;
    st.ng = g1 - g0;
    for (int g = 0; g < st.ng; ++g) S += st.gcp[g];
  } else if (s_copies) {
    S = s_copies[seg];
  }
  st.S = S;
  const int P = L - S * B;
  st.P = P < 0 ? 0 : P;
  return st;
}

// Clean keys seen by copy c: the prefix end of its group.
__device__ __forceinline__ int copy_prefix_end(const Stair& st, int c) {
  if (!st.gpe) return st.P;
  int acc = 0;
  for (int g = 0; g < st.ng; ++g) {
    acc += st.gcp[g];
    if (c < acc) return st.gpe[g];
  }
  return st.P;
}

// First copy whose group sees clean key j (j < P); S if none does.
__device__ __forceinline__ int first_copy_seeing(const Stair& st, int j) {
  if (!st.gpe) return 0;
  int acc = 0;
  for (int g = 0; g < st.ng; ++g) {
    if (st.gpe[g] > j) return acc;
    acc += st.gcp[g];
  }
  return acc;
}

struct RowKeys {
  int e1;  // first interval is [0, e1)
  int s2;  // second interval is [s2, e2) (empty for prefix rows)
  int e2;
};

__device__ __forceinline__ RowKeys row_keys(int i, const Stair& st) {
  RowKeys r;
  if (i < st.P) {
    int e = (i / st.B + 1) * st.B;
    r.e1 = e < st.P ? e : st.P;
    r.s2 = 0;
    r.e2 = 0;
  } else {
    int c = (i - st.P) / st.B;
    int e = st.P + (c + 1) * st.B;
    r.e1 = copy_prefix_end(st, c);
    r.s2 = st.P + c * st.B;
    r.e2 = e < st.L ? e : st.L;
  }
  return r;
}

__device__ __forceinline__ bool admitted(const RowKeys& r, int j) {
  return j < r.e1 || (j >= r.s2 && j < r.e2);
}

// The query rows that admit key j (0 <= j < L): at most two intervals.  A
// clean key of block floor(j/B) is seen by the prefix rows of that block and
// later ones, [lo, P), and by the copies of every group with pe > j -- with
// groups ordered by pe, a final run of copies [c_lo, L); a key of copy c only
// by the rows of copy c.
struct KeyRows {
  int lo, hi;    // first interval
  int lo2, hi2;  // second interval (empty if lo2 >= hi2)
};

__device__ __forceinline__ KeyRows key_rows(int j, const Stair& st) {
  KeyRows r;
  if (j < st.P) {
    r.lo = (j / st.B) * st.B;
    r.hi = st.P;
    r.lo2 = st.P + first_copy_seeing(st, j) * st.B;
    r.hi2 = st.L;
    if (r.lo2 == r.hi) {  // every copy sees the key: one interval
      r.hi = st.L;
      r.lo2 = r.hi2 = 0;
    }
  } else {
    const int c = (j - st.P) / st.B;
    const int e = st.P + (c + 1) * st.B;
    r.lo = st.P + c * st.B;
    r.hi = e < st.L ? e : st.L;
    r.lo2 = r.hi2 = 0;
  }
  return r;
}

__device__ __forceinline__ bool row_sees(const KeyRows& r, int i) {
  return (i >= r.lo && i < r.hi) || (i >= r.lo2 && i < r.hi2);
}

// Key ranges a tile of query rows [q_first, q_last] (inclusive, all inside
// the segment) must visit: [0, r1e) and [r2s, r2e), merged when they touch.
struct TileKeys {
  int r1e;
  int r2s;
  int r2e;
};

__device__ __forceinline__ TileKeys tile_keys(int q_first, int q_last, const Stair& st) {
  TileKeys t;
  const int P = st.P, B = st.B;
  if (q_last < P) {
    int e = (q_last / B + 1) * B;
    t.r1e = e < P ? e : P;
    t.r2s = t.r2e = 0;
  } else {
    const int c_first = q_first >= P ? (q_first - P) / B : 0;
    const int c_last = (q_last - P) / B;
    // clean keys: the largest prefix end among the tile's rows (prefix ends
    // grow with the copy index; prefix rows reach at most P)
    int e1 = copy_prefix_end(st, c_last);
    if (q_first < P) e1 = P;
    t.r1e = e1;
    t.r2s = P + c_first * B;
    t.r2e = P + (c_last + 1) * B;
    if (t.r2e > st.L) t.r2e = st.L;
  }
  if (t.r2e > t.r2s && t.r2s <= t.r1e) {  // contiguous: one range
    t.r1e = t.r2e > t.r1e ? t.r2e : t.r1e;
    t.r2s = t.r2e = 0;
  }
  return t;
}

// Smallest clean-key end among rows [q_first, q_last]: prefix ends grow along
// the prefix and along the copies, so it is the first row's or the first copy
// row's.
__device__ __forceinline__ int min_prefix_end(int q_first, int q_last, const Stair& st) {
  int e = row_keys(q_first, st).e1;
  if (q_first < st.P && q_last >= st.P) {
    const int e2 = row_keys(st.P, st).e1;
    e = e2 < e ? e2 : e;
  }
  return e;
}

}  // namespace bca
