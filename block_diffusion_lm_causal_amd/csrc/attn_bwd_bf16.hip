// Backward of block-causal / staircase attention (bf16 in, float32
// accumulation) on gfx950.
//
// The attention is the one of the forward ("On-Policy Residual Learning for
// Diffusion Language Models": block-causal attention, thread page highlight 3;
// staircase packed replay used to train on captured denoising states, paper
// cards page Figure 3 caption and thread page Insight 3).  With
// P = softmax(scale * Q K^T) over admitted keys, O = P V and upstream dO:
//   dV = P^T dO,  dP = dO V^T,  delta = rowsum(dO * O),
//   dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,
// and P is recomputed from Q, K and the forward's LSE.
//
// Three kernels, no atomics (results are bit-reproducible):
//   1. delta = rowsum(dO * O) in float32.
//   2. dK/dV: an 8-wave workgroup owns 128 keys of one KV head.  Waves 0-3
//      ("V waves", 32 keys each) compute S = Q K^T -> P and dV += P^T dO;
//      waves 4-7 ("K waves", the same keys) compute dP = dO V^T, take P from
//      their V wave through LDS, form dS and dK += dS^T Q.  S is computed
//      once, and each SIMD pairs one wave of each kind, so one's MFMA work
//      overlaps the other's exponentials.  K and V fragments and the dK/dV
//      accumulators stay in registers; each step streams a 32-row tile of Q
//      and dO (one query head) through LDS, loaded straight from HBM two steps
//      ahead.  S is computed with queries on the M axis, so the P and dS
//      accumulators are, unchanged, the A operands of the dV and dK products;
//      their B operands (dO and Q with queries on K) come from the row-major
//      tiles through the transposed LDS read.
//   3. dQ: shaped like the forward's ping-pong kernel -- two groups of four
//      waves, one phase apart, over 32-key tiles: MFMA phase S^T(t) = K Q^T,
//      dP^T(t) = V dO^T and dQ^T += K^T dS^T(t-1); VALU phase P and dS of
//      tile t.  K^T comes from the row-major K tile through the transposed read.
#include <type_traits>

#include "bca_device.hpp"
#include "bca_kernels.hpp"

namespace bca {
namespace {

constexpr int kBN = 32;    // keys per tile in the dQ kernel
constexpr int kQt = 32;    // query rows per dK/dV step
constexpr int kKvKeys = 128;  // keys per dK/dV workgroup

// ---------------------------------------------------------------------------
// 1. delta[h][i] = sum_d dO[i,h,d] * O[i,h,d], and lse2[h][i] = LSE[h][i] log2(e)

__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  const int d = a.d;
  const int lanes_per_row = d / 8;  // 16 (d = 128) or 8 (d = 64)
  const long long row = (long long)blockIdx.x * (256 / lanes_per_row) + threadIdx.x / lanes_per_row;
  const int sub = threadIdx.x % lanes_per_row;
  const long long nrows = (long long)a.total * a.hq;
  float acc = 0.f;
  if (row < nrows) {
    const u32x4 o = *reinterpret_cast<const u32x4*>(a.o + row * d + sub * 8);
    const u32x4 g = *reinterpret_cast<const u32x4*>(a.dout + row * d + sub * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16_to_f32(o[w] & 0xffffu), bf16_to_f32(g[w] & 0xffffu), acc);
      acc = fmaf(bf16_to_f32(o[w] >> 16), bf16_to_f32(g[w] >> 16), acc);
    }
  }
  for (int off = lanes_per_row / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < nrows && sub == 0) {
    const long long i = row / a.hq;
    const int h = (int)(row % a.hq);
    a.delta[(size_t)h * a.total + i] = acc;
    a.lse2[(size_t)h * a.total + i] = a.lse[(size_t)h * a.total + i] * kLog2e;
  }
}

// s_waitcnt vmcnt(n), n < 64 (expcnt and lgkmcnt left unconstrained; the
// two high bits of vmcnt sit at bits 14-15 of the immediate).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// A operand fragment of a row-major swizzled tile: row lane%32 (+ row_base),
// logical 16-byte chunk 2kk + half.
template <int D>
__device__ __forceinline__ uint32_t row_frag_off(int lane, int kk) {
  const int half = lane >> 5;
  return (uint32_t)((lane & 31) * D * 2 + (((2 * kk + half) ^ swz<D>(lane & 15)) * 16));
}

// Transposed-read offsets: 16-lane group G, address-lane 4r + q reads rows
// 8sub + 4half + r (of a 16-row chunk), columns 32dt + 16(G%2) + 4q.
template <int D>
__device__ __forceinline__ uint32_t tr_off(int lane, int dt, int sub) {
  const int half = lane >> 5;
  const int a = lane & 15, r = a >> 2, q = a & 3, g2 = (lane >> 4) & 1;
  const int row = 8 * sub + 4 * half + r;
  const int chunk = 4 * dt + 2 * g2 + (q >> 1);
  return (uint32_t)(row * D * 2 + ((chunk ^ swz<D>(row)) * 16) + (q & 1) * 8);
}

__device__ __forceinline__ bf16x8 tr_pair(const char* p0, const char* p1) {
  const u32x2 l2 = __builtin_bit_cast(u32x2, lds_read_tr16(p0));
  const u32x2 h2 = __builtin_bit_cast(u32x2, lds_read_tr16(p1));
  return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}

// ---------------------------------------------------------------------------
// 2. dK / dV

// Per-tile side values of the dK/dV kernel: [buffer][0] the LSE of the
// tile's rows times log2(e), [buffer][1] their delta (64 slots, rows past the
// tile's 32 land in the upper half and are not read).
struct __attribute__((aligned(16))) KvSide {
  float v[4][2][64];
};

template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdArgs a, int nkt_max) {
  // Four tile buffers, each a Q tile then a dO tile (32 rows x D, row-major,
  // swizzled), filled by direct loads that the compiler does not see (so it
  // adds no waits for them); explicit waits and barriers order them.
  constexpr int kTileBytes = 2 * kQt * D * 2;
  __shared__ __attribute__((aligned(16))) uint16_t tiles[4][2 * kQt * D];
  __shared__ KvSide lds;
  // P of a tile (bf16 pairs, two 16-byte words per lane) from each V wave to
  // the K wave of the same keys, double-buffered by step parity.
  __shared__ __attribute__((aligned(16))) uint32_t p_xchg[2][4][2][64 * 4];
  const int group = a.hq / a.hkv;
  // Order: KV head fastest, then the key tiles of one segment (earliest keys,
  // i.e. most query rows, first), then the next segment.  Every workgroup
  // sweeps its query tiles from the last one down, so the workgroups resident
  // on an XCD stream the same Q/dO rows at the same time and share them in L2.
  const int w = blockIdx.x;
  const int g = w % a.hkv;
  const int rest = w / a.hkv;
  const int ktile = rest % nkt_max;
  const int seg = rest / nkt_max;
  const int base = a.cu_seqlens[seg];
  const int L = a.cu_seqlens[seg + 1] - base;
  const int k0 = ktile * kKvKeys;
  if (k0 >= L) return;
  const Stair stair = make_stair(seg, L, a.block_size, a.s_copies, a.group_start, a.group_pe,
                                 a.group_copies);
  const int P = stair.P;
  const int B = a.block_size;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool kwave = wave >= 4;           // K waves compute dK, V waves dV
  const int kw0 = k0 + (wave & 3) * 32;   // this wave's first key
  const int key = kw0 + (lane & 31);      // key of this lane's accumulator column
  const int k_last_wg = min(k0 + kKvKeys, L) - 1;

  // Query rows that admit any key of the workgroup: up to two ranges,
  // [qs1, qe1) (prefix rows from the first key's block, and the copies that
  // own keys of the workgroup) and [qs2, qe2) (the copies of the groups that
  // see the first clean key).
  int qs1, qe1, qs2 = 0, qe2 = 0;
  if (k0 < P) {
    qs1 = (k0 / B) * B;
    qe1 = k_last_wg >= P ? min(L, P + ((k_last_wg - P) / B + 1) * B) : P;
    qs2 = P + first_copy_seeing(stair, k0) * B;
    qe2 = L;
    if (qs2 <= qe1) {
      qe1 = max(qe1, qe2);
      qs2 = qe2 = 0;
    }
  } else {
    const int c_first = (k0 - P) / B, c_last = (k_last_wg - P) / B;
    qs1 = P + c_first * B;
    qe1 = min(L, P + (c_last + 1) * B);
  }
  const int nqt1 = (qe1 - qs1 + kQt - 1) / kQt;
  const int nqt2 = qe2 > qs2 ? (qe2 - qs2 + kQt - 1) / kQt : 0;
  const int nsteps = (nqt1 + nqt2) * group;

  // Loads: Q and dO tiles (32 rows x D) by DMA.  A tile is kInstPerTile
  // 1 KB instructions per tensor; instruction i of the 2 * kInstPerTile is
  // issued by wave i % 8 (Q blocks first, then dO blocks).  Wave 0 also loads
  // the tile's LSE * log2(e) and delta rows (two 256-byte loads).
  constexpr int kChunks = D / 8;
  constexpr int kRowsPerInst = 64 / kChunks;               // 4 (D=128) or 8 (D=64)
  constexpr int kInstPerTile = kQt / kRowsPerInst;         // 8 or 4
  constexpr int kDmaPerWave = 2 * kInstPerTile / 8;        // 2 or 1 per step
  const int q_row_elems = a.hq * D;
  uint32_t dma_voff[kDmaPerWave];
  int dma_row0[kDmaPerWave];
  bool dma_is_q[kDmaPerWave];
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int i = wave + 8 * j;
    dma_is_q[j] = i < kInstPerTile;
    dma_row0[j] = (dma_is_q[j] ? i : i - kInstPerTile) * kRowsPerInst;
    const int R = dma_row0[j] + lane / kChunks;
    const int c = (lane % kChunks) ^ swz<D>(R);
    dma_voff[j] = (uint32_t)(R * q_row_elems * 2 + c * 16);
  }
  // Steps sweep the query tiles of range 2, then of range 1, each from its
  // last tile down, every tile once per query head of the group.  A cursor
  // holds the step's tile (first row), head within the group and range
  // [lo, end); rows of a tile past `end` are loaded as zeros and masked.
  struct Cursor {
    int qt0, h, lo, end;
  };
  auto advance = [&](Cursor& c) {
    if (++c.h == group) {
      c.h = 0;
      c.qt0 -= kQt;
      if (c.qt0 < c.lo && c.lo != qs1) {  // range 2 done: continue with range 1
        c.qt0 = qs1 + (nqt1 - 1) * kQt;
        c.lo = qs1;
        c.end = qe1;
      }
    }
  };
  const uint32_t tiles_lds = lds_addr_of(&tiles[0][0]);
  const uint32_t side_lds = lds_addr_of(&lds.v[0][0][0]);
  auto issue_step = [&](const Cursor& c, int buf) {
    const int qt0 = c.qt0;
    const int head = g * group + c.h;
    const int rows = min(c.end - qt0, kQt);
    const uint32_t nbytes = (uint32_t)((rows - 1) * q_row_elems * 2 + D * 2);
    const size_t off = (size_t)(base + qt0) * q_row_elems + (size_t)head * D;
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      const i32x4 r = rsrc_words((dma_is_q[j] ? a.q : a.dout) + off, nbytes);
      const uint32_t dst = tiles_lds + (uint32_t)(buf * kTileBytes) +
                           (dma_is_q[j] ? 0u : (uint32_t)(kQt * D * 2)) +
                           (uint32_t)(dma_row0[j] * D * 2);
      buffer_load_lds16_asm(r, dst, dma_voff[j]);
    }
    if (wave == 0) {
      const size_t so = (size_t)head * a.total + base + qt0;
      const uint32_t sbytes = (uint32_t)(rows * 4);
      const uint32_t dst = side_lds + (uint32_t)(buf * 2 * 64 * 4);
      buffer_load_lds4_asm(rsrc_words(a.lse2 + so, sbytes), dst, (uint32_t)lane * 4);
      buffer_load_lds4_asm(rsrc_words(a.delta + so, sbytes), dst + 64 * 4, (uint32_t)lane * 4);
    }
  };
  // Wait until only the newest step's loads may be outstanding.
  auto wait_all_but_newest = [&]() {
    if (wave == 0) wait_vmem_le<kDmaPerWave + 2>();
    else wait_vmem_le<kDmaPerWave>();
  };

  // K fragments of this wave's keys in V waves (B operand of S = Q K^T), V
  // fragments in K waves (B operand of dP = dO V^T).
  bf16x8 kvf[D / 16];
  {
    const uint16_t* src = kwave ? a.v : a.k;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 r = u32x4{0, 0, 0, 0};
      if (key < L) {
        const size_t off = ((size_t)(base + key) * a.hkv + g) * D + kk * 16 + half * 8;
        r = *reinterpret_cast<const u32x4*>(src + off);
      }
      kvf[kk] = __builtin_bit_cast(bf16x8, r);
    }
  }
  f32x16 acc[D / 32];  // dV (V waves) or dK (K waves): keys on M, dims on N
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

  // LDS offsets of this lane's fragments in a row-major swizzled tile, with
  // the tensor each role reads folded in: the A operand of S / dP comes from
  // the Q rows (V waves) or the dO rows (K waves), the transposed B operand of
  // dV / dK from dO (V waves) or Q (K waves).  Buffer and 16-row chunk
  // offsets are immediates.  The swizzle permutes the 16-byte chunks of a row
  // (offset bits 4-7), so A fragment kk sits at roff0 ^ (32 kk): each step
  // rebuilds these from roff0 (an empty asm hides that they do not change),
  // which keeps seven registers free.
  constexpr uint32_t kGOff = kQt * D * 2;  // dO tile after the Q tile
  const uint32_t roff0 = row_frag_off<D>(lane, 0) + (kwave ? kGOff : 0u);
  uint32_t toff[D / 32][2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    toff[dt][0] = tr_off<D>(lane, dt, 0) + (kwave ? 0u : kGOff);
    toff[dt][1] = tr_off<D>(lane, dt, 1) + (kwave ? 0u : kGOff);
  }
  const char* const tiles_c = reinterpret_cast<const char*>(&tiles[0][0]);

  const int wave_key_last = min(kw0 + 31, L - 1);
  const bool wave_has_keys = kw0 < L;
  // Rows admitting this lane's key (at most two intervals), and for the wave
  // the rows admitting any of its keys [w1lo, w1hi) u [w2lo, w2hi) and the
  // rows admitting all 32 of them [f1lo, f1hi) u [f2lo, f2hi).  Along the
  // clean keys both the prefix-row interval and the run of copies seeing the
  // key start later for later keys; a copy key is seen by its copy only.
  KeyRows kr = KeyRows{0, 0, 0, 0};
  if (key < L) kr = key_rows(key, stair);
  int w1lo = 0, w1hi = 0, w2lo = 0, w2hi = 0, f1lo = 0, f1hi = 0, f2lo = 0, f2hi = 0;
  if (wave_has_keys) {
    const KeyRows first = key_rows(kw0, stair), last = key_rows(wave_key_last, stair);
    if (kw0 < P) {
      w1lo = first.lo;
      w1hi = wave_key_last >= P ? max(first.hi, last.hi) : first.hi;  // owned copies extend it
      w2lo = first.lo2;
      w2hi = first.hi2;
    } else {
      w1lo = first.lo;
      w1hi = last.hi;
    }
    const bool all_clean = wave_key_last < P;
    const bool one_copy_keys = kw0 >= P && (kw0 - P) / B == (wave_key_last - P) / B;
    if (kw0 + 31 < L && (all_clean || one_copy_keys)) {
      f1lo = last.lo;
      f1hi = last.hi;
      f2lo = last.lo2;
      f2hi = last.hi2;
    }
  }

  // Steps are software-pipelined.  Tile t (a step's Q and dO rows with their
  // side values) lives in buffer t % 4.  In step st the V waves compute
  // dV += P(st)^T dO(st) from the P(st) they made one step earlier, and
  // S(st+1) -> P(st+1), which they hand to the K waves through LDS; the K
  // waves compute dP(st) = dO(st) V^T, dS(st) = P(st) (dP(st) - delta) and
  // dK += dS(st)^T Q(st).  Each step ends with one barrier.  Tile st+3 is
  // loaded into the buffer tile st-1 left; tile st+2 must have landed by the
  // step's end.  The loop runs in groups of four steps (buffers and LDS
  // offsets fixed at compile time, the handed-over P registers alternating);
  // steps past the last do nothing.
  Cursor cur = nqt2 > 0 ? Cursor{qs2 + (nqt2 - 1) * kQt, 0, qs2, qe2}
                        : Cursor{qs1 + (nqt1 - 1) * kQt, 0, qs1, qe1};  // tile st
  Cursor nx1 = cur;                                                     // tile st + 1
  advance(nx1);
  Cursor ld = cur;                                                      // next tile to load
  // Prologue: tiles 0-2 issued, 0 and 1 landed.
  if (nsteps > 0) {
    issue_step(ld, 0);
    advance(ld);
    if (nsteps > 1) {
      issue_step(ld, 1);
      advance(ld);
    }
    if (nsteps > 2) {
      issue_step(ld, 2);
      advance(ld);
    }
  }
  // Everything landed, the K/V fragments included: the compiler does not
  // count the direct loads, so a partial wait here would leave it waiting
  // for those fragments (and with them every load in flight) inside the loop.
  wait_vmem();
  barrier_lds();

  auto active = [&](const Cursor& c) {
    return wave_has_keys &&
           ((c.qt0 < w1hi && c.qt0 + kQt > w1lo) || (c.qt0 < w2hi && c.qt0 + kQt > w2lo));
  };
  // Side values of this lane's accumulator rows 8 r4 + 4 half + 0..3 of the
  // tile in buffer `buf`: LSE * log2(e) (V waves) or delta (K waves).
  auto read_side = [&](auto bc, int r4) {
    constexpr int buf = decltype(bc)::value;
    return *reinterpret_cast<const f32x4*>(&lds.v[buf][kwave ? 1 : 0][8 * r4 + 4 * half]);
  };
  // V waves: S = Q K^T of the tile in buffer `buf` (queries on M, keys on N).
  // K waves: dP = dO V^T of the same tile.
  auto qk_product = [&](auto bc) {
    constexpr int buf = decltype(bc)::value;
    uint32_t r0 = roff0;
    asm volatile("" : "+v"(r0));
    auto frag = [&](int kk) {
      return *reinterpret_cast<const bf16x8*>(tiles_c + buf * kTileBytes + (r0 ^ (32u * kk)));
    };
    // fragments read kQA MFMAs ahead of use, so that LDS latency hides
    // behind the MFMAs between; the scheduling groups below pin that order
    // (left alone, the compiler reads one ahead)
    constexpr int kQA = 4;
    constexpr int kK = D / 16;
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 fr[kQA];
#pragma unroll
    for (int i = 0; i < kQA; ++i) fr[i] = frag(i);
    f32x16 sc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kK; ++kk) {
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[kk % kQA], kvf[kk], sc, 0, 0, 0);
      if (kk + kQA < kK) fr[kk % kQA] = frag(kk + kQA);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kQA, 0);
#pragma unroll
    for (int i = 0; i < kK - kQA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kQA, 0);
    __builtin_amdgcn_sched_barrier(0);
    return sc;
  };
  // V waves: P = exp2(S scale log2 e - LSE log2 e) over admitted (row, key)
  // pairs, as bf16 pairs; register r of a lane holds query row 8(r/4) +
  // 4 half + r%4 of the tile at cursor c.  In a tile not wholly admitted, a
  // 32-bit row mask of this lane's key selects the pairs.
  auto make_p = [&](const f32x16& sc, auto bc, const Cursor& c, uint32_t (&pk)[2][4]) {
    const int qt0 = c.qt0, qe = c.end;
    const bool full = qt0 + kQt <= qe && ((qt0 >= f1lo && qt0 + kQt <= f1hi) ||
                                          (qt0 >= f2lo && qt0 + kQt <= f2hi));
    auto rows = [&](bool masked, uint32_t m) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l2v = read_side(bc, r4);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = fast_exp2(fmaf(sc[4 * r4 + e], a.scale_log2, -l2v[e]));
          v[e] = !masked || ((m >> (8 * r4 + e)) & 1u) ? pv : 0.f;
        }
        pk[r4 >> 1][(r4 & 1) * 2 + 0] = pack_bf16x2(v[0], v[1]);
        pk[r4 >> 1][(r4 & 1) * 2 + 1] = pack_bf16x2(v[2], v[3]);
      }
    };
    if (full) {
      rows(false, 0u);
    } else {
      auto bits = [&](int lo, int hi) -> uint64_t {  // rows [lo, hi) of the tile
        const int x = min(max(lo - qt0, 0), 32), y = min(max(hi - qt0, 0), 32);
        return ((1ull << y) - 1) & ~((1ull << x) - 1);
      };
      const uint32_t m =
          (uint32_t)((bits(kr.lo, kr.hi) | bits(kr.lo2, kr.hi2)) & bits(qt0, qe));
      rows(true, m >> (4 * half));
    }
  };
  // acc += X^T Y over the tile's 32 query rows: X (keys on M, queries on K)
  // from the P or dS registers, Y (queries on K, dims on N) from the
  // row-major tile in buffer `buf` (dO or Q) through the transposed read.
  auto accumulate = [&](const uint32_t (&pk)[2][4], auto bc) {
    constexpr int buf = decltype(bc)::value;
    constexpr int kM = 2 * (D / 32);  // MFMA m: c = m / (D/32), dt = m % (D/32)
    constexpr int kAA = 3;        // B operands read kAA MFMAs ahead
    auto frag = [&](int m) {
      const char* bt = tiles_c + buf * kTileBytes + (m / (D / 32)) * 16 * D * 2;
      return tr_pair(bt + toff[m % (D / 32)][0], bt + toff[m % (D / 32)][1]);
    };
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 fr[kAA];
#pragma unroll
    for (int i = 0; i < kAA; ++i) fr[i] = frag(i);
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const int c = m / (D / 32), dt = m % (D / 32);
      const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pk[c][0], pk[c][1], pk[c][2], pk[c][3]});
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, fr[m % kAA], acc[dt], 0, 0, 0);
      if (m + kAA < kM) fr[m % kAA] = frag(m + kAA);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAA, 0);
#pragma unroll
    for (int i = 0; i < kM - kAA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAA, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  uint32_t* const pex = &p_xchg[0][wave & 3][0][lane * 4];
  constexpr int kPexParity = 4 * 2 * 64 * 4;  // words between the two parities
  auto put_p = [&](int parity, const uint32_t (&pk)[2][4]) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
      *reinterpret_cast<u32x4*>(pex + parity * kPexParity + c * 64 * 4) =
          u32x4{pk[c][0], pk[c][1], pk[c][2], pk[c][3]};
  };
  // P(st+1) (bf16 pairs) handed from a step to the next in V waves.
  struct Carry {
    uint32_t w[2][4];
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // Pre-step: P(0) (V waves, also handed over through LDS).
  Carry carry_a = {}, carry_b = {};
  if (nsteps > 0 && !kwave && active(cur)) {
    const f32x16 sc = qk_product(I0{});
    make_p(sc, I0{}, cur, carry_a.w);
    put_p(0, carry_a.w);
  }
  barrier_lds();

  auto step = [&](int st, auto bc, const Carry& cin, Carry& cout) {
    constexpr int b = decltype(bc)::value;  // st % 4
    using B1 = std::integral_constant<int, (b + 1) & 3>;
    // Loads of tile st+3 into the buffer tile st-1 left, issued behind the
    // first MFMAs of the step so that their issue overlaps the MFMA pipe.
    auto issue = [&]() {
      if (st + 3 < nsteps) {
        issue_step(ld, (b + 3) & 3);
        advance(ld);
      }
    };
    const bool act = st < nsteps && active(cur);
    const bool act1 = st + 1 < nsteps && active(nx1);
    // V waves: S(st+1), then dV += P(st)^T dO(st), then P(st+1) (its
    // exponentials overlap the dV products).  K waves: dP(st), dS(st) =
    // P(st) (dP(st) - delta), then dK += dS(st)^T Q(st).  One accumulate
    // for both roles keeps the accumulators in one set of registers.
    f32x16 sc;  // S(st+1) or dP(st)
    uint32_t xw[2][4];
    if (!kwave) {
      if (act1) sc = qk_product(B1{});
      issue();
#pragma unroll
      for (int j = 0; j < 8; ++j) xw[j >> 2][j & 3] = cin.w[j >> 2][j & 3];
    } else if (act) {
      u32x4 pw[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
        pw[c] = *reinterpret_cast<const u32x4*>(pex + (b & 1) * kPexParity + c * 64 * 4);
      sc = qk_product(bc);
      issue();
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 dlv = read_side(bc, r4);
        const uint32_t w0 = pw[r4 >> 1][(r4 & 1) * 2 + 0];
        const uint32_t w1 = pw[r4 >> 1][(r4 & 1) * 2 + 1];
        const float p[4] = {bf16_to_f32(w0 & 0xffffu), bf16_to_f32(w0 >> 16),
                            bf16_to_f32(w1 & 0xffffu), bf16_to_f32(w1 >> 16)};
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = p[e] * (sc[4 * r4 + e] - dlv[e]);
        xw[r4 >> 1][(r4 & 1) * 2 + 0] = pack_bf16x2(v[0], v[1]);
        xw[r4 >> 1][(r4 & 1) * 2 + 1] = pack_bf16x2(v[2], v[3]);
      }
    } else {
      issue();
    }
    if (act) accumulate(xw, bc);
    if (!kwave && act1) {
      make_p(sc, B1{}, nx1, cout.w);
      put_p((b + 1) & 1, cout.w);
    }
    advance(cur);
    advance(nx1);
    // Tile st+2 must have landed; tile st+3 stays in flight across the
    // barrier.
    if (st + 3 < nsteps) wait_all_but_newest();
    else wait_vmem();
    barrier_lds();
  };
  for (int st = 0; st < nsteps; st += 4) {
    step(st, I0{}, carry_a, carry_b);
    step(st + 1, I1{}, carry_b, carry_a);
    step(st + 2, I2{}, carry_a, carry_b);
    step(st + 3, I3{}, carry_b, carry_a);
  }

  // Epilogue: lane holds dims 32 dt + lane%32 of keys 8(r/4) + 4 half + r%4.
  if (!wave_has_keys) return;
  uint16_t* out = kwave ? a.dk : a.dv;
  const float mul = kwave ? a.scale : 1.f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (kr < L) {
        const size_t off = ((size_t)(base + kr) * a.hkv + g) * D + dt * 32 + (lane & 31);
        out[off] = static_cast<uint16_t>(pack_bf16x2(acc[dt][r] * mul, 0.f) & 0xffffu);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ (ping-pong)

template <int D>
struct DqLds {
  uint16_t k[4][kBN * D];  // K(t) in k[t & 3]
  uint16_t v[2][kBN * D];  // V(t) in v[t & 1]
};

template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(BwdArgs a, int hpw, int ntiles_max) {
  __shared__ DqLds<D> lds;
  const int ngroups = a.hq / hpw;
  const int tok = 32 * (8 / hpw);
  // Order as the forward: head group fastest, then one segment's query tiles.
  const int w = blockIdx.x;
  const int hg = w % ngroups;
  const int rest = w / ngroups;
  const int rank = rest % ntiles_max;
  const int seg = rest / ntiles_max;
  const int base = a.cu_seqlens[seg];
  const int L = a.cu_seqlens[seg + 1] - base;
  const int ntiles_q = (L + tok - 1) / tok;
  if (rank >= ntiles_q) return;
  const int tile = ntiles_q - 1 - rank;
  const Stair stair = make_stair(seg, L, a.block_size, a.s_copies, a.group_start, a.group_pe,
                                 a.group_copies);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int head = hg * hpw + wave % hpw;
  const int g = (hg * hpw) / (a.hq / a.hkv);
  const int q0 = tile * tok;
  const int q_last = min(q0 + tok, L) - 1;
  const TileKeys tk = tile_keys(q0, q_last, stair);
  const int qw0 = q0 + (wave / hpw) * 32;
  const int qi = qw0 + (lane & 31);
  const bool wave_active = qw0 < L;
  const int qw_last = min(qw0 + 32, L) - 1;

  const int kv_elems = a.hkv * D;
  const uint16_t* kb = a.k + (size_t)base * kv_elems + (size_t)g * D;
  const uint16_t* vb = a.v + (size_t)base * kv_elems + (size_t)g * D;
  const int n1 = (tk.r1e + kBN - 1) / kBN;
  const int n2 = tk.r2e > tk.r2s ? (tk.r2e - tk.r2s + kBN - 1) / kBN : 0;
  const int ntile = n1 + n2;
  auto tile_k0 = [&](int t) { return t < n1 ? t * kBN : tk.r2s + (t - n1) * kBN; };
  auto tile_end = [&](int t) { return t < n1 ? tk.r1e : tk.r2e; };

  // DMA, by the four waves of group A only: a kBN x D tile is kInstPerTensor
  // 1 KB instructions per tensor; wave w issues instructions w + 4 j.
  constexpr int kChunks = D / 8;
  constexpr int kRowsPerInst = 64 / kChunks;
  constexpr int kInstPerTensor = kBN / kRowsPerInst;  // 8 (D=128) or 4 (D=64)
  constexpr int kInstPerWave = kInstPerTensor / 4;
  uint32_t dvoff[kInstPerWave];
  int drow0[kInstPerWave];
#pragma unroll
  for (int j = 0; j < kInstPerWave; ++j) {
    drow0[j] = ((wave & 3) + 4 * j) * kRowsPerInst;
    const int R = drow0[j] + lane / kChunks;
    dvoff[j] = (uint32_t)(R * kv_elems * 2 + (((lane % kChunks) ^ swz<D>(R)) * 16));
  }
  auto issue = [&](const uint16_t* src, int t, uint16_t* dst) {
    const int k0 = tile_k0(t);
    const int rows = min(tile_end(t) - k0, kBN);
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(src + (size_t)k0 * kv_elems, (uint32_t)((rows - 1) * kv_elems * 2 + D * 2));
#pragma unroll
    for (int j = 0; j < kInstPerWave; ++j) buffer_load_lds16(r, dst + drow0[j] * D, dvoff[j]);
  };
  if (ntile > 0 && grp == 0) {
    issue(kb, 0, lds.k[0]);
    issue(vb, 0, lds.v[0]);
  }

  bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 rq = u32x4{0, 0, 0, 0}, rg = u32x4{0, 0, 0, 0};
    if (qi < L) {
      const size_t off = ((size_t)(base + qi) * a.hq + head) * D + kk * 16 + half * 8;
      rq = *reinterpret_cast<const u32x4*>(a.q + off);
      rg = *reinterpret_cast<const u32x4*>(a.dout + off);
    }
    qf[kk] = __builtin_bit_cast(bf16x8, rq);
    gf[kk] = __builtin_bit_cast(bf16x8, rg);
  }
  float lse2 = 0.f, dl = 0.f;
  if (qi < L) {
    lse2 = a.lse[(size_t)head * a.total + base + qi] * kLog2e;
    dl = a.delta[(size_t)head * a.total + base + qi];
  }
  const RowKeys rk = row_keys(qi < L ? qi : qw_last, stair);
  const RowKeys rkA = row_keys(wave_active ? qw0 : 0, stair);
  const RowKeys rkB = row_keys(wave_active ? qw_last : 0, stair);
  const bool one_copy = rkA.e2 > rkA.s2 && rkA.s2 == rkB.s2;
  // every row of the wave sees the clean keys [0, e1_all)
  const int e1_all = wave_active ? min_prefix_end(qw0, qw_last, stair) : 0;

  uint32_t koff[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = row_frag_off<D>(lane, kk);
  uint32_t toff[D / 32][2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    toff[dt][0] = tr_off<D>(lane, dt, 0);
    toff[dt][1] = tr_off<D>(lane, dt, 1);
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

  if (ntile > 0) {
    wait_vmem();
    __syncthreads();
    f32x16 s[kBN / 32], dp[kBN / 32];
    // dS^T of the tile between its VALU and dQ phases; zero before the first
    uint32_t pk[kBN / 16][4] = {};
    // MFMA phase t: dQ^T += K^T dS^T of tile t-1 and S^T, dP^T of tile t.
    // Every phase runs the same straight-line code (a second code path
    // pushes the kernel past its register budget): in phase 0 the dQ^T
    // MFMAs add K^T times the zero dS^T (K of tile 0, finite), and in phase
    // ntile the S^T and dP^T of stale tile memory are computed and dropped.
    // The MFMAs run dQ^T first (dS^T(t-1) is dead before S^T(t) and dP^T(t)
    // are live), then S^T and dP^T alternating; the LDS operands of each
    // MFMA (two transposed K reads for dQ^T, one K or V read otherwise) are
    // read kAh MFMAs ahead, so LDS latency hides behind the MFMAs between.
    auto mfma_phase = [&](int kti, int kdi, int vti) {
      const char* kd = reinterpret_cast<const char*>(lds.k[kdi]);
      const char* kt = reinterpret_cast<const char*>(lds.k[kti]);
      const char* vt = reinterpret_cast<const char*>(lds.v[vti]);
      constexpr int kN = D / 16;   // dQ^T MFMAs = S^T MFMAs = dP^T MFMAs
      constexpr int kM = 3 * kN;   // MFMAs of the phase
      constexpr int kAh = 3;
      static_assert(kBN == 32, "one S^T / dP^T accumulator per tile");
      static_assert(kAh <= kN, "lookahead within the dQ^T MFMAs");
      // MFMA m: m < kN is dQ^T MFMA m (c = m / (D/32), dt = m % (D/32)),
      // then S^T and dP^T alternate over kk = (m - kN) / 2.
      auto frag = [&](int m) {
        if (m < kN) {
          const int c = m / (D / 32), dt = m % (D / 32);
          return tr_pair(kd + toff[dt][0] + c * 16 * D * 2, kd + toff[dt][1] + c * 16 * D * 2);
        }
        const int kk = (m - kN) / 2;
        return *reinterpret_cast<const bf16x8*>(((m - kN) % 2 ? vt : kt) + koff[kk]);
      };
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 fr[kAh];
#pragma unroll
      for (int m = 0; m < kAh; ++m) fr[m] = frag(m);
      s[0] = f32x16{};
      dp[0] = f32x16{};
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        if (m < kN) {
          const int c = m / (D / 32), dt = m % (D / 32);
          const bf16x8 db = __builtin_bit_cast(bf16x8, u32x4{pk[c][0], pk[c][1], pk[c][2], pk[c][3]});
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % kAh], db, acc[dt], 0, 0, 0);
        } else if ((m - kN) % 2 == 0) {
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % kAh], qf[(m - kN) / 2], s[0], 0, 0, 0);
        } else {
          dp[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % kAh], gf[(m - kN) / 2], dp[0], 0, 0, 0);
        }
        if (m + kAh < kM) fr[m % kAh] = frag(m + kAh);
      }
      // issue order: the reads of the first kAh MFMAs (two per dQ^T MFMA),
      // then each MFMA followed by the reads of the MFMA kAh later (group
      // masks: 0x100 LDS read, 0x008 MFMA)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAh, 0);
#pragma unroll
      for (int m = 0; m < kN - kAh; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int m = kN - kAh; m < kM - kAh; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kAh, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    // VALU phase of tile t: P^T and dS^T.  Masked scores are set to -inf
    // first (only in tiles not wholly admitted for the wave), so that the
    // loop below is straight-line code: P = 0 there, and with it dS.
    auto valu_phase = [&](int t) {
      const int k0 = tile_k0(t), kend = tile_end(t);
      const bool full = wave_active && (k0 + kBN <= kend) &&
                        ((k0 + kBN <= e1_all) ||
                         (one_copy && k0 >= rkA.s2 && k0 + kBN <= rkA.e2));
      if (!full) {
#pragma unroll
        for (int h = 0; h < kBN / 32; ++h) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = k0 + h * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool ok = (j < kend) & ((j < rk.e1) | ((j >= rk.s2) & (j < rk.e2)));
            s[h][r] = ok ? s[h][r] : kNegInf;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kBN / 32; ++h) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float dsv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float p = fast_exp2(fmaf(s[h][r + e], a.scale_log2, -lse2));
            dsv[e] = p * (dp[h][r + e] - dl);
          }
          pk[h * 2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(dsv[0], dsv[1]);
        }
      }
    };
    // Group A's loads in phase 2t, after its own LDS reads: K and V of tile t+1.
    // The barrier closing phase 2t leaves them in flight; A waits for them at
    // the end of phase 2t+1.
    auto issue_next = [&](int t) {
      if (t + 1 < ntile) {
        issue(kb, t + 1, lds.k[(t + 1) & 3]);
        issue(vb, t + 1, lds.v[(t + 1) & 1]);
      }
    };
    // Two groups one phase apart, each in its own straight-line loop (as the
    // forward): A runs MFMA(t) then VALU(t), B runs VALU(t-1) then MFMA(t);
    // every iteration passes two barriers in both groups.  The loops are
    // unrolled by four, so the buffers each phase reads -- K(t) in k[t & 3],
    // K(t-1) in k[(t-1) & 3], V(t) in v[t & 1] -- are constants in the code
    // and every LDS address is a lane offset plus an immediate; phase 0
    // takes its dQ^T operand from k[0] (tile 0; dS^T is zero there).
    auto phase_a = [&](int t, int kti, int kdi, int vti) {
      mfma_phase(kti, kdi, vti);
      issue_next(t);
      barrier_lds();
      if (t < ntile) valu_phase(t);
      wait_vmem_barrier();
    };
    auto phase_b = [&](int t, int kti, int kdi, int vti) {
      if (t >= 1) valu_phase(t - 1);
      barrier_lds();
      mfma_phase(kti, kdi, vti);
      barrier_lds();
    };
    auto run = [&](auto&& phase) {
      phase(0, 0, 0, 0);
      int t = 1;
      for (; t + 3 <= ntile; t += 4) {
        phase(t, 1, 0, 1);
        phase(t + 1, 2, 1, 0);
        phase(t + 2, 3, 2, 1);
        phase(t + 3, 0, 3, 0);
      }
      for (; t <= ntile; ++t) phase(t, t & 3, (t - 1) & 3, t & 1);
    };
    if (grp == 0) {
      run(phase_a);
    } else {
      run(phase_b);
    }
  }

  if (!(qi < L)) return;
  uint16_t* dst = a.dq + ((size_t)(base + qi) * a.hq + head) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = dt * 32 + 8 * gq + 4 * half;
      *reinterpret_cast<u32x2*>(dst + d) =
          u32x2{pack_bf16x2(acc[dt][4 * gq] * a.scale, acc[dt][4 * gq + 1] * a.scale),
                pack_bf16x2(acc[dt][4 * gq + 2] * a.scale, acc[dt][4 * gq + 3] * a.scale)};
    }
  }
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int max_seqlen, hipStream_t stream) {
  if (a.nseq <= 0 || a.total <= 0) return hipSuccess;
  // 1. delta
  {
    const long long nrows = (long long)a.total * a.hq;
    const int rows_per_wg = 256 / (a.d / 8);
    const long long nwg = (nrows + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)nwg), dim3(256), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // 2. dK, dV
  {
    const long long nkt = (max_seqlen + kKvKeys - 1) / kKvKeys;
    const long long nwg = nkt * a.nseq * a.hkv;
    if (a.d == 128) {
      hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3((unsigned)nwg), dim3(512), 0, stream, a,
                         (int)nkt);
    } else {
      hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3((unsigned)nwg), dim3(512), 0, stream, a,
                         (int)nkt);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // 3. dQ
  {
    const int hpw = heads_per_wg(a.hq, a.hkv);
    const int tok = 32 * (8 / hpw);
    const long long ntiles = (max_seqlen + tok - 1) / tok;
    const long long nwg = ntiles * a.nseq * (a.hq / hpw);
    if (a.d == 128) {
      hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3((unsigned)nwg), dim3(512), 0, stream, a, hpw,
                         (int)ntiles);
    } else {
      hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3((unsigned)nwg), dim3(512), 0, stream, a, hpw,
                         (int)ntiles);
    }
    return hipGetLastError();
  }
}

}  // namespace bca
