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
//   2. dK/dV (bwd_dkdv_kernel, used for head_dim 64; bwd_dkdv_pp_kernel, the
//      same roles in a two-phase ping-pong over 64-row steps, for head_dim
//      128): an 8-wave workgroup owns 128 keys of one KV head.  Waves 0-3
//      ("V waves", 32 keys each) compute S = Q K^T -> P and dV += P^T dO;
//      waves 4-7 ("K waves", the same keys) compute dP = dO V^T, take P from
//      their V wave through LDS, form dS and dK += dS^T Q.  S is computed
//      once, and each SIMD pairs one wave of each kind.  In bwd_dkdv_kernel
//      each wave issues its own elementwise work between its MFMAs: a V wave the
//      exponentials of the next tile between its dV MFMAs, a K wave the dS
//      of the current tile between the MFMAs of the next tile's dP.  K and V
//      fragments and the dK/dV accumulators stay in registers; each step
//      streams a 32-row (ping-pong: 64-row) tile of Q and dO of one query head
//      through LDS, loaded straight from HBM two or three steps ahead.  S is computed with queries on the
//      M axis, so the P and dS accumulators are, unchanged, the A operands of
//      the dV and dK products; their B operands (dO and Q with queries on K)
//      come from the row-major tiles through the transposed LDS read.
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

// One workgroup takes kDeltaPasses x (256 / (d/8)) consecutive query rows of
// one head (d/8 lanes per row, 16 bytes each), all loads issued before any
// arithmetic so that every lane has 2 kDeltaPasses loads in flight; the rows
// it writes are consecutive in the [hq, total] side arrays.  Workgroups are
// ordered head fastest, so neighbouring workgroups read neighbouring bytes
// of the token-major O and dO.
constexpr int kDeltaPasses = 4;

__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  const int d = a.d;
  const int lanes_per_row = d / 8;                     // 16 (d = 128) or 8 (d = 64)
  const int rows_per_pass = 256 / lanes_per_row;       // 16 or 32
  const int h = (int)(blockIdx.x % (unsigned)a.hq);
  const long long i0 = (long long)(blockIdx.x / (unsigned)a.hq) * rows_per_pass * kDeltaPasses;
  const int sub = threadIdx.x % lanes_per_row;
  const int r = threadIdx.x / lanes_per_row;
  u32x4 o[kDeltaPasses], g[kDeltaPasses];
#pragma unroll
  for (int p = 0; p < kDeltaPasses; ++p) {
    const long long i = i0 + p * rows_per_pass + r;
    o[p] = g[p] = u32x4{0, 0, 0, 0};
    if (i < a.total) {
      const size_t off = ((size_t)i * a.hq + h) * d + sub * 8;
      o[p] = *reinterpret_cast<const u32x4*>(a.o + off);
      g[p] = *reinterpret_cast<const u32x4*>(a.dout + off);
    }
  }
#pragma unroll
  for (int p = 0; p < kDeltaPasses; ++p) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16_to_f32(o[p][w] & 0xffffu), bf16_to_f32(g[p][w] & 0xffffu), acc);
      acc = fmaf(bf16_to_f32(o[p][w] >> 16), bf16_to_f32(g[p][w] >> 16), acc);
    }
    for (int off = lanes_per_row / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    const long long i = i0 + p * rows_per_pass + r;
    if (i < a.total && sub == 0) {
      a.delta[(size_t)h * a.total + i] = acc;
      a.lse2[(size_t)h * a.total + i] = a.lse[(size_t)h * a.total + i] * kLog2e;
    }
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
  // holds a step's tile t (in sweep order) and head h within the group; the
  // tile's first row and the end of its range follow by selects, so the step
  // loop has no data-dependent branches (a taken branch costs a SIMD about
  // as much as several MFMA issue slots).  Rows of a tile past the end are
  // loaded as zeros and masked.
  struct Cursor {
    int t, h;
  };
  const int row0_r2 = qs2 + (nqt2 - 1) * kQt;         // tile t of range 2: row0_r2 - 32 t
  const int row0_r1 = qs1 + (nqt1 - 1 + nqt2) * kQt;  // tile t of range 1: row0_r1 - 32 t
  auto tile_row0 = [&](int t) { return (t < nqt2 ? row0_r2 : row0_r1) - t * kQt; };
  auto tile_end = [&](int t) { return t < nqt2 ? qe2 : qe1; };
  auto advance = [&](Cursor& c) {
    const int h1 = c.h + 1;
    const bool wrap = h1 == group;
    c.h = wrap ? 0 : h1;
    c.t += wrap ? 1 : 0;
  };
  const uint32_t tiles_lds = lds_addr_of(&tiles[0][0]);
  // Side values: wave 0 loads the tile's LSE * log2(e) rows, wave 4 its delta
  // rows (every load instruction costs the issuing wave address-unit time, so
  // the other waves issue none and wait for one load fewer).
  const bool side_real = wave == 0 || wave == 4;
  const float* const side_src = wave == 0 ? a.lse2 : a.delta;
  const uint32_t side_dst = lds_addr_of(&lds.v[0][wave == 0 ? 0 : 1][0]);
  // A step past the last issues zero-length loads: they write zeros to a
  // buffer that only steps past the last read.
  auto issue_step = [&](const Cursor& c, int buf, bool valid) {
    const int qt0 = valid ? tile_row0(c.t) : 0;
    const int head = g * group + c.h;
    const int rows = valid ? min(tile_end(c.t) - qt0, kQt) : 0;
    const uint32_t nbytes = rows > 0 ? (uint32_t)((rows - 1) * q_row_elems * 2 + D * 2) : 0u;
    const size_t off = (size_t)(base + qt0) * q_row_elems + (size_t)head * D;
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      const i32x4 r = rsrc_words((dma_is_q[j] ? a.q : a.dout) + off, nbytes);
      const uint32_t dst = tiles_lds + (uint32_t)(buf * kTileBytes) +
                           (dma_is_q[j] ? 0u : (uint32_t)(kQt * D * 2)) +
                           (uint32_t)(dma_row0[j] * D * 2);
      buffer_load_lds16_asm(r, dst, dma_voff[j]);
    }
    if (side_real) {
      const size_t so = (size_t)head * a.total + base + qt0;
      buffer_load_lds4_asm(rsrc_words(side_src + so, (uint32_t)(rows * 4)),
                           side_dst + (uint32_t)(buf * 2 * 64 * 4), (uint32_t)lane * 4);
    }
  };
  // Wait until only the newest step's loads may be outstanding.
  auto wait_all_but_newest = [&]() {
    if (side_real) wait_vmem_le<kDmaPerWave + 1>();
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
  // (bitwise & and |: short-circuit operators become branches)
  auto active = [&](int qt0) {
    return wave_has_keys &
           (((qt0 < w1hi) & (qt0 + kQt > w1lo)) | ((qt0 < w2hi) & (qt0 + kQt > w2lo)));
  };

  // Tiles: tile t (a step's Q and dO rows with their side values) lives in
  // buffer t % 4; tiles 0-2 are loaded before the loop and step st loads
  // tile st+3 into the buffer tile st-1 left.
  Cursor ld = Cursor{0, 0};
  issue_step(ld, 0, nsteps > 0);
  advance(ld);
  issue_step(ld, 1, nsteps > 1);
  advance(ld);
  issue_step(ld, 2, nsteps > 2);
  advance(ld);
  // Everything landed, the K/V fragments included: the compiler does not
  // count the direct loads, so a partial wait here would leave it waiting
  // for those fragments (and with them every load in flight) inside the loop.
  wait_vmem();
  barrier_lds();

  // S = Q K^T (V waves) or dP = dO V^T (K waves) of the tile in buffer
  // `buf`, queries on M, keys on N; A fragments read kQA MFMAs ahead of use
  // (the scheduling groups pin that order; left alone, the compiler reads one
  // ahead).
  auto qk_product = [&](auto bc) {
    constexpr int buf = decltype(bc)::value;
    uint32_t r0 = roff0;
    asm volatile("" : "+v"(r0));
    auto frag = [&](int kk) {
      return *reinterpret_cast<const bf16x8*>(tiles_c + buf * kTileBytes + (r0 ^ (32u * kk)));
    };
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
  // acc += X^T Y over the tile's 32 query rows: X (keys on M, queries on K)
  // from the P or dS words, Y (queries on K, dims on N) from the row-major
  // tile in buffer `buf` (dO or Q) through the transposed read, its
  // fragments read kAA MFMAs ahead.  chunk(j), j = 0..7, is VALU work
  // independent of these MFMAs, issued in order behind them (8 / kM chunks
  // after each MFMA; scheduling fences keep the order), so that it runs
  // while the MFMA pipe is busy instead of after it.
  auto accumulate = [&](f32x16 (&acc)[D / 32], const uint32_t (&xw)[2][4], auto bc,
                        auto&& chunk) {
    constexpr int buf = decltype(bc)::value;
    constexpr int kM = 2 * (D / 32);  // MFMA m: c = m / (D/32), dt = m % (D/32)
    constexpr int kAA = 3;
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
      const bf16x8 xa = __builtin_bit_cast(bf16x8, u32x4{xw[c][0], xw[c][1], xw[c][2], xw[c][3]});
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, fr[m % kAA], acc[dt], 0, 0, 0);
      if (m + kAA < kM) fr[m % kAA] = frag(m + kAA);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = m * 8 / kM; j < (m + 1) * 8 / kM; ++j) chunk(j);  // 8 words in all
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The side values of this lane's accumulator rows 8 r4 + 4 half + 0..3 of
  // the tile in buffer `buf`: LSE * log2(e) (V waves) or delta (K waves).
  auto read_side = [&](auto bc, int r4) {
    constexpr int buf = decltype(bc)::value;
    return *reinterpret_cast<const f32x4*>(&lds.v[buf][kwave ? 1 : 0][8 * r4 + 4 * half]);
  };
  // P of tile `c` from its scores (V waves): exp2(S scale log2(e) - LSE
  // log2(e)) over admitted (row, key) pairs, bf16 pairs; register r of a
  // lane holds query row 8(r/4) + 4 half + r%4.  A tile not wholly admitted
  // selects the pairs with a 32-bit row mask of this lane's key; a tile
  // that sees none of the wave's keys (or past the last step) gets P = 0.
  // p_mask gives the mask, p_word(j) one packed word (registers 2j, 2j+1).
  auto p_mask = [&](const Cursor& c, bool valid) -> uint32_t {
    const int qt0 = tile_row0(c.t), qe = tile_end(c.t);
    const bool act = valid & active(qt0);
    const bool full = act & (qt0 + kQt <= qe) &
                      (((qt0 >= f1lo) & (qt0 + kQt <= f1hi)) | ((qt0 >= f2lo) & (qt0 + kQt <= f2hi)));
    auto bits = [&](int lo, int hi) -> uint64_t {  // rows [lo, hi) of the tile
      const int x = min(max(lo - qt0, 0), 32), y = min(max(hi - qt0, 0), 32);
      return ((1ull << y) - 1) & ~((1ull << x) - 1);
    };
    const uint32_t m = (uint32_t)((bits(kr.lo, kr.hi) | bits(kr.lo2, kr.hi2)) & bits(qt0, qe));
    return full ? 0xffffffffu : (act ? m >> (4 * half) : 0u);
  };
  auto p_word = [&](const f32x16& sc, const f32x4 (&side)[4], uint32_t m, int j) {
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * j + e;
      const float pv = fast_exp2(fmaf(sc[r], a.scale_log2, -side[r >> 2][r & 3]));
      v[e] = ((m >> (8 * (r >> 2) + (r & 3))) & 1u) ? pv : 0.f;
    }
    return pack_bf16x2(v[0], v[1]);
  };
  uint32_t* const pex = &p_xchg[0][wave & 3][0][lane * 4];
  constexpr int kPexParity = 4 * 2 * 64 * 4;  // words between the two parities
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  f32x16 acc[D / 32];  // dV (V waves) or dK (K waves): keys on M, dims on N
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

  // The two roles run separate loops with one barrier per step each (the
  // same count), so each keeps only its own live registers and its
  // accumulator has one definition per step.  Steps past the last run the
  // same code on zero P (their tiles are zero-length loads), which adds
  // nothing.  The loops run in groups of four steps: buffer offsets are
  // compile-time constants and the carried registers alternate.
  if (!kwave) {
    // V waves, step st: S(st+1) = Q(st+1) K^T; dV += P(st)^T dO(st) with the
    // exponentials of P(st+1) between those MFMAs; P(st+1) to the K wave.
    struct Carry {
      uint32_t w[2][4];
    };
    Carry pa = {}, pb = {};
    Cursor cur = Cursor{0, 0};  // tile st
    {
      const f32x16 sc = qk_product(I0{});
      f32x4 side[4];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) side[r4] = read_side(I0{}, r4);
      const uint32_t m = p_mask(cur, nsteps > 0);
#pragma unroll
      for (int j = 0; j < 8; ++j) pa.w[j >> 2][j & 3] = p_word(sc, side, m, j);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        *reinterpret_cast<u32x4*>(pex + c * 64 * 4) =
            u32x4{pa.w[c][0], pa.w[c][1], pa.w[c][2], pa.w[c][3]};
    }
    barrier_lds();
    auto step = [&](int st, auto bc, const Carry& pin, Carry& pout) {
      constexpr int b = decltype(bc)::value;  // st % 4
      using B1 = std::integral_constant<int, (b + 1) & 3>;
      Cursor nx = cur;
      advance(nx);
      f32x4 side[4];  // read before the MFMAs they are scheduled among
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) side[r4] = read_side(B1{}, r4);
      const f32x16 sc = qk_product(B1{});
      issue_step(ld, (b + 3) & 3, st + 3 < nsteps);
      advance(ld);
      const uint32_t m = p_mask(nx, st + 1 < nsteps);
      accumulate(acc, pin.w, bc,
                 [&](int j) {
                   uint32_t word = p_word(sc, side, m, j);
                   asm volatile("" : "+v"(word));  // keep it among the MFMAs
                   pout.w[j >> 2][j & 3] = word;
                 });
#pragma unroll
      for (int c = 0; c < 2; ++c)
        *reinterpret_cast<u32x4*>(pex + ((b + 1) & 1) * kPexParity + c * 64 * 4) =
            u32x4{pout.w[c][0], pout.w[c][1], pout.w[c][2], pout.w[c][3]};
      cur = nx;
      wait_all_but_newest();
      barrier_lds();
    };
    for (int st = 0; st < nsteps; st += 4) {
      step(st, I0{}, pa, pb);
      step(st + 1, I1{}, pb, pa);
      step(st + 2, I2{}, pa, pb);
      step(st + 3, I3{}, pb, pa);
    }
  } else {
    // K waves, step st: dP(st+1) = dO(st+1) V^T with dS(st) = P(st)
    // (dP(st) - delta) between those MFMAs; dK += dS(st)^T Q(st).
    f32x16 dpa = qk_product(I0{}), dpb = f32x16{};  // dP(0)
    barrier_lds();
    auto step = [&](int st, auto bc, const f32x16& dp_in, f32x16& dp_out) {
      constexpr int b = decltype(bc)::value;
      using B1 = std::integral_constant<int, (b + 1) & 3>;
      u32x4 pw[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
        pw[c] = *reinterpret_cast<const u32x4*>(pex + (b & 1) * kPexParity + c * 64 * 4);
      f32x4 side[4];  // read before the MFMAs they are scheduled among
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) side[r4] = read_side(bc, r4);
      uint32_t xw[2][4];
      // dP(st+1) MFMAs with dS(st) between them: after MFMA j, word j of
      // dS(st) = P(st) (dP(st) - delta) (registers 2j, 2j+1)
      {
        uint32_t r0 = roff0;
        asm volatile("" : "+v"(r0));
        auto frag = [&](int kk) {
          return *reinterpret_cast<const bf16x8*>(tiles_c + B1::value * kTileBytes +
                                                  (r0 ^ (32u * kk)));
        };
        constexpr int kQA = 4;
        constexpr int kK = D / 16;
        static_assert(kK == 8 || kK == 4, "dS words per MFMA");
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 fr[kQA];
#pragma unroll
        for (int i = 0; i < kQA; ++i) fr[i] = frag(i);
        f32x16 dpn = f32x16{};
        auto ds_word = [&](int j) {
          const uint32_t w = pw[j >> 2][j & 3];
          const float p0 = bf16_to_f32(w & 0xffffu), p1 = bf16_to_f32(w >> 16);
          const int r = 2 * j;
          const float v0 = p0 * (dp_in[r] - side[r >> 2][r & 3]);
          const float v1 = p1 * (dp_in[r + 1] - side[(r + 1) >> 2][(r + 1) & 3]);
          uint32_t word = pack_bf16x2(v0, v1);
          asm volatile("" : "+v"(word));  // keep it here: IR passes sink it to its use
          xw[j >> 2][j & 3] = word;
        };
#pragma unroll
        for (int kk = 0; kk < kK; ++kk) {
          dpn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[kk % kQA], kvf[kk], dpn, 0, 0, 0);
          if (kk + kQA < kK) fr[kk % kQA] = frag(kk + kQA);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = kk * 8 / kK; j < (kk + 1) * 8 / kK; ++j) ds_word(j);
          __builtin_amdgcn_sched_barrier(0);
        }
        dp_out = dpn;
      }
      issue_step(ld, (b + 3) & 3, st + 3 < nsteps);
      advance(ld);
      accumulate(acc, xw, bc, [](int) {});
      wait_all_but_newest();
      barrier_lds();
    };
    for (int st = 0; st < nsteps; st += 4) {
      step(st, I0{}, dpa, dpb);
      step(st + 1, I1{}, dpb, dpa);
      step(st + 2, I2{}, dpa, dpb);
      step(st + 3, I3{}, dpb, dpa);
    }
  }

  // Epilogue: lane holds dims 32 dt + lane%32 of keys 8(r/4) + 4 half + r%4.
  if (!wave_has_keys) return;
  uint16_t* out = kwave ? a.dk : a.dv;
  const float mul = kwave ? a.scale : 1.f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr2 = kw0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (kr2 < L) {
        const size_t off = ((size_t)(base + kr2) * a.hkv + g) * D + dt * 32 + (lane & 31);
        out[off] = static_cast<uint16_t>(pack_bf16x2(acc[dt][r] * mul, 0.f) & 0xffffu);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2b. dK / dV, ping-pong (head_dim 128): the roles of the kernel above (V
// waves and K waves of 32 keys each, one of each per SIMD), over 64-row steps
// and in two phases per step, as the forward's wave groups:
//   phase 1: V waves  S(t) = Q(t) K^T and dV += P(t-1)^T dO(t-1)   (32 MFMAs)
//            K waves  dS(t-1) = P(t-1) (dP(t-1) - delta)           (VALU)
//   phase 2: K waves  dP(t) = dO(t) V^T and dK += dS(t-1)^T Q(t-1) (32 MFMAs)
//            V waves  P(t) from S(t), handed to the K waves in LDS (VALU)
// so each SIMD issues MFMAs in both phases, 32 per wave per phase (with
// 32-row steps a phase held 16, too few to cover the LDS latency at its
// start).  Tiles t-1 and t are read in step t; tile t+2 is loaded during it,
// all by the K waves, into the buffer tile t-2 left, and they wait for tile
// t+1 at the end of the step.
constexpr int kQt2 = 64;  // query rows per ping-pong step

template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_pp_kernel(BwdArgs a, int nkt_max) {
  static_assert(D == 128, "ping-pong dK/dV kernel is for head_dim 128");
  constexpr int kTileBytes = 2 * kQt2 * D * 2;  // Q rows then dO rows
  constexpr uint32_t kGOff = kQt2 * D * 2;
  constexpr int kK = D / 16;   // 16-dim chunks
  constexpr int kDT = D / 32;  // 32-dim tiles of dK / dV
  __shared__ __attribute__((aligned(16))) uint16_t tiles[4][2 * kQt2 * D];
  __shared__ KvSide lds;
  // P(t) of V wave h for K wave h: [h][mb][c][lane] (u32x4 = 8 bf16)
  __shared__ __attribute__((aligned(16))) u32x4 p_xchg[4][2][2][64];
  const int group = a.hq / a.hkv;
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
  const bool kwave = wave >= 4;
  const int kw0 = k0 + (wave & 3) * 32;
  const int key = kw0 + (lane & 31);
  const int k_last_wg = min(k0 + kKvKeys, L) - 1;

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
  const int nqt1 = (qe1 - qs1 + kQt2 - 1) / kQt2;
  const int nqt2 = qe2 > qs2 ? (qe2 - qs2 + kQt2 - 1) / kQt2 : 0;
  const int nsteps = (nqt1 + nqt2) * group;

  // Loads, all by the K waves (load issue in the V waves' phase 2, the longer
  // one, lengthened the step): a tile is 16 1 KB instructions per tensor, four
  // per K wave for each of Q and dO; wave 4 also loads the tile's delta rows,
  // wave 5 its LSE * log2(e) rows.  A K wave issues the side rows and its Q
  // rows in phase 1 and its dO rows after its MFMA phase, where it would
  // otherwise wait.
  constexpr int kChunks = D / 8;
  constexpr int kRowsPerInst = 64 / kChunks;  // 4
  constexpr int kDmaPerWave = kQt2 / kRowsPerInst / 4;  // 4
  const int q_row_elems = a.hq * D;
  uint32_t dma_voff[kDmaPerWave];
  int dma_row0[kDmaPerWave];
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    dma_row0[j] = ((wave & 3) + 4 * j) * kRowsPerInst;
    const int R = dma_row0[j] + lane / kChunks;
    const int c = (lane % kChunks) ^ swz<D>(R);
    dma_voff[j] = (uint32_t)(R * q_row_elems * 2 + c * 16);
  }
  struct Cursor {
    int t, h;
  };
  const int row0_r2 = qs2 + (nqt2 - 1) * kQt2;
  const int row0_r1 = qs1 + (nqt1 - 1 + nqt2) * kQt2;
  auto tile_row0 = [&](int t) { return (t < nqt2 ? row0_r2 : row0_r1) - t * kQt2; };
  auto tile_end = [&](int t) { return t < nqt2 ? qe2 : qe1; };
  auto advance = [&](Cursor& c) {
    const int h1 = c.h + 1;
    const bool wrap = h1 == group;
    c.h = wrap ? 0 : h1;
    c.t += wrap ? 1 : 0;
  };
  const uint32_t tiles_lds = lds_addr_of(&tiles[0][0]);
  const bool side_real = wave == 4 || wave == 5;
  const float* const side_src = wave == 5 ? a.lse2 : a.delta;
  const uint32_t side_dst = lds_addr_of(&lds.v[0][wave == 5 ? 0 : 1][0]);
  // Part `part` of this K wave's share of a step's loads (tile of cursor c
  // into buffer buf): part 0 (in phase 1) the side rows of waves 4 and 5
  // first, then the Q rows; part 1 the dO rows (after the MFMA phase, where
  // the K waves have time to spare).
  auto issue_part = [&](const Cursor& c, int buf, bool valid, int part) {
    const int qt0 = valid ? tile_row0(c.t) : 0;
    const int head = g * group + c.h;
    const int rows = valid ? min(tile_end(c.t) - qt0, kQt2) : 0;
    const uint32_t nbytes = rows > 0 ? (uint32_t)((rows - 1) * q_row_elems * 2 + D * 2) : 0u;
    const size_t off = (size_t)(base + qt0) * q_row_elems + (size_t)head * D;
    if (side_real & (part == 0)) {
      const size_t so = (size_t)head * a.total + base + qt0;
      buffer_load_lds4_asm(rsrc_words(side_src + so, (uint32_t)(rows * 4)),
                           side_dst + (uint32_t)(buf * 2 * 64 * 4), (uint32_t)lane * 4);
    }
    const uint32_t dst0 = tiles_lds + (uint32_t)(buf * kTileBytes) + (part ? kGOff : 0u);
    const i32x4 r = rsrc_words((part ? a.dout : a.q) + off, nbytes);
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j)
      buffer_load_lds16_asm(r, dst0 + (uint32_t)(dma_row0[j] * D * 2), dma_voff[j]);
  };
  // K waves, end of step t: tile t+1 landed.  Only the newest step's Q and
  // dO rows may still be outstanding; its side rows, issued before them, have
  // landed too, so tile t+2's LSE rows are readable from step t+1 on.
  auto wait_all_but_newest = [&]() { wait_vmem_le<2 * kDmaPerWave>(); };

  // K fragments (V waves, B operand of S) or V fragments (K waves, of dP).
  bf16x8 kvf[kK];
  {
    const uint16_t* src = kwave ? a.v : a.k;
#pragma unroll
    for (int kk = 0; kk < kK; ++kk) {
      u32x4 r = u32x4{0, 0, 0, 0};
      if (key < L) {
        const size_t off = ((size_t)(base + key) * a.hkv + g) * D + kk * 16 + half * 8;
        r = *reinterpret_cast<const u32x4*>(src + off);
      }
      kvf[kk] = __builtin_bit_cast(bf16x8, r);
    }
  }
  // A fragments of S / dP: Q rows (V waves) or dO rows (K waves); transposed
  // B fragments of dV / dK: dO (V waves) or Q (K waves).
  const uint32_t roff0 = row_frag_off<D>(lane, 0) + (kwave ? kGOff : 0u);
  uint32_t toff[kDT][2];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    toff[dt][0] = tr_off<D>(lane, dt, 0) + (kwave ? 0u : kGOff);
    toff[dt][1] = tr_off<D>(lane, dt, 1) + (kwave ? 0u : kGOff);
  }
  const char* const tiles_c = reinterpret_cast<const char*>(&tiles[0][0]);

  const int wave_key_last = min(kw0 + 31, L - 1);
  const bool wave_has_keys = kw0 < L;
  KeyRows kr = KeyRows{0, 0, 0, 0};
  if (key < L) kr = key_rows(key, stair);
  int w1lo = 0, w1hi = 0, w2lo = 0, w2hi = 0, f1lo = 0, f1hi = 0, f2lo = 0, f2hi = 0;
  if (wave_has_keys) {
    const KeyRows first = key_rows(kw0, stair), last = key_rows(wave_key_last, stair);
    if (kw0 < P) {
      w1lo = first.lo;
      w1hi = wave_key_last >= P ? max(first.hi, last.hi) : first.hi;
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
  // Row mask of this lane's key over the 64 rows of tile c: bit 16 mb + r for
  // row 32 mb + 8 (r/4) + 4 half + r%4 (the rows of accumulator register r
  // of M block mb); all ones for a tile wholly admitted, zero past the end.
  auto p_mask = [&](const Cursor& c, bool valid) -> uint32_t {
    const int qt0 = tile_row0(c.t), qe = tile_end(c.t);
    const bool act = valid & wave_has_keys &
                     (((qt0 < w1hi) & (qt0 + kQt2 > w1lo)) | ((qt0 < w2hi) & (qt0 + kQt2 > w2lo)));
    const bool full = act & (qt0 + kQt2 <= qe) &
                      (((qt0 >= f1lo) & (qt0 + kQt2 <= f1hi)) |
                       ((qt0 >= f2lo) & (qt0 + kQt2 <= f2hi)));
    auto bits = [&](int lo, int hi) -> uint64_t {  // rows [lo, hi) of the tile
      const int x = min(max(lo - qt0, 0), 64), y = min(max(hi - qt0, 0), 64);
      const uint64_t hy = y >= 64 ? ~0ull : ((1ull << y) - 1);
      const uint64_t hx = x >= 64 ? ~0ull : ((1ull << x) - 1);
      return hy & ~hx;
    };
    const uint64_t m = (bits(kr.lo, kr.hi) | bits(kr.lo2, kr.hi2)) & bits(qt0, qe);
    // rows 32 mb + 8 q + 4 half + e  ->  bit 16 mb + 4 q + e
    uint32_t out = 0;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const uint32_t w32 = (uint32_t)(m >> (32 * mb)) >> (4 * half);
#pragma unroll
      for (int q = 0; q < 4; ++q) out |= ((w32 >> (8 * q)) & 0xfu) << (16 * mb + 4 * q);
    }
    return full ? 0xffffffffu : (act ? out : 0u);
  };
  // whether tile c is wholly admitted for the wave's 32 keys (wave-uniform)
  auto p_full = [&](const Cursor& c, bool valid) -> bool {
    const int qt0 = tile_row0(c.t), qe = tile_end(c.t);
    return valid & wave_has_keys & (qt0 + kQt2 <= qe) &
           (((qt0 >= f1lo) & (qt0 + kQt2 <= f1hi)) | ((qt0 >= f2lo) & (qt0 + kQt2 <= f2hi)));
  };
  auto read_side = [&](int buf, int mb, int r4) {
    return *reinterpret_cast<const f32x4*>(
        &lds.v[buf][kwave ? 1 : 0][32 * mb + 8 * r4 + 4 * half]);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  f32x16 acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) acc[dt] = f32x16{};

  // Tiles 0 and 1 before the loop; buffer 3 (the "tile -1" of step 0), its
  // side values and the P hand-over start as zeros, so step 0's products of
  // the previous tile add nothing.
  Cursor ld = Cursor{0, 0};
  if (kwave) {
    issue_part(ld, 0, nsteps > 0, 0);
    issue_part(ld, 0, nsteps > 0, 1);
    advance(ld);
    issue_part(ld, 1, nsteps > 1, 0);
    issue_part(ld, 1, nsteps > 1, 1);
    advance(ld);
  }
  {
    u32x4* z = reinterpret_cast<u32x4*>(&tiles[3][0]);
    for (int i = tid; i < kTileBytes / 16; i += 512) z[i] = u32x4{0, 0, 0, 0};
    for (int i = tid; i < 2 * 64; i += 512) lds.v[3][i / 64][i % 64] = 0.f;
    u32x4* px = &p_xchg[0][0][0][0];
    for (int i = tid; i < 4 * 2 * 2 * 64; i += 512) px[i] = u32x4{0, 0, 0, 0};
  }
  wait_vmem();
  barrier_lds();

  // MFMA phase of step t (buffers bt = t % 4, bp = (t - 1) % 4): out[mb] =
  // X(t) Y^T over the 64 rows (X = Q or dO rows, Y = this wave's K or V) and
  // acc += W(t-1)^T Z(t-1) with W from the words xw (P or dS of tile t-1,
  // keys on M, rows on K) and Z (dO or Q rows of tile t-1) by transposed
  // reads.  The two products alternate MFMA by MFMA, with the operands of
  // each read kAh MFMA pairs ahead.
  auto mfma_phase = [&](auto cbt, auto cbp, const uint32_t (&xw)[2][2][4], f32x16 (&out)[2],
                        bool zero_out) {
    constexpr int bt = decltype(cbt)::value, bp = decltype(cbp)::value;
    uint32_t r0 = roff0;
    asm volatile("" : "+v"(r0));
    auto afrag = [&](int i) {  // i = 2 kk + mb
      const int kk = i >> 1, mb = i & 1;
      return *reinterpret_cast<const bf16x8*>(tiles_c + bt * kTileBytes + mb * 32 * D * 2 +
                                              (r0 ^ (32u * kk)));
    };
    auto tfrag = [&](int i) {  // i = kDT c + dt, c = 16-row chunk of tile t-1
      const int c = i / kDT, dt = i % kDT;
      const char* tb = tiles_c + bp * kTileBytes + c * 16 * D * 2;
      return tr_pair(tb + toff[dt][0], tb + toff[dt][1]);
    };
    constexpr int kN = 2 * kK;  // 16 MFMAs of each product
    constexpr int kAh = 2;
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 fa[kAh], ft[kAh];
#pragma unroll
    for (int i = 0; i < kAh; ++i) {
      fa[i] = afrag(i);
      ft[i] = tfrag(i);
    }
    if (zero_out) {
      out[0] = f32x16{};
      out[1] = f32x16{};
    }
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int c = i / kDT, dt = i % kDT;
      const bf16x8 xa = __builtin_bit_cast(
          bf16x8, u32x4{xw[c >> 1][c & 1][0], xw[c >> 1][c & 1][1], xw[c >> 1][c & 1][2],
                        xw[c >> 1][c & 1][3]});
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, ft[i % kAh], acc[dt], 0, 0, 0);
      out[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i % kAh], kvf[i >> 1], out[i & 1],
                                                          0, 0, 0);
      if (i + kAh < kN) {
        fa[i % kAh] = afrag(i + kAh);
        ft[i % kAh] = tfrag(i + kAh);
      }
    }
    // issue order: the reads of kAh pairs, then (2 MFMAs, 3 reads) groups,
    // then the last MFMAs (group masks: 0x100 LDS read, 0x008 MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, 3 * kAh, 0);
#pragma unroll
    for (int i = 0; i < kN - kAh; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kAh, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  if (!kwave) {
    // V waves: phase 1 MFMAs (S(t), dV from P(t-1)); phase 2 P(t).  The S
    // accumulators start at -LSE(t) log2(e) / (scale log2(e)) of their rows,
    // so P = exp2(scale log2(e) S') needs no LDS read in phase 2: tile t+1's
    // LSE rows are read at the end of step t.
    uint32_t pw[2][2][4] = {};  // P(t-1), then P(t): [mb][c][word]
    u32x4* const pex = &p_xchg[wave & 3][0][0][lane];
    const float neg_inv = -1.f / a.scale_log2;
    f32x16 s[2];
    auto load_lse = [&](int buf) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 v = read_side(buf, mb, r4);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[mb][4 * r4 + e] = v[e] * neg_inv;
        }
    };
    load_lse(0);
    auto step = [&](int st, auto cbt) {
      constexpr int bt = decltype(cbt)::value;
      using BP = std::integral_constant<int, (bt + 3) & 3>;
      // the wave in its MFMA phase gets the higher issue priority, so the
      // other wave's VALU work fills the gaps between MFMAs instead of
      // delaying them
      __builtin_amdgcn_s_setprio(2);
      mfma_phase(cbt, BP{}, pw, s, false);
      __builtin_amdgcn_s_setprio(0);
      barrier_lds();
      const Cursor cur = Cursor{st / group, st % group};
      // scores outside the admitted pairs to -inf (exp2 gives 0), only on
      // tiles not wholly admitted
      if (!p_full(cur, st < nsteps)) {
        const uint32_t m = p_mask(cur, st < nsteps);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[mb][r] = ((m >> (16 * mb + r)) & 1u) ? s[mb][r] : kNegInf;
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float v0 = fast_exp2(s[mb][2 * j] * a.scale_log2);
          const float v1 = fast_exp2(s[mb][2 * j + 1] * a.scale_log2);
          pw[mb][j >> 2][j & 3] = pack_bf16x2(v0, v1);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
          pex[(mb * 2 + c) * 64] = u32x4{pw[mb][c][0], pw[mb][c][1], pw[mb][c][2], pw[mb][c][3]};
      }
      load_lse((bt + 1) & 3);
      barrier_lds();
    };
    for (int st = 0; st <= nsteps; st += 4) {
      step(st, I0{});
      step(st + 1, I1{});
      step(st + 2, I2{});
      step(st + 3, I3{});
    }
  } else {
    // K waves: phase 1 dS(t-1); phase 2 MFMAs (dP(t), dK from dS(t-1)).
    f32x16 dp[2] = {f32x16{}, f32x16{}};  // dP(t-1), then dP(t)
    const u32x4* const pex = &p_xchg[wave & 3][0][0][lane];
    auto step = [&](int st, auto cbt) {
      constexpr int bt = decltype(cbt)::value;
      using BP = std::integral_constant<int, (bt + 3) & 3>;
      issue_part(ld, (bt + 2) & 3, st + 2 < nsteps, 0);
      uint32_t xw[2][2][4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x4 side[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) side[r4] = read_side(BP::value, mb, r4);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4 pwc = pex[(mb * 2 + c) * 64];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t wd = pwc[q];
            const int r = 8 * c + 2 * q;
            const float v0 = bf16_to_f32(wd & 0xffffu) * (dp[mb][r] - side[r >> 2][r & 3]);
            const float v1 =
                bf16_to_f32(wd >> 16) * (dp[mb][r + 1] - side[(r + 1) >> 2][(r + 1) & 3]);
            xw[mb][c][q] = pack_bf16x2(v0, v1);
          }
        }
      }
      // dS complete before the barrier (IR passes would sink it into the MFMA phase)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          asm volatile("" ::"v"(xw[mb][c][0]), "v"(xw[mb][c][1]), "v"(xw[mb][c][2]),
                       "v"(xw[mb][c][3]));
      barrier_lds();
      __builtin_amdgcn_s_setprio(2);  // as the V waves' MFMA phase
      mfma_phase(cbt, BP{}, xw, dp, true);
      __builtin_amdgcn_s_setprio(0);
      issue_part(ld, (bt + 2) & 3, st + 2 < nsteps, 1);
      advance(ld);
      wait_all_but_newest();
      barrier_lds();
    };
    for (int st = 0; st <= nsteps; st += 4) {
      step(st, I0{});
      step(st + 1, I1{});
      step(st + 2, I2{});
      step(st + 3, I3{});
    }
  }

  if (!wave_has_keys) return;
  uint16_t* out = kwave ? a.dk : a.dv;
  const float mul = kwave ? a.scale : 1.f;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr2 = kw0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (kr2 < L) {
        const size_t off = ((size_t)(base + kr2) * a.hkv + g) * D + dt * 32 + (lane & 31);
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

hipError_t launch_bwd_bf16(const BwdArgs& a, int max_seqlen, int stage, hipStream_t stream) {
  if (a.nseq <= 0 || a.total <= 0) return hipSuccess;
  // 1. delta
  if (stage == 0 || stage == 1) {
    const int rows_per_wg = 256 / (a.d / 8) * kDeltaPasses;
    const long long nwg = (long long)((a.total + rows_per_wg - 1) / rows_per_wg) * a.hq;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)nwg), dim3(256), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // 2. dK, dV
  if (stage == 0 || stage == 2) {
    const long long nkt = (max_seqlen + kKvKeys - 1) / kKvKeys;
    const long long nwg = nkt * a.nseq * a.hkv;
    if (a.d == 128) {
      hipLaunchKernelGGL(bwd_dkdv_pp_kernel<128>, dim3((unsigned)nwg), dim3(512), 0, stream, a,
                         (int)nkt);
    } else {
      hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3((unsigned)nwg), dim3(512), 0, stream, a,
                         (int)nkt);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // 3. dQ
  if (stage == 0 || stage == 3) {
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
  return hipSuccess;
}

}  // namespace bca
