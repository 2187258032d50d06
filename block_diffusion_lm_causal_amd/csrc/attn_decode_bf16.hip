// The decode step of block-causal attention on gfx950 (CDNA4): the B noisy
// queries of the current block against the prefix KV cache plus the block's
// own keys ("On-Policy Residual Learning for Diffusion Language Models",
// thread page, Result 4: each block's denoising loop at batch 1), with a bf16
// or an FP8 E4M3 cache, split over key chunks and merged by log-sum-exp
// weights.  The per-tile math is the forward's (attn_fwd_bf16.hip): S^T =
// K Q^T on v_mfma_f32_32x32x16_bf16, log2-domain softmax with a lazy rescale,
// O^T += V^T P^T with V^T from the transposed LDS read.
#include "attn_common.hpp"

namespace bca {
namespace {

// ---------------------------------------------------------------------------
// Decode step: one workgroup per (KV head group, 32-token tile, key chunk).
// Eight waves in two groups of four hold the same query rows (the hpw heads of
// a KV head x 32 tokens); for every 64-key tile group A takes keys 0-31 and
// group B keys 32-63, so both groups work on each tile as soon as it lands.
// Up to kDecTiles tiles of the chunk are requested from HBM at once, each
// wave issuing its share tile by tile; tile t becomes readable once every wave
// has seen its own loads for tiles <= t complete (vmcnt) and passed a barrier,
// while later tiles are still in flight.  The query rows come the same way
// (HBM -> LDS, then each wave reads its fragments into registers), and every
// load is the inline-assembly direct-to-LDS form with plain s_barrier
// barriers: the compiler then inserts no vmcnt waits of its own.  With the
// compiler-visible forms it waited for every outstanding load before each
// tile (a barrier's fence, and a may-alias wait before LDS reads that follow
// a direct-to-LDS load), so no tile was multiplied before the last had
// landed.  The two groups merge their (max, sum, O) through LDS at the end;
// the result is the final O and LSE (one chunk) or a bf16 partial that the
// combine kernel merges by log-sum-exp weights.

constexpr int kDecTiles = 5;  // key tiles of a chunk staged in LDS at once

// One slot holds a K tile and its V tile; the last slot first holds the
// workgroup's 128 query rows (the same 2 * 64 * D bf16), which every wave
// copies to registers before that slot's tile is requested.
template <int D>
struct LdsDec {
  struct Slot {
    uint16_t k[kBN * D];
    uint16_t v[kBN * D];
  } slot[kDecTiles];
};

// s_waitcnt vmcnt(N) immediate (vmcnt is split over bits 3:0 and 15:14;
// expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 0xF) | (((n >> 4) & 0x3) << 14); }

// s_waitcnt vmcnt(n) for n = STEP * k, 0 <= k <= 5, chosen at run time.
template <int STEP>
__device__ __forceinline__ void wait_vmem_upto(int n) {
  switch (n / STEP) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1 * STEP)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * STEP)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * STEP)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * STEP)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * STEP)); break;
  }
}

// Per-wave constants of the decode kernels: which rows, heads, keys and LDS
// offsets this wave works with.
template <int D>
struct DecWave {
  int lane, half, wave, grp, wv, head, kv_head;
  int split, ntile_all;  // this workgroup's split and its number of key tiles
  int kv_len;            // keys attended (the host's kv_len, or the device-resident length)
  int ntiles_kv;         // 64-key tiles of the whole cache
  int hg, tok0;          // KV head group, first query token of the workgroup
  int qw0, qi;           // first query row of the wave, the lane's row
  bf16x8 qf[D / 16];     // the lane's query, B operand of S^T = K Q^T
  uint32_t koff[D / 16];     // K fragment offsets in a bf16 tile
  uint32_t voff[D / 32][2];  // V^T transposed-read offsets in a bf16 tile
};

// Key tile i (0-based) of split `split`: tiles are dealt to the splits in
// turn (split s takes tiles s, s + nsplit, s + 2 nsplit, ...), so at any
// moment the workgroups of a KV head read one contiguous stretch of the cache.
__device__ __forceinline__ int split_tile(int split, int nsplit, int i) {
  return split + i * nsplit;
}

template <int D>
__device__ __forceinline__ void dec_wave_init(const DecodeArgs& a, DecWave<D>& dw) {
  const int ngroups = a.hq / a.hpw;
  const int tok = kRows * (4 / a.hpw);
  const int ntok = (a.q_len + tok - 1) / tok;
  const int w = blockIdx.x;
  const int hg = w % ngroups;  // one KV head per XCD when there are 8 groups
  const int rest = w / ngroups;
  const int tile = rest % ntok;
  dw.split = rest / ntok;
  const int tid = threadIdx.x;
  dw.lane = tid & 63;
  dw.half = dw.lane >> 5;
  dw.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  dw.grp = dw.wave >> 2;  // key half of every tile
  dw.wv = dw.wave & 3;    // wave within its group
  dw.head = hg * a.hpw + dw.wv % a.hpw;
  dw.kv_head = (hg * a.hpw) / (a.hq / a.hkv);
  // The cache length: fixed at launch, or read from device memory (a
  // captured loop whose prefix grows between replays), clamped to
  // [q_len, kv_len] -- the grid and the partials were planned for kv_len.
  dw.kv_len = a.kv_len;
  if (a.kv_len_dev) dw.kv_len = min(max(*a.kv_len_dev, a.q_len), a.kv_len);
  dw.ntiles_kv = (dw.kv_len + kBN - 1) / kBN;
  dw.ntile_all = dw.split < dw.ntiles_kv ? (dw.ntiles_kv - dw.split + a.nsplit - 1) / a.nsplit : 0;
  dw.hg = hg;
  dw.tok0 = tile * tok;
  dw.qw0 = tile * tok + (dw.wv / a.hpw) * kRows;
  dw.qi = dw.qw0 + (dw.lane & 31);
  // K rows of this group's key half (32 rows from 32 grp); V rows of that half
  // through the transposed read.
  const int sw = swz<D>(dw.lane & 15);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    dw.koff[kk] = (uint32_t)((32 * dw.grp + (dw.lane & 31)) * D * 2 +
                             (((2 * kk + dw.half) ^ sw) * 16));
  const int aa = dw.lane & 15, r = aa >> 2, q = aa & 3, g2 = (dw.lane >> 4) & 1;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int row = 32 * dw.grp + 8 * sub + 4 * dw.half + r;
      const int chunk = 4 * dt + 2 * g2 + (q >> 1);
      dw.voff[dt][sub] = (uint32_t)(row * D * 2 + ((chunk ^ swz<D>(row)) * 16) + (q & 1) * 8);
    }
  }
}

// This wave's share of the direct-to-LDS loads of the workgroup's query
// rows into `qlds` (128 rows of D bf16 in the K-tile layout and swizzle):
// row 32 w + r is token r of the 32-token sub-tile of wave w's head, so
// every wave w of either group later reads rows 32 (w mod 4) + 0..31.  Rows
// past q_len lie past the buffer's end and arrive as zeros.
template <int D>
__device__ __forceinline__ void dec_issue_q(const DecodeArgs& a, const DecWave<D>& dw,
                                            uint32_t qlds) {
  constexpr int kChunks = D / 8;
  constexpr int kRowsPerInst = 64 / kChunks;
  constexpr int kInst = 4 * kRows / kRowsPerInst / 8;  // per wave
  const int tok = kRows * (4 / a.hpw);
  const int ntok = min(a.q_len - dw.tok0, tok);
  const i32x4 r = rsrc_words(a.q + (size_t)dw.tok0 * a.hq * D, (uint32_t)(ntok * a.hq * D * 2));
#pragma unroll
  for (int j = 0; j < kInst; ++j) {
    const int row0 = (dw.wave + 8 * j) * kRowsPerInst;
    const int R = row0 + dw.lane / kChunks;
    const int w = R / kRows;
    const int t = (w / a.hpw) * kRows + R % kRows;
    const int head = dw.hg * a.hpw + w % a.hpw;
    const uint32_t voff =
        (uint32_t)(((t * a.hq + head) * D) * 2 + (((dw.lane % kChunks) ^ swz<D>(R)) * 16));
    buffer_load_lds16_asm(r, qlds + (uint32_t)(row0 * D * 2), voff);
  }
}

// The lane's query fragments from the rows dec_issue_q staged (after they
// have landed for every wave).
template <int D>
__device__ __forceinline__ void dec_read_q(const char* qlds, DecWave<D>& dw) {
  const int sw = swz<D>(dw.lane & 15);
  const char* row = qlds + (kRows * dw.wv + (dw.lane & 31)) * D * 2;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    dw.qf[kk] = *reinterpret_cast<const bf16x8*>(row + (((2 * kk + dw.half) ^ sw) * 16));
}

// One 64-key tile for this wave's key half: S^T in two accumulator chains,
// mask past the cache end, online softmax with the lazy rescale, O^T +=
// V^T P^T.  k0 is the first key of the half.  The MFMA A operands come from
// the fetchers: kfrag(kk) the K fragment of dims 16 kk.. (keys on M), vfrag(c,
// dt) the V^T fragment of dims 32 dt.. and keys 16 c.. of the half (dims on M),
// each eight bf16 values per lane in the 32x32x16 operand layout.
template <int D, typename KFrag, typename VFrag>
__device__ __forceinline__ void dec_tile_with(KFrag kfrag, VFrag vfrag, const DecWave<D>& dw,
                                              int k0, int kend, float scale_log2,
                                              WaveState<D>& ws) {
  f32x16 s = f32x16{}, s1 = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; kk += 2) {
    const bf16x8 a0 = kfrag(kk);
    const bf16x8 a1 = kfrag(kk + 1);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, dw.qf[kk], s, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, dw.qf[kk + 1], s1, 0, 0, 0);
  }
  s += s1;
  if (k0 + 32 > kend) {  // keys past the cache's end (zero-filled) are masked
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = k0 + 8 * (r >> 2) + 4 * dw.half + (r & 3);
      s[r] = j < kend ? s[r] : kNegInf;
    }
  }
  float mt[8];
#pragma unroll
  for (int r = 0; r < 16; r += 2) mt[r / 2] = fmaxf(s[r], s[r + 1]);
#pragma unroll
  for (int ww = 4; ww >= 1; ww >>= 1) {
#pragma unroll
    for (int i = 0; i < ww; ++i) mt[i] = fmaxf(mt[i], mt[i + ww]);
  }
  const float mloc = xhalf_max(mt[0]) * scale_log2;
  const bool grow = mloc > ws.m + kRescaleSlack;
  const float m_new = grow ? mloc : ws.m;
  const float alpha = fast_exp2(ws.m - m_new);
  ws.m = m_new;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) ws.acc[dt] *= alpha;
  }
  const float neg_m = -m_new;
  float lsum = ws.l * alpha;
  uint32_t pk[2][4];
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float p0 = fast_exp2(fmaf(s[r], scale_log2, neg_m));
    const float p1 = fast_exp2(fmaf(s[r + 1], scale_log2, neg_m));
    lsum += p0 + p1;
    pk[r >> 3][(r & 7) >> 1] = pack_bf16x2(p0, p1);
  }
  ws.l = lsum;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[c][0], pk[c][1], pk[c][2], pk[c][3]});
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      ws.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag(c, dt), pb, ws.acc[dt], 0, 0, 0);
  }
}

// The tile body on a bf16 tile pair (K at kt, V at vt, row-major, swizzled).
template <int D>
__device__ __forceinline__ void dec_tile(const char* kt, const char* vt, const DecWave<D>& dw,
                                         int k0, int kend, float scale_log2, WaveState<D>& ws) {
  auto kfrag = [&](int kk) { return *reinterpret_cast<const bf16x8*>(kt + dw.koff[kk]); };
  auto vfrag = [&](int c, int dt) {
    const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(vt + dw.voff[dt][0] + c * 16 * D * 2));
    const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(vt + dw.voff[dt][1] + c * 16 * D * 2));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  };
  dec_tile_with<D>(kfrag, vfrag, dw, k0, kend, scale_log2, ws);
}

// End of a decode workgroup: group B's (max, sum, O) merge into group A's
// through LDS scratch `mrg` (free tile memory, (D/32*16*64 + 128) floats per
// wave of group A), then group A writes the final rows (one chunk) or the
// float32 partial of its (split, head, 32-token tile).  O is scaled by o_mul.
// Contains a workgroup barrier: every wave calls it.
template <int D>
__device__ __forceinline__ void dec_finish(const DecodeArgs& a, const DecWave<D>& dw, float* mrg,
                                           WaveState<D>& ws) {
  const int lane = dw.lane;
  constexpr int kWaveFloats = (D / 32) * 16 * 64 + 128;
  // 16 bytes per lane and instruction: element (dt, r) of lane l at
  // float 4 ((dt * 4 + r / 4) * 64 + l) + r % 4 of the wave's area.
  if (dw.grp == 1) {
    float* dst = mrg + dw.wv * kWaveFloats;
    f32x4* dst4 = reinterpret_cast<f32x4*>(dst);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        dst4[(dt * 4 + r4) * 64 + lane] =
            f32x4{ws.acc[dt][4 * r4], ws.acc[dt][4 * r4 + 1], ws.acc[dt][4 * r4 + 2],
                  ws.acc[dt][4 * r4 + 3]};
    }
    dst[(D / 32) * 16 * 64 + lane] = ws.m;
    dst[(D / 32) * 16 * 64 + 64 + lane] = ws.l;
  }
  __syncthreads();
  if (dw.grp == 1) return;
  {
    const float* src = mrg + dw.wv * kWaveFloats;
    const f32x4* src4 = reinterpret_cast<const f32x4*>(src);
    const float mb = src[(D / 32) * 16 * 64 + lane];
    const float lb = src[(D / 32) * 16 * 64 + 64 + lane];
    const float m_new = fmaxf(ws.m, mb);
    const float sa = fast_exp2(ws.m - m_new), sb = fast_exp2(mb - m_new);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 b = src4[(dt * 4 + r4) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          ws.acc[dt][r] = (ws.acc[dt][r] * sa + b[e] * sb) * a.o_mul;
        }
      }
    }
    ws.l = ws.l * sa + lb * sb;
    ws.m = m_new;
  }
  const bool valid = dw.qi < a.q_len;
  if (a.nsplit == 1) {
    write_rows<D, false>(ws, valid, a.o + ((size_t)dw.qi * a.hq + dw.head) * D,
                         a.lse + (size_t)dw.head * a.q_len + dw.qi);
    return;
  }
  if (dw.qw0 >= a.q_len) return;  // a wave past the block's last query has no partial
  // Partial of this (split, head, 32-token tile), normalised and rounded to
  // bf16, in the accumulator's own layout: the 8-byte group (dt, g, lane)
  // holds dims 32 dt + 8 g + 4 (lane / 32) + 0..3 of token lane % 32.  Every
  // store instruction writes 512 bytes contiguous.  (The per-CU memory pipe
  // sets the pace of this kernel, so the partial's bytes cost as much time as
  // key/value bytes; the LSE stays float32.)
  // A split with no keys (a device-resident cache length shorter than the
  // plan) leaves l = 0: its partial is O = 0 with LSE = -inf, weight 0 in
  // the merge.
  const float l = xhalf_sum(ws.l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int ntok32 = (a.q_len + kRows - 1) / kRows;
  const size_t ptile = ((size_t)dw.split * a.hq + dw.head) * ntok32 + dw.qw0 / kRows;
  u32x2* po = reinterpret_cast<u32x2*>(a.part_o + ptile * (size_t)(kRows * D));
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      po[(dt * 4 + gq) * 64 + lane] =
          u32x2{pack_bf16x2(ws.acc[dt][4 * gq] * inv, ws.acc[dt][4 * gq + 1] * inv),
                pack_bf16x2(ws.acc[dt][4 * gq + 2] * inv, ws.acc[dt][4 * gq + 3] * inv)};
    }
  }
  if (dw.half == 0) a.part_lse[ptile * kRows + (lane & 31)] = (ws.m + fast_log2(l)) * kLn2;
}

template <int D>
__global__ __launch_bounds__(kPPThreads, 1) void decode_bf16_kernel(DecodeArgs a) {
  if (a.steps_dev && a.step >= *a.steps_dev) return;  // a step the loop skips
  __shared__ LdsDec<D> lds;
  constexpr int kChunks = D / 8;
  constexpr int kRowsPerInst = 64 / kChunks;
  constexpr int kInstPerTile = 2 * (kBN / kRowsPerInst);  // K and V, 1 KB each
  constexpr int kInstPerWaveTile = kInstPerTile / 8;      // 4 (D=128) or 2 (D=64)
  static_assert(kInstPerWaveTile * (kDecTiles - 1) < 64 && kDecTiles <= 6, "vmcnt range");
  DecWave<D> dw;
  dec_wave_init<D>(a, dw);
  const int kv_elems = a.hkv * D;
  const uint16_t* kb = a.k + (size_t)dw.kv_head * D;
  const uint16_t* vb = a.v + (size_t)dw.kv_head * D;
  const uint32_t slots = lds_addr_of(&lds.slot[0]);
  constexpr uint32_t kSlotBytes = sizeof(typename LdsDec<D>::Slot);

  // This wave's loads of one tile into slot `sl`: instructions wave + 8 j of
  // the tile's kInstPerTile (K blocks, then V blocks).
  auto load_tile = [&](int sl, int i) {
    const int k0 = split_tile(dw.split, a.nsplit, i) * kBN;
    const int rows = min(dw.kv_len - k0, kBN);
    const uint32_t nbytes = (uint32_t)((rows - 1) * kv_elems * 2 + D * 2);
    const i32x4 rk = rsrc_words(kb + (size_t)k0 * kv_elems, nbytes);
    const i32x4 rv = rsrc_words(vb + (size_t)k0 * kv_elems, nbytes);
#pragma unroll
    for (int j = 0; j < kInstPerWaveTile; ++j) {
      const int ii = dw.wave + 8 * j;
      const bool is_k = ii < kInstPerTile / 2;
      const int row0 = (is_k ? ii : ii - kInstPerTile / 2) * kRowsPerInst;
      const int R = row0 + dw.lane / kChunks;
      const uint32_t voff = (uint32_t)(R * kv_elems * 2 + (((dw.lane % kChunks) ^ swz<D>(R)) * 16));
      const uint32_t dst = slots + (uint32_t)sl * kSlotBytes + (is_k ? 0u : (uint32_t)(kBN * D * 2)) +
                           (uint32_t)(row0 * D * 2);
      buffer_load_lds16_asm(is_k ? rk : rv, dst, voff);
    }
  };
  // Tiles t = 0 .. nt-1 of a round, in slots 0 .. nt-1, all requested: tile t
  // has landed for this wave once at most the loads of the later tiles are
  // outstanding, and for every wave after the barrier.
  auto consume = [&](int r0, int nt, WaveState<D>& ws) {
    for (int t = 0; t < nt; ++t) {
      wait_vmem_upto<kInstPerWaveTile>(kInstPerWaveTile * (nt - 1 - t));
      barrier_lds();
      dec_tile<D>(reinterpret_cast<const char*>(lds.slot[t].k),
                  reinterpret_cast<const char*>(lds.slot[t].v), dw,
                  split_tile(dw.split, a.nsplit, r0 + t) * kBN + 32 * dw.grp, dw.kv_len,
                  a.scale_log2, ws);
    }
  };

  WaveState<D> ws;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) ws.acc[dt] = f32x16{};
  ws.m = kNegBig;
  ws.l = 0.f;
  // Round 0: the query rows into the last slot, then tiles 0 .. nt0-1; once
  // the query rows have landed and every wave holds its fragments, the last
  // slot takes tile kDecTiles-1.
  const int nt = min(kDecTiles, dw.ntile_all);
  const int nt0 = min(kDecTiles - 1, dw.ntile_all);
  dec_issue_q<D>(a, dw, slots + (uint32_t)(kDecTiles - 1) * kSlotBytes);
  for (int t = 0; t < nt0; ++t) load_tile(t, t);
  wait_vmem_upto<kInstPerWaveTile>(kInstPerWaveTile * nt0);
  barrier_lds();
  dec_read_q<D>(reinterpret_cast<const char*>(&lds.slot[kDecTiles - 1]), dw);
  barrier_lds();  // every wave's query reads are done: the slot is free
  if (nt > nt0) load_tile(kDecTiles - 1, kDecTiles - 1);
  consume(0, nt, ws);
  for (int r0 = kDecTiles; r0 < dw.ntile_all; r0 += kDecTiles) {
    const int ntr = min(kDecTiles, dw.ntile_all - r0);
    barrier_lds();  // the previous round's tiles have been consumed
    for (int t = 0; t < ntr; ++t) load_tile(t, r0 + t);
    consume(r0, ntr, ws);
  }
  __syncthreads();  // the tile buffers are free for the merge
  dec_finish<D>(a, dw, reinterpret_cast<float*>(&lds.slot[0]), ws);
}

// FP8 K/V cache (OCP E4M3; the pages run their decode with an FP8 KV cache,
// paper cards page, Table 11 configurations).  The E4M3 bytes of up to
// kDec8Tiles 64-key tiles per round go to LDS (half the bytes of bf16) and
// every wave widens its own operand fragments in registers right before its
// MFMAs: K rows with an 8-byte LDS read, V^T with the transposed byte read
// (ds_read_b64_tr_b8), then v_cvt_pk_f32_fp8 and bf16 packing -- exact, since
// every E4M3 value is a bf16 value.  The K scale is folded into scale_log2
// and the V scale into o_mul.
constexpr int kDec8Tiles = 5;

template <int D>
struct LdsDec8 {
  uint8_t k8[kDec8Tiles][kBN * D];
  uint8_t v8[kDec8Tiles][kBN * D];
  uint16_t q[4 * kRows * D];  // the workgroup's query rows (dec_issue_q)
};

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// 16-byte chunk swizzle of an E4M3 tile (D / 16 chunks of a D-byte row): the
// 8-byte K reads of 32 rows at one logical chunk and the transposed reads of
// 8 rows at one chunk spread over the LDS banks.
template <int D>
__device__ __forceinline__ int swz8(int row) {
  return (row >> 1) & (D / 16 - 1);
}

// Eight E4M3 bytes (in byte order) to eight bf16 values.
__device__ __forceinline__ bf16x8 widen_e4m3x8(i32x2 raw) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(raw[0], false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(raw[0], true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(raw[1], false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(raw[1], true);
  return __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]),
                                          pack_bf16x2(c[0], c[1]), pack_bf16x2(d[0], d[1])});
}

template <int D>
__global__ __launch_bounds__(kPPThreads, 1) void decode_fp8_kernel(DecodeArgs a) {
  if (a.steps_dev && a.step >= *a.steps_dev) return;  // a step the loop skips
  __shared__ LdsDec8<D> lds;
  constexpr int kChunks8 = D / 16;                         // 16-byte chunks per fp8 row
  constexpr int kRowsPerInst = 64 / kChunks8;              // 8 (D=128) or 16 (D=64)
  constexpr int kInstPerTile = 2 * (kBN / kRowsPerInst);   // K and V, 1 KB each
  constexpr int kInstPerWaveTile = kInstPerTile / 8;       // 2 (D=128) or 1 (D=64)
  static_assert(kInstPerWaveTile * (kDec8Tiles - 1) < 64 && kDec8Tiles <= 6, "vmcnt range");
  DecWave<D> dw;
  dec_wave_init<D>(a, dw);
  dec_issue_q<D>(a, dw, lds_addr_of(&lds.q[0]));
  const int row_bytes = a.hkv * D;
  const uint8_t* kb = a.k8 + (size_t)dw.kv_head * D;
  const uint8_t* vb = a.v8 + (size_t)dw.kv_head * D;
  const int lane = dw.lane;
  // K fragment kk: row 32 grp + lane % 32, bytes 16 kk + 8 (lane / 32) .. +8.
  uint32_t koff8[D / 16];
  {
    const int R = 32 * dw.grp + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      koff8[kk] = (uint32_t)(R * D + ((kk ^ swz8<D>(R)) * 16) + 8 * dw.half);
  }
  // V^T fragment (c, dt) through the transposed byte read: in each 16-lane
  // group g = lane / 16, address-lane 2 r + q points at 8 bytes (dims +8 q)
  // of one key row, and lane i of the group receives byte i of the group's
  // 16-byte segment from each of its 8 rows, in row order.  The rows are
  // the keys the P operand pairs with element r of this lane: from the S^T
  // accumulator layout, keys 16 c + 4 h + 0..3 and 16 c + 8 + 4 h + 0..3 of
  // the half (h = lane / 32 = g / 2); the dims are 32 dt + 16 (g % 2) + i.
  uint32_t voff8[2][D / 32];
  {
    const int g = (lane >> 4) & 3, i = lane & 15, r = i >> 1, q = i & 1;
    const int kr = (r < 4 ? 0 : 8) + 4 * (g >> 1) + (r & 3);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int R = 32 * dw.grp + 16 * c + kr;
        const int chunk = 2 * dt + (g & 1);
        voff8[c][dt] = (uint32_t)(R * D + ((chunk ^ swz8<D>(R)) * 16) + 8 * q);
      }
    }
  }

  // This wave's loads of one tile: instructions wave + 8 j of the tile's
  // kInstPerTile (K blocks, then V blocks); lane l of an instruction fills
  // physical chunk l % kChunks8 of its row with the logical chunk the
  // swizzle puts there.
  const uint32_t k8_lds = lds_addr_of(&lds.k8[0][0]);
  const uint32_t v8_lds = lds_addr_of(&lds.v8[0][0]);
  auto load_tile = [&](int t_round, int i) {
    const int k0 = split_tile(dw.split, a.nsplit, i) * kBN;
    const int rows = min(dw.kv_len - k0, kBN);
    const uint32_t nbytes = (uint32_t)((rows - 1) * row_bytes + D);
    const i32x4 rk = rsrc_words(kb + (size_t)k0 * row_bytes, nbytes);
    const i32x4 rv = rsrc_words(vb + (size_t)k0 * row_bytes, nbytes);
#pragma unroll
    for (int j = 0; j < kInstPerWaveTile; ++j) {
      const int ii = dw.wave + 8 * j;
      const bool is_k = ii < kInstPerTile / 2;
      const int row0 = (is_k ? ii : ii - kInstPerTile / 2) * kRowsPerInst;
      const int R = row0 + lane / kChunks8;
      const uint32_t voff = (uint32_t)(R * row_bytes + (((lane % kChunks8) ^ swz8<D>(R)) * 16));
      const uint32_t dst = (is_k ? k8_lds : v8_lds) + (uint32_t)(t_round * kBN * D + row0 * D);
      buffer_load_lds16_asm(is_k ? rk : rv, dst, voff);
    }
  };

  WaveState<D> ws;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) ws.acc[dt] = f32x16{};
  ws.m = kNegBig;
  ws.l = 0.f;
  // The query rows were requested first: once at most the first round's
  // tile loads are outstanding they have landed for this wave, and for every
  // wave after the barrier.  (All loads here are the inline-assembly form, so
  // the compiler adds no vmcnt waits of its own; see the bf16 kernel.)
  {
    const int nt = min(kDec8Tiles, dw.ntile_all);
    for (int t = 0; t < nt; ++t) load_tile(t, t);
    wait_vmem_upto<kInstPerWaveTile>(kInstPerWaveTile * nt);
    barrier_lds();
    dec_read_q<D>(reinterpret_cast<const char*>(&lds.q[0]), dw);
  }
  for (int r0 = 0; r0 < dw.ntile_all; r0 += kDec8Tiles) {
    const int nt = min(kDec8Tiles, dw.ntile_all - r0);
    if (r0 > 0) {
      barrier_lds();  // the previous round's tiles have been consumed
      for (int t = 0; t < nt; ++t) load_tile(t, r0 + t);
    }
    for (int t = 0; t < nt; ++t) {
      wait_vmem_upto<kInstPerWaveTile>(kInstPerWaveTile * (nt - 1 - t));
      barrier_lds();  // tile t has landed for every wave
      const char* kt = reinterpret_cast<const char*>(lds.k8[t]);
      const char* vt = reinterpret_cast<const char*>(lds.v8[t]);
      auto kfrag = [&](int kk) {
        return widen_e4m3x8(*reinterpret_cast<const i32x2*>(kt + koff8[kk]));
      };
      auto vfrag = [&](int c, int dt) {
        return widen_e4m3x8(__builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vt + voff8[c][dt])));
      };
      dec_tile_with<D>(kfrag, vfrag, dw, split_tile(dw.split, a.nsplit, r0 + t) * kBN + 32 * dw.grp,
                       dw.kv_len, a.scale_log2, ws);
    }
  }
  __syncthreads();  // the tile buffers are free for the merge
  dec_finish<D>(a, dw, reinterpret_cast<float*>(&lds.k8[0][0]), ws);
}

// Merge the split partials: one 4-wave workgroup per (head, 32-token tile,
// 1 KB slice of the partial), so that the merge runs on many compute units
// with several loads in flight per lane.  Wave w takes the splits c = w mod 4;
// lane l serves token l % 32.  Each wave forms lse_w = log sum exp(lse_c) and
// O_w = sum_c exp(lse_c - lse_w) O_c over its splits (the loads of up to
// kChunk splits issued together), then wave 0 merges the four (lse_w, O_w)
// the same way through LDS.
constexpr int kCombineWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kCombineWaves) void decode_combine_kernel(DecodeArgs a) {
  if (a.steps_dev && a.step >= *a.steps_dev) return;  // a step the loop skips
  constexpr int kSlices = D / 8;  // 512-byte slices of a 32 x D bf16 partial
  constexpr int kChunk = 8;
  __shared__ f32x4 red_o[kCombineWaves][64];
  __shared__ float red_m[kCombineWaves][64], red_s[kCombineWaves][64];
  const int ntok32 = (a.q_len + 31) / 32;
  // Workgroup order: head group fastest, as in the decode kernel, so that the
  // partials of a head group are merged on the XCD whose L2 holds them.
  const int ngroups = a.hq / a.hpw;
  const int hg = blockIdx.x % ngroups;
  int rest = blockIdx.x / ngroups;
  const int slice = rest % kSlices;
  rest /= kSlices;
  const int tile = rest % ntok32;
  const int head = hg * a.hpw + rest / ntok32;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane & 31;
  const size_t tile_stride = (size_t)a.hq * ntok32;  // partial tiles per split
  const size_t my_tile = (size_t)head * ntok32 + tile;
  const float* lse_src = a.part_lse + my_tile * 32 + row;
  const u32x2* o_src = reinterpret_cast<const u32x2*>(a.part_o + my_tile * (size_t)(32 * D)) +
                       slice * 64 + lane;
  const size_t lse_step = tile_stride * 32;             // floats between splits
  const size_t o_step = tile_stride * (size_t)(8 * D);  // 8-byte groups between splits
  float m = kNegBig, sum = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = wave; c0 < a.nsplit; c0 += kChunk * kCombineWaves) {
    float x[kChunk];
    f32x4 y[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int c = c0 + u * kCombineWaves;
      x[u] = kNegBig;
      y[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (c < a.nsplit) {
        x[u] = lse_src[(size_t)c * lse_step] * kLog2e;
        const u32x2 w2 = o_src[(size_t)c * o_step];
        y[u] = f32x4{__uint_as_float(w2[0] << 16), __uint_as_float(w2[0] & 0xffff0000u),
                     __uint_as_float(w2[1] << 16), __uint_as_float(w2[1] & 0xffff0000u)};
      }
    }
    float mc = m;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) mc = fmaxf(mc, x[u]);
    const float sc = fast_exp2(m - mc);
    acc *= sc;
    sum *= sc;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const float wv = fast_exp2(x[u] - mc);  // 0 for missing splits
      acc += wv * y[u];
      sum += wv;
    }
    m = mc;
  }
  red_o[wave][lane] = acc;
  red_m[wave][lane] = m;
  red_s[wave][lane] = sum;
  __syncthreads();
  if (wave != 0) return;
  float mt = kNegBig;
#pragma unroll
  for (int w = 0; w < kCombineWaves; ++w) mt = fmaxf(mt, red_m[w][lane]);
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  float st = 0.f;
#pragma unroll
  for (int w = 0; w < kCombineWaves; ++w) {
    const float wv = fast_exp2(red_m[w][lane] - mt);
    o += wv * red_o[w][lane];
    st += wv * red_s[w][lane];
  }
  o *= 1.f / st;
  // slice = dt * 4 + g: dims 32 dt + 8 g + 4 (lane / 32) + 0..3 of token row
  const int qi = tile * 32 + row;
  if (qi < a.q_len) {
    const int d = (slice >> 2) * 32 + (slice & 3) * 8 + 4 * (lane >> 5);
    *reinterpret_cast<u32x2*>(a.o + ((size_t)qi * a.hq + head) * D + d) =
        u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    if (slice == 0 && lane < 32) a.lse[(size_t)head * a.q_len + qi] = (mt + fast_log2(st)) * kLn2;
  }
}

}  // namespace

namespace {

// Decode kernel (bf16 or fp8 cache), then the combine when the keys are split.
hipError_t launch_decode(const DecodeArgs& a, bool fp8, hipStream_t stream) {
  const int ngroups = a.hq / a.hpw;
  const int tok = kRows * (4 / a.hpw);
  const int ntok = (a.q_len + tok - 1) / tok;
  const long long nwg = (long long)ngroups * ntok * a.nsplit;
  if (nwg <= 0) return hipSuccess;
  const dim3 grid((unsigned)nwg), block(kPPThreads);
  if (fp8) {
    if (a.d == 128) hipLaunchKernelGGL(decode_fp8_kernel<128>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(decode_fp8_kernel<64>, grid, block, 0, stream, a);
  } else {
    if (a.d == 128) hipLaunchKernelGGL(decode_bf16_kernel<128>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(decode_bf16_kernel<64>, grid, block, 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nsplit == 1) return err;
  const unsigned ncomb = (unsigned)((a.q_len + 31) / 32) * a.hq * (a.d / 8);
  if (a.d == 128) {
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(ncomb), dim3(64 * kCombineWaves), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(ncomb), dim3(64 * kCombineWaves), 0,
                       stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  return launch_decode(a, false, stream);
}

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t stream) {
  return launch_decode(a, true, stream);
}

}  // namespace bca
