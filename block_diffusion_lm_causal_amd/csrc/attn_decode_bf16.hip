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
// while later tiles are still in flight.  The two groups merge their
// (max, sum, O) through LDS at the end; the result is the final O and LSE
// (one chunk) or a float32 partial that the combine kernel merges by
// log-sum-exp weights.

constexpr int kDecTiles = 5;  // key tiles of a chunk staged in LDS at once

template <int D>
struct LdsDec {
  uint16_t k[kDecTiles][kBN * D];
  uint16_t v[kDecTiles][kBN * D];
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
  int split, kbeg, kend, ntile_all;  // this workgroup's key chunk
  int qw0, qi;                       // first query row of the wave, the lane's row
  bf16x8 qf[D / 16];                 // the lane's query, B operand of S^T = K Q^T
  uint32_t koff[D / 16];             // K fragment offsets in a bf16 tile
  uint32_t voff[D / 32][2];          // V^T transposed-read offsets in a bf16 tile
};

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
  // key tiles are dealt to the splits as evenly as they go
  const int ntiles_kv = (a.kv_len + kBN - 1) / kBN;
  const int t_first = (int)((long long)dw.split * ntiles_kv / a.nsplit);
  const int t_end = (int)((long long)(dw.split + 1) * ntiles_kv / a.nsplit);
  dw.kbeg = t_first * kBN;
  dw.kend = min(a.kv_len, t_end * kBN);
  dw.ntile_all = t_end - t_first;
  dw.qw0 = tile * tok + (dw.wv / a.hpw) * kRows;
  dw.qi = dw.qw0 + (dw.lane & 31);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 raw = u32x4{0, 0, 0, 0};
    if (dw.qi < a.q_len) {
      raw = *reinterpret_cast<const u32x4*>(a.q + ((size_t)dw.qi * a.hq + dw.head) * D +
                                            kk * 16 + dw.half * 8);
    }
    dw.qf[kk] = __builtin_bit_cast(bf16x8, raw);
  }
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

// One 64-key bf16 tile (K at kt, V at vt) for this wave's key half: S^T in
// two accumulator chains, mask past the chunk end, online softmax with the
// lazy rescale, O^T += V^T P^T.  k0 is the first key of the half.
template <int D>
__device__ __forceinline__ void dec_tile(const char* kt, const char* vt, const DecWave<D>& dw,
                                         int k0, int kend, float scale_log2, WaveState<D>& ws) {
  f32x16 s = f32x16{}, s1 = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; kk += 2) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kt + dw.koff[kk]);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kt + dw.koff[kk + 1]);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, dw.qf[kk], s, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, dw.qf[kk + 1], s1, 0, 0, 0);
  }
  s += s1;
  if (k0 + 32 > kend) {  // keys past the chunk's end (zero-filled) are masked
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
    for (int dt = 0; dt < D / 32; ++dt) {
      const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(vt + dw.voff[dt][0] + c * 16 * D * 2));
      const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(vt + dw.voff[dt][1] + c * 16 * D * 2));
      const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
      ws.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, ws.acc[dt], 0, 0, 0);
    }
  }
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
  if (dw.grp == 1) {
    float* dst = mrg + dw.wv * kWaveFloats;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(dt * 16 + r) * 64 + lane] = ws.acc[dt][r];
    }
    dst[(D / 32) * 16 * 64 + lane] = ws.m;
    dst[(D / 32) * 16 * 64 + 64 + lane] = ws.l;
  }
  __syncthreads();
  if (dw.grp == 1) return;
  {
    const float* src = mrg + dw.wv * kWaveFloats;
    const float mb = src[(D / 32) * 16 * 64 + lane];
    const float lb = src[(D / 32) * 16 * 64 + 64 + lane];
    const float m_new = fmaxf(ws.m, mb);
    const float sa = fast_exp2(ws.m - m_new), sb = fast_exp2(mb - m_new);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ws.acc[dt][r] = (ws.acc[dt][r] * sa + src[(dt * 16 + r) * 64 + lane] * sb) * a.o_mul;
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
  // Partial of this (split, head, 32-token tile), normalised, in the
  // accumulator's own layout: float4 (dt, g, lane) holds dims
  // 32 dt + 8 g + 4 (lane / 32) + 0..3 of token lane % 32.  Every store
  // instruction writes 1 KB contiguous.
  const float l = xhalf_sum(ws.l);
  const float inv = 1.f / l;
  const int ntok32 = (a.q_len + kRows - 1) / kRows;
  const size_t ptile = ((size_t)dw.split * a.hq + dw.head) * ntok32 + dw.qw0 / kRows;
  f32x4* po = reinterpret_cast<f32x4*>(a.part_o + ptile * (size_t)(kRows * D));
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      po[(dt * 4 + gq) * 64 + lane] = f32x4{ws.acc[dt][4 * gq] * inv, ws.acc[dt][4 * gq + 1] * inv,
                                            ws.acc[dt][4 * gq + 2] * inv, ws.acc[dt][4 * gq + 3] * inv};
    }
  }
  if (dw.half == 0) a.part_lse[ptile * kRows + (lane & 31)] = (ws.m + fast_log2(l)) * kLn2;
}

template <int D>
__global__ __launch_bounds__(kPPThreads, 1) void decode_bf16_kernel(DecodeArgs a) {
  __shared__ LdsDec<D> lds;
  constexpr int kChunks = D / 8;
  constexpr int kRowsPerInst = 64 / kChunks;
  constexpr int kInstPerTile = 2 * (kBN / kRowsPerInst);  // K and V, 1 KB each
  constexpr int kInstPerWaveTile = kInstPerTile / 8;      // 4 (D=128) or 2 (D=64)
  static_assert(kInstPerWaveTile * (kDecTiles - 1) < 64 && kDecTiles <= 6, "vmcnt range");
  DecWave<D> dw;
  dec_wave_init<D>(a, dw);  // query fragments first: every later vmcnt wait covers them
  const int kv_elems = a.hkv * D;
  const uint16_t* kb = a.k + (size_t)dw.kv_head * D;
  const uint16_t* vb = a.v + (size_t)dw.kv_head * D;

  // This wave's loads of one tile: instructions wave + 8 j of the tile's
  // kInstPerTile (K blocks, then V blocks).
  auto load_tile = [&](int t_round, int t_abs) {
    const int k0 = dw.kbeg + t_abs * kBN;
    const int rows = min(dw.kend - k0, kBN);
    const uint32_t nbytes = (uint32_t)((rows - 1) * kv_elems * 2 + D * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb + (size_t)k0 * kv_elems, nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb + (size_t)k0 * kv_elems, nbytes);
#pragma unroll
    for (int j = 0; j < kInstPerWaveTile; ++j) {
      const int i = dw.wave + 8 * j;
      const bool is_k = i < kInstPerTile / 2;
      const int row0 = (is_k ? i : i - kInstPerTile / 2) * kRowsPerInst;
      const int R = row0 + dw.lane / kChunks;
      const uint32_t voff = (uint32_t)(R * kv_elems * 2 + (((dw.lane % kChunks) ^ swz<D>(R)) * 16));
      if (is_k) buffer_load_lds16(rk, lds.k[t_round] + row0 * D, voff);
      else buffer_load_lds16(rv, lds.v[t_round] + row0 * D, voff);
    }
  };

  WaveState<D> ws;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) ws.acc[dt] = f32x16{};
  ws.m = kNegBig;
  ws.l = 0.f;
  for (int r0 = 0; r0 < dw.ntile_all; r0 += kDecTiles) {
    const int nt = min(kDecTiles, dw.ntile_all - r0);
    if (r0 > 0) __syncthreads();  // the previous round's tiles have been consumed
    for (int t = 0; t < nt; ++t) load_tile(t, r0 + t);
    for (int t = 0; t < nt; ++t) {
      // tile t has landed once at most the loads of tiles t+1.. are outstanding
      wait_vmem_upto<kInstPerWaveTile>(kInstPerWaveTile * (nt - 1 - t));
      __syncthreads();
      dec_tile<D>(reinterpret_cast<const char*>(lds.k[t]), reinterpret_cast<const char*>(lds.v[t]),
                  dw, dw.kbeg + (r0 + t) * kBN + 32 * dw.grp, dw.kend, a.scale_log2, ws);
    }
  }
  __syncthreads();  // the tile buffers are free for the merge
  dec_finish<D>(a, dw, reinterpret_cast<float*>(&lds.k[0][0]), ws);
}

// FP8 K/V cache (OCP E4M3; the pages run their decode with an FP8 KV cache,
// paper cards page, Table 11 configurations).  Up to kDec8Tiles 64-key tiles
// of raw bytes are requested at once (half the bytes of bf16); each tile,
// once landed, is widened exactly to bf16 (v_cvt_pk_f32_fp8, then bf16
// packing: every E4M3 value is a bf16 value) into one bf16 K/V tile pair
// shared by the workgroup, and attended as in the bf16 kernel.  The K scale
// is folded into scale_log2 and the V scale into o_mul.
constexpr int kDec8Tiles = 6;

template <int D>
struct LdsDec8 {
  uint8_t k8[kDec8Tiles][kBN * D];
  uint8_t v8[kDec8Tiles][kBN * D];
  uint16_t k[kBN * D];
  uint16_t v[kBN * D];
};

template <int D>
__global__ __launch_bounds__(kPPThreads, 1) void decode_fp8_kernel(DecodeArgs a) {
  __shared__ LdsDec8<D> lds;
  constexpr int kChunks8 = D / 16;                         // 16-byte chunks per fp8 row
  constexpr int kRowsPerInst = 64 / kChunks8;              // 8 (D=128) or 16 (D=64)
  constexpr int kInstPerTile = 2 * (kBN / kRowsPerInst);   // K and V, 1 KB each
  constexpr int kInstPerWaveTile = kInstPerTile / 8;       // 2 (D=128) or 1 (D=64)
  static_assert(kInstPerWaveTile * (kDec8Tiles - 1) < 64 && kDec8Tiles <= 6, "vmcnt range");
  DecWave<D> dw;
  dec_wave_init<D>(a, dw);
  const int row_bytes = a.hkv * D;
  const uint8_t* kb = a.k8 + (size_t)dw.kv_head * D;
  const uint8_t* vb = a.v8 + (size_t)dw.kv_head * D;

  auto load_tile = [&](int t_round, int t_abs) {
    const int k0 = dw.kbeg + t_abs * kBN;
    const int rows = min(dw.kend - k0, kBN);
    const uint32_t nbytes = (uint32_t)((rows - 1) * row_bytes + D);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb + (size_t)k0 * row_bytes, nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb + (size_t)k0 * row_bytes, nbytes);
#pragma unroll
    for (int j = 0; j < kInstPerWaveTile; ++j) {
      const int i = dw.wave + 8 * j;
      const bool is_k = i < kInstPerTile / 2;
      const int row0 = (is_k ? i : i - kInstPerTile / 2) * kRowsPerInst;
      const int R = row0 + dw.lane / kChunks8;
      const uint32_t voff = (uint32_t)(R * row_bytes + (dw.lane % kChunks8) * 16);
      if (is_k) buffer_load_lds16(rk, lds.k8[t_round] + row0 * D, voff);
      else buffer_load_lds16(rv, lds.v8[t_round] + row0 * D, voff);
    }
  };
  // Widen fp8 tile t to the bf16 tile pair: 16-byte chunk c of a tensor is
  // dims 16 (c % kChunks8) .. +15 of row c / kChunks8, written as the two
  // swizzled bf16 chunks of those dims.
  auto widen = [&](int t) {
    for (int ci = threadIdx.x; ci < 2 * kBN * kChunks8; ci += kPPThreads) {
      const bool is_k = ci < kBN * kChunks8;
      const int c = is_k ? ci : ci - kBN * kChunks8;
      const int R = c / kChunks8, c16 = c % kChunks8;
      const u32x4 raw = *reinterpret_cast<const u32x4*>((is_k ? lds.k8[t] : lds.v8[t]) + R * D + c16 * 16);
      uint32_t outw[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[e], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[e], true);
        outw[2 * e] = pack_bf16x2(lo[0], lo[1]);
        outw[2 * e + 1] = pack_bf16x2(hi[0], hi[1]);
      }
      char* dst = reinterpret_cast<char*>(is_k ? lds.k : lds.v) + R * D * 2;
      *reinterpret_cast<u32x4*>(dst + (((2 * c16) ^ swz<D>(R)) * 16)) =
          u32x4{outw[0], outw[1], outw[2], outw[3]};
      *reinterpret_cast<u32x4*>(dst + (((2 * c16 + 1) ^ swz<D>(R)) * 16)) =
          u32x4{outw[4], outw[5], outw[6], outw[7]};
    }
  };

  WaveState<D> ws;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) ws.acc[dt] = f32x16{};
  ws.m = kNegBig;
  ws.l = 0.f;
  for (int r0 = 0; r0 < dw.ntile_all; r0 += kDec8Tiles) {
    const int nt = min(kDec8Tiles, dw.ntile_all - r0);
    for (int t = 0; t < nt; ++t) load_tile(t, r0 + t);
    for (int t = 0; t < nt; ++t) {
      wait_vmem_upto<kInstPerWaveTile>(kInstPerWaveTile * (nt - 1 - t));
      __syncthreads();  // fp8 tile t landed; the bf16 pair is no longer read
      widen(t);
      __syncthreads();  // bf16 pair complete
      dec_tile<D>(reinterpret_cast<const char*>(lds.k), reinterpret_cast<const char*>(lds.v),
                  dw, dw.kbeg + (r0 + t) * kBN + 32 * dw.grp, dw.kend, a.scale_log2, ws);
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
  constexpr int kSlices = D / 8;  // 1 KB slices of a 32 x D fp32 partial
  constexpr int kChunk = 8;
  __shared__ f32x4 red_o[kCombineWaves][64];
  __shared__ float red_m[kCombineWaves][64], red_s[kCombineWaves][64];
  const int ntok32 = (a.q_len + 31) / 32;
  const int slice = blockIdx.x % kSlices;
  const int rest = blockIdx.x / kSlices;
  const int tile = rest % ntok32;
  const int head = rest / ntok32;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane & 31;
  const size_t tile_stride = (size_t)a.hq * ntok32;  // partial tiles per split
  const size_t my_tile = (size_t)head * ntok32 + tile;
  const float* lse_src = a.part_lse + my_tile * 32 + row;
  const f32x4* o_src = reinterpret_cast<const f32x4*>(a.part_o + my_tile * (size_t)(32 * D)) +
                       slice * 64 + lane;
  const size_t lse_step = tile_stride * 32;             // floats between splits
  const size_t o_step = tile_stride * (size_t)(8 * D);  // float4s between splits
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
        y[u] = o_src[(size_t)c * o_step];
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
