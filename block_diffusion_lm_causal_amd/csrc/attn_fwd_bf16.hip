// bf16 MFMA forward for block-causal / staircase attention and the split-KV
// decode step on gfx950 (CDNA4).
//
// Attention computed: "On-Policy Residual Learning for Diffusion Language
// Models" -- block-causal attention (thread page, highlight 3), staircase
// packed replay of captured denoising states (paper cards page, Figure 3
// caption; thread page, Insight 3) and the per-block denoising step against a
// prefix KV cache (thread page, Result 4).  The admitted-key rule is in
// bca_device.hpp.
//
// Work decomposition.  A forward workgroup is 8 wave64s.  Each wave owns 32
// query rows of one query head; the waves are `hpw` query heads that share a
// KV head (GQA) times 8/hpw consecutive 32-row sub-tiles, so K/V tiles
// staged in LDS serve all of them.  The workgroup walks only the key tiles its rows admit (whole masked
// tiles are never issued), 64 keys at a time.
//
// Data movement.  K and V tiles go from HBM straight into LDS
// (buffer_load ... lds, 16 bytes per lane), double-buffered, with the next
// tiles in flight while the current one is multiplied.  The buffer resource of
// each tile ends at the tile's last valid key, so rows past it arrive as zeros
// without any per-lane work.  Tiles are stored row-major with a 16-byte chunk
// swizzle (bca_device.hpp) that keeps both LDS read patterns conflict-free.
//
// Math.  Per 64-key tile each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (keys on M, its 32 queries on N, Q held in
// registers), so each lane holds 32 scores of one query: the row max needs a
// single cross-lane step (lane ^ 32) and the row sum stays lane-local until
// the epilogue.  Probabilities are rounded to bf16 and fed back unchanged as
// the B operand of O^T += V^T P^T; the V^T operand comes from the row-major V
// tile through the transposed LDS read (ds_read_b64_tr_b16), in the key order
// the S^T accumulator already has.  Softmax runs in the log2 domain: one FMA
// applies scale * log2(e) and subtracts the running max before v_exp_f32.
// The running max is only moved (and O rescaled) when a row's maximum grows
// by more than 2^8, which keeps P <= 256 and skips almost every rescale.
#include "bca_device.hpp"
#include "bca_kernels.hpp"

namespace bca {
namespace {

constexpr int kBN = 64;    // keys per tile
constexpr int kRows = 32;  // query rows per wave
constexpr float kRescaleSlack = 8.0f;  // log2 units a row max may grow before rescaling

// Everything a workgroup needs to know about its rows and keys.
struct WgPlan {
  const uint16_t* q;     // query rows of this workgroup's segment (row 0 = segment start)
  const uint16_t* k;     // key rows of the segment, already offset to the KV head
  const uint16_t* v;
  int q_rows;            // valid query rows (segment length, or q_len for decode)
  int r1s, r1e, r2s, r2e;  // key ranges to visit
  Stair stair;           // admitted-key rule of the segment
  int qw0;               // first query row of the calling wave
};

template <int D>
struct WaveState {
  f32x16 acc[D / 32];  // O^T accumulator: lane holds query lane%32
  float m;             // running max (log2 domain), identical in lanes l and l^32
  float l;             // lane-local partial running sum
};

// O^T += V^T P^T for one 64-key tile: V^T fragments through the transposed LDS
// read, P^T as the B operand straight from the S^T accumulator layout.
template <int D>
__device__ __forceinline__ void pv_update(const char* vt, const uint32_t (&voff)[D / 32][2],
                                          const uint32_t (&pk)[kBN / 16][4], WaveState<D>& ws) {
#pragma unroll
  for (int c = 0; c < kBN / 16; ++c) {
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[c][0], pk[c][1], pk[c][2], pk[c][3]});
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const s16x4 lo = lds_read_tr16(vt + voff[dt][0] + c * 16 * D * 2);
      const s16x4 hi = lds_read_tr16(vt + voff[dt][1] + c * 16 * D * 2);
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
      ws.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, ws.acc[dt], 0, 0, 0);
    }
  }
}

// Write the normalised rows of a wave: O as bf16 (or float32 partials) and LSE.
template <int D, bool PARTIAL>
__device__ __forceinline__ void write_rows(const WaveState<D>& ws, bool valid, void* o_row,
                                           float* lse_out) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const float l = xhalf_sum(ws.l);
  const float inv = 1.f / l;
  if (!valid) return;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = dt * 32 + 8 * g + 4 * half;
      const float a0 = ws.acc[dt][4 * g + 0] * inv, a1 = ws.acc[dt][4 * g + 1] * inv;
      const float a2 = ws.acc[dt][4 * g + 2] * inv, a3 = ws.acc[dt][4 * g + 3] * inv;
      if (PARTIAL) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(o_row) + d) = f32x4{a0, a1, a2, a3};
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o_row) + d) =
            u32x2{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
      }
    }
  }
  if (half == 0) *lse_out = (ws.m + fast_log2(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// Ping-pong forward: 8 waves in two groups of 4 (A = waves 0-3, B = waves 4-7,
// one wave of each group per SIMD).  Both groups consume the same K/V tiles;
// B runs one phase behind A, so on every SIMD one wave is in an MFMA phase
// (S^T of tile t and O^T += V^T P^T of tile t-1) while the other is in its
// softmax phase (VALU), and they swap at each barrier.  Phases 2t and 2t+1:
//   A: MFMA(t), then softmax(t);   B: softmax(t-1), then MFMA(t).
// Each group runs its own straight-line loop (two barriers per iteration, so
// both groups pass the same barriers), which keeps S and P in fixed registers.
// Only group A loads K/V: in phase 2t, after its own LDS reads, it issues
// K(t+1) and V(t) into the buffers last read in phase 2t-1 (double buffers),
// and waits for them at the end of phase 2t+1.  Group B never has a tile
// load in flight, so none of its LDS reads waits on one.

constexpr int kPPThreads = 512;

template <int D>
struct LdsPP {
  uint16_t k[2][kBN * D];
  uint16_t v[2][kBN * D];
};

// Direct HBM -> LDS loads of one 64-key tile, issued by the 4 waves of group A.
template <int D>
struct PPLoader {
  static constexpr int kChunks = D / 8;                        // 16-byte chunks per row
  static constexpr int kRowsPerInst = 64 / kChunks;            // rows one instruction fills
  static constexpr int kInstPerWave = kBN / kRowsPerInst / 4;  // per tensor
  uint32_t voff[kInstPerWave];
  int lds_row0[kInstPerWave];

  __device__ __forceinline__ void init(int row_bytes, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kInstPerWave; ++i) {
      const int row0 = (i * 4 + wave) * kRowsPerInst;
      const int R = row0 + lane / kChunks;
      const int c = (lane % kChunks) ^ swz<D>(R);  // logical chunk landing in this lane's slot
      voff[i] = (uint32_t)(R * row_bytes + c * 16);
      lds_row0[i] = row0;
    }
  }
  // keys [k0, min(k0 + 64, kend)); rows past kend arrive as zeros
  __device__ __forceinline__ void issue(const uint16_t* base, int row_elems, int k0, int kend,
                                        uint16_t* dst) {
    const int rows = min(kend - k0, kBN);
    const uint32_t nbytes = (uint32_t)((rows - 1) * row_elems * 2 + D * 2);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (size_t)k0 * row_elems, nbytes);
#pragma unroll
    for (int i = 0; i < kInstPerWave; ++i) buffer_load_lds16(r, dst + lds_row0[i] * D, voff[i]);
  }
};

template <int D>
__device__ __forceinline__ void attend_pp(const WgPlan& p, int q_stride, int kv_stride,
                                          float scale_log2, LdsPP<D>& lds, WaveState<D>& ws) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: A, 1: B (one phase behind)
  const int qi = p.qw0 + (lane & 31);
  const bool wave_active = p.qw0 < p.q_rows;
  const int qw_last = min(p.qw0 + kRows, p.q_rows) - 1;

  PPLoader<D> ld;
  ld.init(kv_stride * 2, wave & 3, lane);
  const int n1 = (p.r1e - p.r1s + kBN - 1) / kBN;
  const int n2 = p.r2e > p.r2s ? (p.r2e - p.r2s + kBN - 1) / kBN : 0;
  const int ntile = n1 + n2;
  auto tile_k0 = [&](int t) { return t < n1 ? p.r1s + t * kBN : p.r2s + (t - n1) * kBN; };
  auto tile_end = [&](int t) { return t < n1 ? p.r1e : p.r2e; };
  if (ntile > 0 && grp == 0) ld.issue(p.k, kv_stride, tile_k0(0), tile_end(0), lds.k[0]);

  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 raw = u32x4{0, 0, 0, 0};
    if (qi < p.q_rows) {
      raw = *reinterpret_cast<const u32x4*>(p.q + (size_t)qi * q_stride + kk * 16 + half * 8);
    }
    qf[kk] = __builtin_bit_cast(bf16x8, raw);
  }
  const RowKeys rk = row_keys(qi < p.q_rows ? qi : qw_last, p.stair);
  const RowKeys rkA = row_keys(wave_active ? p.qw0 : 0, p.stair);
  const RowKeys rkB = row_keys(wave_active ? qw_last : 0, p.stair);
  const bool one_copy = rkA.e2 > rkA.s2 && rkA.s2 == rkB.s2;
  // every row of the wave sees the clean keys [0, e1_all)
  const int e1_all = wave_active ? min_prefix_end(p.qw0, qw_last, p.stair) : 0;

  uint32_t koff[D / 16];
  {
    const int sw = swz<D>(lane & 15);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      koff[kk] = (uint32_t)((lane & 31) * D * 2 + (((2 * kk + half) ^ sw) * 16));
  }
  uint32_t voff[D / 32][2];
  {
    const int a = lane & 15, r = a >> 2, q = a & 3, g2 = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int row = 8 * sub + 4 * half + r;
        const int chunk = 4 * dt + 2 * g2 + (q >> 1);
        voff[dt][sub] = (uint32_t)(row * D * 2 + ((chunk ^ swz<D>(row)) * 16) + (q & 1) * 8);
      }
    }
  }

#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) ws.acc[dt] = f32x16{};
  ws.m = kNegBig;
  ws.l = 0.f;
  if (ntile == 0) return;
  wait_vmem();
  __syncthreads();

  f32x16 s[kBN / 32];         // S^T of the tile between its MFMA and softmax phases
  uint32_t pk[kBN / 16][4];   // P^T of the tile between its softmax and P V phases
  float alpha_prev = 1.f;
  bool rescale_prev = false;

  // MFMA phase: the rescale pending from the previous softmax, O^T += V^T P^T
  // of tile t-1 (t >= 1), then S^T of tile t (t < ntile).
  auto mfma_phase = [&](int t, bool do_pv, bool do_s) {
    if (rescale_prev) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) ws.acc[dt] *= alpha_prev;
    }
    if (do_pv) pv_update<D>(reinterpret_cast<const char*>(lds.v[(t - 1) & 1]), voff, pk, ws);
    if (do_s) {
      // K fragments (kk, h) in order i = 2 kk + h, read kAhead ahead of use
      // so that LDS latency hides behind the MFMAs; the scheduling groups
      // below pin that order (left alone, the scheduler reads only two ahead).
      const char* kt = reinterpret_cast<const char*>(lds.k[t & 1]);
      constexpr int kFrags = (D / 16) * (kBN / 32);
      constexpr int kAhead = 4;
      auto frag = [&](int i) {
        return *reinterpret_cast<const bf16x8*>(kt + koff[i / 2] + (i % 2) * 32 * D * 2);
      };
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 kb[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) kb[i] = frag(i);
#pragma unroll
      for (int h = 0; h < kBN / 32; ++h) s[h] = f32x16{};
#pragma unroll
      for (int i = 0; i < kFrags; ++i) {
        s[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[i % kAhead], qf[i / 2], s[i % 2], 0, 0, 0);
        if (i + kAhead < kFrags) kb[i % kAhead] = frag(i + kAhead);
      }
      // issue order: kAhead LDS reads, then (MFMA, read) pairs, then MFMAs
      // (group masks: 0x100 LDS read, 0x008 MFMA)
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
      for (int i = 0; i < kFrags - kAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Softmax phase of tile t: mask (only where the tile is not wholly
  // admitted for this wave), running max with lazy rescale, P in bf16.
  auto softmax_phase = [&](int t) {
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
    float mt[kBN / 4];
#pragma unroll
    for (int h = 0; h < kBN / 32; ++h) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) mt[h * 8 + r / 2] = fmaxf(s[h][r], s[h][r + 1]);
    }
#pragma unroll
    for (int w = kBN / 8; w >= 1; w >>= 1) {
#pragma unroll
      for (int i = 0; i < w; ++i) mt[i] = fmaxf(mt[i], mt[i + w]);
    }
    const float mloc = xhalf_max(mt[0]) * scale_log2;
    const bool grow = mloc > ws.m + kRescaleSlack;
    const float m_new = grow ? mloc : ws.m;
    const float alpha = fast_exp2(ws.m - m_new);
    ws.m = m_new;
    const float neg_m = -m_new;
    float lsum = ws.l * alpha;
#pragma unroll
    for (int h = 0; h < kBN / 32; ++h) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(s[h][r], scale_log2, neg_m));
        const float p1 = fast_exp2(fmaf(s[h][r + 1], scale_log2, neg_m));
        lsum += p0 + p1;
        pk[h * 2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(p0, p1);
      }
    }
    ws.l = lsum;
    rescale_prev = __builtin_amdgcn_ballot_w64(grow) != 0;
    alpha_prev = alpha;
  };

  // Group A's loads in phase 2t: K(t+1) and V(t).
  auto issue = [&](int t) {
    if (t + 1 < ntile) ld.issue(p.k, kv_stride, tile_k0(t + 1), tile_end(t + 1), lds.k[(t + 1) & 1]);
    if (t < ntile) ld.issue(p.v, kv_stride, tile_k0(t), tile_end(t), lds.v[t & 1]);
  };

  // Phase barriers are barrier_lds(): the loads issued in phase 2t stay in
  // flight across the barrier that ends it and are waited for (vmcnt) only at
  // the end of phase 2t+1.
  if (grp == 0) {
    mfma_phase(0, false, true);
    issue(0);
    barrier_lds();
    softmax_phase(0);
    wait_vmem_barrier();
    for (int t = 1; t < ntile; ++t) {
      mfma_phase(t, true, true);
      issue(t);
      barrier_lds();
      softmax_phase(t);
      wait_vmem_barrier();
    }
    mfma_phase(ntile, true, false);
    barrier_lds();
    barrier_lds();
  } else {
    barrier_lds();
    mfma_phase(0, false, true);
    barrier_lds();
    for (int t = 1; t < ntile; ++t) {
      softmax_phase(t - 1);
      barrier_lds();
      mfma_phase(t, true, true);
      barrier_lds();
    }
    softmax_phase(ntile - 1);
    barrier_lds();
    mfma_phase(ntile, true, false);
    barrier_lds();
  }
}

template <int D>
__global__ __launch_bounds__(kPPThreads, 1) void fwd_pp_kernel(FwdArgs a, int ntiles_max) {
  __shared__ LdsPP<D> lds;
  const int ngroups = a.hq / a.hpw;
  const int tok = kRows * (8 / a.hpw);
  // Workgroup order: head group fastest (one KV head per XCD when there are 8),
  // then the tiles of one segment, costliest first, then the next segment --
  // so the workgroups resident on an XCD share one segment's K/V in L2.
  const int w = blockIdx.x;
  const int hg = w % ngroups;
  const int rest = w / ngroups;
  const int rank = rest % ntiles_max;
  const int seg = rest / ntiles_max;

  const int base = a.cu_seqlens[seg];
  const int L = a.cu_seqlens[seg + 1] - base;
  const int ntiles = (L + tok - 1) / tok;
  if (rank >= ntiles) return;
  const int tile = ntiles - 1 - rank;
  const Stair stair = make_stair(seg, L, a.block_size, a.s_copies, a.group_start, a.group_pe,
                                 a.group_copies);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int head = hg * a.hpw + wave % a.hpw;
  const int kv_head = (hg * a.hpw) / (a.hq / a.hkv);
  const int q0 = tile * tok;
  const int q_last = min(q0 + tok, L) - 1;
  const TileKeys tk = tile_keys(q0, q_last, stair);

  WgPlan p;
  p.q = a.q + (size_t)base * a.hq * D + (size_t)head * D;
  p.k = a.k + (size_t)base * a.hkv * D + (size_t)kv_head * D;
  p.v = a.v + (size_t)base * a.hkv * D + (size_t)kv_head * D;
  p.q_rows = L;
  p.r1s = 0;
  p.r1e = tk.r1e;
  p.r2s = tk.r2s;
  p.r2e = tk.r2e;
  p.stair = stair;
  p.qw0 = q0 + (wave / a.hpw) * kRows;

  WaveState<D> ws;
  attend_pp<D>(p, a.hq * D, a.hkv * D, a.scale_log2, lds, ws);

  const int lane = threadIdx.x & 63;
  const int qi = p.qw0 + (lane & 31);
  write_rows<D, false>(ws, qi < L, a.o + ((size_t)(base + qi) * a.hq + head) * D,
                       a.lse + (size_t)head * a.total + base + qi);
}

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

hipError_t launch_fwd_bf16(const FwdArgs& a, int max_seqlen, hipStream_t stream) {
  const int ngroups = a.hq / a.hpw;
  const int tok = kRows * (8 / a.hpw);  // query tokens per 8-wave workgroup
  const long long ntiles = (max_seqlen + tok - 1) / tok;
  const long long nwg = ntiles * a.nseq * ngroups;
  if (nwg <= 0) return hipSuccess;
  if (a.d == 128) {
    hipLaunchKernelGGL(fwd_pp_kernel<128>, dim3((unsigned)nwg), dim3(kPPThreads), 0, stream, a,
                       (int)ntiles);
  } else {
    hipLaunchKernelGGL(fwd_pp_kernel<64>, dim3((unsigned)nwg), dim3(kPPThreads), 0, stream, a,
                       (int)ntiles);
  }
  return hipGetLastError();
}

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
