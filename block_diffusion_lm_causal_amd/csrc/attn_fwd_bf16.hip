// bf16 MFMA forward for block-causal / staircase attention on gfx950 (CDNA4).
//
// Attention computed: "On-Policy Residual Learning for Diffusion Language
// Models" -- block-causal attention (thread page, highlight 3), staircase
// packed replay of captured denoising states (paper cards page, Figure 3
// caption; thread page, Insight 3).  The admitted-key rule is in
// bca_device.hpp; the decode step is in attn_decode_bf16.hip.
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
#include "attn_common.hpp"


namespace bca {
namespace {

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

// ---------------------------------------------------------------------------
// Ping-pong forward: 8 waves in two groups of 4 (A = waves 0-3, B = waves 4-7,
// one wave of each group per SIMD).  Both groups consume the same K/V tiles;
// B runs one phase behind A, so on every SIMD one wave is in an MFMA phase
// (S^T of tile t and O^T += V^T P^T of tile t-1) while the other is in its
// softmax phase (VALU), and they swap at each barrier.  Phases 2t and 2t+1:
//   A: MFMA(t), then softmax(t);   B: softmax(t-1), then MFMA(t).
// Each group runs its own straight-line loop (two barriers per iteration, so
// both groups pass the same barriers), which keeps S and P in fixed registers.
// Each group loads at the start of its softmax phase, where the issue (a few
// hundred cycles of the address unit) does not lengthen an MFMA phase: B
// issues V(t) in phase 2t, A issues K(t+1) in phase 2t+1, into the buffers
// last read in phase 2t-1 (double buffers), and each waits for its own loads
// at the end of phase 2t+1.


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
  // of tile t-1 (t >= 1) and S^T of tile t (t < ntile).  With both products
  // the MFMAs alternate (P V, S, P V, S, ...), so the two transposed V reads
  // of one and the K read of the other spread evenly over the phase instead
  // of the 32 V reads crowding the LDS at its start.  par = t & 1 selects the
  // buffers: K(t) in k[par], V(t-1) in v[par ^ 1].
  auto mfma_phase = [&](int t, bool do_pv, bool do_s, int par) {
    if (rescale_prev) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) ws.acc[dt] *= alpha_prev;
    }
    if (do_pv && do_s) {
      const char* vt = reinterpret_cast<const char*>(lds.v[par ^ 1]);
      const char* kt = reinterpret_cast<const char*>(lds.k[par]);
      constexpr int kN = kBN * D / 512;  // MFMAs of each product per tile
      constexpr int kAh = 2;             // MFMA pairs whose operands are read ahead
      auto vfrag = [&](int i) {
        const int c = i / (D / 32), dt = i % (D / 32);
        const s16x4 lo = lds_read_tr16(vt + voff[dt][0] + c * 16 * D * 2);
        const s16x4 hi = lds_read_tr16(vt + voff[dt][1] + c * 16 * D * 2);
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
      };
      auto kfrag = [&](int i) {
        return *reinterpret_cast<const bf16x8*>(kt + koff[i / 2] + (i % 2) * 32 * D * 2);
      };
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 va[kAh], kb[kAh];
#pragma unroll
      for (int i = 0; i < kAh; ++i) {
        va[i] = vfrag(i);
        kb[i] = kfrag(i);
      }
#pragma unroll
      for (int h = 0; h < kBN / 32; ++h) s[h] = f32x16{};
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        const int c = i / (D / 32), dt = i % (D / 32);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[c][0], pk[c][1], pk[c][2], pk[c][3]});
        ws.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % kAh], pb, ws.acc[dt], 0, 0, 0);
        s[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[i % kAh], qf[i / 2], s[i % 2], 0, 0, 0);
        if (i + kAh < kN) {
          va[i % kAh] = vfrag(i + kAh);
          kb[i % kAh] = kfrag(i + kAh);
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
    } else if (do_pv) {
      pv_update<D>(reinterpret_cast<const char*>(lds.v[par ^ 1]), voff, pk, ws);
    } else if (do_s) {
      // K fragments (kk, h) in order i = 2 kk + h, read kAhead ahead of use
      // so that LDS latency hides behind the MFMAs; the scheduling groups
      // below pin that order (left alone, the scheduler reads only two ahead).
      const char* kt = reinterpret_cast<const char*>(lds.k[par]);
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
    // Row max of the lane's 32 scores: four independent chains of
    // three-input maxima (v_max3_f32), 18 instructions.
    float mc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& v = s[c >> 1];
      const int o = (c & 1) * 8;
      float m = fmaxf(fmaxf(v[o + 0], v[o + 1]), v[o + 2]);
      m = fmaxf(fmaxf(m, v[o + 3]), v[o + 4]);
      m = fmaxf(fmaxf(m, v[o + 5]), v[o + 6]);
      mc[c] = fmaxf(m, v[o + 7]);
    }
    const float mloc = xhalf_max(fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]))) * scale_log2;
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
    // P must be complete within this phase: the compiler would otherwise move
    // the exponentials past the barrier, next to the P V product that uses
    // them, which puts this group's VALU work into its own MFMA phase.
#pragma unroll
    for (int c = 0; c < kBN / 16; ++c)
      asm volatile("" ::"v"(pk[c][0]), "v"(pk[c][1]), "v"(pk[c][2]), "v"(pk[c][3]), "v"(lsum));
  };

  // Loads, each at the start of its group's softmax phase, where the issue
  // (a few hundred cycles of the address unit) does not lengthen an MFMA
  // phase: group B issues V(t) in phase 2t, group A K(t+1) in phase 2t+1.
  // Both go into buffers last read in phase 2t-1 and are waited for (vmcnt)
  // by their issuer at the end of phase 2t+1, before phase 2t+2 reads them.
  auto issue_k = [&](int t) {
    if (t < ntile) ld.issue(p.k, kv_stride, tile_k0(t), tile_end(t), lds.k[t & 1]);
  };
  auto issue_v = [&](int t) {
    if (t < ntile) ld.issue(p.v, kv_stride, tile_k0(t), tile_end(t), lds.v[t & 1]);
  };

  // Phase barriers are barrier_lds(), except the one ending phase 2t+1,
  // which first waits (vmcnt) for the loads of the iteration.
  // The loops are unrolled by two, so the parity of t -- which LDS buffer
  // each phase reads -- is a constant in the code, and every LDS address is
  // a lane offset plus an immediate.
  if (grp == 0) {
    auto step = [&](int t, int par) {
      mfma_phase(t, true, true, par);
      barrier_lds();
      issue_k(t + 1);
      softmax_phase(t);
      wait_vmem_barrier();
    };
    mfma_phase(0, false, true, 0);
    barrier_lds();
    issue_k(1);
    softmax_phase(0);
    wait_vmem_barrier();
    int t = 1;
    for (; t + 1 < ntile; t += 2) {
      step(t, 1);
      step(t + 1, 0);
    }
    if (t < ntile) step(t, 1);
    mfma_phase(ntile, true, false, ntile & 1);
    barrier_lds();
    barrier_lds();
  } else {
    auto step = [&](int t, int par) {
      issue_v(t);
      softmax_phase(t - 1);
      barrier_lds();
      mfma_phase(t, true, true, par);
      wait_vmem_barrier();
    };
    issue_v(0);
    barrier_lds();
    mfma_phase(0, false, true, 0);
    wait_vmem_barrier();
    int t = 1;
    for (; t + 1 < ntile; t += 2) {
      step(t, 1);
      step(t + 1, 0);
    }
    if (t < ntile) step(t, 1);
    softmax_phase(ntile - 1);
    barrier_lds();
    mfma_phase(ntile, true, false, ntile & 1);
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

}  // namespace bca
