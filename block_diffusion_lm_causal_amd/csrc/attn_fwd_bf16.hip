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
// Work decomposition.  A workgroup is 4 wave64s.  Each wave owns 32 query rows
// of one query head; the workgroup's waves are `hpw` query heads that share a
// KV head (GQA) times 4/hpw consecutive 32-row sub-tiles, so K/V tiles staged
// in LDS serve all of them.  The workgroup walks only the key tiles its rows
// admit (whole masked tiles are never issued), 64 keys at a time, with
// double-buffered LDS and the next tile's global loads in flight while the
// current tile is multiplied.
//
// Per 64-key tile each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (keys on the M axis, its 32 queries on the N axis), so every lane holds 32
// scores of a single query: the row max needs one cross-lane step (lane^32)
// and the running sum stays lane-local until the epilogue.  Probabilities are
// rounded to bf16 and fed straight back as the B operand of O^T += V^T P^T;
// V is stored transposed in LDS with the key order inside each 16-key chunk
// permuted to match the accumulator layout of S^T, so no register shuffles are
// needed between the two products.  Softmax runs in the log2 domain
// (scale * log2(e) folded into one multiply, exp2 on v_exp_f32).
#include "bca_device.hpp"
#include "bca_kernels.hpp"

namespace bca {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;    // keys per tile
constexpr int kRows = 32;  // query rows per wave

template <int D>
struct Lds {
  static constexpr int kKPitch = D + 8;    // bf16 per K row  (row = 68 dwords for D = 128)
  static constexpr int kVPitch = kBN + 8;  // bf16 per V^T row (row = 36 dwords)
  uint16_t k[2][kBN * kKPitch];
  uint16_t vt[2][D * kVPitch];
};

// Position, inside a 16-key chunk of the V^T tile, of key kk (bits 2 and 3
// swapped): lane half 0 of the S^T accumulator holds keys {0-3, 8-11} of every
// 16-key chunk and lane half 1 keys {4-7, 12-15}.
__device__ __forceinline__ int vt_pos(int key) {
  int kk = key & 15;
  return (key & ~15) | (kk & 3) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

template <int D>
struct TileLoader {
  // K: BN*D/8 16-byte chunks, D/8 per key row.  V: (BN/4)*(D/8) items of
  // 4 keys x 8 dims, transposed into V^T on the way into LDS.
  static constexpr int kKChunks = kBN * D / 8 / kThreads;          // per thread
  static constexpr int kVItems = (kBN / 4) * (D / 8);              // total
  static constexpr int kVPerThread = (kVItems + kThreads - 1) / kThreads;
  u32x4 kr[kKChunks];
  u32x4 vr[kVPerThread][4];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ kbase,
                                       const uint16_t* __restrict__ vbase, int row_stride,
                                       int k0, int kend, int tid) {
#pragma unroll
    for (int i = 0; i < kKChunks; ++i) {
      int id = tid + i * kThreads;
      int key = id / (D / 8), ch = id % (D / 8);
      int j = k0 + key;
      if (j < kend) {
        kr[i] = *reinterpret_cast<const u32x4*>(kbase + (size_t)j * row_stride + ch * 8);
      } else {
        kr[i] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < kVPerThread; ++i) {
      int item = tid + i * kThreads;
      int m = item % (kBN / 4), ch = item / (kBN / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int j = k0 + 4 * m + e;
        if (item < kVItems && j < kend) {
          vr[i][e] = *reinterpret_cast<const u32x4*>(vbase + (size_t)j * row_stride + ch * 8);
        } else {
          vr[i][e] = u32x4{0, 0, 0, 0};
        }
      }
    }
  }

  __device__ __forceinline__ void store(Lds<D>& lds, int buf, int tid) {
#pragma unroll
    for (int i = 0; i < kKChunks; ++i) {
      int id = tid + i * kThreads;
      int key = id / (D / 8), ch = id % (D / 8);
      *reinterpret_cast<u32x4*>(&lds.k[buf][key * Lds<D>::kKPitch + ch * 8]) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < kVPerThread; ++i) {
      int item = tid + i * kThreads;
      if (item < kVItems) {
        int m = item % (kBN / 4), ch = item / (kBN / 4);
        int pos = vt_pos(4 * m);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          int w = dd >> 1, sh = (dd & 1) * 16;
          uint32_t lo = ((vr[i][0][w] >> sh) & 0xffffu) | (((vr[i][1][w] >> sh) & 0xffffu) << 16);
          uint32_t hi = ((vr[i][2][w] >> sh) & 0xffffu) | (((vr[i][3][w] >> sh) & 0xffffu) << 16);
          *reinterpret_cast<u32x2*>(&lds.vt[buf][(ch * 8 + dd) * Lds<D>::kVPitch + pos]) =
              u32x2{lo, hi};
        }
      }
    }
  }
};

// Everything a workgroup needs to know about its rows and keys.
struct WgPlan {
  const uint16_t* q;     // query rows of this workgroup's segment (row 0 = segment start)
  const uint16_t* k;     // key rows of the segment, already offset to the KV head
  const uint16_t* v;
  int q_rows;            // valid query rows (segment length, or q_len for decode)
  int q0;                // first query row of the workgroup tile
  int r1s, r1e, r2s, r2e;  // key ranges to visit
  int P, L, B;           // admitted-key rule (decode: P = L = key end, everything admitted)
  int head_wave;         // query head of the calling wave
  int qw0;               // first query row of the calling wave
};

template <int D>
struct WaveState {
  f32x16 acc[D / 32];  // O^T accumulator: lane holds query lane%32
  float m;             // running max (log2 domain), identical in lanes l and l^32
  float l;             // lane-local partial running sum
};

// The tile loop: accumulates softmax(scale * q K^T) V over the planned key
// ranges into ws (unnormalised, with running max and partial sums).
template <int D>
__device__ __forceinline__ void attend(const WgPlan& p, int q_stride, int kv_stride,
                                       float scale_log2, Lds<D>& lds, WaveState<D>& ws) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int qi = p.qw0 + (lane & 31);
  const bool wave_active = p.qw0 < p.q_rows;
  const int qw_last = min(p.qw0 + kRows, p.q_rows) - 1;

  // Query fragments: B operand of S^T = K Q^T, 8 consecutive dims per lane.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 raw = u32x4{0, 0, 0, 0};
    if (qi < p.q_rows) {
      raw = *reinterpret_cast<const u32x4*>(p.q + (size_t)qi * q_stride + kk * 16 + half * 8);
    }
    qf[kk] = __builtin_bit_cast(bf16x8, raw);
  }

  const RowKeys rk = row_keys(qi < p.q_rows ? qi : qw_last, p.P, p.L, p.B);
  const RowKeys rkA = row_keys(p.qw0 < p.q_rows ? p.qw0 : 0, p.P, p.L, p.B);
  const RowKeys rkB = row_keys(wave_active ? qw_last : 0, p.P, p.L, p.B);
  const int first_copy_row = p.qw0 > p.P ? p.qw0 : p.P;
  const int s2_first = (qw_last >= p.P) ? row_keys(first_copy_row, p.P, p.L, p.B).s2 : 0x7fffffff;
  const bool one_copy = rkA.e2 > rkA.s2 && rkA.s2 == rkB.s2;

#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) ws.acc[dt] = f32x16{};
  ws.m = kNegBig;
  ws.l = 0.f;

  const int n1 = (p.r1e - p.r1s + kBN - 1) / kBN;
  const int n2 = p.r2e > p.r2s ? (p.r2e - p.r2s + kBN - 1) / kBN : 0;
  const int ntile = n1 + n2;
  if (ntile == 0) return;

  TileLoader<D> ld;
  ld.load(p.k, p.v, kv_stride, p.r1s, p.r1e, tid);
  ld.store(lds, 0, tid);
  __syncthreads();

  for (int t = 0; t < ntile; ++t) {
    const int buf = t & 1;
    const int k0 = t < n1 ? p.r1s + t * kBN : p.r2s + (t - n1) * kBN;
    const int kend = t < n1 ? p.r1e : p.r2e;
    if (t + 1 < ntile) {
      const int t1 = t + 1;
      const int k0n = t1 < n1 ? p.r1s + t1 * kBN : p.r2s + (t1 - n1) * kBN;
      const int kendn = t1 < n1 ? p.r1e : p.r2e;
      ld.load(p.k, p.v, kv_stride, k0n, kendn, tid);
    }

    const bool skip = !wave_active ||
                      (k0 >= rkB.e1 && (k0 + kBN <= s2_first || k0 >= rkB.e2));
    if (!skip) {
      const bool full = (k0 + kBN <= kend) &&
                        ((k0 + kBN <= rkA.e1) ||
                         (one_copy && k0 >= rkA.s2 && k0 + kBN <= rkA.e2));
      // S^T tile: two 32-key halves.
      f32x16 s[kBN / 32];
#pragma unroll
      for (int h = 0; h < kBN / 32; ++h) s[h] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int h = 0; h < kBN / 32; ++h) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              &lds.k[buf][(h * 32 + (lane & 31)) * Lds<D>::kKPitch + kk * 16 + half * 8]);
          s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[h], 0, 0, 0);
        }
      }
      // Scale, mask, row max.
      float mloc = kNegInf;
#pragma unroll
      for (int h = 0; h < kBN / 32; ++h) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[h][r] * scale_log2;
          if (!full) {
            const int j = k0 + h * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (!(j < kend && admitted(rk, j))) x = kNegInf;
          }
          s[h][r] = x;
          mloc = fmaxf(mloc, x);
        }
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(ws.m, mloc);
      const float alpha = fast_exp2(ws.m - m_new);
      ws.m = m_new;
      float lsum = 0.f;
      uint32_t pk[kBN / 16][4];
#pragma unroll
      for (int h = 0; h < kBN / 32; ++h) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(s[h][r] - m_new);
          const float p1 = fast_exp2(s[h][r + 1] - m_new);
          lsum += p0 + p1;
          pk[h * 2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(p0, p1);
        }
      }
      ws.l = ws.l * alpha + lsum;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) ws.acc[dt] *= alpha;
      // O^T += V^T P^T
#pragma unroll
      for (int c = 0; c < kBN / 16; ++c) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[c][0], pk[c][1], pk[c][2], pk[c][3]});
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              &lds.vt[buf][(dt * 32 + (lane & 31)) * Lds<D>::kVPitch + c * 16 + half * 8]);
          ws.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, ws.acc[dt], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntile) ld.store(lds, buf ^ 1, tid);
    __syncthreads();
  }
}

// Write the normalised rows of a wave: O as bf16 (or float32 partials) and LSE.
template <int D, bool PARTIAL>
__device__ __forceinline__ void write_rows(const WaveState<D>& ws, int qi, bool valid,
                                           void* o_row, float* lse_out) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const float l = ws.l + __shfl_xor(ws.l, 32);
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
  (void)qi;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  __shared__ Lds<D> lds;
  const int ngroups = a.hq / a.hpw;
  const int tok = kRows * (4 / a.hpw);
  const int w = blockIdx.x;
  const int hg = w % ngroups;
  const int rest = w / ngroups;
  const int seg = rest % a.nseq;
  const int rank = rest / a.nseq;

  const int base = a.cu_seqlens[seg];
  const int L = a.cu_seqlens[seg + 1] - base;
  const int ntiles = (L + tok - 1) / tok;
  if (rank >= ntiles) return;
  const int tile = ntiles - 1 - rank;  // costliest (last) tiles of every segment first
  const int S = a.s_copies ? a.s_copies[seg] : 0;
  int P = L - S * a.block_size;
  if (P < 0) P = 0;

  const int wave = threadIdx.x >> 6;
  const int head = hg * a.hpw + wave % a.hpw;
  const int g = head / (a.hq / a.hkv);
  const int kv_head_wg = (hg * a.hpw) / (a.hq / a.hkv);
  (void)g;
  const int q0 = tile * tok;
  const int q_last = min(q0 + tok, L) - 1;
  const TileKeys tk = tile_keys(q0, q_last, P, L, a.block_size);

  WgPlan p;
  p.q = a.q + (size_t)base * a.hq * D + (size_t)head * D;
  p.k = a.k + (size_t)base * a.hkv * D + (size_t)kv_head_wg * D;
  p.v = a.v + (size_t)base * a.hkv * D + (size_t)kv_head_wg * D;
  p.q_rows = L;
  p.q0 = q0;
  p.r1s = 0;
  p.r1e = tk.r1e;
  p.r2s = tk.r2s;
  p.r2e = tk.r2e;
  p.P = P;
  p.L = L;
  p.B = a.block_size;
  p.head_wave = head;
  p.qw0 = q0 + (wave / a.hpw) * kRows;

  WaveState<D> ws;
  attend<D>(p, a.hq * D, a.hkv * D, a.scale_log2, lds, ws);

  const int lane = threadIdx.x & 63;
  const int qi = p.qw0 + (lane & 31);
  const bool valid = qi < L;
  write_rows<D, false>(ws, qi, valid,
                       a.o + ((size_t)(base + qi) * a.hq + head) * D,
                       a.lse + (size_t)head * a.total + base + qi);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void decode_bf16_kernel(DecodeArgs a) {
  __shared__ Lds<D> lds;
  const int ngroups = a.hq / a.hpw;
  const int tok = kRows * (4 / a.hpw);
  const int ntok = (a.q_len + tok - 1) / tok;
  const int w = blockIdx.x;
  const int hg = w % ngroups;
  const int rest = w / ngroups;
  const int tile = rest % ntok;
  const int split = rest / ntok;

  const int wave = threadIdx.x >> 6;
  const int head = hg * a.hpw + wave % a.hpw;
  const int kv_head_wg = (hg * a.hpw) / (a.hq / a.hkv);
  const int kbeg = split * a.chunk;
  const int kend = min(a.kv_len, kbeg + a.chunk);

  WgPlan p;
  p.q = a.q + (size_t)head * D;
  p.k = a.k + (size_t)kv_head_wg * D;
  p.v = a.v + (size_t)kv_head_wg * D;
  p.q_rows = a.q_len;
  p.q0 = tile * tok;
  p.r1s = kbeg;
  p.r1e = kend;
  p.r2s = p.r2e = 0;
  p.P = kend;  // every query row admits every key below the chunk end
  p.L = kend;
  p.B = 0x40000000;
  p.head_wave = head;
  p.qw0 = p.q0 + (wave / a.hpw) * kRows;

  WaveState<D> ws;
  attend<D>(p, a.hq * D, a.hkv * D, a.scale_log2, lds, ws);

  const int lane = threadIdx.x & 63;
  const int qi = p.qw0 + (lane & 31);
  const bool valid = qi < a.q_len;
  if (a.nsplit == 1) {
    write_rows<D, false>(ws, qi, valid, a.o + ((size_t)qi * a.hq + head) * D,
                         a.lse + (size_t)head * a.q_len + qi);
  } else {
    write_rows<D, true>(ws, qi, valid,
                        a.part_o + (((size_t)split * a.q_len + qi) * a.hq + head) * D,
                        a.part_lse + ((size_t)split * a.hq + head) * a.q_len + qi);
  }
}

// Merge the split partials of one (query row, head) per wave:
// lse = log sum_c exp(lse_c);  O = sum_c exp(lse_c - lse) O_c.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // row = qi * hq + head
  if (row >= a.q_len * a.hq) return;
  const int qi = row / a.hq, head = row % a.hq;
  float mx = kNegInf;
  for (int c = lane; c < a.nsplit; c += 64) {
    mx = fmaxf(mx, a.part_lse[((size_t)c * a.hq + head) * a.q_len + qi]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float sum = 0.f;
  for (int c = lane; c < a.nsplit; c += 64) {
    sum += fast_exp2((a.part_lse[((size_t)c * a.hq + head) * a.q_len + qi] - mx) * kLog2e);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  const float lse = mx + fast_log2(sum) * kLn2;
  constexpr int kPer = D / 64;  // dims per lane
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  for (int c = 0; c < a.nsplit; ++c) {
    const float wgt = fast_exp2((a.part_lse[((size_t)c * a.hq + head) * a.q_len + qi] - lse) *
                                kLog2e);
    const float* src = a.part_o + (((size_t)c * a.q_len + qi) * a.hq + head) * D + lane * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[e] += wgt * src[e];
  }
  uint16_t* dst = a.o + ((size_t)qi * a.hq + head) * D + lane * kPer;
  if constexpr (kPer == 2) {
    *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[0], acc[1]);
  } else {
    dst[0] = static_cast<uint16_t>(pack_bf16x2(acc[0], 0.f) & 0xffffu);
  }
  if (lane == 0) a.lse[(size_t)head * a.q_len + qi] = lse;
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int ntiles_max, hipStream_t stream) {
  const int ngroups = a.hq / a.hpw;
  const long long nwg = (long long)ntiles_max * a.nseq * ngroups;
  if (nwg <= 0) return hipSuccess;
  if (a.d == 128) {
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  const int ngroups = a.hq / a.hpw;
  const int tok = kRows * (4 / a.hpw);
  const int ntok = (a.q_len + tok - 1) / tok;
  const long long nwg = (long long)ngroups * ntok * a.nsplit;
  if (nwg <= 0) return hipSuccess;
  if (a.d == 128) {
    hipLaunchKernelGGL(decode_bf16_kernel<128>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_bf16_kernel<64>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nsplit == 1) return err;
  const unsigned nrows = (unsigned)a.q_len * a.hq;
  if (a.d == 128) {
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((nrows + 3) / 4), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((nrows + 3) / 4), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace bca
