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
//   1. delta = rowsum(dO * O) in float32, one row per 16 lanes.
//   2. dK/dV: a workgroup owns 128 keys of one KV head (32 per wave), keeps
//      its K and V fragments in registers and its dK, dV accumulators in
//      registers, and sweeps every 32-row query tile of every query head of
//      the group that admits any of its keys.  S = Q K^T is computed with
//      queries on the M axis so that the accumulators of P and dS are,
//      unchanged, the A operands of dV += P^T dO and dK += dS^T Q (queries
//      permuted inside each 16-row chunk, matched by the transposed dO and Q
//      tiles staged in LDS).
//   3. dQ: shaped like the forward -- a workgroup owns 32 query rows of up to
//      four query heads sharing a KV head and sweeps the admitted key tiles;
//      S^T = K Q^T and dP^T = V dO^T put one query per lane, so dS^T is the B
//      operand of dQ^T += K^T dS^T with K^T staged in LDS.
#include "bca_device.hpp"
#include "bca_kernels.hpp"

namespace bca {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int perm16(int idx) {
  // bits 2 and 3 swapped: order of rows/keys inside a 16-chunk that matches
  // the register order of a 32x32 MFMA accumulator's lane halves.
  int kk = idx & 15;
  return (idx & ~15) | (kk & 3) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

__device__ __forceinline__ uint32_t bf16_pair(uint32_t a, uint32_t b, int sh) {
  return ((a >> sh) & 0xffffu) | (((b >> sh) & 0xffffu) << 16);
}

// ---------------------------------------------------------------------------
// 1. delta[h][i] = sum_d dO[i,h,d] * O[i,h,d]

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
  }
}

// ---------------------------------------------------------------------------
// 2. dK / dV

constexpr int kKvKeys = 128;  // keys per workgroup (32 per wave)
constexpr int kQt = 32;       // query rows per tile

template <int D>
struct KvLds {
  static constexpr int kRowPitch = D + 8;   // bf16, row-major [32][D]
  static constexpr int kTPitch = kQt + 8;   // bf16, transposed [D][32] (queries permuted)
  uint16_t q[2][kQt * kRowPitch];
  uint16_t qt[2][D * kTPitch];
  uint16_t g[2][kQt * kRowPitch];   // dO
  uint16_t gt[2][D * kTPitch];
  float lse2[2][kQt];   // LSE * log2(e)
  float delta[2][kQt];
};

// One (query tile, head) step's global loads: item = 4 rows x 8 dims of Q or dO.
template <int D>
struct QTileLoader {
  static constexpr int kItems = (kQt / 4) * (D / 8);  // per tensor: 128 (D=128) or 64
  u32x4 r[4];
  float side;  // lse or delta of one row (threads < 2 * kQt)

  __device__ __forceinline__ void load(const BwdArgs& a, int base, int L, int qt0, int head,
                                       int tid) {
    const int tensor = tid / kItems;  // 0: Q, 1: dO, >= 2 idle (D = 64)
    const int item = tid % kItems;
    const int m = item % (kQt / 4), ch = item / (kQt / 4);
    const uint16_t* src = tensor == 0 ? a.q : a.dout;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = qt0 + 4 * m + e;
      if (tensor < 2 && i < L) {
        r[e] = *reinterpret_cast<const u32x4*>(src + ((size_t)(base + i) * a.hq + head) * D + ch * 8);
      } else {
        r[e] = u32x4{0, 0, 0, 0};
      }
    }
    side = 0.f;
    if (tid < 2 * kQt) {
      const int i = qt0 + (tid % kQt);
      if (i < L) {
        side = tid < kQt ? a.lse[(size_t)head * a.total + base + i] * kLog2e
                         : a.delta[(size_t)head * a.total + base + i];
      }
    }
  }

  __device__ __forceinline__ void store(KvLds<D>& s, int buf, int tid) {
    const int tensor = tid / kItems;
    const int item = tid % kItems;
    const int m = item % (kQt / 4), ch = item / (kQt / 4);
    if (tensor < 2) {
      uint16_t* rowm = tensor == 0 ? s.q[buf] : s.g[buf];
      uint16_t* tr = tensor == 0 ? s.qt[buf] : s.gt[buf];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<u32x4*>(&rowm[(4 * m + e) * KvLds<D>::kRowPitch + ch * 8]) = r[e];
      }
      const int pos = perm16(4 * m);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int w = dd >> 1, sh = (dd & 1) * 16;
        *reinterpret_cast<u32x2*>(&tr[(ch * 8 + dd) * KvLds<D>::kTPitch + pos]) =
            u32x2{bf16_pair(r[0][w], r[1][w], sh), bf16_pair(r[2][w], r[3][w], sh)};
      }
    }
    if (tid < kQt) s.lse2[buf][tid] = side;
    else if (tid < 2 * kQt) s.delta[buf][tid - kQt] = side;
  }
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ KvLds<D> lds;
  const int group = a.hq / a.hkv;
  const int w = blockIdx.x;
  const int g = w % a.hkv;
  const int rest = w / a.hkv;
  const int seg = rest % a.nseq;
  const int ktile = rest / a.nseq;  // earliest keys (most query rows) first
  const int base = a.cu_seqlens[seg];
  const int L = a.cu_seqlens[seg + 1] - base;
  const int k0 = ktile * kKvKeys;
  if (k0 >= L) return;
  const int S = a.s_copies ? a.s_copies[seg] : 0;
  int P = L - S * a.block_size;
  if (P < 0) P = 0;
  const int B = a.block_size;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = tid >> 6;
  const int kw0 = k0 + wave * 32;           // this wave's first key
  const int key = kw0 + (lane & 31);        // key of this lane's B-operand column
  const int k_last_wg = min(k0 + kKvKeys, L) - 1;

  // Query rows that admit any key of the workgroup.
  int qs, qe;
  if (k0 < P) {
    qs = (k0 / B) * B;
    qe = L;
  } else {
    const int c_first = (k0 - P) / B, c_last = (k_last_wg - P) / B;
    qs = P + c_first * B;
    qe = min(L, P + (c_last + 1) * B);
  }

  // K and V fragments (B operands of S = Q K^T and dP = dO V^T) stay in registers.
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 rk = u32x4{0, 0, 0, 0}, rv = u32x4{0, 0, 0, 0};
    if (key < L) {
      const size_t off = ((size_t)(base + key) * a.hkv + g) * D + kk * 16 + half * 8;
      rk = *reinterpret_cast<const u32x4*>(a.k + off);
      rv = *reinterpret_cast<const u32x4*>(a.v + off);
    }
    kf[kk] = __builtin_bit_cast(bf16x8, rk);
    vf[kk] = __builtin_bit_cast(bf16x8, rv);
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  const int wave_key_last = min(kw0 + 31, L - 1);
  const bool wave_has_keys = kw0 < L;
  const int nqt = (qe - qs + kQt - 1) / kQt;
  const int nsteps = nqt * group;

  QTileLoader<D> ld;
  if (nsteps > 0) {
    ld.load(a, base, qe, qs, g * group, tid);
    ld.store(lds, 0, tid);
  }
  __syncthreads();

  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    const int qt0 = qs + (st / group) * kQt;
    if (st + 1 < nsteps) {
      const int st1 = st + 1;
      ld.load(a, base, qe, qs + (st1 / group) * kQt, g * group + st1 % group, tid);
    }

    // Does any row of this query tile admit any key of this wave?
    const int qa = qt0, qb = min(qt0 + kQt, qe) - 1;
    const RowKeys ra = row_keys(qa, P, L, B);
    const RowKeys rb = row_keys(qb, P, L, B);
    bool active = wave_has_keys;
    if (active) {
      // rows admit prefix keys up to e1 (non-decreasing in the row) and,
      // for copy rows, their own copy
      const bool hits_prefix = kw0 < rb.e1;
      const int first_copy_row = qa > P ? qa : P;
      const bool hits_copy = qb >= P && kw0 < rb.e2 &&
                             wave_key_last >= row_keys(first_copy_row, P, L, B).s2;
      active = hits_prefix || hits_copy;
    }
    if (active) {
      // every (row, key) of the tile admitted: no padding rows or keys, and the
      // keys inside the prefix part all rows see, or inside the one copy they share
      const bool full = qt0 + kQt <= qe && kw0 + 31 < L &&
                        ((kw0 + 31 < ra.e1) ||
                         (ra.e2 > ra.s2 && ra.s2 == rb.s2 && kw0 >= ra.s2 && kw0 + 31 < ra.e2));
      // S = Q K^T and dP = dO V^T, queries on M, keys on N.
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 qa8 = *reinterpret_cast<const bf16x8*>(
            &lds.q[buf][(lane & 31) * KvLds<D>::kRowPitch + kk * 16 + half * 8]);
        const bf16x8 ga8 = *reinterpret_cast<const bf16x8*>(
            &lds.g[buf][(lane & 31) * KvLds<D>::kRowPitch + kk * 16 + half * 8]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa8, kf[kk], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga8, vf[kk], dp, 0, 0, 0);
      }
      // P and dS; accumulator register r holds query row 8(r/4) + 4 half + r%4.
      uint32_t pp[2][4], pds[2][4];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float pv[2], dsv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int qr = 8 * ((r + e) >> 2) + 4 * half + ((r + e) & 3);
          const float l2 = lds.lse2[buf][qr];
          const float dl = lds.delta[buf][qr];
          float p = fast_exp2(s[r + e] * a.scale_log2 - l2);
          if (!full) {
            const int i = qt0 + qr;
            if (!(i < qe && key < L && admitted(row_keys(i, P, L, B), key))) p = 0.f;
          }
          pv[e] = p;
          dsv[e] = p * (dp[r + e] - dl);
        }
        pp[r >> 3][(r & 7) >> 1] = pack_bf16x2(pv[0], pv[1]);
        pds[r >> 3][(r & 7) >> 1] = pack_bf16x2(dsv[0], dsv[1]);
      }
      // dV += P^T dO and dK += dS^T Q: keys on M, dims on N, queries contracted.
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pp[c][0], pp[c][1], pp[c][2], pp[c][3]});
        const bf16x8 da = __builtin_bit_cast(bf16x8, u32x4{pds[c][0], pds[c][1], pds[c][2], pds[c][3]});
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int row = (dt * 32 + (lane & 31)) * KvLds<D>::kTPitch + c * 16 + half * 8;
          const bf16x8 gb = *reinterpret_cast<const bf16x8*>(&lds.gt[buf][row]);
          const bf16x8 qb8 = *reinterpret_cast<const bf16x8*>(&lds.qt[buf][row]);
          dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, gb, dv[dt], 0, 0, 0);
          dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, qb8, dk[dt], 0, 0, 0);
        }
      }
    }
    if (st + 1 < nsteps) ld.store(lds, buf ^ 1, tid);
    __syncthreads();
  }

  // Epilogue: lane holds dims 32 dt + lane%32 of keys 8(r/4) + 4 half + r%4.
  if (!wave_has_keys) return;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (kr < L) {
        const size_t off = ((size_t)(base + kr) * a.hkv + g) * D + dt * 32 + (lane & 31);
        a.dk[off] = static_cast<uint16_t>(pack_bf16x2(dk[dt][r] * a.scale, 0.f) & 0xffffu);
        a.dv[off] = static_cast<uint16_t>(pack_bf16x2(dv[dt][r], 0.f) & 0xffffu);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ

constexpr int kBN = 64;  // keys per tile

template <int D>
struct DqLds {
  static constexpr int kKPitch = D + 8;
  static constexpr int kTPitch = kBN + 8;
  uint16_t k[2][kBN * kKPitch];
  uint16_t v[2][kBN * kKPitch];
  uint16_t kt[2][D * kTPitch];
};

template <int D>
struct KvTileLoader {
  // item = 4 keys x 8 dims of K and of V
  static constexpr int kItems = (kBN / 4) * (D / 8);  // 256 (D=128) or 128
  u32x4 kr[4], vr[4];

  __device__ __forceinline__ void load(const uint16_t* kb, const uint16_t* vb, int stride, int k0,
                                       int kend, int tid) {
    const int m = tid % (kBN / 4), ch = tid / (kBN / 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = k0 + 4 * m + e;
      if (tid < kItems && j < kend) {
        kr[e] = *reinterpret_cast<const u32x4*>(kb + (size_t)j * stride + ch * 8);
        vr[e] = *reinterpret_cast<const u32x4*>(vb + (size_t)j * stride + ch * 8);
      } else {
        kr[e] = u32x4{0, 0, 0, 0};
        vr[e] = u32x4{0, 0, 0, 0};
      }
    }
  }

  __device__ __forceinline__ void store(DqLds<D>& s, int buf, int tid) {
    if (tid >= kItems) return;
    const int m = tid % (kBN / 4), ch = tid / (kBN / 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<u32x4*>(&s.k[buf][(4 * m + e) * DqLds<D>::kKPitch + ch * 8]) = kr[e];
      *reinterpret_cast<u32x4*>(&s.v[buf][(4 * m + e) * DqLds<D>::kKPitch + ch * 8]) = vr[e];
    }
    const int pos = perm16(4 * m);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int w = dd >> 1, sh = (dd & 1) * 16;
      *reinterpret_cast<u32x2*>(&s.kt[buf][(ch * 8 + dd) * DqLds<D>::kTPitch + pos]) =
          u32x2{bf16_pair(kr[0][w], kr[1][w], sh), bf16_pair(kr[2][w], kr[3][w], sh)};
    }
  }
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a, int hpw) {
  __shared__ DqLds<D> lds;
  const int ngroups = a.hq / hpw;
  const int tok = 32 * (4 / hpw);
  const int w = blockIdx.x;
  const int hg = w % ngroups;
  const int rest = w / ngroups;
  const int seg = rest % a.nseq;
  const int rank = rest / a.nseq;
  const int base = a.cu_seqlens[seg];
  const int L = a.cu_seqlens[seg + 1] - base;
  const int ntiles = (L + tok - 1) / tok;
  if (rank >= ntiles) return;
  const int tile = ntiles - 1 - rank;
  const int S = a.s_copies ? a.s_copies[seg] : 0;
  int P = L - S * a.block_size;
  if (P < 0) P = 0;
  const int B = a.block_size;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = tid >> 6;
  const int head = hg * hpw + wave % hpw;
  const int g = (hg * hpw) / (a.hq / a.hkv);
  const int q0 = tile * tok;
  const int q_last = min(q0 + tok, L) - 1;
  const TileKeys tk = tile_keys(q0, q_last, P, L, B);
  const int qw0 = q0 + (wave / hpw) * 32;
  const int qi = qw0 + (lane & 31);
  const bool wave_active = qw0 < L;
  const int qw_last = min(qw0 + 32, L) - 1;

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
  const RowKeys rk = row_keys(qi < L ? qi : qw_last, P, L, B);
  const RowKeys rkA = row_keys(wave_active ? qw0 : 0, P, L, B);
  const RowKeys rkB = row_keys(wave_active ? qw_last : 0, P, L, B);
  const int first_copy_row = qw0 > P ? qw0 : P;
  const int s2_first = (qw_last >= P) ? row_keys(first_copy_row, P, L, B).s2 : 0x7fffffff;
  const bool one_copy = rkA.e2 > rkA.s2 && rkA.s2 == rkB.s2;

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

  const uint16_t* kb = a.k + (size_t)base * a.hkv * D + (size_t)g * D;
  const uint16_t* vb = a.v + (size_t)base * a.hkv * D + (size_t)g * D;
  const int n1 = (tk.r1e + kBN - 1) / kBN;
  const int n2 = tk.r2e > tk.r2s ? (tk.r2e - tk.r2s + kBN - 1) / kBN : 0;
  const int ntile = n1 + n2;

  KvTileLoader<D> ld;
  if (ntile > 0) {
    ld.load(kb, vb, a.hkv * D, 0, tk.r1e, tid);
    ld.store(lds, 0, tid);
  }
  __syncthreads();
  for (int t = 0; t < ntile; ++t) {
    const int buf = t & 1;
    const int k0 = t < n1 ? t * kBN : tk.r2s + (t - n1) * kBN;
    const int kend = t < n1 ? tk.r1e : tk.r2e;
    if (t + 1 < ntile) {
      const int t1 = t + 1;
      ld.load(kb, vb, a.hkv * D, t1 < n1 ? t1 * kBN : tk.r2s + (t1 - n1) * kBN,
              t1 < n1 ? tk.r1e : tk.r2e, tid);
    }
    const bool skip = !wave_active || (k0 >= rkB.e1 && (k0 + kBN <= s2_first || k0 >= rkB.e2));
    if (!skip) {
      const bool full = (k0 + kBN <= kend) &&
                        ((k0 + kBN <= rkA.e1) || (one_copy && k0 >= rkA.s2 && k0 + kBN <= rkA.e2));
      f32x16 s[kBN / 32], dp[kBN / 32];
#pragma unroll
      for (int h = 0; h < kBN / 32; ++h) {
        s[h] = f32x16{};
        dp[h] = f32x16{};
      }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int h = 0; h < kBN / 32; ++h) {
          const int off = (h * 32 + (lane & 31)) * DqLds<D>::kKPitch + kk * 16 + half * 8;
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&lds.k[buf][off]);
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(&lds.v[buf][off]);
          s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[h], 0, 0, 0);
          dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[kk], dp[h], 0, 0, 0);
        }
      }
      uint32_t pk[kBN / 16][4];
#pragma unroll
      for (int h = 0; h < kBN / 32; ++h) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float dsv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float p = fast_exp2(s[h][r + e] * a.scale_log2 - lse2);
            if (!full) {
              const int j = k0 + h * 32 + 8 * ((r + e) >> 2) + 4 * half + ((r + e) & 3);
              if (!(j < kend && admitted(rk, j))) p = 0.f;
            }
            dsv[e] = p * (dp[h][r + e] - dl);
          }
          pk[h * 2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(dsv[0], dsv[1]);
        }
      }
#pragma unroll
      for (int c = 0; c < kBN / 16; ++c) {
        const bf16x8 db = __builtin_bit_cast(bf16x8, u32x4{pk[c][0], pk[c][1], pk[c][2], pk[c][3]});
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
              &lds.kt[buf][(dt * 32 + (lane & 31)) * DqLds<D>::kTPitch + c * 16 + half * 8]);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, db, acc[dt], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntile) ld.store(lds, buf ^ 1, tid);
    __syncthreads();
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
      hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
    } else {
      hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // 3. dQ
  {
    const int hpw = heads_per_wg(a.hq, a.hkv);
    const int tok = 32 * (4 / hpw);
    const long long ntiles = (max_seqlen + tok - 1) / tok;
    const long long nwg = ntiles * a.nseq * (a.hq / hpw);
    if (a.d == 128) {
      hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, a, hpw);
    } else {
      hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, a, hpw);
    }
    return hipGetLastError();
  }
}

}  // namespace bca
