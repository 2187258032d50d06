// float32 forward for block-causal / staircase attention (VALU, no MFMA).
//
// Same attention as the bf16 path ("On-Policy Residual Learning for Diffusion
// Language Models": block-causal attention, thread page highlight 3; staircase
// replay, paper cards page Figure 3 caption), kept in float32 end to end for
// callers that need full single precision.  A workgroup of two waves owns 64
// query rows of one head; two lanes share a row, each holding half of the
// head dimension, and combine their partial dot products with one lane swap.
// K and V tiles of 32 keys are staged in LDS and read as broadcasts.
#include "bca_device.hpp"
#include "bca_kernels.hpp"

namespace bca {
namespace {

constexpr int kF32Threads = 128;
constexpr int kF32Rows = 64;  // query rows per workgroup
constexpr int kF32BN = 32;    // keys per tile

template <int D>
__global__ __launch_bounds__(kF32Threads) void fwd_f32_kernel(FwdF32Args a) {
  constexpr int DH = D / 2;  // dims per lane
  __shared__ float ks[kF32BN][D];
  __shared__ float vs[kF32BN][D];

  const int w = blockIdx.x;
  const int head = w % a.hq;
  const int rest = w / a.hq;
  const int seg = rest % a.nseq;
  const int rank = rest / a.nseq;
  const int base = a.cu_seqlens[seg];
  const int L = a.cu_seqlens[seg + 1] - base;
  const int ntiles = (L + kF32Rows - 1) / kF32Rows;
  if (rank >= ntiles) return;
  const int tile = ntiles - 1 - rank;
  const Stair stair = make_stair(seg, L, a.block_size, a.s_copies, a.group_start, a.group_pe,
                                 a.group_copies);
  const int g = head / (a.hq / a.hkv);

  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int q0 = tile * kF32Rows;
  const int qi = q0 + (tid >> 1);
  const bool valid = qi < L;
  const int q_last = min(q0 + kF32Rows, L) - 1;
  const TileKeys tk = tile_keys(q0, q_last, stair);
  const RowKeys rk = row_keys(valid ? qi : q_last, stair);

  float qv[DH];
  const float* qrow = a.q + ((size_t)(base + (valid ? qi : q_last)) * a.hq + head) * D + half * DH;
#pragma unroll
  for (int e = 0; e < DH; ++e) qv[e] = qrow[e];
  float acc[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) acc[e] = 0.f;
  float m = kNegBig, l = 0.f;

  const float* kb = a.k + (size_t)base * a.hkv * D + (size_t)g * D;
  const float* vb = a.v + (size_t)base * a.hkv * D + (size_t)g * D;
  const int n1 = (tk.r1e + kF32BN - 1) / kF32BN;
  const int n2 = tk.r2e > tk.r2s ? (tk.r2e - tk.r2s + kF32BN - 1) / kF32BN : 0;
  for (int t = 0; t < n1 + n2; ++t) {
    const int k0 = t < n1 ? t * kF32BN : tk.r2s + (t - n1) * kF32BN;
    const int kend = t < n1 ? tk.r1e : tk.r2e;
    for (int idx = tid; idx < kF32BN * D; idx += kF32Threads) {
      const int key = idx / D, e = idx % D;
      const int j = k0 + key;
      const bool in = j < kend;
      ks[key][e] = in ? kb[(size_t)j * a.hkv * D + e] : 0.f;
      vs[key][e] = in ? vb[(size_t)j * a.hkv * D + e] : 0.f;
    }
    __syncthreads();
    float sc[kF32BN];
    float mloc = kNegInf;
#pragma unroll
    for (int key = 0; key < kF32BN; ++key) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DH; ++e) dot = fmaf(qv[e], ks[key][half * DH + e], dot);
      dot += __shfl_xor(dot, 1);
      const int j = k0 + key;
      float x = dot * a.scale_log2;
      if (!(j < kend && admitted(rk, j))) x = kNegInf;
      sc[key] = x;
      mloc = fmaxf(mloc, x);
    }
    const float m_new = fmaxf(m, mloc);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DH; ++e) acc[e] *= alpha;
#pragma unroll
    for (int key = 0; key < kF32BN; ++key) {
      const float p = fast_exp2(sc[key] - m_new);
      l += p;
#pragma unroll
      for (int e = 0; e < DH; ++e) acc[e] = fmaf(p, vs[key][half * DH + e], acc[e]);
    }
    __syncthreads();
  }
  if (!valid) return;
  const float inv = 1.f / l;
  float* orow = a.o + ((size_t)(base + qi) * a.hq + head) * D + half * DH;
#pragma unroll
  for (int e = 0; e < DH; ++e) orow[e] = acc[e] * inv;
  if (half == 0) a.lse[(size_t)head * a.total + base + qi] = (m + fast_log2(l)) * kLn2;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdF32Args& a, int max_seqlen, hipStream_t stream) {
  const int ntiles = (max_seqlen + kF32Rows - 1) / kF32Rows;
  const long long nwg = (long long)ntiles * a.nseq * a.hq;
  if (nwg <= 0) return hipSuccess;
  if (a.d == 128) {
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3((unsigned)nwg), dim3(kF32Threads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3((unsigned)nwg), dim3(kF32Threads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace bca
