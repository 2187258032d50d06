// Machine microbenchmarks for the benchmark's "measured peak" figures
// (libbca_probe.so; not part of the attention library).
//
//   bca_probe_read   -- streaming read of a device buffer: every byte once,
//                       16 bytes per lane per load, eight loads in flight per
//                       lane; the sum of the words goes to one int per
//                       workgroup so the loads cannot be dropped.
//   bca_probe_mfma   -- back-to-back v_mfma_f32_32x32x16_bf16 on every SIMD
//                       (eight independent accumulator chains per wave), with
//                       the shader clock and the 100 MHz real-time counter
//                       read at the start and end of every workgroup, so the
//                       caller gets both the MFMA rate and the clock it ran at.
//   bca_probe_empty  -- a kernel that does nothing (launch cost).
//   bca_probe_mfma_lds -- the MFMA stream of bca_probe_mfma with one 16-byte
//                       LDS read per lane (1 KB per wave) for every MFMA, or
//                       for every second MFMA, each read feeding the next
//                       MFMA's A operand: what the attention kernels' operand
//                       traffic costs the MFMA rate and the clock.
//   bca_probe_valu   -- VALU issue cost: independent v_exp_f32, or v_fma_f32,
//                       or v_exp_f32 beside MFMAs, in eight-wave workgroups.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4_t* __restrict__ src,
                                                         size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4_t v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc += v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = src[i];
    acc += v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int t = 0; t < (int)blockDim.x; ++t) s += red[t];
    sink[blockIdx.x] = s;
  }
}

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* out,
                                                         unsigned long long* clocks) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16_t{};
  const unsigned long long t0 = wall_clock64();
  const unsigned long long c0 = clock64();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  const unsigned long long c1 = clock64();
  const unsigned long long t1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = t1 - t0;
  }
}

__global__ void probe_empty_kernel() {}

// 8 waves; each wave reads its own 1 KB slot of a 64 KB LDS area (conflict
// free) and folds the words into the next MFMA's A operand.
template <int kReadsPer8>
__global__ __launch_bounds__(512) void probe_mfma_lds_kernel(int iters, float* out,
                                                             unsigned long long* clocks) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[16384];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 16384; i += 512) buf[i] = (uint32_t)(i * 2654435761u) & 0x3f803f80u;
  __syncthreads();
  const char* base = reinterpret_cast<const char*>(buf) + wave * 1024 + lane * 16;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
  }
  f32x16_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16_t{};
  const unsigned long long t0 = wall_clock64();
  const unsigned long long c0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      asm volatile("" ::: "memory");  // every read is issued
      if (j % (8 / kReadsPer8) == 0) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(base + ((it * 8 + j) & 7) * 8192);
        a = __builtin_bit_cast(bf16x8_t, v);
      }
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j & 3], 0, 0, 0);
    }
  }
  const unsigned long long c1 = clock64();
  const unsigned long long t1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * blockDim.x + tid] = s;
  if (tid == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = t1 - t0;
  }
}

// Per wave and iteration: kind 0, 16 v_exp_f32 (each after a v_mul_f32);
// kind 1, 64 v_fma_f32; kind 2, 8 MFMAs with 16 v_exp_f32 between them.
// Sixteen independent chains, so issue and not latency sets the pace.
template <int kKind>
__global__ __launch_bounds__(512) void probe_valu_kernel(int iters, float* out,
                                                         unsigned long long* clocks) {
  const int tid = threadIdx.x, lane = tid & 63;
  float e[16], f[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    e[j] = 0.01f * (float)(lane + j);
    f[j] = 0.02f * (float)(lane - j);
  }
  bf16x8_t a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(0.001f * (float)((lane + k) & 7));
    b[k] = (__bf16)(0.002f * (float)k);
  }
  f32x16_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16_t{};
  const unsigned long long t0 = wall_clock64();
  const unsigned long long c0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (kKind == 2) acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j & 3], 0, 0, 0);
      if (kKind != 1) {
        e[2 * j] = __builtin_amdgcn_exp2f(e[2 * j] * -0.5f);
        e[2 * j + 1] = __builtin_amdgcn_exp2f(e[2 * j + 1] * -0.5f);
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) f[(j * 8 + r) & 15] = fmaf(f[(j * 8 + r) & 15], 0.999f, 0.001f);
      }
    }
  }
  const unsigned long long c1 = clock64();
  const unsigned long long t1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += e[j] + f[j];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * blockDim.x + tid] = s;
  if (tid == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = t1 - t0;
  }
}

}  // namespace

extern "C" {

// Reads n_bytes (a multiple of 16) from src with `wgs` workgroups of 256
// threads; sink needs `wgs` uint32 slots.  Returns a hipError_t code.
int bca_probe_read(const void* src, size_t n_bytes, int wgs, void* sink, void* stream) {
  if (!src || !sink || wgs < 1 || (n_bytes & 15)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_read_kernel, dim3(wgs), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4_t*)src, n_bytes / 16, (uint32_t*)sink);
  return (int)hipGetLastError();
}

// `wgs` workgroups of four waves, each wave issuing iters * 8 MFMAs of
// 32x32x16 (32,768 FLOP each); out needs wgs * 256 floats, clocks 2 * wgs
// uint64 (per workgroup: shader clock cycles, then 100 MHz real-time ticks).
int bca_probe_mfma(int iters, int wgs, void* out, void* clocks, void* stream) {
  if (!out || !clocks || wgs < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(wgs), dim3(256), 0, (hipStream_t)stream, iters,
                     (float*)out, (unsigned long long*)clocks);
  return (int)hipGetLastError();
}

// `wgs` workgroups of eight waves, each wave issuing iters * 8 MFMAs with an
// LDS read before every MFMA (every = 1) or every second one (every = 2);
// out needs wgs * 512 floats, clocks as bca_probe_mfma.
int bca_probe_mfma_lds(int iters, int wgs, int every, void* out, void* clocks, void* stream) {
  if (!out || !clocks || wgs < 1 || iters < 1 || (every != 1 && every != 2))
    return (int)hipErrorInvalidValue;
  if (every == 1)
    hipLaunchKernelGGL(probe_mfma_lds_kernel<8>, dim3(wgs), dim3(512), 0, (hipStream_t)stream,
                       iters, (float*)out, (unsigned long long*)clocks);
  else
    hipLaunchKernelGGL(probe_mfma_lds_kernel<4>, dim3(wgs), dim3(512), 0, (hipStream_t)stream,
                       iters, (float*)out, (unsigned long long*)clocks);
  return (int)hipGetLastError();
}

// `wgs` workgroups of eight waves running probe kind 0, 1 or 2 (see above);
// out needs wgs * 512 floats, clocks as bca_probe_mfma.
int bca_probe_valu(int kind, int iters, int wgs, void* out, void* clocks, void* stream) {
  if (!out || !clocks || wgs < 1 || iters < 1 || kind < 0 || kind > 2)
    return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  unsigned long long* c = (unsigned long long*)clocks;
  if (kind == 0)
    hipLaunchKernelGGL(probe_valu_kernel<0>, dim3(wgs), dim3(512), 0, s, iters, (float*)out, c);
  else if (kind == 1)
    hipLaunchKernelGGL(probe_valu_kernel<1>, dim3(wgs), dim3(512), 0, s, iters, (float*)out, c);
  else
    hipLaunchKernelGGL(probe_valu_kernel<2>, dim3(wgs), dim3(512), 0, s, iters, (float*)out, c);
  return (int)hipGetLastError();
}

int bca_probe_empty(void* stream) {
  hipLaunchKernelGGL(probe_empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

}  // extern "C"
