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
//                       read at the start and end of workgroup 0, so the
//                       caller gets both the MFMA rate and the clock it ran at.
//   bca_probe_empty  -- a kernel that does nothing (launch cost).
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
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = c1 - c0;
    clocks[1] = t1 - t0;
  }
}

__global__ void probe_empty_kernel() {}

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
// 32x32x16 (32,768 FLOP each); out needs wgs * 256 floats, clocks two
// uint64 (shader clock cycles, then 100 MHz real-time ticks, of workgroup 0).
int bca_probe_mfma(int iters, int wgs, void* out, void* clocks, void* stream) {
  if (!out || !clocks || wgs < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(wgs), dim3(256), 0, (hipStream_t)stream, iters,
                     (float*)out, (unsigned long long*)clocks);
  return (int)hipGetLastError();
}

int bca_probe_empty(void* stream) {
  hipLaunchKernelGGL(probe_empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

}  // extern "C"
