// Pieces shared by the bf16 forward and decode kernels (gfx950): tile sizes,
// the per-wave online-softmax state and the epilogue that writes a wave's rows.
#pragma once

#include "bca_device.hpp"
#include "bca_kernels.hpp"

namespace bca {
namespace {
constexpr int kBN = 64;    // keys per tile
constexpr int kRows = 32;  // query rows per wave
constexpr float kRescaleSlack = 8.0f;  // log2 units a row max may grow before rescaling
constexpr int kPPThreads = 512;  // 8-wave workgroups

template <int D>
struct WaveState {
  f32x16 acc[D / 32];  // O^T accumulator: lane holds query lane%32
  float m;             // running max (log2 domain), identical in lanes l and l^32
  float l;             // lane-local partial running sum
};

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

}  // namespace
}  // namespace bca
