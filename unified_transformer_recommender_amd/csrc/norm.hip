// Row normalisation (pre-norm of fun-rec-mdbook 7.5.1: RMSNorm, or LayerNorm where configured).
//
// One wave per row; each lane holds d / 64 consecutive elements in fp32 registers, so the row
// is read once and the two reductions (mean for LayerNorm, then the centred sum of squares) are
// wave shuffles. The output is the storage dtype that the following GEMM consumes.

#include "common.hpp"
#include "launch.hpp"

namespace ot {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename TI, typename TO, int PER>
__global__ __launch_bounds__(256) void norm_kernel(const NormArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.n_seq * a.rows) return;
  const int b = row / a.rows, i = row - b * a.rows;
  const TI *x = (const TI *)a.in + b * a.in_sb + (long long)(a.in_i0 + i) * a.d + lane * PER;
  TO *y = (TO *)a.out + b * a.out_sb + (long long)(a.out_i0 + i) * a.d + lane * PER;
  const TO *gm = (const TO *)a.gamma + lane * PER;
  const TO *bt = (const TO *)a.beta + lane * PER;
  float v[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) v[e] = to_f32(x[e]);
  const float inv_d = 1.0f / (float)a.d;
  float mean = 0.0f;
  if (a.layer) {
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < PER; ++e) s += v[e];
    mean = wave_sum(s) * inv_d;
  }
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float c = v[e] - mean;
    ss += c * c;
  }
  const float r = 1.0f / sqrtf(wave_sum(ss) * inv_d + a.eps);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    float o = (v[e] - mean) * r * to_f32(gm[e]);
    if (a.layer) o += to_f32(bt[e]);
    y[e] = from_f32<TO>(o);
  }
}

template <typename TI, typename TO>
static hipError_t launch_per(const NormArgs &a, hipStream_t s) {
  const int rows = a.n_seq * a.rows;
  dim3 gd((rows + 3) / 4), bd(256);
  switch (a.d / 64) {
    case 1: hipLaunchKernelGGL((norm_kernel<TI, TO, 1>), gd, bd, 0, s, a); break;
    case 2: hipLaunchKernelGGL((norm_kernel<TI, TO, 2>), gd, bd, 0, s, a); break;
    case 3: hipLaunchKernelGGL((norm_kernel<TI, TO, 3>), gd, bd, 0, s, a); break;
    case 4: hipLaunchKernelGGL((norm_kernel<TI, TO, 4>), gd, bd, 0, s, a); break;
    case 5: hipLaunchKernelGGL((norm_kernel<TI, TO, 5>), gd, bd, 0, s, a); break;
    case 6: hipLaunchKernelGGL((norm_kernel<TI, TO, 6>), gd, bd, 0, s, a); break;
    case 7: hipLaunchKernelGGL((norm_kernel<TI, TO, 7>), gd, bd, 0, s, a); break;
    case 8: hipLaunchKernelGGL((norm_kernel<TI, TO, 8>), gd, bd, 0, s, a); break;
    case 9: hipLaunchKernelGGL((norm_kernel<TI, TO, 9>), gd, bd, 0, s, a); break;
    case 10: hipLaunchKernelGGL((norm_kernel<TI, TO, 10>), gd, bd, 0, s, a); break;
    case 11: hipLaunchKernelGGL((norm_kernel<TI, TO, 11>), gd, bd, 0, s, a); break;
    case 12: hipLaunchKernelGGL((norm_kernel<TI, TO, 12>), gd, bd, 0, s, a); break;
    case 13: hipLaunchKernelGGL((norm_kernel<TI, TO, 13>), gd, bd, 0, s, a); break;
    case 14: hipLaunchKernelGGL((norm_kernel<TI, TO, 14>), gd, bd, 0, s, a); break;
    case 15: hipLaunchKernelGGL((norm_kernel<TI, TO, 15>), gd, bd, 0, s, a); break;
    case 16: hipLaunchKernelGGL((norm_kernel<TI, TO, 16>), gd, bd, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_norm(int dtype, int in_f32, const NormArgs &a, hipStream_t s) {
  if (a.n_seq * a.rows == 0) return hipSuccess;
  if (dtype == 1) return in_f32 ? launch_per<float, bf16>(a, s) : launch_per<bf16, bf16>(a, s);
  return launch_per<float, float>(a, s);
}

}  // namespace ot
