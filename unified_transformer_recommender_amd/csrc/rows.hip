// Row-wise kernels of the training step (fun-rec-mdbook 7.5.1: pre-norm RMSNorm / LayerNorm; the
// backward of each norm and of the attention softmax's row term).
//
// One workgroup takes 32 consecutive rows of one row set (a wave takes 8 of them, one row at a
// time; a lane holds E = d / 64 consecutive features). Feature-major outputs are staged in LDS as a
// [d][32] tile and written as 16-byte pieces of consecutive tokens of one feature.
//
// Norm backward (per row, r = 1 / sqrt(mean(x^2) + eps) or 1 / sqrt(var(x) + eps), xhat the
// normalised row, gy = dy * g):
//   RMSNorm:   dx = r (gy - xhat mean(gy xhat))
//   LayerNorm: dx = r (gy - mean(gy) - xhat mean(gy xhat))
//   dg = sum over rows of dy xhat,  db = sum over rows of dy (per-tile partials, summed by colsum)

#include "bwd.hpp"

namespace ot {
namespace {

template <int E, typename T>
__device__ __forceinline__ void load_row(const T *p, float (&v)[E]) {
  if constexpr (sizeof(T) == 4) {
    if constexpr (E >= 4) {
#pragma unroll
      for (int i = 0; i < E; i += 4) {
        const f32x4 x = *(const f32x4 *)(p + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[i + k] = x[k];
      }
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = p[i];
    }
  } else {
    if constexpr (E >= 4) {
#pragma unroll
      for (int i = 0; i < E; i += 4) {
        const bf16x4 x = *(const bf16x4 *)(p + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[i + k] = (float)x[k];
      }
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = (float)p[i];
    }
  }
}

template <int E, typename T>
__device__ __forceinline__ void store_row(T *p, const float (&v)[E]) {
#pragma unroll
  for (int i = 0; i < E; ++i) p[i] = from_f32<T>(v[i]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) x += __shfl_xor(x, k, 64);
  return x;
}

template <typename T>
__device__ __forceinline__ long long row_at(const RowView &v, int b, int t) {
  return (long long)b * v.sb + (long long)(t - v.t_off) * v.rs;
}

template <typename T, int E, int MODE>
__global__ __launch_bounds__(256) void rows_kernel(const RowsArgs a) {
  constexpr int D = 64 * E;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int LDT = 32 + EPC;
  constexpr bool NEED_T = true;
  __shared__ __attribute__((aligned(16))) T sT[NEED_T ? D * LDT : 1];
  __shared__ float sCol[MODE == ROWS_NORM_BWD ? 4 * 2 * D : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int ji = 0;
  if (a.n_jobs > 1 && (int)blockIdx.x >= a.job[1].tile0) ji = 1;
  const RowsJob &J = a.job[ji];
  const int local = blockIdx.x - J.tile0;
  const int j = local / J.m_tiles, mt = local % J.m_tiles;
  const int m = J.rs.n_seq * J.rs.rows;
  const int r0 = mt * 32;
  const int f0 = lane * E;

  float g[E], be[E];
  if constexpr (MODE == ROWS_NORM_FWD || MODE == ROWS_NORM_BWD) {
    load_row<E>((const T *)a.gamma + f0, g);
    if (a.layer) load_row<E>((const T *)a.beta + f0, be);
    else {
#pragma unroll
      for (int i = 0; i < E; ++i) be[i] = 0.0f;
    }
  }
  float cg[E] = {}, cb[E] = {};

  for (int k = 0; k < 8; ++k) {
    const int rr = wave * 8 + k;
    const int r = r0 + rr;
    if (r >= m) break;
    const int b = r / J.rs.rows;
    const int t = J.rs.t0 + j * J.rs.t_step + (r - b * J.rs.rows);
    float x[E], y[E];
    if (a.x_f32) load_row<E>((const float *)a.x.base + row_at<T>(a.x, b, t) + f0, x);
    else load_row<E>((const T *)a.x.base + row_at<T>(a.x, b, t) + f0, x);

    if constexpr (MODE == ROWS_NORM_FWD || MODE == ROWS_NORM_BWD) {
      float mu = 0.0f;
      if (a.layer) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < E; ++i) s += x[i];
        mu = wave_sum(s) * (1.0f / D);
      }
      float s2 = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) s2 += (x[i] - mu) * (x[i] - mu);
      const float rstd = 1.0f / sqrtf(wave_sum(s2) * (1.0f / D) + a.eps);
      float xh[E];
#pragma unroll
      for (int i = 0; i < E; ++i) xh[i] = (x[i] - mu) * rstd;
      if constexpr (MODE == ROWS_NORM_FWD) {
#pragma unroll
        for (int i = 0; i < E; ++i) y[i] = fmaf(xh[i], g[i], be[i]);
      } else {
        float dy[E];
        load_row<E>((const float *)a.dy.base + row_at<T>(a.dy, b, t) + f0, dy);
        float sg = 0.0f, sgx = 0.0f;
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const float gy = dy[i] * g[i];
          sg += gy;
          sgx += gy * xh[i];
          cg[i] += dy[i] * xh[i];
          cb[i] += dy[i];
        }
        const float mgx = wave_sum(sgx) * (1.0f / D);
        const float mg = a.layer ? wave_sum(sg) * (1.0f / D) : 0.0f;
#pragma unroll
        for (int i = 0; i < E; ++i) y[i] = rstd * (dy[i] * g[i] - mg - xh[i] * mgx);
        if (a.res.base && t >= a.res_from) {
          float rv[E];
          load_row<E>((const float *)a.res.base + row_at<T>(a.res, b, t) + f0, rv);
#pragma unroll
          for (int i = 0; i < E; ++i) y[i] += rv[i];
        }
        if (a.out_f32.base) {
          float *o = (float *)a.out_f32.base + row_at<T>(a.out_f32, b, t) + f0;
#pragma unroll
          for (int i = 0; i < E; ++i) o[i] = y[i];
        }
      }
    } else if constexpr (MODE == ROWS_CONVERT) {
#pragma unroll
      for (int i = 0; i < E; ++i) y[i] = x[i];
    } else {   // ROWS_DOT: x = O, dy = dO (storage dtype); D per head
      float dO[E];
      load_row<E>((const T *)a.dy.base + row_at<T>(a.dy, b, t) + f0, dO);
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) s += x[i] * dO[i];
      const int dh = D / a.n_heads;
      const int lph = dh / E;   // lanes per head (a power of two, at least 2 ... 16)
      for (int kk = 1; kk < lph; kk <<= 1) s += __shfl_xor(s, kk, 64);
      if ((lane & (lph - 1)) == 0) a.dvec[(long long)b * a.d_sb + (long long)(f0 / dh) * a.d_R + (t - a.d_p0)] = s;
#pragma unroll
      for (int i = 0; i < E; ++i) y[i] = x[i];
    }

    if (a.out_t.base) store_row<E>((T *)a.out_t.base + row_at<T>(a.out_t, b, t) + f0, y);
    if (J.outT) {
#pragma unroll
      for (int i = 0; i < E; ++i) sT[(f0 + i) * LDT + rr] = from_f32<T>(y[i]);
    }
  }

  if constexpr (MODE == ROWS_NORM_BWD) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      sCol[(wave * 2 + 0) * D + f0 + i] = cg[i];
      sCol[(wave * 2 + 1) * D + f0 + i] = cb[i];
    }
  }
  __syncthreads();
  if constexpr (MODE == ROWS_NORM_BWD) {
    float *dst = a.colpart + (long long)blockIdx.x * 2 * D;
    for (int f = tid; f < 2 * D; f += 256) {
      const int kind = f / D, c = f - kind * D;
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) s += sCol[(w * 2 + kind) * D + c];
      dst[f] = s;
    }
  }
  if (J.outT) {
    // piece pc of feature f: tokens r0 + pc * EPC .. + EPC - 1
    constexpr int PPF = 32 / EPC;
    T *base = (T *)J.outT + j * J.tr_g + r0;
    for (int idx = tid; idx < D * PPF; idx += 256) {
      const int f = idx / PPF, pc = idx - f * PPF;
      const int rb = pc * EPC;
      T *dst = base + (long long)f * J.tr_ld + rb;
      const T *src = &sT[f * LDT + rb];
      if (r0 + rb + EPC <= m) {
        st16(dst, ld16(src));
      } else {
        for (int e = 0; e < EPC && r0 + rb + e < m; ++e) dst[e] = src[e];
      }
    }
  }
}

// Column sums of per-tile partials: one workgroup per 64 columns of one kind (g or b).
__global__ __launch_bounds__(256) void colsum_kernel(const float *part, int n_tiles, int d, float *dst_g, float *dst_b) {
  __shared__ float s[4][64];
  const int groups = d / 64;
  const int kind = blockIdx.x / groups, c0 = (blockIdx.x - kind * groups) * 64;
  float *dst = kind == 0 ? dst_g : dst_b;
  if (!dst) return;
  const int c = c0 + (threadIdx.x & 63), ph = threadIdx.x >> 6;
  float acc = 0.0f;
  for (int t = ph; t < n_tiles; t += 4) acc += part[((long long)t * 2 + kind) * d + c];
  s[ph][threadIdx.x & 63] = acc;
  __syncthreads();
  if (ph == 0) dst[c] = (s[0][threadIdx.x] + s[1][threadIdx.x]) + (s[2][threadIdx.x] + s[3][threadIdx.x]);
}

template <typename T, int E>
hipError_t launch_e(const RowsArgs &a, int grid, hipStream_t s) {
  switch (a.mode) {
    case ROWS_NORM_FWD: hipLaunchKernelGGL((rows_kernel<T, E, ROWS_NORM_FWD>), dim3(grid), dim3(256), 0, s, a); break;
    case ROWS_NORM_BWD: hipLaunchKernelGGL((rows_kernel<T, E, ROWS_NORM_BWD>), dim3(grid), dim3(256), 0, s, a); break;
    case ROWS_CONVERT: hipLaunchKernelGGL((rows_kernel<T, E, ROWS_CONVERT>), dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((rows_kernel<T, E, ROWS_DOT>), dim3(grid), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const RowsArgs &a, int grid, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_e<T, 1>(a, grid, s);
    case 128: return launch_e<T, 2>(a, grid, s);
    case 256: return launch_e<T, 4>(a, grid, s);
    case 512: return launch_e<T, 8>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rows(int dtype, const RowsArgs &a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  return dtype == 1 ? launch_t<bf16>(a, grid, s) : launch_t<float>(a, grid, s);
}

hipError_t launch_colsum(const float *colpart, int n_tiles, int d, float *dst_g, float *dst_b, hipStream_t s) {
  hipLaunchKernelGGL(colsum_kernel, dim3(2 * (d / 64)), dim3(256), 0, s, colpart, n_tiles, d, dst_g, dst_b);
  return hipGetLastError();
}

}  // namespace ot
