// Row-wise and data-movement kernels of the training step (fun-rec-mdbook 7.5.1: pre-norm RMSNorm /
// LayerNorm; the backward of each norm and of the attention softmax's row term), plus the weight
// transposes and zero fills the backward products need.
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

// Column sums of per-tile partials [n_tiles][2][d]: workgroup (p, group) adds tiles
// [p * per, (p + 1) * per) for 64 columns of one kind (g or b) and writes the sum to
// out[p][kind][c]; with one range that is the final column sum. Fixed order, no atomics.
__global__ __launch_bounds__(256) void colsum_kernel(const float *part, int n_tiles, int per, int d, float *out_g,
                                                     float *out_b, long long out_split) {
  __shared__ float s[4][64];
  const int groups = 2 * (d / 64);
  const int gi = blockIdx.x % groups, p = blockIdx.x / groups;
  const int kind = gi / (d / 64), c0 = (gi - kind * (d / 64)) * 64;
  float *dst = kind == 0 ? out_g : out_b;
  if (!dst) return;
  const int c = c0 + (threadIdx.x & 63), ph = threadIdx.x >> 6;
  const int t0 = p * per, t1 = min(n_tiles, t0 + per);
  float acc = 0.0f;
  for (int t = t0 + ph; t < t1; t += 4) acc += part[((long long)t * 2 + kind) * d + c];
  s[ph][threadIdx.x & 63] = acc;
  __syncthreads();
  if (ph == 0)
    dst[p * out_split + c] = (s[0][threadIdx.x] + s[1][threadIdx.x]) + (s[2][threadIdx.x] + s[3][threadIdx.x]);
}

// ---- weight transposes (32 x 32 tiles through LDS) --------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const TrArgs a) {
  __shared__ T tile[32][33];
  const int b = blockIdx.x;
  int ji = 0;
#pragma unroll
  for (int i = 1; i < TR_MAX_JOBS; ++i)
    if (i < a.n_jobs && b >= a.job[i].tile0) ji = i;
  const TrJob &J = a.job[ji];
  const int rt = (J.rows + 31) / 32, ct = (J.cols + 31) / 32;
  int local = b - J.tile0;
  const int tc = local % ct;
  local /= ct;
  const int tr = local % rt;
  const int set = local / rt;
  const T *src = (const T *)J.src + set * J.src_set;
  T *dst = (T *)J.dst + set * J.dst_set;
  const int x = threadIdx.x & 31, y0 = threadIdx.x >> 5;
  for (int y = y0; y < 32; y += 8) {
    const int r = tr * 32 + y, c = tc * 32 + x;
    if (r < J.rows && c < J.cols) tile[y][x] = src[(long long)r * J.cols + c];
  }
  __syncthreads();
  for (int y = y0; y < 32; y += 8) {
    const int c = tc * 32 + y, r = tr * 32 + x;
    if (r < J.rows && c < J.cols) dst[(long long)c * J.dst_ld + J.dst_off + r] = tile[x][y];
  }
}

// ---- zero fills ----------------------------------------------------------------------------------
// One workgroup per contiguous segment (row i of group j of a job): its elements [c0, c1), written
// by consecutive threads (coalesced; 4-byte stores for 4-byte elements, 2-byte otherwise).
__global__ __launch_bounds__(256) void fill_kernel(const FillArgs a) {
  const long long seg = blockIdx.x;
  int ji = 0;
#pragma unroll
  for (int i = 1; i < FILL_MAX_JOBS; ++i)
    if (i < a.n_jobs && seg >= a.job[i].start) ji = i;
  const FillJob &J = a.job[ji];
  const long long x = seg - J.start;
  const int i = (int)(x % J.rows), jg = (int)(x / J.rows);
  char *row = (char *)J.base + ((long long)jg * J.g + (long long)i * J.ld) * J.esz;
  for (int c = J.c0 + (int)threadIdx.x; c < J.c1; c += 256) {
    if (J.esz == 2) *(uint16_t *)(row + (long long)c * 2) = 0;
    else *(uint32_t *)(row + (long long)c * 4) = 0;
  }
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

hipError_t launch_colsum(const float *colpart, int n_tiles, int d, float *dst_g, float *dst_b, float *scratch,
                         hipStream_t s) {
  const int groups = 2 * (d / 64);
  if (n_tiles > COLSUM_PER) {
    // first level: ranges of COLSUM_PER tiles into scratch [ranges][2][d], then their sum
    const int ranges = (n_tiles + COLSUM_PER - 1) / COLSUM_PER;
    hipLaunchKernelGGL(colsum_kernel, dim3(groups * ranges), dim3(256), 0, s, colpart, n_tiles, COLSUM_PER, d,
                       scratch, scratch + d, 2LL * d);
    colpart = scratch;
    n_tiles = ranges;
  }
  hipLaunchKernelGGL(colsum_kernel, dim3(groups), dim3(256), 0, s, colpart, n_tiles, n_tiles, d, dst_g, dst_b, 0LL);
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype, const TrArgs &a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  if (dtype == 1) hipLaunchKernelGGL(transpose_kernel<bf16>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(transpose_kernel<float>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill(const FillArgs &a, hipStream_t s) {
  if (a.total == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)a.total), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ot
