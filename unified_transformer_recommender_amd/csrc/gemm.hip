// Contractions of the training step on MFMA: the recomputed projections (W^O + residual, W1 + b1 +
// GELU), the backward products (dX = dY W for every mixed linear layer, dY * GELU' fused), and the
// weight gradients dW = sum over tokens dY^T X (plus the bias gradients as row sums of dY^T), all as
// one grouped NT kernel: both operands hold the contraction index contiguously.
//
// Work unit: one workgroup of GM_NW waves computes GM_NW * 32 token-operand rows by GM_NT
// feature-operand rows. Orientation as in the forward kernels (C^T = B A^T): an accumulator column
// is a token-operand row (lane % 32), its rows are feature-operand rows. The contraction is consumed
// in chunks of 128 bytes per row, brought into LDS by direct global->LDS loads into two chunk
// buffers (the next chunk loads while the current one is multiplied). A chunk's 16-byte pieces p of
// row r sit at slot r * 8 + (p ^ (r & 7)), so a fragment read (one piece of 32 consecutive rows)
// touches every bank once. Lane group g (lane / 32) owns pieces 4g..4g+3 of each chunk for both
// operands, so the contraction order is the same on both sides.
//
// Split contraction: a job may cut k into n_split contiguous chunk ranges, each workgroup writing
// its fp32 partial; launch_reduce sums them in a fixed order (results do not depend on timing).

#include "bwd.hpp"

namespace ot {
namespace {

constexpr int GM_NW = 4;       // waves per workgroup, 32 token rows each
constexpr int GM_NT = 64;      // feature rows per workgroup
constexpr int GM_CB = 128;     // bytes of k per row and chunk
constexpr int GM_NB = 2;       // chunk buffers
constexpr int GM_W_BYTES = GM_NT * GM_CB;
constexpr int GM_X_BYTES = GM_NW * 32 * GM_CB;
constexpr int GM_STAGE_BYTES = GM_W_BYTES + GM_X_BYTES;
static_assert(GM_NT == 64 && GM_NW == 4, "direct-to-LDS load split: 2 feature and 4 token loads per wave");

__device__ __forceinline__ uint32_t slot_byte(int r, int p) { return (uint32_t)(r * 8 + (p ^ (r & 7))) * 16u; }

__device__ __forceinline__ long long row_off(const Mat2 &m, int j, int i) {
  return j * m.g + (long long)(i / m.rpb) * m.sb + (long long)(i % m.rpb) * m.rs;
}

// Workgroup b runs on XCD b % 8; consecutive tiles (the feature tiles of one token tile, which read
// the same token rows) go to one XCD so that its L2 serves the repeats.
__device__ __forceinline__ int xcd_tile(int b, int n) {
  const int per = n / 8;
  return b < 8 * per ? (b % 8) * per + b / 8 : b;
}

// Derivative of the erf-form GELU, Phi(x) + x phi(x), with Phi from Abramowitz & Stegun 7.1.26 in
// the same form as gelu_as (|error| of Phi <= 1.5e-7 / 2).
__device__ __forceinline__ float gelu_grad(float x) {
  constexpr float p = 0.3275911f * 0.70710678118654752f;
  constexpr float a1 = 0.5f * 0.254829592f, a2 = 0.5f * -0.284496736f, a3 = 0.5f * 1.421413741f,
                  a4 = 0.5f * -1.453152027f, a5 = 0.5f * 1.061405429f;
  constexpr float neg_half_log2e = -0.72134752044448170f;
  constexpr float inv_sqrt_2pi = 0.3989422804014327f;
  const float ax = fabsf(x);
  const float t = 1.0f / fmaf(p, ax, 1.0f);
  const float q = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);   // 0.5 erfc(|x| / sqrt 2) / e
  const float e = __builtin_amdgcn_exp2f(x * x * neg_half_log2e);              // exp(-x^2 / 2)
  const float tail = q * e;
  const float cdf = x >= 0.0f ? 1.0f - tail : tail;
  return fmaf(x * inv_sqrt_2pi, e, cdf);
}

// Four consecutive values of a row (storage dtype or fp32) as floats.
template <typename T>
__device__ __forceinline__ f32x4 load4(const T *p) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4 v = *(const bf16x4 *)p;
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  } else {
    return *(const f32x4 *)p;
  }
}

template <typename T>
__global__ __launch_bounds__(GM_NW * 64, 2) void gemm_kernel(const GemmArgs a) {
  using MM = Mma<T>;
  constexpr int ESZ = (int)sizeof(T);
  constexpr int KC = GM_CB / ESZ;             // k elements per chunk
  constexpr int EPP = 16 / ESZ;               // elements per 16-byte piece
  constexpr int SPP = EPP / MM::KPL;          // MFMA k-steps per piece (bf16: 1, fp32: 4)
  constexpr int NTT = GM_NT / 32;             // accumulator tiles per wave
  static_assert(GM_NW * TileStage<float>::SIZE * 4 <= GM_NB * GM_STAGE_BYTES, "staging fits in the ring");
  __shared__ __attribute__((aligned(16))) char ring[GM_NB * GM_STAGE_BYTES];

  const int tile = xcd_tile((int)blockIdx.x, (int)gridDim.x);
  int ji = 0;
#pragma unroll
  for (int i = 1; i < GEMM_MAX_JOBS; ++i)
    if (i < a.n_jobs && tile >= a.job[i].tile0) ji = i;
  const GemmJob &J = a.job[ji];
  int local = tile - J.tile0;
  const int nt = local % J.n_tiles;
  local /= J.n_tiles;
  const int mt = local % J.m_tiles;
  local /= J.m_tiles;
  const int j = local % J.n_groups;
  const int split = local / J.n_groups;
  const int n0 = nt * GM_NT;
  const int mw0 = mt * (GM_NW * 32);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int lc = lane & 31, g = lane >> 5;
  const int m0 = mw0 + wave * 32;

  const int n_all = J.k_len / KC;
  const int per = (n_all + J.n_split - 1) / J.n_split;
  const int c_lo = min(n_all, split * per), c_hi = min(n_all, c_lo + per);
  const int n_chunks = c_hi - c_lo;

  // direct-to-LDS sources: feature rows n0.. of the tile, token rows of this wave (clamped to the
  // last row in the ragged tail, whose results are never stored); byte offsets from the first row
  const long long wrow0 = row_off(J.b, j, n0), xrow0 = row_off(J.a, j, mw0);
  const char *wsrc = (const char *)J.b.base + (wrow0 + (long long)c_lo * KC) * ESZ;
  const char *xsrc = (const char *)J.a.base + (xrow0 + (long long)c_lo * KC) * ESZ;
  uint32_t w_off[2], x_off[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int s = (2 * wave + i) * 64 + lane, r = s / 8, p = (s % 8) ^ (r & 7);
    w_off[i] = (uint32_t)((row_off(J.b, j, n0 + r) - wrow0) * ESZ + p * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = i * 64 + lane, r = s / 8, p = (s % 8) ^ (r & 7);
    const int row = min(m0 + r, J.m - 1);
    x_off[i] = (uint32_t)((row_off(J.a, j, row) - xrow0) * ESZ + p * 16);
  }
  const uint32_t ring_lds = lds_addr(ring);
  auto issue = [&](int c) {
    const uint32_t st = ring_lds + (uint32_t)((c % GM_NB) * GM_STAGE_BYTES);
    const uint32_t cb = (uint32_t)c * GM_CB;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16s(wsrc, w_off[i] + cb, __builtin_amdgcn_readfirstlane(st + (uint32_t)((2 * wave + i) * 1024)));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16s(xsrc, x_off[i] + cb, __builtin_amdgcn_readfirstlane(st + GM_W_BYTES + (uint32_t)(wave * 4096 + i * 1024)));
  };

  // bias of this lane's accumulator rows, loaded before the first direct-to-LDS load
  float bv[NTT][16] = {};
  if (J.bias) {
    const T *bias = (const T *)J.bias + j * J.bias_g + n0;
#pragma unroll
    for (int t = 0; t < NTT; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 b4 = load4<T>(bias + t * 32 + 8 * jj + 4 * g);   // acc_row(4 jj + i, g) = 8 jj + 4 g + i
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[t][4 * jj + i] = b4[i];
      }
  }
  const bool rowsum = J.epi == EPI_PARTIAL && J.rowsum && nt == 0;
  float rsum = 0.0f;
  asm volatile("" ::: "memory");

  f32x16 acc[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) acc[t] = f32x16{};

  if (n_chunks > 0) issue(0);
  for (int c = 0; c < n_chunks; ++c) {
    wait_vm<0>();
    wait_lgkm0();
    bare_barrier();
    if (c + 1 < n_chunks) issue(c + 1);

    const char *st = ring + (c % GM_NB) * GM_STAGE_BYTES;
    const char *xs = st + GM_W_BYTES + wave * 4096;
    u32x4 xb[4], wa[4][NTT];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xb[q] = *(const u32x4 *)(xs + slot_byte(lc, 4 * g + q));
#pragma unroll
      for (int t = 0; t < NTT; ++t) wa[q][t] = *(const u32x4 *)(st + slot_byte(t * 32 + lc, 4 * g + q));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        if constexpr (ESZ == 2) {
          acc[t] = MM::mma(__builtin_bit_cast(bf16x8, wa[q][t]), __builtin_bit_cast(bf16x8, xb[q]), acc[t]);
        } else {
          const f32x4 af = __builtin_bit_cast(f32x4, wa[q][t]), bf = __builtin_bit_cast(f32x4, xb[q]);
#pragma unroll
          for (int e = 0; e < SPP; ++e) acc[t] = MM::mma(af[e], bf[e], acc[t]);
        }
      }
    sched_lds_mfma<4 * (1 + NTT), 4 * NTT * SPP, 6>();
    if (rowsum) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (ESZ == 2) {
          const bf16x8 v = __builtin_bit_cast(bf16x8, xb[q]);
#pragma unroll
          for (int e = 0; e < 8; ++e) rsum += (float)v[e];
        } else {
          const f32x4 v = __builtin_bit_cast(f32x4, xb[q]);
          rsum += (v[0] + v[1]) + (v[2] + v[3]);
        }
      }
    }
  }

  // ---- epilogue ----------------------------------------------------------------------------
  wait_lgkm0();
  bare_barrier();   // every wave is done with the ring; it becomes the staging area
  if (rowsum) {
    const float other = __shfl_xor(rsum, 32, 64);
    if (g == 0 && m0 + lc < J.m) J.rowsum[split * J.rowsum_split + (long long)j * J.m + m0 + lc] = rsum + other;
  }
  const bool tok_ok = m0 + lc < J.m;
  const int my_row = min(m0 + lc, J.m - 1);
#pragma unroll
  for (int t = 0; t < NTT; ++t) {
    f32x16 v = acc[t];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] += bv[t][e];
    const int nb = n0 + t * 32;
    if (J.epi == EPI_STORE && J.resid.base) {
      const long long ro = row_off(J.resid, j, my_row) + nb + 4 * g;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 r4 = J.resid_f32 ? load4<float>((const float *)J.resid.base + ro + 8 * jj)
                                     : load4<T>((const T *)J.resid.base + ro + 8 * jj);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * jj + i] += r4[i];
      }
    }
    if (J.epi == EPI_DGELU) {
      const long long ro = row_off(J.aux, j, my_row) + nb + 4 * g;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 h4 = load4<T>((const T *)J.aux.base + ro + 8 * jj);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * jj + i] *= gelu_grad(h4[i]);
      }
    }
    // feature-major copy: lanes of a half-wave write 32 consecutive tokens of one feature
    if (J.outT.base && tok_ok) {
      T *dst = (T *)J.outT.base + j * J.outT.g + m0 + lc;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float y = J.epi == EPI_GELU ? gelu_as(v[e]) : v[e];
        dst[(long long)(nb + acc_row(e, g)) * J.outT.ld] = from_f32<T>(y);
      }
    }
    // row-major output through the wave's LDS staging tile
    if (J.out.base) {
      const long long split_off = J.epi == EPI_PARTIAL ? split * J.part_split : 0;
      auto store_rows = [&](auto tag) {
        using U = decltype(tag);
        using TS = TileStage<U>;
        U *stg = reinterpret_cast<U *>(ring) + wave * TS::SIZE;
        TS::put(stg, v, lc, g);
        wait_lgkm0();
#pragma unroll
        for (int k = 0; k < TS::NI; ++k) {
          const int m = m0 + TS::token(k, lane);
          const u32x4 piece = TS::get(stg, k, lane);
          if (m < J.m) st16((U *)J.out.base + split_off + row_off(J.out, j, m) + nb + TS::feature(lane), piece);
        }
        wait_lgkm0();
      };
      if (J.epi == EPI_PARTIAL || J.out_f32) store_rows(0.0f);
      else store_rows(T{});
    }
  }
}

// ---- split partial sums ----------------------------------------------------------------------
__global__ __launch_bounds__(256) void reduce_kernel(const RedArgs a) {
  const long long e4 = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e4 >= a.total) return;
  int ji = 0;
#pragma unroll
  for (int i = 1; i < RED_MAX_JOBS; ++i)
    if (i < a.n_jobs && e4 >= a.job[i].start) ji = i;
  const RedJob &J = a.job[ji];
  const long long e = e4 - J.start;
  if (e + 4 <= J.count && ((J.split | e) & 3) == 0) {
    f32x4 s = *(const f32x4 *)(J.src + e);
    for (int k = 1; k < J.n_split; ++k) {
      const f32x4 v = *(const f32x4 *)(J.src + k * J.split + e);
      s += v;
    }
    *(f32x4 *)(J.dst + e) = s;
  } else {
    for (long long x = e; x < min(e + 4, J.count); ++x) {
      float s = J.src[x];
      for (int k = 1; k < J.n_split; ++k) s += J.src[k * J.split + x];
      J.dst[x] = s;
    }
  }
}

}  // namespace

int gemm_tokens_per_tile() { return GM_NW * 32; }
int gemm_features_per_tile() { return GM_NT; }

hipError_t launch_gemm(int dtype, const GemmArgs &a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  if (dtype == 1) hipLaunchKernelGGL(gemm_kernel<bf16>, dim3(grid), dim3(GM_NW * 64), 0, s, a);
  else hipLaunchKernelGGL(gemm_kernel<float>, dim3(grid), dim3(GM_NW * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce(const RedArgs &a, hipStream_t s) {
  if (a.total == 0) return hipSuccess;
  const long long groups = (a.total + 3) / 4;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ot
