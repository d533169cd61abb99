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
//
// The GELU-derivative product runs two contractions through the same chunk ring: first the
// pre-activation Z = A2 B2^T + bias of its output tile, kept in registers as GELU'(Z), then the main
// product. The FFN's pre-activation rows thus never go to memory: its output is as wide as the
// hidden layer, and writing and re-reading it cost more than forming it again on the matrix units.

#include "bwd.hpp"

namespace ot {
namespace {

constexpr int GM_CB = 128;     // bytes of k per row and chunk
constexpr int GM_TOK = 128;    // token-operand rows per workgroup (both layouts)

// Wave layouts of a 4-wave workgroup: WGM x WGN waves, each computing TM x TN accumulator tiles of
// 32 x 32 (TM token tiles, TN feature tiles). Narrow: 4 x 1 waves of 1 x 2 tiles (128 tokens x 64
// features; every feature fragment read feeds one MFMA). Wide: 2 x 2 waves of 2 x 2 tiles
// (128 x 128; every fragment read feeds two MFMAs).
template <int TM_, int TN_, int WGM_, int WGN_, int NB_>
struct Layout {
  static constexpr int TM = TM_, TN = TN_, WGM = WGM_, WGN = WGN_;
  static constexpr int NB = NB_;             // chunk buffers: NB - 1 chunks in flight
  static constexpr int FR = 32 * TN * WGN;   // feature rows per workgroup
  static constexpr int TR = 32 * TM * WGM;   // token rows per workgroup
  static constexpr int STAGE = (FR + TR) * GM_CB;
  static constexpr int LOADS = (FR + TR) * 8 / 256;   // 16-byte direct loads per thread and chunk
  static_assert(WGM * WGN == 4 && TR == GM_TOK, "4 waves, 128 token rows");
  static_assert(NB >= 2 && NB <= 4, "chunk buffers");
};
// Two chunk buffers: measured on the OneTransS training step, three or four buffers (fewer
// workgroups per CU) made the contractions 12-58 % slower.
using Narrow = Layout<1, 2, 4, 1, 2>;
using Wide = Layout<2, 2, 2, 2, 2>;

// Wait until chunk c's direct loads have landed: the loads of the chunks issued after it (at most
// NB - 2, fewer near the end) may stay outstanding.
template <typename LY>
__device__ __forceinline__ void wait_chunk(int after) {
  if constexpr (LY::NB >= 4) {
    if (after >= 2) { wait_vm<2 * LY::LOADS>(); return; }
  }
  if constexpr (LY::NB >= 3) {
    if (after >= 1) { wait_vm<LY::LOADS>(); return; }
  }
  wait_vm<0>();
}

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
// the same form as gelu_as (|error| of Phi <= 1.5e-7 / 2). fp32 storage.
__device__ __forceinline__ float gelu_grad_as(float x) {
  constexpr float p = 0.3275911f * 0.70710678118654752f;
  constexpr float a1 = 0.5f * 0.254829592f, a2 = 0.5f * -0.284496736f, a3 = 0.5f * 1.421413741f,
                  a4 = 0.5f * -1.453152027f, a5 = 0.5f * 1.061405429f;
  constexpr float neg_half_log2e = -0.72134752044448170f;
  constexpr float inv_sqrt_2pi = 0.3989422804014327f;
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(p, ax, 1.0f));
  const float q = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);   // 0.5 erfc(|x| / sqrt 2) / e
  const float e = __builtin_amdgcn_exp2f(x * x * neg_half_log2e);              // exp(-x^2 / 2)
  const float tail = q * e;
  const float cdf = x >= 0.0f ? 1.0f - tail : tail;
  return fmaf(x * inv_sqrt_2pi, e, cdf);
}

// Derivative of the bf16 paths' GELU x sigma(z), z = x (A1 + A3 x^2) (gelu_fit, the function the
// bf16 forward evaluates): sigma(z) (1 + x (1 - sigma(z)) (A1 + 3 A3 x^2)), with
// 1 - sigma(z) = e^-z sigma(z).
__device__ __forceinline__ float gelu_grad_fit(float x) {
  constexpr float L = -1.4426950408889634f;   // -log2(e)
  const float x2 = x * x;
  const float e = __builtin_amdgcn_exp2f(x * fmaf(x2, GELU_FIT_A3 * L, GELU_FIT_A1 * L));   // e^-z
  const float sg = __builtin_amdgcn_rcpf(1.0f + e);
  const float dz = fmaf(3.0f * GELU_FIT_A3, x2, GELU_FIT_A1);
  return sg * fmaf(x * e * sg, dz, 1.0f);
}

template <typename T> __device__ __forceinline__ float gelu_of(float x) {
  return sizeof(T) == 2 ? gelu_fit(x) : gelu_as(x);
}
template <typename T> __device__ __forceinline__ float gelu_grad_of(float x) {
  return sizeof(T) == 2 ? gelu_grad_fit(x) : gelu_grad_as(x);
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

template <typename T, typename LY>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const GemmArgs a) {
  using MM = Mma<T>;
  constexpr int ESZ = (int)sizeof(T);
  constexpr int KC = GM_CB / ESZ;             // k elements per chunk
  constexpr int EPP = 16 / ESZ;               // elements per 16-byte piece
  constexpr int SPP = EPP / MM::KPL;          // MFMA k-steps per piece (bf16: 1, fp32: 4)
  constexpr int TM = LY::TM, TN = LY::TN;
  static_assert(4 * TileStage<float>::SIZE * 4 + 4 * 32 * (32 + 16 / ESZ) * ESZ <= LY::NB * LY::STAGE,
                "row-major and feature-major staging fit in the ring");
  __shared__ __attribute__((aligned(16))) char ring[LY::NB * LY::STAGE];

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
  const int n0 = nt * LY::FR;
  const int mw0 = mt * LY::TR;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int lc = lane & 31, g = lane >> 5;
  const int wm = wave % LY::WGM, wn = wave / LY::WGM;
  const int m0 = mw0 + wm * 32 * TM;          // this wave's first token row
  const int f0 = wn * 32 * TN;                // this wave's first feature row within the tile

  // bias of this lane's accumulator rows, loaded before the first direct-to-LDS load
  float bv[TN][16] = {};
  if (J.bias) {
    const T *bias = (const T *)J.bias + j * J.bias_g + n0 + f0;
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 b4 = load4<T>(bias + t * 32 + 8 * jj + 4 * g);   // acc_row(4 jj + i, g) = 8 jj + 4 g + i
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[t][4 * jj + i] = b4[i];
      }
  }
  const bool rowsum = J.epi == EPI_PARTIAL && J.rowsum && nt == 0 && wn == 0;
  float rsum[TM] = {};
  asm volatile("" ::: "memory");

  f32x16 acc[TM][TN];
  const uint32_t ring_lds = lds_addr(ring);

  // acc = sum over chunks [c_lo, c_lo + n_chunks) of A's token rows times Bw's feature rows (the
  // chunk ring starts empty and is free again when this returns)
  auto contract = [&](const Mat2 &A, const Mat2 &Bw, int c_lo, int n_chunks, bool rs) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int t = 0; t < TN; ++t) acc[i][t] = f32x16{};
    // direct-to-LDS loads: instruction i of wave w covers stage slots [(4 i + w) 64, + 64); slot s
    // holds piece (s % 8) ^ (row & 7) of stage row s / 8 (feature rows first, then token rows; a
    // token row past the end re-reads the last row, whose results are never stored)
    const long long wrow0 = row_off(Bw, j, n0), xrow0 = row_off(A, j, mw0);
    const char *wsrc = (const char *)Bw.base + (wrow0 + (long long)c_lo * KC) * ESZ;
    const char *xsrc = (const char *)A.base + (xrow0 + (long long)c_lo * KC) * ESZ;
    uint32_t off[LY::LOADS];
#pragma unroll
    for (int i = 0; i < LY::LOADS; ++i) {
      const int s = (4 * i + wave) * 64 + lane, r = s / 8, p = (s % 8) ^ (r & 7);
      if (r < LY::FR) {
        off[i] = (uint32_t)((row_off(Bw, j, n0 + r) - wrow0) * ESZ + p * 16);
      } else {
        const int row = min(mw0 + r - LY::FR, J.m - 1);
        off[i] = (uint32_t)((row_off(A, j, row) - xrow0) * ESZ + p * 16);
      }
    }
    auto issue = [&](int c) {
      const uint32_t st = ring_lds + (uint32_t)((c % LY::NB) * LY::STAGE);
      const uint32_t cb = (uint32_t)c * GM_CB;
#pragma unroll
      for (int i = 0; i < LY::LOADS; ++i) {
        const bool feat = (4 * i + wave) * 8 < LY::FR;   // wave-uniform: 8 rows per instruction
        dma16s(feat ? (const void *)wsrc : (const void *)xsrc, off[i] + cb,
               __builtin_amdgcn_readfirstlane(st + (uint32_t)((4 * i + wave) * 1024)));
      }
    };
#pragma unroll
    for (int c = 0; c < LY::NB - 1; ++c)
      if (c < n_chunks) issue(c);
    for (int c = 0; c < n_chunks; ++c) {
      wait_chunk<LY>(min(LY::NB - 2, n_chunks - 1 - c));
      wait_lgkm0();
      bare_barrier();   // every wave's loads of chunk c have landed; chunk c - 1's buffer is free
      if (c + LY::NB - 1 < n_chunks) issue(c + LY::NB - 1);

      const char *st = ring + (c % LY::NB) * LY::STAGE;
      const char *xs = st + LY::FR * GM_CB;
      u32x4 xb[4][TM], wa[4][TN];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int i = 0; i < TM; ++i) xb[q][i] = *(const u32x4 *)(xs + slot_byte(wm * 32 * TM + i * 32 + lc, 4 * g + q));
#pragma unroll
        for (int t = 0; t < TN; ++t) wa[q][t] = *(const u32x4 *)(st + slot_byte(f0 + t * 32 + lc, 4 * g + q));
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            if constexpr (ESZ == 2) {
              acc[i][t] = MM::mma(__builtin_bit_cast(bf16x8, wa[q][t]), __builtin_bit_cast(bf16x8, xb[q][i]), acc[i][t]);
            } else {
              const f32x4 af = __builtin_bit_cast(f32x4, wa[q][t]), bf = __builtin_bit_cast(f32x4, xb[q][i]);
#pragma unroll
              for (int e = 0; e < SPP; ++e) acc[i][t] = MM::mma(af[e], bf[e], acc[i][t]);
            }
          }
      sched_lds_mfma<4 * (TM + TN), 4 * TM * TN * SPP, 6>();
      if (rs) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            if constexpr (ESZ == 2) {
              const bf16x8 v = __builtin_bit_cast(bf16x8, xb[q][i]);
#pragma unroll
              for (int e = 0; e < 8; ++e) rsum[i] += (float)v[e];
            } else {
              const f32x4 v = __builtin_bit_cast(f32x4, xb[q][i]);
              rsum[i] += (v[0] + v[1]) + (v[2] + v[3]);
            }
          }
      }
    }
    wait_lgkm0();
    bare_barrier();   // every wave is done with the ring
  };

  // DGELU: the gate GELU'(Z) from a first contraction (the pre-activation never goes to memory)
  f32x16 gate[TM][TN];
  if (J.epi == EPI_DGELU) {
    contract(J.a2, J.b2, 0, J.k_len2 / KC, false);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) gate[i][t][e] = gelu_grad_of<T>(acc[i][t][e] + bv[t][e]);
  }

  const int n_all = J.k_len / KC;
  const int per = (n_all + J.n_split - 1) / J.n_split;
  const int c_lo = min(n_all, split * per), c_hi = min(n_all, c_lo + per);
  contract(J.a, J.b, c_lo, c_hi - c_lo, rowsum);

  // ---- epilogue (the ring becomes the staging area) -------------------------------------------
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int mi = m0 + i * 32;               // first token row of this accumulator tile
    if (rowsum) {
      const float other = __shfl_xor(rsum[i], 32, 64);
      if (g == 0 && mi + lc < J.m) J.rowsum[split * J.rowsum_split + (long long)j * J.m + mi + lc] = rsum[i] + other;
    }
    const int my_row = min(mi + lc, J.m - 1);
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      f32x16 v = acc[i][t];
      if (J.epi != EPI_DGELU) {   // (DGELU: the bias belongs to the pre-activation)
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] += bv[t][e];
      }
      const int nb = n0 + f0 + t * 32;
      if (J.epi == EPI_STORE && J.resid.base) {
        const long long ro = row_off(J.resid, j, my_row) + nb + 4 * g;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 r4 = J.resid_f32 ? load4<float>((const float *)J.resid.base + ro + 8 * jj)
                                       : load4<T>((const T *)J.resid.base + ro + 8 * jj);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * jj + e] += r4[e];
        }
      }
      if (J.epi == EPI_DGELU) {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] *= gate[i][t][e];
      }
      // feature-major copy through the wave's transposed staging tile [32 features][32 tokens]:
      // each 16-byte store holds consecutive tokens of one feature
      if (J.outT.base) {
        constexpr int EPC = 16 / ESZ, LDT = 32 + EPC, PPF = 32 / EPC;
        T *stT = reinterpret_cast<T *>(ring + 4 * TileStage<float>::SIZE * 4) + wave * 32 * LDT;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float y = J.epi == EPI_GELU ? gelu_of<T>(v[e]) : v[e];
          stT[acc_row(e, g) * LDT + lc] = from_f32<T>(y);
        }
        wait_lgkm0();
        T *dst = (T *)J.outT.base + j * J.outT.g + mi;
#pragma unroll
        for (int k = 0; k < 32 * PPF / 64; ++k) {
          const int idx = k * 64 + lane, f = idx / PPF, r = (idx - f * PPF) * EPC;
          const u32x4 piece = *(const u32x4 *)(stT + f * LDT + r);
          T *d = dst + (long long)(nb + f) * J.outT.ld + r;
          if (mi + r + EPC <= J.m) {
            st16(d, piece);
          } else {
            const T *pe = (const T *)&piece;
            for (int e = 0; e < EPC && mi + r + e < J.m; ++e) d[e] = pe[e];
          }
        }
        wait_lgkm0();
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
            const int m = mi + TS::token(k, lane);
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

int gemm_tokens_per_tile() { return GM_TOK; }
int gemm_features_per_tile() { return Narrow::FR; }

// The plan counts Narrow tiles (64 features); when every job's feature rows are a multiple of 128
// the launch uses the Wide layout with its own tile numbering.
hipError_t launch_gemm(int dtype, const GemmArgs &a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  bool wide = true;
  for (int i = 0; i < a.n_jobs; ++i) wide &= a.job[i].n_feat % Wide::FR == 0;
  if (wide) {
    GemmArgs w = a;
    long long tiles = 0;
    for (int i = 0; i < w.n_jobs; ++i) {
      GemmJob &J = w.job[i];
      J.n_tiles = J.n_feat / Wide::FR;
      J.tile0 = (int)tiles;
      tiles += (long long)J.n_split * J.n_groups * J.m_tiles * J.n_tiles;
    }
    if (dtype == 1) hipLaunchKernelGGL((gemm_kernel<bf16, Wide>), dim3((unsigned)tiles), dim3(256), 0, s, w);
    else hipLaunchKernelGGL((gemm_kernel<float, Wide>), dim3((unsigned)tiles), dim3(256), 0, s, w);
  } else {
    if (dtype == 1) hipLaunchKernelGGL((gemm_kernel<bf16, Narrow>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<float, Narrow>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const RedArgs &a, hipStream_t s) {
  if (a.total == 0) return hipSuccess;
  const long long groups = (a.total + 3) / 4;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ot
