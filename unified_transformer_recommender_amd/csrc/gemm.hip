// Mixed-parameter grouped GEMM with fused epilogues (gfx950, MFMA 32x32).
//
// The OneTrans projections apply W_S to every S row and W_NS,j to NS token j (fun-rec-mdbook
// 7.5.1, conditional parameterization; the same for the Mixed FFN). One launch covers every
// parameter set of a projection: the S rows of all sequences form one group multiplied by W_S,
// and NS token j of all sequences forms group j multiplied by W_NS,j. Each workgroup computes a
// BM x BN tile of one group with one parameter set, so the weights of a tile are one contiguous
// [BN][K] slab and the A rows are gathered by (sequence, position).
//
// Dataflow per workgroup: 256 threads = 4 waves in a 2x2 grid, each wave owning (BM/2) x (BN/2)
// of the tile as 32x32 MFMA accumulators. A and W tiles [rows][BK] (k contiguous, the layout of
// both operands in memory) are staged through LDS in two buffers: the global loads of k-tile
// kt+1 are issued before the MFMAs of k-tile kt, stored to the other buffer afterwards, and one
// barrier per k-tile separates the two.
//
// Epilogue: each fp32 accumulator is rounded to the storage dtype and written to its head-split
// Q/K/V (or K/V cache) row.

#include "common.hpp"
#include "launch.hpp"

namespace ot {

template <typename T, int BM, int BN, int BK>
struct GemmTile {
  static constexpr int EPC = 16 / (int)sizeof(T);    // elements per 16-byte chunk
  static constexpr int LDK = BK + EPC;                // padded LDS row (elements)
  static constexpr int WM = BM / 2, WN = BN / 2;      // wave tile
  static constexpr int TM = WM / 32, TN = WN / 32;    // MFMA tiles per wave
  static constexpr int CPR = BK / EPC;                // chunks per tile row
  static constexpr int A_CPT = BM * CPR / 256;        // A chunks per thread
  static constexpr int B_CPT = BN * CPR / 256;
  static_assert(A_CPT >= 1 && B_CPT >= 1, "tile too small for 256 threads");
  static_assert(BM * CPR % 256 == 0 && BN * CPR % 256 == 0, "tile/thread mismatch");
};

__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

template <typename T, int BM, int BN, int BK>
__global__ __launch_bounds__(256) void mixed_gemm_kernel(const GemmArgs args) {
  using G = GemmTile<T, BM, BN, BK>;
  using M = Mma<T>;
  using frag = typename M::frag;
  __shared__ __attribute__((aligned(16))) T sA[2][BM * G::LDK];
  __shared__ __attribute__((aligned(16))) T sB[2][BN * G::LDK];
  __shared__ int s_b[BM];
  __shared__ int s_t[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lc = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- which job / parameter group / tile --------------------------------------------------
  const int bid = blockIdx.x;
  int ji = 0;
  for (int j = 1; j < args.n_jobs; ++j)
    if (bid >= args.job[j].tile_start) ji = j;
  const GemmJob &jb = args.job[ji];
  const int nt_seg = args.N / BN;
  int local = bid - jb.tile_start;
  const int tn = local % (jb.n_seg * nt_seg);
  local /= jb.n_seg * nt_seg;
  const int tm = local % jb.m_tiles;
  const int grp = local / jb.m_tiles;
  const int seg = tn / nt_seg;
  const int n0 = (tn - seg * nt_seg) * BN;
  const int wgrp = jb.rs.wg0 + grp;
  const int M_rows = jb.rs.n_seq * jb.rs.rows;
  const int d_head = args.d_head;
  const int m0 = tm * BM;
  const int K = args.K, N = args.N;

  // ---- row map of this tile: (sequence, position) per tile row -----------------------------
  for (int r = tid; r < BM; r += 256) {
    const int gr = m0 + r;
    int b = -1, t = 0;
    if (gr < M_rows) {
      b = gr / jb.rs.rows;
      t = jb.rs.t0 + grp * jb.rs.t_step + (gr - b * jb.rs.rows);
    }
    s_b[r] = b;
    s_t[r] = t;
  }
  __syncthreads();

  const T *W = (const T *)jb.w[seg] + ((size_t)wgrp * N + n0) * (size_t)K;
  const T *a_src[G::A_CPT];
  int a_dst[G::A_CPT];
#pragma unroll
  for (int i = 0; i < G::A_CPT; ++i) {
    const int ch = tid + i * 256;
    const int row = ch / G::CPR, kc = (ch % G::CPR) * G::EPC;
    const int b = s_b[row];
    a_src[i] = b >= 0 ? (const T *)args.a.base + b * args.a.sb + (long long)(s_t[row] - args.a.t_off) * args.a.rs + kc
                      : nullptr;
    a_dst[i] = row * G::LDK + kc;
  }
  const T *b_src[G::B_CPT];
  int b_dst[G::B_CPT];
#pragma unroll
  for (int i = 0; i < G::B_CPT; ++i) {
    const int ch = tid + i * 256;
    const int row = ch / G::CPR, kc = (ch % G::CPR) * G::EPC;
    b_src[i] = W + (size_t)row * K + kc;
    b_dst[i] = row * G::LDK + kc;
  }

  u32x4 ra[G::A_CPT], rb[G::B_CPT];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < G::A_CPT; ++i) ra[i] = a_src[i] ? ld16(a_src[i] + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < G::B_CPT; ++i) rb[i] = ld16(b_src[i] + k0);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < G::A_CPT; ++i) st16(&sA[buf][a_dst[i]], ra[i]);
#pragma unroll
    for (int i = 0; i < G::B_CPT; ++i) st16(&sB[buf][b_dst[i]], rb[i]);
  };

  f32x16 acc[G::TM][G::TN];
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j) acc[i][j] = f32x16{};

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const T *pa = &sA[cur][(wm * G::WM + lc) * G::LDK + g * M::KPL];
    const T *pb = &sB[cur][(wn * G::WN + lc) * G::LDK + g * M::KPL];
#pragma unroll
    for (int kk = 0; kk < BK / M::KSTEP; ++kk) {
      frag af[G::TM], bfr[G::TN];
#pragma unroll
      for (int i = 0; i < G::TM; ++i) af[i] = *(const frag *)(pa + i * 32 * G::LDK + kk * M::KSTEP);
#pragma unroll
      for (int j = 0; j < G::TN; ++j) bfr[j] = *(const frag *)(pb + j * 32 * G::LDK + kk * M::KSTEP);
#pragma unroll
      for (int i = 0; i < G::TM; ++i)
#pragma unroll
        for (int j = 0; j < G::TN; ++j) acc[i][j] = M::mma(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: head-split rows ------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < G::TM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = wm * G::WM + i * 32 + acc_row(v, g);
      const int b = s_b[row];
      if (b < 0) continue;
      const int t = s_t[row];
      const HeadView &hv = jb.out_heads[seg];
#pragma unroll
      for (int j = 0; j < G::TN; ++j) {
        const int col = n0 + wn * G::WN + j * 32 + lc;
        const int h = col / d_head, c = col - h * d_head;
        ((T *)hv.base)[b * hv.sb + h * hv.sh + (long long)(t - hv.t_off) * d_head + c] = from_f32<T>(acc[i][j][v]);
      }
    }
  }
}

template <typename T, int BM, int BN>
static hipError_t launch_t(const GemmArgs &a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((mixed_gemm_kernel<T, BM, BN, GEMM_BK>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int tile, const GemmArgs &a, int grid, hipStream_t s) {
  if (dtype == 1) return tile ? launch_t<bf16, 128, 128>(a, grid, s) : launch_t<bf16, 64, 64>(a, grid, s);
  return tile ? launch_t<float, 128, 128>(a, grid, s) : launch_t<float, 64, 64>(a, grid, s);
}

}  // namespace ot
