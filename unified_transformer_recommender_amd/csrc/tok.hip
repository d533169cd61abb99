// Tokenizers ahead of block 1 (fun-rec-mdbook 7.5.0, "Unified Tokenization").
//
// Both tokenizers are two-layer MLPs applied row by row: each behaviour-specific MLP_i maps
// every event embedding of sequence type i to width d, and the Auto-Split MLP maps a sample's
// concatenated non-sequential features to l_ns * d values that are cut into l_ns rows. All of
// them are dense contractions, so the work is one grouped linear-layer kernel on MFMA, launched
// once per layer for every MLP together:
//   launch 1: H_i = GELU(E_i W1_i^T + b1_i) for every sequence type, and the same for NS;
//   launch 2: rows of X(0) = H_i W2_i^T + b2_i, written straight into their merged positions;
// plus a copy of the [SEP] rows into theirs. With the timestamp-aware merge, rank_kernel first finds
// every event's row in time order, and launch 2 writes each row there and adds its type's embedding
// instead. GELU: the shared erf-form evaluations (bf16: the fitted
// sigmoid form, whose error is below the bf16 rounding of the hidden activation it produces).
//
// Work unit: one workgroup of LIN_NW waves computes a tile of LIN_NW * 32 rows by LIN_NT output
// features. Orientation as in the block kernels (C^T = W X^T): an accumulator column is a row
// of the input (lane % 32), its rows are output features. k is consumed in chunks of 128 bytes
// per row; the weight rows of the tile and the wave's own input rows of a chunk are brought into
// LDS by direct global->LDS loads into LIN_NB chunk buffers. Two buffers (the next chunk loads
// while the current one is multiplied) measured faster than three: with K of 64..256 a tile has
// few chunks, and the smaller LDS footprint lets three workgroups share a CU.
//
// LDS layout of a chunk: 16-byte pieces p = 0..7 of row r sit at slot r * 8 + (p ^ (r & 7)), so a
// fragment read (one piece of 32 consecutive rows) touches every bank once.
//
// k order inside a chunk: lane group g (lane / 32) owns the chunk's k elements
// [g * KC / 2, (g + 1) * KC / 2), in MFMA steps of KPL. Both operands use that same order, so the
// contraction is unchanged and every fragment is one 16-byte piece.

#include "common.hpp"
#include "launch.hpp"

namespace ot {
namespace {

constexpr int LIN_NW = 4;      // waves per workgroup, 32 input rows each
constexpr int LIN_NT = 64;     // output features per workgroup
constexpr int LIN_CB = 128;    // bytes of k per row and chunk
constexpr int LIN_NB = 2;      // chunk buffers (2: 48 KB of LDS, three workgroups per CU)
constexpr int LIN_W_BYTES = LIN_NT * LIN_CB;             // weight rows of one chunk
constexpr int LIN_X_BYTES = LIN_NW * 32 * LIN_CB;        // input rows of one chunk
constexpr int LIN_STAGE_BYTES = LIN_W_BYTES + LIN_X_BYTES;
static_assert(LIN_NB == 2 || LIN_NB == 3, "chunks in flight behind the current one: LIN_NB - 2");
static_assert(LIN_NT == 64 && LIN_NW == 4, "direct-to-LDS load split: 2 weight and 4 input loads per wave");

__device__ __forceinline__ uint32_t slot_byte(int r, int p) { return (uint32_t)(r * 8 + (p ^ (r & 7))) * 16u; }

// Workgroup b of a launch of n runs on XCD b % 8. Tile t = (b % 8) * (n / 8) + b / 8 (for the first
// 8 * (n / 8) workgroups) gives each XCD a contiguous run of tiles, so the output tiles of one row
// tile, which read the same input rows, share that XCD's L2 instead of fetching the rows from HBM
// once per XCD.
__device__ __forceinline__ int xcd_tile(int b, int n) {
  const int per = n / 8;
  return b < 8 * per ? (b % 8) * per + b / 8 : b;
}

// MAP: some group of the launch has a row map and a second bias (layer 2 of the time merge).
template <typename T, bool MAP>
__global__ __launch_bounds__(LIN_NW * 64, 2) void lin_kernel(const LinArgs a) {
  using MM = Mma<T>;
  using TS = TileStage<T>;
  constexpr int ESZ = (int)sizeof(T);
  constexpr int KC = LIN_CB / ESZ;             // k elements per chunk
  constexpr int EPP = 16 / ESZ;                // elements per 16-byte piece
  constexpr int SPP = EPP / MM::KPL;           // MFMA k-steps per piece (bf16: 1, fp32: 4)
  constexpr int NTT = LIN_NT / 32;             // accumulator tiles per wave
  static_assert(LIN_NW * TS::SIZE * ESZ <= LIN_NB * LIN_STAGE_BYTES, "staging fits in the ring");
  __shared__ __attribute__((aligned(16))) char ring[LIN_NB * LIN_STAGE_BYTES];

  // tile and group of this workgroup (uniform)
  const int tile = xcd_tile((int)blockIdx.x, (int)gridDim.x);
  int gi = 0;
#pragma unroll
  for (int i = 1; i < LIN_MAX_GROUPS; ++i)
    if (i < a.n_groups && tile >= a.g[i].tile0) gi = i;
  const LinGroup &G = a.g[gi];
  const int local = tile - G.tile0;
  const int n_tiles = G.n / LIN_NT;
  const int n0 = (local % n_tiles) * LIN_NT;
  const int mw0 = (local / n_tiles) * (LIN_NW * 32);   // first row of the workgroup
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int lc = lane & 31, g = lane >> 5;
  const int m0 = mw0 + wave * 32;                      // first row of this wave
  const long long kb = (long long)G.k * ESZ;           // bytes per weight / input row

  // direct-to-LDS sources: weight rows n0.. of the tile; input rows of this wave (clamped to the
  // last row in the ragged tail, whose results are never stored)
  const char *wsrc = (const char *)G.w + (long long)n0 * kb;
  const char *xsrc = (const char *)G.x + (long long)mw0 * G.x_ld * ESZ;
  const long long xrb = G.x_ld * ESZ;
  uint32_t w_off[2], x_off[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int s = (2 * wave + i) * 64 + lane, r = s / 8, p = (s % 8) ^ (r & 7);
    w_off[i] = (uint32_t)(r * kb + p * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = i * 64 + lane, r = s / 8, p = (s % 8) ^ (r & 7);
    const int row = min(m0 + r, G.m - 1) - mw0;
    x_off[i] = (uint32_t)(row * xrb + p * 16);
  }
  const uint32_t ring_lds = lds_addr(ring);
  auto issue = [&](int c) {
    const uint32_t st = ring_lds + (uint32_t)((c % LIN_NB) * LIN_STAGE_BYTES);
    const uint32_t cb = (uint32_t)c * LIN_CB;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16s(wsrc, w_off[i] + cb, __builtin_amdgcn_readfirstlane(st + (uint32_t)((2 * wave + i) * 1024)));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16s(xsrc, x_off[i] + cb, __builtin_amdgcn_readfirstlane(st + LIN_W_BYTES + (uint32_t)(wave * 4096 + i * 1024)));
  };
  constexpr int PER_CHUNK = 6;   // direct-to-LDS loads per wave and chunk

  // bias (plus the second bias) of this lane's accumulator rows, loaded before the first
  // direct-to-LDS load so that they are not counted among the loads the chunk waits below leave
  // outstanding
  float bv[NTT][16] = {};
  auto load_bias = [&](const void *src, float (&out)[NTT][16]) {
    const T *bias = (const T *)src + n0;
#pragma unroll
    for (int t = 0; t < NTT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const T *bp = bias + t * 32 + 8 * j + 4 * g;   // acc_row(4 j + i, g) = 8 j + 4 g + i
        if constexpr (ESZ == 2) {
          const bf16x4 b4 = *(const bf16x4 *)bp;
#pragma unroll
          for (int i = 0; i < 4; ++i) out[t][4 * j + i] += (float)b4[i];
        } else {
          const f32x4 b4 = *(const f32x4 *)bp;
#pragma unroll
          for (int i = 0; i < 4; ++i) out[t][4 * j + i] += b4[i];
        }
      }
  };
  load_bias(G.b, bv);
  if (MAP && G.b_add) load_bias(G.b_add, bv);   // only on layers without activation
  asm volatile("" ::: "memory");

  f32x16 acc[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) acc[t] = f32x16{};

  const int n_chunks = G.k / KC;
#pragma unroll
  for (int c = 0; c < LIN_NB - 1; ++c)
    if (c < n_chunks) issue(c);

  for (int c = 0; c < n_chunks; ++c) {
    // chunk c has landed once at most the loads of the chunks issued after it are outstanding
    if (LIN_NB == 3 && c + 1 < n_chunks) wait_vm<PER_CHUNK * (LIN_NB - 2)>();
    else wait_vm<0>();
    wait_lgkm0();
    bare_barrier();
    if (c + LIN_NB - 1 < n_chunks) issue(c + LIN_NB - 1);

    const char *st = ring + (c % LIN_NB) * LIN_STAGE_BYTES;
    const char *xs = st + LIN_W_BYTES + wave * 4096;
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
          // reinterpret the whole piece, then take its lanes (4 k-steps of the fp32 MFMA)
          const f32x4 af = __builtin_bit_cast(f32x4, wa[q][t]), bf = __builtin_bit_cast(f32x4, xb[q]);
#pragma unroll
          for (int e = 0; e < SPP; ++e) acc[t] = MM::mma(af[e], bf[e], acc[t]);
        }
      }
    sched_lds_mfma<4 * (1 + NTT), 4 * NTT * SPP, 6>();
  }

  // epilogue: bias, optional GELU, staged coalesced store of each 32 x 32 tile
  wait_lgkm0();
  bare_barrier();   // every wave is done with the ring; it becomes the staging area
  T *stg = reinterpret_cast<T *>(ring) + wave * TS::SIZE;
#pragma unroll
  for (int t = 0; t < NTT; ++t) {
    f32x16 v = acc[t];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float y = v[e] + bv[t][e];
      if (G.gelu) y = ESZ == 2 ? gelu_fit(y) : gelu_as(y);
      v[e] = y;
    }
    TS::put(stg, v, lc, g);
    wait_lgkm0();
#pragma unroll
    for (int k = 0; k < TS::NI; ++k) {
      const int tok = TS::token(k, lane);
      const int m = m0 + tok;
      const u32x4 piece = TS::get(stg, k, lane);
      if (m < G.m) {
        const int r = MAP && G.y_row ? G.y_row[m] : m % G.y_rps;
        T *dst = (T *)G.y + (long long)(m / G.y_rps) * G.y_ss + (long long)r * G.y_rs + n0 + t * 32 + TS::feature(lane);
        st16(dst, piece);
      }
    }
    wait_lgkm0();
  }
}

// [SEP] rows: row j of `sep` to row sep_row[j] of every sample of X(0).
template <typename T>
__global__ __launch_bounds__(256) void sep_kernel(const SepArgs a) {
  constexpr int EPP = 16 / (int)sizeof(T);
  const int ppr = a.d / EPP;                                // pieces per row
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)a.batch * a.n_sep * ppr;
  if (i >= total) return;
  const int piece = (int)(i % ppr);
  const int j = (int)((i / ppr) % a.n_sep);
  const long long b = i / ((long long)ppr * a.n_sep);
  const T *src = (const T *)a.sep + (long long)j * a.d + piece * EPP;
  T *dst = (T *)a.x0 + b * a.sample_stride + (long long)a.sep_row[j] * a.d + piece * EPP;
  st16(dst, ld16(src));
}

// One workgroup per sample. The sample's timestamps go to LDS; an event's row is the number of the
// sample's events with a smaller key (time, type, position). When every type's timestamps are
// non-decreasing (the usual case: a behaviour log is chronological), that count is, per other type
// j, a binary search: the events of an earlier type j < i at times <= t, of a later type at times
// < t, plus the event's own position. Otherwise the workgroup counts by comparing with every event
// (O(n^2), exact for any order). Either way the rows are a permutation of 0..total-1.
__global__ __launch_bounds__(256) void rank_kernel(const RankArgs a) {
  extern __shared__ long long s_t[];
  __shared__ int s_unsorted;
  const long long b = blockIdx.x;
  if (threadIdx.x == 0) s_unsorted = 0;
  int off = 0;
  for (int i = 0; i < a.n_seq; ++i) {
    const long long *src = a.t[i] + b * a.len[i];
    for (int l = threadIdx.x; l < a.len[i]; l += 256) s_t[off + l] = src[l];
    off += a.len[i];
  }
  __syncthreads();
  off = 0;
  int bad = 0;
  for (int i = 0; i < a.n_seq; ++i) {
    for (int l = 1 + threadIdx.x; l < a.len[i]; l += 256) bad |= s_t[off + l - 1] > s_t[off + l];
    off += a.len[i];
  }
  if (bad) atomicOr(&s_unsorted, 1);
  __syncthreads();
  const bool sorted = s_unsorted == 0;
  off = 0;
  for (int i = 0; i < a.n_seq; ++i) {
    for (int l = threadIdx.x; l < a.len[i]; l += 256) {
      const int e = off + l;
      const long long t = s_t[e];
      int r = 0;
      if (sorted) {
        r = l;
        int o = 0;
        for (int j = 0; j < a.n_seq; ++j) {
          if (j != i) {
            // first position in type j whose time is > t (j < i) or >= t (j > i)
            int lo = 0, hi = a.len[j];
            while (lo < hi) {
              const int mid = (lo + hi) >> 1;
              const long long v = s_t[o + mid];
              if (j < i ? v <= t : v < t) lo = mid + 1;
              else hi = mid;
            }
            r += lo;
          }
          o += a.len[j];
        }
      } else {
        for (int u = 0; u < a.total; ++u) {
          const long long v = s_t[u];
          r += (v < t) | ((v == t) & (u < e));
        }
      }
      a.pos[i][b * a.len[i] + l] = r;
    }
    off += a.len[i];
  }
}

}  // namespace

hipError_t launch_rank(const RankArgs &a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(rank_kernel, dim3(batch), dim3(256), (size_t)a.total * sizeof(long long), s, a);
  return hipGetLastError();
}

int lin_rows_per_tile() { return LIN_NW * 32; }
int lin_features_per_tile() { return LIN_NT; }

hipError_t launch_lin(int dtype, const LinArgs &a, int grid, hipStream_t s) {
  bool map = false;
  for (int i = 0; i < a.n_groups; ++i) map |= a.g[i].y_row != nullptr || a.g[i].b_add != nullptr;
  if (dtype == 1) {
    if (map) hipLaunchKernelGGL((lin_kernel<bf16, true>), dim3(grid), dim3(LIN_NW * 64), 0, s, a);
    else hipLaunchKernelGGL((lin_kernel<bf16, false>), dim3(grid), dim3(LIN_NW * 64), 0, s, a);
  } else {
    if (map) hipLaunchKernelGGL((lin_kernel<float, true>), dim3(grid), dim3(LIN_NW * 64), 0, s, a);
    else hipLaunchKernelGGL((lin_kernel<float, false>), dim3(grid), dim3(LIN_NW * 64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_sep(int dtype, const SepArgs &a, hipStream_t s) {
  const int epp = dtype == 1 ? 8 : 4;
  const long long total = (long long)a.batch * a.n_sep * (a.d / epp);
  const int grid = (int)((total + 255) / 256);
  if (grid == 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(sep_kernel<bf16>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(sep_kernel<float>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ot
