// Fused pre-norm 1 + mixed-parameter Q/K/V projection (fun-rec-mdbook 7.5.1: q_i, k_i, v_i =
// W_i x_i with W_i = W_S for S rows and W_NS,j for NS token j; pre-norm before the sub-layer;
// 7.5.2: keys/values from every row of the block, queries only from the tail rows).
//
// Orientation as in the post-attention kernel: products are formed transposed, C^T = W Xh^T, so
// each lane owns one token of each of its wave's token groups (two groups of 32 for bf16 at
// d <= 256: every weight fragment read from LDS then feeds two MFMAs). A lane loads its token's
// input row, forms the norm statistics with one cross-half shuffle (or reads them from the
// previous block's post kernel), and keeps the normalised row as bf16 B fragments in registers;
// where the previous block's post kernel handed the normalised rows over (bf16, xh_piece order),
// the lane loads those fragments instead, one contiguous 1 KB wave load per k-chunk.
// The projection weights stream through LDS in chunks of 32 output features x d (direct
// global->LDS loads by all four waves, XOR-swizzled rows, double-buffered): with d_head = 32 a
// chunk is exactly one head, and each accumulator tile is written into the head-major Q/K/V (or
// K/V cache) rows through a per-wave LDS staging tile. Chunks of W_Q are skipped by workgroups
// holding no query row.
//
// Waits: loads and stores share one vector-memory counter on this architecture. Every wave
// issues exactly NS output stores per chunk (lanes with nothing to store write their piece to a
// trash slot), so waiting for a chunk's weights is a fixed partial wait that leaves the previous
// chunk's stores in flight; the chunk handoff is a plain s_barrier (no memory fence).

#include "common.hpp"
#include "launch.hpp"

namespace ot {

namespace {

template <int RP, int RB>
__device__ __forceinline__ constexpr int chunk_swz(int r) {
  constexpr int rpb = RB >= 256 ? 1 : 256 / RB;
  constexpr int P = RP < 16 / rpb ? RP : 16 / rpb;
  return (r / rpb) & (P - 1);
}

constexpr int QKV_NW = 4;                 // waves per workgroup
constexpr int QKV_NB = 2;                 // weight-chunk ring slots; loads run QKV_NB - 1 chunks ahead

// Token groups of 32 per wave: with two, every weight fragment read from LDS feeds two MFMAs
// (half the LDS operand traffic and half the weight stream per token). The normalised rows of
// both groups stay in registers, which bounds it to bf16 at d <= 256.
// A launch with fewer than QKV_SMALL_LAUNCH two-group tiles (half the GPU's CUs) runs one token
// group per wave instead: twice the workgroups, each with half the work, since the workgroups'
// latency, not the LDS traffic, bounds such a launch.
template <typename T, int D>
constexpr int qkv_tg() { return (sizeof(T) == 2 && D <= 256) ? 2 : 1; }

// Workgroups per CU the register budget is set for: two (256 registers per lane), except fp32 at
// d = 512, whose normalised row alone takes 256 registers per lane (one workgroup, 512 registers).
template <typename T, int D>
constexpr int qkv_wgs_per_cu() { return (sizeof(T) == 4 && D >= 512) ? 1 : 2; }

template <typename T, typename TI, int D, bool LAYER, int TG>
__global__ __launch_bounds__(QKV_NW * 64, (qkv_wgs_per_cu<T, D>())) void qkv_kernel(const QkvArgs a) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int NW = QKV_NW;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int DT = D / 32;                    // 32-feature chunks per projection
  constexpr int KC = D / M::KSTEP;
  constexpr int RPA = D / EPC;                  // 16-byte pieces per weight row
  constexpr int CH = 32 * D;
  constexpr int BLOCKS = CH / EPC / 64;         // 1 KB wave loads per chunk
  constexpr int LPW = BLOCKS / NW;              // wave loads per chunk per wave
  static_assert(BLOCKS % NW == 0 && LPW >= 1, "chunk must split into whole wave loads");
  constexpr bool BF = sizeof(T) == 2;
  using TS = TileStage<T>;
  constexpr int NS = TS::NI * TG;               // output stores per chunk per wave
  constexpr int NB = QKV_NB;
  constexpr int PD = 4;                         // LDS operand reads in flight ahead of the MFMAs
  static_assert(NB == 2, "the chunk waits below assume one chunk in flight");
  __shared__ __attribute__((aligned(16))) T lds[NB][CH];
  __shared__ __attribute__((aligned(16))) T stage[NW][TS::SIZE];
  __shared__ float s_gm[D], s_bt[D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lc = lane & 31;
  const int dh = a.d_head;

  // ---- job / group / token tile --------------------------------------------------------------
  // The workgroup's tile is NW * TG * 32 rows of one parameter group; wave w holds token groups
  // w * TG .. w * TG + TG - 1 of it, and the lane's token lc of each.
  // workgroup -> (token tile, chunk range): the n_split workgroups of a tile split its chunk stream
  const int nsp = a.n_split > 1 ? a.n_split : 1;
  const int bid = blockIdx.x / nsp, split = blockIdx.x - bid * nsp;
  const QkvJob &jb = (a.n_jobs > 1 && bid >= a.job[1].tile_start) ? a.job[1] : a.job[0];
  const int local = bid - jb.tile_start;
  const int tm = local % jb.m_tiles, grp = local / jb.m_tiles;
  const int wg = jb.rs.wg0 + grp;
  const int M_rows = jb.rs.n_seq * jb.rs.rows;
  int b[TG], t[TG];
  bool valid[TG], lane_q[TG];
  bool any_q = false;
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int r0 = (tm * NW + wave) * (TG * 32) + tg * 32 + lc;
    valid[tg] = r0 < M_rows;
    const int r = valid[tg] ? r0 : 0;
    b[tg] = r / jb.rs.rows;
    t[tg] = jb.rs.t0 + grp * jb.rs.t_step + (r - b[tg] * jb.rs.rows);
    lane_q[tg] = valid[tg] && t[tg] >= jb.q_from;
    any_q = any_q || lane_q[tg];
  }
  const bool tile_q = __syncthreads_or(any_q);   // does any token of this workgroup issue a query?
  // this workgroup's chunks [c0, c1) of the stream K 0..DT-1, V, then Q (Q only if tile_q)
  const int per_split = (3 * DT + nsp - 1) / nsp;
  const int c0 = split * per_split;
  const int c1 = min(tile_q ? 3 * DT : 2 * DT, c0 + per_split);
  if (c0 >= c1) return;                          // uniform over the workgroup: no later barrier is missed
  // Output pieces this lane stores (one per store instruction): the piece's token within its
  // group, and whether it is written at all. Every store instruction is issued; a lane with
  // nothing to write sends its piece to a trash slot, so the number of outstanding vector-memory
  // operations after each chunk is a constant the chunk waits rely on.
  int sb[TG][TS::NI], stt[TG][TS::NI], ssh[TG][TS::NI];
  bool sval[TG][TS::NI], sq[TG][TS::NI];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int k = 0; k < TS::NI; ++k) {
      const int tok = TS::token(k, lane);
      sb[tg][k] = __shfl(b[tg], tok, 64);
      stt[tg][k] = __shfl(t[tg], tok, 64);
      sval[tg][k] = __shfl((int)valid[tg], tok, 64) != 0;
      sq[tg][k] = __shfl((int)lane_q[tg], tok, 64) != 0;
      ssh[tg][k] = a.kv_shift ? a.kv_shift[sb[tg][k]] : 0;   // ragged cache: the sequence's row offset
    }
  T *stg = stage[wave];

  // ---- weight chunk stream: K chunks 0..DT-1, V chunks, then (if any query row) Q chunks -------
  const T *wk = (const T *)a.wk + (size_t)wg * D * D;
  const T *wv = (const T *)a.wv + (size_t)wg * D * D;
  const T *wq = (const T *)a.wq + (size_t)wg * D * D;
  // byte offset of this lane's 16-byte piece j within a chunk (32 rows of d, pieces XOR-swizzled);
  // piece j of the wave lands at LDS piece (j * NW + wave) * 64 + lane of the chunk buffer
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t off[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int P = (j * NW + wave) * 64 + lane;
    const int row = P / RPA, q = P % RPA;
    off[j] = (uint32_t)((row * D + (q ^ chunk_swz<RPA, RPA * 16>(row)) * EPC) * (int)sizeof(T));
  }
  auto issue = [&](int i) {
    const int seg = i / DT, ci = i - seg * DT;
    const T *base = (seg == 0 ? wk : seg == 1 ? wv : wq) + (size_t)(32 * ci) * D;
    const uint32_t dst = lds_addr(lds[i % NB]);
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma16s(base, off[j], dst + (uint32_t)((j * NW + wave_s) * 64 * 16));
  };
  issue(c0);

  // handed-over rows are normalised already: no norm parameters to stage, and their loads go out
  // right behind the first chunk's
  const bool from_xh = BF && a.xh != nullptr;
  if (!from_xh) {
    for (int i = tid; i < D; i += NW * 64) {
      s_gm[i] = to_f32(((const T *)a.gamma)[i]);
      s_bt[i] = LAYER ? to_f32(((const T *)a.beta)[i]) : 0.0f;
    }
    __syncthreads();                             // gamma / beta staged
  }

  // ---- norm1 of this lane's tokens -> bf16 B fragments (k = 16 kc + 8 g + e) -----------------
  // A lane holds half of its token's row (the other half sits in lane +- 32). For bf16 storage at
  // d >= 256 the row's statistics come from the previous block's post-attention kernel when it
  // wrote them (one read of the row); otherwise the row is read twice: once for the statistics, in
  // two halves, and once more (from cache) to normalise, which keeps at most a quarter row live in
  // registers. LayerNorm statistics are taken about the row's first element, which keeps the
  // one-pass variance free of cancellation. Token groups are normalised one after the other.
  frag xfr[TG][KC];
  bool handed = false;
  if constexpr (BF) {
    // rows normalised by the previous block's post-attention kernel, already in fragment order:
    // one contiguous 1 KB wave load per k-chunk. A row group wholly past the job's rows (the last
    // tile's spare waves) reads the job's last group instead; its results are never stored.
    if (from_xh) {
      handed = true;
      const int last = ((M_rows + 31) >> 5) - 1;
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        const int G = min((tm * NW + wave) * TG + tg, last);
        const frag *src = (const frag *)a.xh + xh_piece(jb.xh_g0, grp, M_rows, G, KC, 0, lane);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) xfr[tg][kc] = src[kc * 64];
      }
    }
  }
  if (!handed) {
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    asm volatile("" ::: "memory");               // one group's row in flight at a time
    const TI *xr = (const TI *)a.x.base + b[tg] * a.x.sb + (long long)(t[tg] - a.x.t_off) * a.x.rs;
    if (BF && D >= 256 && a.stats.base != nullptr) {
      const float *sp = (const float *)a.stats.base + b[tg] * a.stats.sb + (long long)(t[tg] - a.stats.t_off) * a.stats.rs;
      const float mean = LAYER ? sp[0] : 0.0f, rstd = sp[1];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if constexpr (BF) {
          const TI *p = xr + 16 * kc + 8 * g;
          frag fr;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int f = 16 * kc + 8 * g + e;
            fr[e] = (bf16)((to_f32(p[e]) - mean) * rstd * s_gm[f] + s_bt[f]);
          }
          xfr[tg][kc] = fr;
        }
      }
    } else if constexpr (BF && D >= 256) {
      constexpr int HALF = KC / 2;
      const float shift = LAYER ? to_f32(xr[0]) : 0.0f;
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        float xv[8 * HALF];
#pragma unroll
        for (int k = 0; k < HALF; ++k) {
          const TI *p = xr + 16 * (part * HALF + k) + 8 * g;
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[8 * k + e] = to_f32(p[e]);
        }
#pragma unroll
        for (int e = 0; e < 8 * HALF; ++e) {
          const float c = xv[e] - shift;
          s1 += c;
          s2 += c * c;
        }
      }
      s1 += __shfl_xor(s1, 32, 64);
      s2 += __shfl_xor(s2, 32, 64);
      const float m1 = s1 * (1.0f / D);
      const float mean = LAYER ? shift + m1 : 0.0f;
      const float var = LAYER ? fmaxf(s2 * (1.0f / D) - m1 * m1, 0.0f) : s2 * (1.0f / D);
      const float rstd = 1.0f / sqrtf(var + a.eps);
      asm volatile("" ::: "memory");             // read the row again rather than keep it live
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const TI *p = xr + 16 * kc + 8 * g;
        frag fr;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int f = 16 * kc + 8 * g + e;
          fr[e] = (bf16)((to_f32(p[e]) - mean) * rstd * s_gm[f] + s_bt[f]);
        }
        xfr[tg][kc] = fr;
      }
    } else {
      constexpr int PER = D / 2;                 // features held by this lane
      float xv[PER];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if constexpr (BF) {
          const TI *p = xr + 16 * kc + 8 * g;
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[8 * kc + e] = to_f32(p[e]);
        } else {
          xv[kc] = to_f32(xr[2 * kc + g]);
        }
      }
      float mean = 0.0f;
      if constexpr (LAYER) {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < PER; ++e) s += xv[e];
        s += __shfl_xor(s, 32, 64);
        mean = s * (1.0f / D);
      }
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float c = xv[e] - mean;
        ss += c * c;
      }
      ss += __shfl_xor(ss, 32, 64);
      const float rstd = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if constexpr (BF) {
          frag fr;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int f = 16 * kc + 8 * g + e;
            fr[e] = (bf16)((xv[8 * kc + e] - mean) * rstd * s_gm[f] + s_bt[f]);
          }
          xfr[tg][kc] = fr;
        } else {
          const int f = 2 * kc + g;
          xfr[tg][kc] = (xv[kc] - mean) * rstd * s_gm[f] + s_bt[f];
        }
      }
    }
  }
  }

  // ---- chunk loop ----------------------------------------------------------------------------
  // Before the barrier of chunk i this wave waits for its own loads of chunk i: after those it
  // has issued only the NS stores of chunk i - 1 (for the first chunk: nothing that is still in flight,
  // the rows above were consumed), and operations complete in issue order. After the barrier
  // every wave has also finished reading chunk i - 1, so its slot takes chunk i + 1.
  T *trash = (T *)a.trash;
  for (int i = c0; i < c1; ++i) {
    // first chunk: its loads are done; with handed-over rows their TG * KC loads, issued after
    // the chunk's, may still be in flight (the MFMAs wait for each fragment as they use it)
    if (i == c0) {
      if constexpr (BF) {
        if (from_xh) wait_vm<TG * KC>();
        else wait_vm<0>();
      } else {
        wait_vm<0>();
      }
    }
    else wait_vm<NS>();
    wait_lgkm0();
    bare_barrier();
    if (i + 1 < c1) issue(i + 1);
    const T *base = lds[i % NB];
    f32x16 acc[TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) acc[tg] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      frag af;
      if constexpr (BF) {
        const int q = (2 * kc + g) ^ chunk_swz<RPA, RPA * 16>(lc);
        af = *(const frag *)(base + lc * D + q * EPC);
      } else {
        const int k = 2 * kc + g;
        af = base[lc * D + ((k / EPC) ^ chunk_swz<RPA, RPA * 16>(lc)) * EPC + k % EPC];
      }
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) acc[tg] = M::mma(af, xfr[tg][kc], acc[tg]);
    }
    if constexpr (BF) sched_lds_mfma<KC, KC * TG, PD>();
    // 32 output features 32 ci .. 32 ci + 31 of every token: stage through LDS, store whole runs
    const int seg = i / DT, ci = i - seg * DT;
    const HeadView &hv = seg == 0 ? jb.k : seg == 1 ? jb.v : jb.q;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      if (seg == 2) {
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[tg][v] *= a.q_scale;
      }
      TS::put(stg, acc[tg], lc, g);
#pragma unroll
      for (int k = 0; k < TS::NI; ++k) {
        const u32x4 piece = TS::get(stg, k, lane);
        const int f = 32 * ci + TS::feature(lane);
        const int h = f / dh, c = f - h * dh;
        const int row = stt[tg][k] - hv.t_off + (seg < 2 ? ssh[tg][k] : 0);
        T *dst = (T *)hv.base + sb[tg][k] * hv.sb + h * hv.sh + (long long)row * dh + c;
        st16((seg < 2 ? sval[tg][k] : sq[tg][k]) ? dst : trash, piece);
      }
    }
  }
}

template <typename T, typename TI, int D, int TG>
hipError_t launch_dlt(const QkvArgs &a, int tiles, hipStream_t s) {
  const int grid = tiles * (a.n_split > 1 ? a.n_split : 1);
  if (a.layer)
    hipLaunchKernelGGL((qkv_kernel<T, TI, D, true, TG>), dim3(grid), dim3(QKV_NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((qkv_kernel<T, TI, D, false, TG>), dim3(grid), dim3(QKV_NW * 64), 0, s, a);
  return hipGetLastError();
}

template <typename T, typename TI, int D>
hipError_t launch_dl(const QkvArgs &a, int grid, hipStream_t s) {
  if constexpr (qkv_tg<T, D>() == 2) {
    if (a.tg == 2) return launch_dlt<T, TI, D, 2>(a, grid, s);
  }
  return launch_dlt<T, TI, D, 1>(a, grid, s);
}

template <typename T, typename TI>
hipError_t launch_d(const QkvArgs &a, int grid, hipStream_t s) {
  switch (a.d_model) {
    case 64: return launch_dl<T, TI, 64>(a, grid, s);
    case 128: return launch_dl<T, TI, 128>(a, grid, s);
    case 256: return launch_dl<T, TI, 256>(a, grid, s);
    case 512: return launch_dl<T, TI, 512>(a, grid, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

int qkv_max_groups(int dtype, int d_model) {
  if (dtype == 1) return d_model <= 256 ? qkv_tg<bf16, 256>() : qkv_tg<bf16, 512>();
  return qkv_tg<float, 256>();
}

int qkv_tokens_per_tile(int tg) { return QKV_NW * 32 * tg; }

int qkv_max_split(int d_model) { return d_model / 32; }   // chunk ranges of at least three chunks

hipError_t launch_qkv(int dtype, int in_f32, const QkvArgs &a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  if (dtype == 1) return in_f32 ? launch_d<bf16, float>(a, grid, s) : launch_d<bf16, bf16>(a, grid, s);
  return launch_d<float, float>(a, grid, s);
}

}  // namespace ot
