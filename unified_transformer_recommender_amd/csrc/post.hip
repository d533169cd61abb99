// Fused post-attention block tail: attention output projection + residual + pre-norm 2 + mixed FFN
// (up, bias, GELU, down, bias) + residual, for the query rows of a block (fun-rec-mdbook 7.5.1:
// Mixed FFN W2_i phi(W1_i x_i + b1_i) + b2_i with S rows sharing one parameter set and NS token j
// owning set 1 + j; pre-norm before each sub-layer).
//
// Orientation: every product is formed transposed, C^T = W X^T, so that the 32 columns of an
// MFMA 32x32 tile are 32 tokens and each lane owns ONE token. Per token the wave keeps
//   Y^T   (d x 32 fp32 accumulators)          -> becomes X'^T after the FFN adds into it
//   Yh^T  (norm2 output, bf16 B fragments)   -> B operand of the FFN up-projection
// and streams the weights (A operand) through LDS in chunks of 32 rows (W^O, W1) or 32 columns
// (W2) shared by the workgroup's waves. The hidden activations of a 32-unit chunk never leave
// registers: up-projection tile -> +b1 -> GELU -> bf16 -> B fragments of the down-projection,
// which accumulates straight into X'^T. An accumulator tile's lane holds the k-indices
// {4g + r + 8j}; two cross-half lane swaps (v_permlane32_swap) turn it into a natural B fragment.
//
// Weight streaming: chunks flow through a ring of NB = 2 LDS buffers (4 in split launches) with
// direct global->LDS loads (each wave instruction writes 64 x 16 bytes), issued NB - 1 chunks
// ahead; a chunk is consumed
// after the issuing waves' own partial vmcnt wait and one fence-free workgroup barrier, so the
// next chunk's loads stay in flight across it. Within a chunk, LDS operand reads are issued a
// few MFMAs ahead of their use. Rows are stored unpadded with their 16-byte pieces XOR-swizzled so
// that 16 lanes reading 16 consecutive rows touch 16 distinct bank groups.
//
// Epilogue: X' rows (fp32) through a per-wave LDS staging tile, the (mean, rstd) of each row for
// the next block's norm 1, and, where the launch hands over, that norm's output in bf16 as the next
// QKV launch's B fragments (xh_piece order); X' rows the next block reads only through those
// fragments are then not stored.
//
// Occupancy: for bf16 at d < 256, and at d = 256 with RMSNorm, the kernel is held to 256 registers
// per lane so that two workgroups share a CU. Each hidden chunk then runs plainly in order
// (up-projection, GELU, down-projection): the other workgroup's MFMAs fill this one's VALU phases,
// waits and activation loads.
//
// GELU is the erf form 0.5 x (1 + erf(x / sqrt 2)): gelu_as (fp32 path) and gelu_fit (bf16 path)
// of the shared header.

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ot {

namespace {


// Waves per workgroup (every chunk is split into whole 1 KB wave loads).
template <typename T, int D>
constexpr int post_nw() { return (sizeof(T) == 2 && D == 128) ? 8 : 4; }

// Workgroups per CU the register budget is set for: two where a lane's d-wide accumulators and
// operand fragments fit in 256 registers (bf16, d <= 256; at d = 256 only for RMSNorm: LayerNorm's
// extra shift vector and mean pass spill at 256), else one (512 registers).
template <typename T, int D, bool LAYER>
constexpr int post_wgs_per_cu() { return (sizeof(T) == 2 && (D < 256 || (D == 256 && !LAYER))) ? 2 : 1; }

// Row layout of a weight chunk in LDS: RP 16-byte pieces per row; piece q of row r is stored at
// slot q ^ swz(r). `rpb` = rows sharing one 256-byte bank line.
template <int RP, int RB>
__device__ __forceinline__ constexpr int chunk_swz(int r) {
  constexpr int rpb = RB >= 256 ? 1 : 256 / RB;
  constexpr int P = RP < 16 / rpb ? RP : 16 / rpb;
  return (r / rpb) & (P - 1);
}

// bf16 accumulator-fed B fragment: lane half g holds k {4g..4g+3, 8+4g..8+4g+3} of a 16-block;
// exchange the middle 8-byte halves between the lane halves to get k {8g .. 8g+7}.
__device__ __forceinline__ bf16x8 natural_kfrag(bf16x8 f) {
  u32x4 u = __builtin_bit_cast(u32x4, f);
  const auto s0 = __builtin_amdgcn_permlane32_swap(u[0], u[2], false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(u[1], u[3], false, false);
  u[0] = s0[0]; u[2] = s0[1];
  u[1] = s1[0]; u[3] = s1[1];
  return __builtin_bit_cast(bf16x8, u);
}

template <typename T, typename TR, int D, bool LAYER, bool SPLIT>
__global__ __launch_bounds__((post_nw<T, D>() * 64), (post_wgs_per_cu<T, D, LAYER>())) void post_kernel(const PostArgs a) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int NW = post_nw<T, D>();
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int DT = D / 32;                    // feature tiles
  constexpr int KC = D / M::KSTEP;              // k-chunks over d
  constexpr int HKC = 32 / M::KSTEP;            // k-chunks over a 32-unit hidden chunk
  constexpr int RPA = D / EPC;                  // pieces per row of a 32 x d chunk (W^O, W1)
  constexpr int RPB = 32 / EPC;                 // pieces per row of a d x 32 chunk (W2)
  constexpr int CH = 32 * D;                    // elements per chunk
  constexpr int BLOCKS = CH / EPC / 64;         // 1 KB wave loads per chunk
  constexpr int LPW = BLOCKS / NW;              // wave loads per chunk per wave
  static_assert(BLOCKS % NW == 0 && LPW >= 1, "chunk must split into whole wave loads");
  // chunk buffers; loads run NB - 1 chunks ahead. A split launch (few token tiles: one workgroup per
  // CU, each with a short chunk stream) runs four, so that chunk load latency is not exposed.
  constexpr int NB = SPLIT ? 4 : 2;
  constexpr int PD = 4;                         // LDS operand reads in flight ahead of the MFMAs
  constexpr bool BF = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) T lds[NB][CH];
  using TS = TileStage<float>;
  __shared__ __attribute__((aligned(16))) float stage[NW][TS::SIZE];
  // per-feature / per-hidden-unit vectors of this parameter set, fp32: gamma, beta, b2 [d], b1 [d_ff]
  __shared__ __attribute__((aligned(16))) float svec[3 * D + POST_MAX_DFF];
  // the next block's norm-1 gamma / beta, fp32, when this launch hands over normalised rows
  __shared__ __attribute__((aligned(16))) float s_xg[D], s_xb[D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lc = lane & 31;
  const int DFF = a.d_ff;
  // workgroup -> (token tile, split): split s of n_split takes hidden chunks [hc0, hc0 + NC)
  const int nsp = SPLIT ? a.n_split : 1;
  const int bid = blockIdx.x / nsp, split = blockIdx.x - bid * nsp;
  const int NC = DFF / 32 / nsp;                // hidden chunks of this workgroup (the host splits evenly)
  const int hc0 = split * NC;
  const int NCH = DT + 2 * NC;                  // chunks in the stream

  // ---- job / group / token tile --------------------------------------------------------------
  const PostJob &jb = (a.n_jobs > 1 && bid >= a.job[1].tile_start) ? a.job[1] : a.job[0];
  const int local = bid - jb.tile_start;
  const int tm = local % jb.m_tiles, grp = local / jb.m_tiles;
  const int wg = jb.rs.wg0 + grp;
  const int M_rows = jb.rs.n_seq * jb.rs.rows;
  const int r0 = tm * (NW * 32) + wave * 32 + lc;   // this lane's token within the group
  const bool valid = r0 < M_rows;
  const int r = valid ? r0 : 0;                     // out-of-range lanes shadow row 0: loads stay in bounds
  const int b = r / jb.rs.rows;
  const int t = jb.rs.t0 + grp * jb.rs.t_step + (r - b * jb.rs.rows);

  const T *wo = (const T *)a.wo + (size_t)wg * D * D;
  // this split's hidden units start at 32 hc0: W1 rows, W2 columns and b1 entries from there
  const T *w1 = (const T *)a.w1 + (size_t)wg * DFF * D + (size_t)(32 * hc0) * D;
  const T *w2 = (const T *)a.w2 + (size_t)wg * D * DFF + 32 * hc0;
  const T *b1 = (const T *)a.b1 + (size_t)wg * DFF + 32 * hc0;
  const T *b2 = (const T *)a.b2 + (size_t)wg * D;

  // ---- weight chunk stream --------------------------------------------------------------------
  // Byte offsets of this lane's 16-byte pieces within a row chunk (W^O, W1: 32 rows of d) and a
  // column chunk (W2: d rows of 32 hidden units); piece j of the wave lands at LDS piece
  // (j * NW + wave) * 64 + lane of the chunk buffer.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t off_r[LPW], off_c[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int P = (j * NW + wave) * 64 + lane;
    const int rr = P / RPA, qr = P % RPA, rc = P / RPB, qc = P % RPB;
    off_r[j] = (uint32_t)((rr * D + (qr ^ chunk_swz<RPA, RPA * 16>(rr)) * EPC) * (int)sizeof(T));
    off_c[j] = (uint32_t)((rc * DFF + (qc ^ chunk_swz<RPB, RPB * 16>(rc)) * EPC) * (int)sizeof(T));
  }
  // chunk i: i < DT            -> W^O rows 32i..32i+31
  //          i == DT + 2c      -> W1 rows of hidden chunk c
  //          i == DT + 2c + 1  -> W2 columns of hidden chunk c
  // This lane's piece of wave load j sits at LDS piece P = (j * NW + wave) * 64 + lane.
  auto issue = [&](int i) {
    const T *base;
    bool cols = false;
    if (i < DT) {
      base = wo + (size_t)(32 * i) * D;
    } else {
      const int c = (i - DT) >> 1;
      if (((i - DT) & 1) == 0) {
        base = w1 + (size_t)(32 * c) * D;
      } else {
        base = w2 + 32 * c;
        cols = true;
      }
    }
    const uint32_t dst = lds_addr(lds[i % NB]);
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      dma16s(base, cols ? off_c[j] : off_r[j], dst + (uint32_t)((j * NW + wave_s) * 64 * 16));
  };
  // Make chunk i visible: this wave's loads of chunk i are done (loads of later chunks may still
  // be in flight) and its LDS accesses so far have completed (so the buffer of chunk i - 1 may be
  // refilled), then every wave's.
  auto arrive = [&](int i) {
    const int later = min(NB - 2, NCH - 1 - i);   // chunks issued after chunk i so far
    if (later >= 2) wait_vm<2 * LPW>();
    else if (later == 1) wait_vm<LPW>();
    else wait_vm<0>();
    wait_lgkm0();
    bare_barrier();
  };

  // A fragment of chunk row `row` for k-chunk kc (row chunks: k = feature; column chunks: k = hidden).
  auto afrag_rows = [&](const T *base, int row, int kc, bool accfed) -> frag {
    if constexpr (BF) {
      (void)accfed;
      const int q = (2 * kc + g) ^ chunk_swz<RPA, RPA * 16>(row);
      return *(const frag *)(base + row * D + q * EPC);
    } else {
      const int k = accfed ? 32 * (kc >> 4) + acc_row(kc & 15, g) : kc * 2 + g;
      return base[row * D + ((k / EPC) ^ chunk_swz<RPA, RPA * 16>(row)) * EPC + k % EPC];
    }
  };
  auto afrag_cols = [&](const T *base, int row, int kc) -> frag {
    if constexpr (BF) {
      const int q = (2 * kc + g) ^ chunk_swz<RPB, RPB * 16>(row);
      return *(const frag *)(base + row * 32 + q * EPC);
    } else {
      const int k = acc_row(kc, g);
      return base[row * 32 + ((k / EPC) ^ chunk_swz<RPB, RPB * 16>(row)) * EPC + k % EPC];
    }
  };

  // prologue: start the weight stream, then the per-token loads
#pragma unroll
  for (int i = 0; i < NB - 1; ++i) issue(i);

  // Per-feature vectors into LDS. Every thread's loads are issued together and waited for once (a
  // plain strided loop waits for each 2-byte load before the next: one memory round trip per
  // element, in front of the first chunk).
  float *s_gm = svec, *s_bt = svec + D, *s_b2 = svec + 2 * D, *s_b1 = svec + 3 * D;
  const bool hand = BF && !SPLIT && a.xh != nullptr;
  {
    constexpr int NT = NW * 64;
    constexpr int SV = (3 * D + POST_MAX_DFF + NT - 1) / NT;   // svec elements per thread, at most
    constexpr int XV = (D + NT - 1) / NT;                      // next-block norm elements per thread
    const int nsv = 3 * D + 32 * NC;
    float sv[SV], xg[XV], xb[XV];
    // every load is issued (elements without a source read gamma[0] and are discarded), so no
    // branch separates them
    const T *const g0 = (const T *)a.gamma;
#pragma unroll
    for (int k = 0; k < SV; ++k) {
      const int i = tid + k * NT;
      const T *src = g0;
      bool use = true;
      if (i < D) src = g0 + i;
      else if (i < 2 * D) { if (LAYER) src = (const T *)a.beta + (i - D); else use = false; }
      else if (i < 3 * D) src = b2 + (i - 2 * D);
      else if (i < nsv) src = b1 + (i - 3 * D);
      else use = false;
      const float v = to_f32(*src);
      sv[k] = use ? v : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < XV; ++k) {
      const int i = min(tid + k * NT, D - 1);
      const float vg = to_f32(*(hand ? (const T *)a.xh_gamma + i : g0));
      const float vb = to_f32(*(hand && LAYER ? (const T *)a.xh_beta + i : g0));
      xg[k] = vg;
      xb[k] = LAYER ? vb : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < SV; ++k)
      if (tid + k * NT < nsv) svec[tid + k * NT] = sv[k];
#pragma unroll
    for (int k = 0; k < XV; ++k)
      if (hand && tid + k * NT < D) {
        s_xg[tid + k * NT] = xg[k];
        s_xb[tid + k * NT] = xb[k];
      }
  }

  frag ofr[KC];
  {
    const T *orow = (const T *)a.o.base + b * a.o.sb + (long long)(t - a.o.t_off) * a.o.rs;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if constexpr (BF)
        ofr[kc] = *(const frag *)(orow + kc * 16 + g * 8);
      else
        ofr[kc] = orow[kc * 2 + g];
    }
  }

  // Y^T accumulators start from the residual rows X^T (fp32, or storage dtype in block 0): the
  // loads are issued here, ahead of the W^O chunks, and each tile's values are needed only by its
  // own chunk's first MFMA, so their latency hides behind the weight stream.
  f32x16 acc[DT];
  {
    const TR *xr = (const TR *)a.resid.base + b * a.resid.sb + (long long)(t - a.resid.t_off) * a.resid.rs + 4 * g;
#pragma unroll
    for (int ti = 0; ti < DT; ++ti)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(TR) == 4) {
          const f32x4 v4 = *(const f32x4 *)(xr + 32 * ti + 8 * j);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[ti][4 * j + q] = v4[q];
        } else {
          const bf16x4 v4 = *(const bf16x4 *)(xr + 32 * ti + 8 * j);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[ti][4 * j + q] = (float)v4[q];
        }
      }
  }

  // ---- W^O: Y^T = X^T + Wo O^T, one 32-feature tile per chunk ---------------------------------
#pragma unroll
  for (int ti = 0; ti < DT; ++ti) {
    arrive(ti);
    if (ti + NB - 1 < NCH) issue(ti + NB - 1);
    const T *base = lds[ti % NB];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) acc[ti] = M::mma(afrag_rows(base, lc, kc, false), ofr[kc], acc[ti]);
    sched_lds_mfma<KC, KC, PD>();
  }

  // ---- norm2, + b2 ----------------------------------------------------------------------------
  frag yfr[KC];
  {
    float mean = 0.0f;
    if constexpr (LAYER) {
      float s = 0.0f;
#pragma unroll
      for (int ti = 0; ti < DT; ++ti)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[ti][v];
      s += __shfl_xor(s, 32, 64);
      mean = s * (1.0f / D);
    }
    float ss = 0.0f;
#pragma unroll
    for (int ti = 0; ti < DT; ++ti)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float c = acc[ti][v] - mean;
        ss += c * c;
      }
    ss += __shfl_xor(ss, 32, 64);
    const float rstd = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
    for (int ti = 0; ti < DT; ++ti) {
      float yh[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int f = 32 * ti + acc_row(v, g);
        float y = (acc[ti][v] - mean) * rstd * s_gm[f];
        if constexpr (LAYER) y += s_bt[f];
        yh[v] = y;
        // split 0 carries Y + b2, the other splits only their part of the FFN
        if (!SPLIT || split == 0) acc[ti][v] += s_b2[f];
        else acc[ti][v] = 0.0f;
      }
      if constexpr (BF) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          frag fr;
#pragma unroll
          for (int e = 0; e < 8; ++e) fr[e] = (bf16)yh[8 * h + e];
          yfr[2 * ti + h] = natural_kfrag(fr);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) yfr[16 * ti + v] = yh[v];
      }
    }
  }

  // ---- FFN: per hidden chunk c, stage A (W1 chunk c): up-projection; GELU; stage B (W2 chunk
  // c): down-projection into X'^T. Two workgroups share a CU, so the VALU work and the waits of
  // one overlap the MFMAs of the other. With two ring slots every W1 chunk sits in slot DT % 2 and
  // every W2 chunk in the other, so each LDS operand address is a fixed per-lane offset.
  for (int c = 0; c < NC; ++c) {
    const int ia = DT + 2 * c;
    const int SA = NB == 2 ? DT % 2 : ia % NB, SB = NB == 2 ? (DT + 1) % 2 : (ia + 1) % NB;
    arrive(ia);
    if (ia + NB - 1 < NCH) issue(ia + NB - 1);
    // the up-projection accumulators start from the bias b1 (accumulator row layout)
    f32x16 h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 b4 = *(const f32x4 *)(s_b1 + 32 * c + 8 * j + 4 * g);
#pragma unroll
      for (int q = 0; q < 4; ++q) h[4 * j + q] = b4[q];
    }
    {
      const T *base = lds[SA];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) h = M::mma(afrag_rows(base, lc, kc, true), yfr[kc], h);
      sched_lds_mfma<KC, KC, PD>();
    }
    frag hfr[HKC];
    {
      float hv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if constexpr (BF) hv[v] = gelu_fit(h[v]);
        else hv[v] = gelu_as(h[v]);
      }
      if constexpr (BF) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          frag fr;
#pragma unroll
          for (int e = 0; e < 8; ++e) fr[e] = (bf16)hv[8 * hh + e];
          hfr[hh] = natural_kfrag(fr);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) hfr[v] = hv[v];
      }
    }
    arrive(ia + 1);
    if (ia + NB < NCH) issue(ia + NB);
    {
      const T *base = lds[SB];
#pragma unroll
      for (int kc = 0; kc < HKC; ++kc)
#pragma unroll
        for (int ti = 0; ti < DT; ++ti) acc[ti] = M::mma(afrag_cols(base, 32 * ti + lc, kc), hfr[kc], acc[ti]);
      sched_lds_mfma<DT * HKC, DT * HKC, PD>();
    }
  }

  // ---- statistics of X' for the next block's norm 1 (exact two-pass over the registers), and
  // that norm's output in the next QKV launch's fragment order --------------------------------
  if (!SPLIT && (a.stats.base != nullptr || hand)) {
    float mean = 0.0f;
    if constexpr (LAYER) {
      float s = 0.0f;
#pragma unroll
      for (int ti = 0; ti < DT; ++ti)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[ti][v];
      s += __shfl_xor(s, 32, 64);
      mean = s * (1.0f / D);
    }
    float ss = 0.0f;
#pragma unroll
    for (int ti = 0; ti < DT; ++ti)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float c = acc[ti][v] - mean;
        ss += c * c;
      }
    ss += __shfl_xor(ss, 32, 64);
    const float rstd = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
    if (a.stats.base != nullptr && g == 0 && valid) {
      float *sp = (float *)a.stats.base + b * a.stats.sb + (long long)(t - a.stats.t_off) * a.stats.rs;
      sp[0] = mean;
      sp[1] = rstd;
    }
    if constexpr (BF && !SPLIT) {
      if (hand) {
        // the same arithmetic as the QKV kernel's norm of a stored X' row, so the fragments are
        // those it would form itself
        u32x4 *dst = (u32x4 *)a.xh + xh_piece(jb.xh_g0, grp, M_rows, (tm * NW + wave), KC, 0, lane);
#pragma unroll
        for (int ti = 0; ti < DT; ++ti)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            frag fr;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int f = 32 * ti + acc_row(8 * h + e, g);
              fr[e] = (bf16)((acc[ti][8 * h + e] - mean) * rstd * s_xg[f] + s_xb[f]);
            }
            const u32x4 piece = __builtin_bit_cast(u32x4, natural_kfrag(fr));
            if (valid) st16(dst + (2 * ti + h) * 64, piece);
          }
      }
    }
  }

  // ---- store X' (fp32) tile by tile through the wave's LDS staging area ------------------------
  {
    float *stg = stage[wave];
    float *rowp[TS::NI];
    bool rv[TS::NI];
#pragma unroll
    for (int k = 0; k < TS::NI; ++k) {
      const int tok = TS::token(k, lane);
      const int tb = __shfl(b, tok, 64), tt = __shfl(t, tok, 64);
      rv[k] = __shfl((int)valid, tok, 64) != 0 && (SPLIT || tt - a.out.t_off >= a.out_from);
      const RowView &ov = SPLIT ? a.part : a.out;
      rowp[k] = (float *)ov.base + (SPLIT ? split * a.part_split : 0) + tb * ov.sb + (long long)(tt - ov.t_off) * ov.rs +
                TS::feature(lane);
    }
#pragma unroll
    for (int ti = 0; ti < DT; ++ti) {
      TS::put(stg, acc[ti], lc, g);
#pragma unroll
      for (int k = 0; k < TS::NI; ++k) {
        const u32x4 piece = TS::get(stg, k, lane);
        if (rv[k]) st16(rowp[k] + 32 * ti, piece);
      }
    }
  }
}

// Sum of the n_split partial X' rows of a split post launch into `out` (fixed order, so results do
// not depend on timing), plus the row statistics for the next block's norm 1 when requested. One
// wave per row, in the job order of the post launch.
template <int D>
__global__ __launch_bounds__(256) void post_reduce_kernel(const PostArgs a, int total) {
  constexpr int PER = D / 64;                   // features per lane
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= total) return;
  const int m0 = a.job[0].rs.n_seq * a.job[0].rs.rows * a.job[0].rs.n_groups;
  const PostJob &jb = (a.n_jobs > 1 && row >= m0) ? a.job[1] : a.job[0];
  const int local = row >= m0 ? row - m0 : row;
  const int M_rows = jb.rs.n_seq * jb.rs.rows;
  const int grp = local / M_rows, r = local - grp * M_rows;
  const int b = r / jb.rs.rows;
  const int t = jb.rs.t0 + grp * jb.rs.t_step + (r - b * jb.rs.rows);
  const long long po = b * a.part.sb + (long long)(t - a.part.t_off) * a.part.rs + PER * lane;
  float x[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) x[e] = 0.0f;
  for (int sp = 0; sp < a.n_split; ++sp) {
    const float *p = (const float *)a.part.base + sp * a.part_split + po;
    if constexpr (PER >= 4) {
#pragma unroll
      for (int e = 0; e < PER; e += 4) {
        const f32x4 v = *(const f32x4 *)(p + e);
#pragma unroll
        for (int q = 0; q < 4; ++q) x[e + q] += v[q];
      }
    } else {
#pragma unroll
      for (int e = 0; e < PER; ++e) x[e] += p[e];
    }
  }
  float *o = (float *)a.out.base + b * a.out.sb + (long long)(t - a.out.t_off) * a.out.rs + PER * lane;
  if constexpr (PER >= 4) {
#pragma unroll
    for (int e = 0; e < PER; e += 4) *(f32x4 *)(o + e) = f32x4{x[e], x[e + 1], x[e + 2], x[e + 3]};
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = x[e];
  }
  if (a.stats.base != nullptr) {
    float mean = 0.0f;
    if (a.layer) {
      float sm = 0.0f;
#pragma unroll
      for (int e = 0; e < PER; ++e) sm += x[e];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sm += __shfl_xor(sm, off, 64);
      mean = sm * (1.0f / D);
    }
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float c = x[e] - mean;
      ss += c * c;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if (lane == 0) {
      float *sp = (float *)a.stats.base + b * a.stats.sb + (long long)(t - a.stats.t_off) * a.stats.rs;
      sp[0] = mean;
      sp[1] = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
    }
  }
}

template <typename T, typename TR, int D, bool SPLIT>
hipError_t launch_dls(const PostArgs &a, int grid, hipStream_t s) {
  if (a.layer)
    hipLaunchKernelGGL((post_kernel<T, TR, D, true, SPLIT>), dim3(grid), dim3(post_nw<T, D>() * 64), 0, s, a);
  else
    hipLaunchKernelGGL((post_kernel<T, TR, D, false, SPLIT>), dim3(grid), dim3(post_nw<T, D>() * 64), 0, s, a);
  return hipGetLastError();
}

template <typename T, typename TR, int D>
hipError_t launch_dl(const PostArgs &a, int tiles, hipStream_t s) {
  if (a.n_split > 1) return launch_dls<T, TR, D, true>(a, tiles * a.n_split, s);
  // bf16 at d = 512: the wave-pair kernel (same 128-token tiles, no register spills)
  if constexpr (sizeof(T) == 2 && D == 512) return launch_post_pair(sizeof(TR) == 4, a, tiles, s);
  return launch_dls<T, TR, D, false>(a, tiles, s);
}

template <typename T, typename TR>
hipError_t launch_d(const PostArgs &a, int grid, hipStream_t s) {
  switch (a.d_model) {
    case 64: return launch_dl<T, TR, 64>(a, grid, s);
    case 128: return launch_dl<T, TR, 128>(a, grid, s);
    case 256: return launch_dl<T, TR, 256>(a, grid, s);
    case 512:
      if constexpr (sizeof(T) == 2) return launch_dl<T, TR, 512>(a, grid, s);
      return launch_post_f32w(512, a, grid, s);   // fp32: the 16-token-tile kernel
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

int post_tokens_per_tile(int dtype, int d_model) {
  if (dtype == 1) return (d_model == 128 ? post_nw<bf16, 128>() : post_nw<bf16, 256>()) * 32;
  if (d_model >= 512) return post_f32w_tokens_per_tile();
  return post_nw<float, 256>() * 32;
}

hipError_t launch_post_reduce(const PostArgs &a, int rows, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const dim3 gd((rows + 3) / 4), bd(256);
  switch (a.d_model) {
    case 64: hipLaunchKernelGGL((post_reduce_kernel<64>), gd, bd, 0, s, a, rows); break;
    case 128: hipLaunchKernelGGL((post_reduce_kernel<128>), gd, bd, 0, s, a, rows); break;
    case 256: hipLaunchKernelGGL((post_reduce_kernel<256>), gd, bd, 0, s, a, rows); break;
    case 512: hipLaunchKernelGGL((post_reduce_kernel<512>), gd, bd, 0, s, a, rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_post(int dtype, int resid_f32, const PostArgs &a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  if (dtype == 1) return resid_f32 ? launch_d<bf16, float>(a, grid, s) : launch_d<bf16, bf16>(a, grid, s);
  return launch_d<float, float>(a, grid, s);
}

}  // namespace ot
