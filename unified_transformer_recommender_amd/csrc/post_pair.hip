// Fused post-attention block tail for bf16 storage at d = 512, wave-pair form: attention
// output projection + residual + pre-norm 2 + mixed FFN (up, bias, GELU, down, bias) + residual
// (fun-rec-mdbook 7.5.1: Mixed FFN W2_i phi(W1_i x_i + b1_i) + b2_i with S rows sharing one
// parameter set and NS token j owning set 1 + j; pre-norm before each sub-layer).
//
// Same orientation as post_kernel (C^T = W X^T: an MFMA tile's 32 columns are 32 tokens, a lane owns
// one token), but the waves work in pairs over G groups of 32 tokens. Wave half hf of a pair owns
// the output features [hf d/2, (hf + 1) d/2) of X'^T for all of the pair's tokens, and the matching
// half of the contraction of the FFN's up-projection:
//   W^O   streamed as column chunks (d rows x 32 input features): each half multiplies its rows by
//         the chunk's 32 features of O (fragments loaded one chunk ahead) into its Y^T half;
//   norm2 per-token sums of the two halves are added through LDS; each half keeps the normalised
//         values of its own features as the up-projection's B fragments;
//   W1    row chunks (32 hidden units x d): each half forms the partial pre-activation over its
//         half of d; the two partials are added through LDS (lane l of both waves holds the same
//         (unit, token) elements), then + b1, GELU, bf16 B fragments;
//   W2    column chunks (d rows x 32 hidden units): each half accumulates its rows into X'^T.
// Every weight fragment read from LDS feeds G MFMAs (one per token group), while a lane's registers
// hold d/2 features of G tokens: at d = 512 with G = 1 that halves the single-wave form's state,
// which does not fit its register budget without spills.
//
// Weight streaming as in post_kernel: a ring of two LDS chunk buffers filled by direct global->LDS
// loads one chunk ahead, one fence-free barrier per chunk, XOR-swizzled 16-byte pieces.

#include "common.hpp"
#include "launch.hpp"

namespace ot {

namespace {

// bf16 accumulator-fed B fragment: lane half g holds k {4g..4g+3, 8+4g..8+4g+3} of a 16-block;
// exchange the middle 8-byte halves between the lane halves to get k {8g .. 8g+7}.
__device__ __forceinline__ bf16x8 natural_kfrag2(bf16x8 f) {
  u32x4 u = __builtin_bit_cast(u32x4, f);
  const auto s0 = __builtin_amdgcn_permlane32_swap(u[0], u[2], false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(u[1], u[3], false, false);
  u[0] = s0[0]; u[2] = s0[1];
  u[1] = s1[0]; u[3] = s1[1];
  return __builtin_bit_cast(bf16x8, u);
}

// Piece q of row r of a chunk whose rows hold RP 16-byte pieces sits at slot q ^ swz(r); rows
// sharing one 256-byte bank line are swizzled together.
template <int RP>
__device__ __forceinline__ constexpr int pswz(int r) {
  constexpr int rb = RP * 16;
  constexpr int rpb = rb >= 256 ? 1 : 256 / rb;
  constexpr int P = RP < 16 / rpb ? RP : 16 / rpb;
  return (r / rpb) & (P - 1);
}

// Pairs per workgroup and token groups per wave. At d = 512 one group: a lane holds 256 features of
// one token (128 accumulator registers) and the kernel fits 256 registers with no spills, two waves
// per SIMD. (Two groups at d = 256 measured 1.8x slower than post_kernel: the doubled state needs
// AGPRs and one wave per SIMD, or spills at two.)
template <int D> struct PairCfg;
template <> struct PairCfg<512> { static constexpr int NP = 4, G = 1, WAVES_PER_SIMD = 2; };   // 8 waves

template <typename TR, int D, bool LAYER>
__global__ __launch_bounds__(2 * PairCfg<D>::NP * 64, PairCfg<D>::WAVES_PER_SIMD) void post_pair_kernel(const PostArgs a) {
  using T = bf16;
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int NP = PairCfg<D>::NP, G = PairCfg<D>::G;
  constexpr int NW = 2 * NP;                    // waves
  constexpr int EPC = 8;                        // bf16 per 16-byte piece
  constexpr int HD = D / 2;                     // features per half
  constexpr int HT = HD / 32;                   // feature tiles per half
  constexpr int HKC = HD / 16;                  // 16-wide k-chunks of a half
  constexpr int RPA = D / EPC;                  // pieces per row of a row chunk (W1: 32 x d)
  constexpr int RPC = 32 / EPC;                 // pieces per row of a column chunk (W^O, W2: d x 32)
  constexpr int CH = 32 * D;                    // elements per chunk
  constexpr int LPW = CH / EPC / 64 / NW;       // 1 KB wave loads per chunk and wave
  static_assert(LPW * NW * 64 * EPC == CH, "chunk must split into whole wave loads");
  constexpr int DT = D / 32;                    // W^O column chunks
  constexpr int PD = 4;                         // LDS operand reads in flight ahead of the MFMAs
  __shared__ __attribute__((aligned(16))) T lds[2][CH];
  // partial pre-activations of the pair halves: [wave][group][element v][lane]
  __shared__ __attribute__((aligned(16))) float hx[NW][G][16][64];
  // per-token partial sums of the two halves (norm 2, and the statistics of X'): [wave][group][token]
  __shared__ float nx[NW][G][32];
  // gamma, beta, b2 [d] and b1 [d_ff] of this parameter set, fp32
  __shared__ __attribute__((aligned(16))) float svec[3 * D + POST_MAX_DFF];
  // the next block's norm-1 gamma / beta, fp32, when this launch hands over normalised rows
  __shared__ __attribute__((aligned(16))) float s_xg[D], s_xb[D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lc = lane & 31;
  const int pair = wave >> 1, hf = wave & 1, partner = wave ^ 1;
  const int DFF = a.d_ff;
  const int NC = DFF / 32;                      // hidden chunks
  const int NCH = DT + 2 * NC;                  // chunks in the stream

  // ---- job / group / token tile --------------------------------------------------------------
  const PostJob &jb = (a.n_jobs > 1 && (int)blockIdx.x >= a.job[1].tile_start) ? a.job[1] : a.job[0];
  const int local = blockIdx.x - jb.tile_start;
  const int tm = local % jb.m_tiles, grp = local / jb.m_tiles;
  const int wg = jb.rs.wg0 + grp;
  const int M_rows = jb.rs.n_seq * jb.rs.rows;
  bool valid[G];
  int tb[G], tt[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int r0 = tm * (NP * G * 32) + pair * (G * 32) + gi * 32 + lc;   // this lane's token in group gi
    valid[gi] = r0 < M_rows;
    const int r = valid[gi] ? r0 : 0;           // out-of-range lanes shadow row 0: loads stay in bounds
    tb[gi] = r / jb.rs.rows;
    tt[gi] = jb.rs.t0 + grp * jb.rs.t_step + (r - tb[gi] * jb.rs.rows);
  }

  const T *wo = (const T *)a.wo + (size_t)wg * D * D;
  const T *w1 = (const T *)a.w1 + (size_t)wg * DFF * D;
  const T *w2 = (const T *)a.w2 + (size_t)wg * D * DFF;
  const T *b1 = (const T *)a.b1 + (size_t)wg * DFF;
  const T *b2 = (const T *)a.b2 + (size_t)wg * D;

  // ---- weight chunk stream --------------------------------------------------------------------
  // chunk i: i < DT           -> W^O columns 32i..32i+31 (all d rows; row stride d)
  //          i == DT + 2c     -> W1 rows of hidden chunk c (32 x d)
  //          i == DT + 2c + 1 -> W2 columns of hidden chunk c (all d rows; row stride d_ff)
  // This lane's piece of wave load j sits at LDS piece P = (j * NW + wave) * 64 + lane.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t off_r[LPW], off_o[LPW], off_2[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int P = (j * NW + wave) * 64 + lane;
    const int rr = P / RPA, qr = P % RPA, rc = P / RPC, qc = P % RPC;
    off_r[j] = (uint32_t)((rr * D + (qr ^ pswz<RPA>(rr)) * EPC) * 2);
    off_o[j] = (uint32_t)((rc * D + (qc ^ pswz<RPC>(rc)) * EPC) * 2);
    off_2[j] = (uint32_t)((rc * DFF + (qc ^ pswz<RPC>(rc)) * EPC) * 2);
  }
  auto issue = [&](int i) {
    const T *base;
    const uint32_t *off;
    if (i < DT) {
      base = wo + 32 * i;
      off = off_o;
    } else {
      const int c = (i - DT) >> 1;
      if (((i - DT) & 1) == 0) {
        base = w1 + (size_t)(32 * c) * D;
        off = off_r;
      } else {
        base = w2 + 32 * c;
        off = off_2;
      }
    }
    const uint32_t dst = lds_addr(lds[i & 1]);
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma16s(base, off[j], dst + (uint32_t)((j * NW + wave_s) * 64 * 16));
  };
  // chunk i has landed for every wave (two buffers: nothing else is in flight behind it)
  auto arrive = [&]() {
    wait_vm<0>();
    wait_lgkm0();
    bare_barrier();
  };
  // A fragments: a row chunk's row `row`, k-chunk kc (16 features); a column chunk's row `row`,
  // k-chunk kc (16 of its 32 columns)
  auto afrag_row = [&](const T *base, int row, int kc) -> frag {
    const int q = (2 * kc + g) ^ pswz<RPA>(row);
    return *(const frag *)(base + row * D + q * EPC);
  };
  auto afrag_col = [&](const T *base, int row, int kc) -> frag {
    const int q = (2 * kc + g) ^ pswz<RPC>(row);
    return *(const frag *)(base + row * 32 + q * EPC);
  };
  // this wave's half of the per-token partial sums s[gi] -> the full sums (one barrier)
  auto pair_sum = [&](float (&s)[G]) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      s[gi] += __shfl_xor(s[gi], 32, 64);
      if (g == 0) nx[wave][gi][lc] = s[gi];
    }
    wait_lgkm0();
    bare_barrier();
#pragma unroll
    for (int gi = 0; gi < G; ++gi) s[gi] += nx[partner][gi][lc];
    wait_lgkm0();
    bare_barrier();   // nx may be written again
  };

  // prologue: start the weight stream, then the per-token loads
  issue(0);

  // Per-feature vectors into LDS: every thread's loads issued together and waited for once
  // (elements without a source read gamma[0] and are discarded, so no branch separates the loads).
  float *s_gm = svec, *s_bt = svec + D, *s_b2 = svec + 2 * D, *s_b1 = svec + 3 * D;
  {
    constexpr int NT = NW * 64;
    constexpr int SV = (3 * D + POST_MAX_DFF + NT - 1) / NT;
    const int nsv = 3 * D + DFF;
    const T *const g0 = (const T *)a.gamma;
    float sv[SV];
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
    for (int k = 0; k < SV; ++k)
      if (tid + k * NT < nsv) svec[tid + k * NT] = sv[k];
  }
  const bool hand = a.xh != nullptr;
  if (hand)
    for (int i = tid; i < D; i += NW * 64) {   // D / (NW * 64) = 1 at d = 512
      s_xg[i] = to_f32(((const T *)a.xh_gamma)[i]);
      s_xb[i] = LAYER ? to_f32(((const T *)a.xh_beta)[i]) : 0.0f;
    }

  // O rows of this lane's tokens; the B fragments of W^O chunk i are O[k = 32 i + 16 kk + 8 g ..]
  const T *orow[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
    orow[gi] = (const T *)a.o.base + tb[gi] * a.o.sb + (long long)(tt[gi] - a.o.t_off) * a.o.rs + 8 * g;
  frag ofr[G][2];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) ofr[gi][kk] = *(const frag *)(orow[gi] + 16 * kk);

  // Y^T accumulators of this half start from the residual rows X^T (fp32, or bf16 in block 0)
  f32x16 acc[G][HT];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const TR *xr = (const TR *)a.resid.base + tb[gi] * a.resid.sb + (long long)(tt[gi] - a.resid.t_off) * a.resid.rs +
                   hf * HD + 4 * g;
#pragma unroll
    for (int ti = 0; ti < HT; ++ti)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(TR) == 4) {
          const f32x4 v4 = *(const f32x4 *)(xr + 32 * ti + 8 * j);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[gi][ti][4 * j + q] = v4[q];
        } else {
          const bf16x4 v4 = *(const bf16x4 *)(xr + 32 * ti + 8 * j);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[gi][ti][4 * j + q] = (float)v4[q];
        }
      }
  }

  // ---- W^O: Y^T = X^T + Wo O^T, one chunk of 32 input features at a time ---------------------
  for (int i = 0; i < DT; ++i) {
    arrive();
    if (i + 1 < NCH) issue(i + 1);
    frag cur[G][2];
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) cur[gi][kk] = ofr[gi][kk];
    if (i + 1 < DT) {   // next chunk's O fragments, in flight during this chunk
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) ofr[gi][kk] = *(const frag *)(orow[gi] + 32 * (i + 1) + 16 * kk);
    }
    const T *base = lds[i & 1];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int ti = 0; ti < HT; ++ti) {
        const frag wa = afrag_col(base, hf * HD + 32 * ti + lc, kk);
#pragma unroll
        for (int gi = 0; gi < G; ++gi) acc[gi][ti] = M::mma(wa, cur[gi][kk], acc[gi][ti]);
      }
    sched_lds_mfma<2 * HT, 2 * HT * G, PD>();
  }

  // ---- norm2, + b2 ----------------------------------------------------------------------------
  frag yfr[G][HKC];
  {
    float mean[G], ss[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) mean[gi] = 0.0f;
    if constexpr (LAYER) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        float s = 0.0f;
#pragma unroll
        for (int ti = 0; ti < HT; ++ti)
#pragma unroll
          for (int v = 0; v < 16; ++v) s += acc[gi][ti][v];
        mean[gi] = s;
      }
      pair_sum(mean);
#pragma unroll
      for (int gi = 0; gi < G; ++gi) mean[gi] *= 1.0f / D;
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      float s = 0.0f;
#pragma unroll
      for (int ti = 0; ti < HT; ++ti)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float c = acc[gi][ti][v] - mean[gi];
          s += c * c;
        }
      ss[gi] = s;
    }
    pair_sum(ss);
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const float rstd = 1.0f / sqrtf(ss[gi] * (1.0f / D) + a.eps);
#pragma unroll
      for (int ti = 0; ti < HT; ++ti) {
        float yh[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int f = hf * HD + 32 * ti + acc_row(v, g);
          float y = (acc[gi][ti][v] - mean[gi]) * rstd * s_gm[f];
          if constexpr (LAYER) y += s_bt[f];
          yh[v] = y;
          acc[gi][ti][v] += s_b2[f];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          frag fr;
#pragma unroll
          for (int e = 0; e < 8; ++e) fr[e] = (bf16)yh[8 * h + e];
          yfr[gi][2 * ti + h] = natural_kfrag2(fr);
        }
      }
    }
  }

  // ---- FFN: per hidden chunk c, the up-projection over this half of d (W1 chunk), the pair's
  // partial pre-activations added through LDS, GELU, then the down-projection of this half's rows
  // (W2 chunk) into X'^T
  for (int c = 0; c < NC; ++c) {
    const int ia = DT + 2 * c;
    arrive();
    if (ia + 1 < NCH) issue(ia + 1);
    f32x16 h[G];
    {
      // half 0's partial starts from the bias b1 (accumulator row layout), half 1's from zero
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 b4 = *(const f32x4 *)(s_b1 + 32 * c + 8 * j + 4 * g);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int gi = 0; gi < G; ++gi) h[gi][4 * j + q] = hf == 0 ? b4[q] : 0.0f;
      }
      const T *base = lds[ia & 1];
#pragma unroll
      for (int kc = 0; kc < HKC; ++kc) {
        const frag wa = afrag_row(base, lc, hf * HKC + kc);
#pragma unroll
        for (int gi = 0; gi < G; ++gi) h[gi] = M::mma(wa, yfr[gi][kc], h[gi]);
      }
      sched_lds_mfma<HKC, HKC * G, PD>();
    }
    // this half's partial pre-activations for the partner (element v of lane l at [v][l]: the
    // partner's lane l holds the same (unit, token) elements)
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int v = 0; v < 16; ++v) hx[wave][gi][v][lane] = h[gi][v];
    arrive();   // W2 chunk landed; the partners' partial pre-activations are visible
    if (ia + 2 < NCH) issue(ia + 2);
    frag hfr[G][2];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      float hv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) hv[v] = gelu_fit(h[gi][v] + hx[partner][gi][v][lane]);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        frag fr;
#pragma unroll
        for (int e = 0; e < 8; ++e) fr[e] = (bf16)hv[8 * hh + e];
        hfr[gi][hh] = natural_kfrag2(fr);
      }
    }
    {
      const T *base = lds[(ia + 1) & 1];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int ti = 0; ti < HT; ++ti) {
          const frag wa = afrag_col(base, hf * HD + 32 * ti + lc, kk);
#pragma unroll
          for (int gi = 0; gi < G; ++gi) acc[gi][ti] = M::mma(wa, hfr[gi][kk], acc[gi][ti]);
        }
      sched_lds_mfma<2 * HT, 2 * HT * G, PD>();
    }
  }

  // ---- statistics of X' for the next block's norm 1 (exact two-pass over the pair's halves), and
  // that norm's output in the next QKV launch's fragment order (this half's 16 k-chunks) -------
  if (a.stats.base != nullptr || hand) {
    float mean[G], ss[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) mean[gi] = 0.0f;
    if constexpr (LAYER) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        float s = 0.0f;
#pragma unroll
        for (int ti = 0; ti < HT; ++ti)
#pragma unroll
          for (int v = 0; v < 16; ++v) s += acc[gi][ti][v];
        mean[gi] = s;
      }
      pair_sum(mean);
#pragma unroll
      for (int gi = 0; gi < G; ++gi) mean[gi] *= 1.0f / D;
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      float s = 0.0f;
#pragma unroll
      for (int ti = 0; ti < HT; ++ti)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float c = acc[gi][ti][v] - mean[gi];
          s += c * c;
        }
      ss[gi] = s;
    }
    pair_sum(ss);
    float rstd[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) rstd[gi] = 1.0f / sqrtf(ss[gi] * (1.0f / D) + a.eps);
    if (a.stats.base != nullptr && hf == 0 && g == 0) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        if (!valid[gi]) continue;
        float *sp = (float *)a.stats.base + tb[gi] * a.stats.sb + (long long)(tt[gi] - a.stats.t_off) * a.stats.rs;
        sp[0] = mean[gi];
        sp[1] = rstd[gi];
      }
    }
    if (hand) {
      // the same arithmetic as the QKV kernel's norm of a stored X' row; k-chunk hf * HD / 16 + 2 ti + h
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        u32x4 *dst = (u32x4 *)a.xh + xh_piece(jb.xh_g0, grp, M_rows, (tm * NP + pair) * G + gi, D / 16, 0, lane);
#pragma unroll
        for (int ti = 0; ti < HT; ++ti)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            frag fr;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int f = hf * HD + 32 * ti + acc_row(8 * h + e, g);
              fr[e] = (bf16)((acc[gi][ti][8 * h + e] - mean[gi]) * rstd[gi] * s_xg[f] + s_xb[f]);
            }
            const u32x4 piece = __builtin_bit_cast(u32x4, natural_kfrag2(fr));
            if (valid[gi]) st16(dst + (hf * (HD / 16) + 2 * ti + h) * 64, piece);
          }
      }
    }
  }

  // ---- store this half of X' (fp32) through the wave's staging tile, which reuses the weight
  // ring once every wave is done with the last chunk
  wait_lgkm0();
  bare_barrier();
  {
    using TS = TileStage<float>;
    static_assert(NW * TS::SIZE * 4 <= 2 * CH * 2, "staging fits in the weight ring");
    float *stg = reinterpret_cast<float *>(&lds[0][0]) + wave * TS::SIZE;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      float *rowp[TS::NI];
      bool rv[TS::NI];
#pragma unroll
      for (int k = 0; k < TS::NI; ++k) {
        const int tok = TS::token(k, lane);
        const int b = __shfl(tb[gi], tok, 64), t = __shfl(tt[gi], tok, 64);
        rv[k] = __shfl((int)valid[gi], tok, 64) != 0 && t - a.out.t_off >= a.out_from;
        rowp[k] = (float *)a.out.base + b * a.out.sb + (long long)(t - a.out.t_off) * a.out.rs + hf * HD +
                  TS::feature(lane);
      }
#pragma unroll
      for (int ti = 0; ti < HT; ++ti) {
        TS::put(stg, acc[gi][ti], lc, g);
        wait_lgkm0();
#pragma unroll
        for (int k = 0; k < TS::NI; ++k) {
          const u32x4 piece = TS::get(stg, k, lane);
          if (rv[k]) st16(rowp[k] + 32 * ti, piece);
        }
        wait_lgkm0();
      }
    }
  }
}

template <typename TR, int D>
hipError_t launch_d2(const PostArgs &a, int grid, hipStream_t s) {
  const dim3 bd(2 * PairCfg<D>::NP * 64);
  if (a.layer) hipLaunchKernelGGL((post_pair_kernel<TR, D, true>), dim3(grid), bd, 0, s, a);
  else hipLaunchKernelGGL((post_pair_kernel<TR, D, false>), dim3(grid), bd, 0, s, a);
  return hipGetLastError();
}

}  // namespace

int post_pair_tokens_per_tile(int d_model) {
  return d_model == 512 ? PairCfg<512>::NP * PairCfg<512>::G * 32 : 0;
}

hipError_t launch_post_pair(int resid_f32, const PostArgs &a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  if (a.d_model == 512) return resid_f32 ? launch_d2<float, 512>(a, grid, s) : launch_d2<bf16, 512>(a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace ot
