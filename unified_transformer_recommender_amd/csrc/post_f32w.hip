// Fused post-attention block tail in fp32 storage at d = 512 (fp32 mode of the widest shape):
// attention output projection + residual + pre-norm 2 + mixed FFN (up, bias, GELU, down, bias) +
// residual (fun-rec-mdbook 7.5.1: Mixed FFN W2_i phi(W1_i x_i + b1_i) + b2_i, S rows sharing one
// parameter set, NS token j owning set 1 + j; pre-norm before each sub-layer).
//
// Same dataflow as the bf16 post kernel (products formed transposed, C^T = W X^T, weights streamed
// through LDS, the hidden activations of a chunk never leaving registers), but on the fp32 MFMA
// 16x16x4 tile: a wave holds 16 tokens, lane l owns token l % 16 and, in every 16-feature
// accumulator tile, features 4 (l / 16) .. 4 (l / 16) + 3 of it. A token's d = 512 accumulators then
// take 128 registers per lane instead of the 256 of a 32-token tile, so Y^T, the normalised row (B
// operand of the up-projection) and the attention output row (B operand of W^O) fit one lane's
// register budget.
//
// k order of every product: instruction kk of a d-long contraction takes, in lane group q = l / 16,
// feature 16 (kk / 4) + 4 q + kk % 4, i.e. exactly the feature that lane holds in accumulator tile
// kk / 4, element kk % 4. The normalised rows are therefore built in place from the accumulators, the
// attention output row is loaded as 16-byte pieces, and the weight rows are read from LDS as 16-byte
// pieces feeding four MFMAs each. The hidden k order of the down-projection is likewise the up-
// projection's accumulator layout (hidden unit 4 q + kk of the 16-unit chunk).
//
// Weight chunks (W^O rows, W1 rows: 16 x d; W2 columns: d x 16) flow through two LDS slots with
// direct global->LDS loads one chunk ahead. Row chunks store the 16-byte pieces of row r at slot
// p ^ (r & 15), so that the 16 lanes of one lane group (16 rows, same piece) hit 16 distinct
// 16-byte bank groups.

#include "common.hpp"
#include "launch.hpp"

namespace ot {

namespace {

constexpr int PW_NW = 4;    // waves per workgroup
constexpr int PW_TOK = 16;  // tokens per wave

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mma16(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(PW_NW * 64, 1) void post_f32w_kernel(const PostArgs a) {
  constexpr int NW = PW_NW;
  constexpr int DT = D / 16;          // 16-feature accumulator tiles
  constexpr int RP = D / 4;           // 16-byte pieces per weight row of a row chunk
  constexpr int CH = 16 * D;          // floats per chunk (16 x d or d x 16)
  constexpr int LPW = CH / 4 / 64 / NW;   // 1 KB wave loads per chunk per wave
  static_assert(LPW * NW * 64 * 4 == CH, "chunk must split into whole wave loads");
  constexpr int NB = 2;
  __shared__ __attribute__((aligned(16))) float lds[NB][CH];
  __shared__ __attribute__((aligned(16))) float svec[3 * D + POST_MAX_DFF];   // gamma, beta, b2, b1

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int DFF = a.d_ff;
  const int NC = DFF / 16;            // hidden chunks of 16 units
  const int NCH = DT + 2 * NC;

  // ---- job / group / token ---------------------------------------------------------------------
  const int bid = blockIdx.x;
  const PostJob &jb = (a.n_jobs > 1 && bid >= a.job[1].tile_start) ? a.job[1] : a.job[0];
  const int local = bid - jb.tile_start;
  const int tm = local % jb.m_tiles, grp = local / jb.m_tiles;
  const int wg = jb.rs.wg0 + grp;
  const int M_rows = jb.rs.n_seq * jb.rs.rows;
  const int r0 = tm * (NW * PW_TOK) + wave * PW_TOK + j;
  const bool valid = r0 < M_rows;
  const int r = valid ? r0 : 0;       // out-of-range lanes shadow row 0: loads stay in bounds
  const int b = r / jb.rs.rows;
  const int t = jb.rs.t0 + grp * jb.rs.t_step + (r - b * jb.rs.rows);

  const float *wo = (const float *)a.wo + (size_t)wg * D * D;
  const float *w1 = (const float *)a.w1 + (size_t)wg * DFF * D;
  const float *w2 = (const float *)a.w2 + (size_t)wg * D * DFF;
  const float *b1 = (const float *)a.b1 + (size_t)wg * DFF;
  const float *b2 = (const float *)a.b2 + (size_t)wg * D;

  // ---- weight chunk stream ---------------------------------------------------------------------
  // chunk i < DT: W^O rows 16 i ..; DT + 2c: W1 rows of hidden chunk c; DT + 2c + 1: W2 columns of c.
  // LDS slot P of a chunk (16 bytes) = piece (j * NW + wave) * 64 + lane of this wave's load j.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t off_r[LPW], off_c[LPW];
#pragma unroll
  for (int l = 0; l < LPW; ++l) {
    const int P = (l * NW + wave) * 64 + lane;
    const int rr = P / RP, pr = P % RP;              // row chunk: row rr, LDS slot pr
    off_r[l] = (uint32_t)((rr * D + (pr ^ (rr & 15)) * 4) * 4);
    const int rc = P / 4, pc = P % 4;                // column chunk: row rc, piece pc
    off_c[l] = (uint32_t)((rc * DFF + pc * 4) * 4);
  }
  auto issue = [&](int i) {
    const float *base;
    bool cols = false;
    if (i < DT) {
      base = wo + (size_t)(16 * i) * D;
    } else {
      const int c = (i - DT) >> 1;
      if (((i - DT) & 1) == 0) {
        base = w1 + (size_t)(16 * c) * D;
      } else {
        base = w2 + 16 * c;
        cols = true;
      }
    }
    const uint32_t dst = lds_addr(lds[i % NB]);
#pragma unroll
    for (int l = 0; l < LPW; ++l)
      dma16s(base, cols ? off_c[l] : off_r[l], dst + (uint32_t)((l * NW + wave_s) * 64 * 16));
  };
  // chunk i visible: every load issued so far has landed (the next chunk is issued after this), this
  // wave's LDS reads of chunk i - 1 are done, then every wave's
  auto arrive = [&]() {
    wait_vm<0>();
    wait_lgkm0();
    bare_barrier();
  };
  // 16-byte piece m (features 16 m + 4 q .. + 3) of row `row` of a row chunk
  auto rpiece = [&](const float *base, int row, int m) -> f32x4_t {
    return *(const f32x4_t *)(base + row * D + (((4 * m + q) ^ (row & 15)) * 4));
  };

  issue(0);
  float *s_gm = svec, *s_bt = svec + D, *s_b2 = svec + 2 * D, *s_b1 = svec + 3 * D;
  for (int i = tid; i < 3 * D + DFF; i += NW * 64) {
    float v;
    if (i < D) v = ((const float *)a.gamma)[i];
    else if (i < 2 * D) v = a.layer ? ((const float *)a.beta)[i - D] : 0.0f;   // RMSNorm: no shift
    else if (i < 3 * D) v = b2[i - 2 * D];
    else v = b1[i - 3 * D];
    svec[i] = v;
  }

  // attention output row (B operand of W^O) and residual row (initial accumulators), 16-byte pieces
  float ofr[D / 4];
  f32x4_t acc[DT];
  {
    const float *orow = (const float *)a.o.base + b * a.o.sb + (long long)(t - a.o.t_off) * a.o.rs + 4 * q;
    const float *xr = (const float *)a.resid.base + b * a.resid.sb + (long long)(t - a.resid.t_off) * a.resid.rs + 4 * q;
#pragma unroll
    for (int m = 0; m < DT; ++m) {
      const f32x4_t o4 = *(const f32x4_t *)(orow + 16 * m);
#pragma unroll
      for (int e = 0; e < 4; ++e) ofr[4 * m + e] = o4[e];
      acc[m] = *(const f32x4_t *)(xr + 16 * m);
    }
  }

  // ---- W^O: Y^T = X^T + Wo O^T, one 16-feature tile per chunk (unrolled: static accumulator index)
#pragma unroll
  for (int ti = 0; ti < DT; ++ti) {
    arrive();
    if (ti + 1 < NCH) issue(ti + 1);
    const float *base = lds[ti % NB];
    f32x4_t c = acc[ti];
#pragma unroll
    for (int m = 0; m < DT; ++m) {
      const f32x4_t w4 = rpiece(base, j, m);
#pragma unroll
      for (int e = 0; e < 4; ++e) c = mma16(w4[e], ofr[4 * m + e], c);
    }
    acc[ti] = c;
  }

  // ---- norm2 (statistics over the 4 lane groups), + b2 ------------------------------------------
  float yfr[D / 4];
  {
    float mean = 0.0f;
    if (a.layer) {
      float s = 0.0f;
#pragma unroll
      for (int m = 0; m < DT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) s += acc[m][e];
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      mean = s * (1.0f / D);
    }
    float ss = 0.0f;
#pragma unroll
    for (int m = 0; m < DT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c = acc[m][e] - mean;
        ss += c * c;
      }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float rstd = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
    for (int m = 0; m < DT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 16 * m + 4 * q + e;
        yfr[4 * m + e] = (acc[m][e] - mean) * rstd * s_gm[f] + s_bt[f];
        acc[m][e] += s_b2[f];
      }
  }

  // ---- FFN: per 16-unit hidden chunk c: up-projection (W1 chunk), + b1, GELU; down-projection (W2
  // chunk) into X'^T ----------------------------------------------------------------------------
  for (int c = 0; c < NC; ++c) {
    const int ia = DT + 2 * c;
    arrive();
    if (ia + 1 < NCH) issue(ia + 1);
    f32x4_t h = *(const f32x4_t *)(s_b1 + 16 * c + 4 * q);
    {
      const float *base = lds[ia % NB];
#pragma unroll
      for (int m = 0; m < DT; ++m) {
        const f32x4_t w4 = rpiece(base, j, m);
#pragma unroll
        for (int e = 0; e < 4; ++e) h = mma16(w4[e], yfr[4 * m + e], h);
      }
    }
    float hv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) hv[e] = gelu_as(h[e]);
    arrive();
    if (ia + 2 < NCH) issue(ia + 2);
    {
      const float *base = lds[(ia + 1) % NB];
      // row 16 m + j of the W2 column chunk, piece q: hidden units 4 q .. 4 q + 3 of the chunk
#pragma unroll
      for (int m = 0; m < DT; ++m) {
        const f32x4_t w4 = *(const f32x4_t *)(base + (16 * m + j) * 16 + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[m] = mma16(w4[e], hv[e], acc[m]);
      }
    }
  }

  // ---- store X' (fp32): tile m of this lane is features 16 m + 4 q .. + 3 of its token ------------
  if (valid) {
    float *orow = (float *)a.out.base + b * a.out.sb + (long long)(t - a.out.t_off) * a.out.rs + 4 * q;
#pragma unroll
    for (int m = 0; m < DT; ++m) *(f32x4_t *)(orow + 16 * m) = acc[m];
  }
}

}  // namespace

int post_f32w_tokens_per_tile() { return PW_NW * PW_TOK; }

hipError_t launch_post_f32w(int d_model, const PostArgs &a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  if (d_model != 512) return hipErrorInvalidValue;
  hipLaunchKernelGGL((post_f32w_kernel<512>), dim3(grid), dim3(PW_NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace ot
