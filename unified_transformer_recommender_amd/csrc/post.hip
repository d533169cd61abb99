// Fused post-attention block tail: attention output projection + residual + pre-norm 2 + mixed FFN
// (up, bias, GELU, down, bias) + residual, for the query rows of a block (fun-rec-mdbook 7.5.1:
// Mixed FFN W2_i phi(W1_i x_i + b1_i) + b2_i with S rows sharing one parameter set and NS token j
// owning set 1 + j; pre-norm before each sub-layer).
//
// Orientation: every product is formed transposed, C^T = W X^T, so that the 32 columns of an
// MFMA 32x32 tile are 32 tokens and each lane owns ONE token. Per token the wave keeps
//   Y^T   (d x 32 fp32 accumulators)          -> becomes X'^T after the FFN adds into it
//   Yh^T  (norm2 output, bf16 B fragments)   -> B operand of the FFN up-projection
// and streams the weights (A operand) through LDS in chunks of 32 rows shared by all waves.
// An accumulator tile's lane holds k-indices {4g + r + 8j}; using it directly as the next
// product's B fragment permutes the k order inside every 16-block (bits 2 and 3 of k swap), so the
// W1 and W2 chunks are written to LDS with the same permutation. The hidden activations of a
// 32-unit chunk never leave registers: up-projection tile -> +b1 -> GELU -> bf16 -> B fragments of
// the down-projection, which accumulates straight into X'^T.
//
// GELU is the exact erf form 0.5 x (1 + erf(x / sqrt 2)); erf is evaluated with Abramowitz &
// Stegun 7.1.26 (|error| <= 1.5e-7): with z = |x|/sqrt2, t = 1/(1 + p z),
//   GELU(x) = max(x, 0) - |x| * 0.5 t (a1 + t(a2 + t(a3 + t(a4 + t a5)))) * exp(-x^2 / 2).

#include "common.hpp"
#include "launch.hpp"

namespace ot {

namespace {

__device__ __forceinline__ float gelu_as(float x) {
  // Abramowitz & Stegun 7.1.26 coefficients, halved so that q = 0.5 t P(t)
  constexpr float p = 0.3275911f * 0.70710678118654752f;   // p / sqrt(2): t = 1 / (1 + p |x| / sqrt 2)
  constexpr float a1 = 0.5f * 0.254829592f, a2 = 0.5f * -0.284496736f, a3 = 0.5f * 1.421413741f,
                  a4 = 0.5f * -1.453152027f, a5 = 0.5f * 1.061405429f;
  constexpr float neg_half_log2e = -0.72134752044448170f;   // -0.5 * log2(e)
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(p, ax, 1.0f));
  const float q = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  const float e = __builtin_amdgcn_exp2f(x * x * neg_half_log2e);
  return fmaf(-ax * q, e, fmaxf(x, 0.0f));
}

// Index of k inside LDS for an accumulator-fed B operand (bf16): bits 2 and 3 of k swapped.
__device__ __forceinline__ constexpr int kperm(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// Waves per workgroup: two per SIMD where the per-token state (d/32 accumulator tiles plus the
// norm2 fragments) fits in half the register file, else one.
template <typename T, int D>
constexpr int post_nw() { return (sizeof(T) == 2 && D <= 128) ? 8 : 4; }

template <typename T, typename TR, int D>
__global__ __launch_bounds__((post_nw<T, D>() * 64)) void post_kernel(const PostArgs a) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int NW = post_nw<T, D>();
  constexpr int NT = NW * 64;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int DT = D / 32;                    // feature tiles
  constexpr int KC = D / M::KSTEP;              // k-chunks over d
  constexpr int LDA = D + EPC;                  // LDS row of a 32 x d chunk (Wo, W1)
  constexpr int LDB = 32 + EPC;                 // LDS row of a d x 32 chunk (W2)
  constexpr int BUF = (32 * LDA > D * LDB) ? 32 * LDA : D * LDB;
  constexpr int PIECES = 32 * D / EPC;          // 16-byte pieces per chunk
  constexpr int PPT = (PIECES + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) T lds[2][BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lc = lane & 31;
  const int DFF = a.d_ff;

  // ---- job / group / token tile --------------------------------------------------------------
  const int bid = blockIdx.x;
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
  const T *w1 = (const T *)a.w1 + (size_t)wg * DFF * D;
  const T *w2 = (const T *)a.w2 + (size_t)wg * D * DFF;
  const T *b1 = (const T *)a.b1 + (size_t)wg * DFF;
  const T *b2 = (const T *)a.b2 + (size_t)wg * D;
  const int n_wo = DT;
  const int n_chunks = n_wo + 2 * (DFF / 32);

  // ---- chunk staging: global -> registers -> LDS ------------------------------------------
  u32x4 pre[PPT];
  auto prefetch = [&](int id) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * NT;
      if (p >= PIECES) break;
      const T *src;
      if (id < n_wo || ((id - n_wo) & 1) == 0) {      // Wo or W1 chunk: 32 rows x d
        const int row = p / (D / EPC), kp = (p - row * (D / EPC)) * EPC;
        const T *base = id < n_wo ? wo + (size_t)(id * 32) * D : w1 + (size_t)(((id - n_wo) >> 1) * 32) * D;
        src = base + (size_t)row * D + kp;
      } else {                                          // W2 chunk: d rows x 32 hidden
        const int row = p / (32 / EPC), kp = (p - row * (32 / EPC)) * EPC;
        src = w2 + (size_t)row * DFF + ((id - n_wo) >> 1) * 32 + kp;
      }
      pre[i] = ld16(src);
    }
  };
  auto commit = [&](int id, int buf) {
    T *dst = lds[buf];
    const bool permute = sizeof(T) == 2 && id >= n_wo;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * NT;
      if (p >= PIECES) break;
      int row, kp, ld;
      if (id < n_wo || ((id - n_wo) & 1) == 0) {
        row = p / (D / EPC); kp = (p - row * (D / EPC)) * EPC; ld = LDA;
      } else {
        row = p / (32 / EPC); kp = (p - row * (32 / EPC)) * EPC; ld = LDB;
      }
      T *d = dst + row * ld;
      if (permute) {
        // 8 consecutive k (k0 = 16m + 8a): first half to 16m + 4a, second half to 16m + 8 + 4a
        const uint2 lo = {pre[i][0], pre[i][1]}, hi = {pre[i][2], pre[i][3]};
        *(uint2 *)(d + kperm(kp)) = lo;
        *(uint2 *)(d + kperm(kp + 4)) = hi;
      } else {
        st16(d + kp, pre[i]);
      }
    }
  };

  // A fragment of row `row` (LDS, leading dim ld) for k-chunk kc; `perm` = accumulator-fed B.
  auto afrag = [&](const T *base, int ld, int row, int kc, bool perm) -> frag {
    if constexpr (sizeof(T) == 2) {
      (void)perm;
      return *(const frag *)(base + row * ld + kc * 16 + g * 8);
    } else {
      const int k = perm ? 32 * (kc >> 4) + acc_row(kc & 15, g) : kc * 2 + g;
      return base[row * ld + k];
    }
  };

  // ---- B fragments of O^T (attention output of this lane's token) -----------------------------
  frag ofr[KC];
  {
    const T *orow = (const T *)a.o.base + b * a.o.sb + (long long)(t - a.o.t_off) * a.o.rs;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if constexpr (sizeof(T) == 2)
        ofr[kc] = *(const frag *)(orow + kc * 16 + g * 8);
      else
        ofr[kc] = orow[kc * 2 + g];
    }
  }

  prefetch(0);
  commit(0, 0);
  __syncthreads();

  f32x16 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x16{};

  // ---- W^O: Y^T = Wo O^T, one 32-feature tile per chunk ---------------------------------------
#pragma unroll
  for (int ti = 0; ti < DT; ++ti) {
    const int cur = ti & 1;
    prefetch(ti + 1);
    const T *base = lds[cur];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) acc[ti] = M::mma(afrag(base, LDA, lc, kc, false), ofr[kc], acc[ti]);
    commit(ti + 1, cur ^ 1);
    __syncthreads();
  }

  // ---- residual, norm2, + b2 ------------------------------------------------------------------
  {
    const TR *xr = (const TR *)a.resid.base + b * a.resid.sb + (long long)(t - a.resid.t_off) * a.resid.rs;
#pragma unroll
    for (int ti = 0; ti < DT; ++ti)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[ti][4 * j + q] += to_f32(xr[32 * ti + 8 * j + 4 * g + q]);
  }
  frag yfr[KC];
  {
    float mean = 0.0f;
    if (a.layer) {
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
    const T *gm = (const T *)a.gamma;
    const T *bt = (const T *)a.beta;
#pragma unroll
    for (int ti = 0; ti < DT; ++ti) {
      float yh[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int f = 32 * ti + acc_row(v, g);
        float y = (acc[ti][v] - mean) * rstd * to_f32(gm[f]);
        if (a.layer) y += to_f32(bt[f]);
        yh[v] = y;
        acc[ti][v] += to_f32(b2[f]);
      }
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          frag fr;
#pragma unroll
          for (int e = 0; e < 8; ++e) fr[e] = (bf16)yh[8 * h + e];
          yfr[2 * ti + h] = fr;
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) yfr[16 * ti + v] = yh[v];
      }
    }
  }

  // ---- FFN: per 32 hidden units, up (+b1, GELU) then down into X'^T ---------------------------
  for (int c = 0; c < DFF / 32; ++c) {
    const int id = n_wo + 2 * c;
    // up-projection chunk (LDS buffer (id & 1))
    prefetch(id + 1);
    f32x16 h = f32x16{};
    {
      const T *base = lds[id & 1];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) h = M::mma(afrag(base, LDA, lc, kc, true), yfr[kc], h);
    }
    commit(id + 1, (id + 1) & 1);
    __syncthreads();
    // bias + GELU -> B fragments of the down-projection
    constexpr int HKC = 32 / M::KSTEP;
    frag hfr[HKC];
    {
      float hv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) hv[v] = gelu_as(h[v] + to_f32(b1[32 * c + acc_row(v, g)]));
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          frag fr;
#pragma unroll
          for (int e = 0; e < 8; ++e) fr[e] = (bf16)hv[8 * hh + e];
          hfr[hh] = fr;
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) hfr[v] = hv[v];
      }
    }
    // down-projection chunk (LDS buffer ((id + 1) & 1))
    if (id + 2 < n_chunks) prefetch(id + 2);
    {
      const T *base = lds[(id + 1) & 1];
#pragma unroll
      for (int ti = 0; ti < DT; ++ti)
#pragma unroll
        for (int kc = 0; kc < HKC; ++kc) acc[ti] = M::mma(afrag(base, LDB, 32 * ti + lc, kc, true), hfr[kc], acc[ti]);
    }
    if (id + 2 < n_chunks) commit(id + 2, id & 1);
    __syncthreads();
  }

  // ---- store X' (fp32, this lane's token) -----------------------------------------------------
  if (valid) {
    float *xo = (float *)a.out.base + b * a.out.sb + (long long)(t - a.out.t_off) * a.out.rs;
#pragma unroll
    for (int ti = 0; ti < DT; ++ti)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(f32x4 *)(xo + 32 * ti + 8 * j + 4 * g) = f32x4{acc[ti][4 * j], acc[ti][4 * j + 1], acc[ti][4 * j + 2], acc[ti][4 * j + 3]};
  }
}

template <typename T, typename TR>
hipError_t launch_d(const PostArgs &a, int grid, hipStream_t s) {
  switch (a.d_model) {
#define OT_POST_CASE(DV)                                                                         \
  case DV:                                                                                        \
    hipLaunchKernelGGL((post_kernel<T, TR, DV>), dim3(grid), dim3(post_nw<T, DV>() * 64), 0, s, a); \
    break;
    OT_POST_CASE(64)
    OT_POST_CASE(128)
    OT_POST_CASE(256)
    OT_POST_CASE(512)
#undef OT_POST_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int post_tokens_per_tile(int dtype, int d_model) {
  if (dtype == 1) return (d_model <= 128 ? post_nw<bf16, 128>() : post_nw<bf16, 512>()) * 32;
  return post_nw<float, 256>() * 32;
}

hipError_t launch_post(int dtype, int resid_f32, const PostArgs &a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  if (dtype == 1) return resid_f32 ? launch_d<bf16, float>(a, grid, s) : launch_d<bf16, bf16>(a, grid, s);
  return launch_d<float, float>(a, grid, s);
}

}  // namespace ot
