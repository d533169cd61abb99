// Backward of the causal mixed attention (fun-rec-mdbook 7.5.1 causal mask, 7.5.2 pyramid tail
// queries) for the training step's activation recomputation (7.5.3, closing paragraph).
//
// With the forward's base-2 convention (queries stored as Qs = Q log2(e) / sqrt(dh), lse the base-2
// log-sum-exp of each query's visible scores), per head:
//   P = exp2(Qs K^T - lse),  dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  D = rowsum(dO * O)
//   dK = dS^T Qs / log2(e),  dQ = dS K / sqrt(dh)
// The probabilities are recomputed, never stored. Two kernels, each owning its outputs (no atomics):
//   attn_dkdv_kernel: a workgroup per (sequence, head, 32 * ATTB_WAVES keys); a wave keeps its 32
//     keys' K and V fragments in registers and walks the query tiles that can see them. Scores are
//     formed as S = Qs K^T with queries as accumulator rows, so that P and dS (per lane: 16
//     queries of one key) are already the B operand of dV^T += dO^T P and dK^T += Qs^T dS, whose
//     contraction index is a permutation of the tile's 32 queries; dO^T and Qs^T are read from
//     transposed LDS copies with the same permutation.
//   attn_dq_kernel: a workgroup per (sequence, head, 32 * ATTB_WAVES queries); a wave keeps its 32
//     queries' Qs and dO fragments in registers and walks the key tiles they can see, forming
//     S^T = K Qs^T (keys as rows, one query per lane column, its lse and D in the lane), and
//     dQ^T += K^T dS^T with K^T from a transposed LDS copy.

#include "bwd.hpp"

namespace ot {
namespace {

constexpr float LN2 = 0.69314718055994531f;

// Fragment of a transposed [row][32 tokens] LDS tile whose k index is the accumulator-row
// permutation of 32 tokens: k-chunk mc, lane group g holds tokens acc_row(v, g) for the chunk's v.
template <typename T> struct TrFrag;
template <> struct TrFrag<bf16> {
  static __device__ __forceinline__ bf16x8 load(const bf16 *row, int mc, int g) {
    const bf16x4 lo = *(const bf16x4 *)(row + 16 * mc + 4 * g);
    const bf16x4 hi = *(const bf16x4 *)(row + 16 * mc + 8 + 4 * g);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  static __device__ __forceinline__ bf16x8 from_acc(const float *p, int mc) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)p[8 * mc + e];
    return r;
  }
};
template <> struct TrFrag<float> {
  static __device__ __forceinline__ float load(const float *row, int mc, int g) { return row[acc_row(mc, g)]; }
  static __device__ __forceinline__ float from_acc(const float *p, int mc) { return p[mc]; }
};

// Stores a 32 x 32 accumulator tile whose columns are tokens (lane % 32) and whose rows are the
// head's features c (rows >= DH unused): row-major into dqkv and feature-major into the S / NS
// copies. tok_pos: this lane's token position t (or -1 when it is not a token of the sequence).
template <typename T, int DH>
__device__ __forceinline__ void store_grad(const AttnBwdArgs &a, T *stg, const f32x16 &acc, int which, int b, int h,
                                           int tok_pos, int lane) {
  using TS = TileStage<T>;
  const int lc = lane & 31, g = lane >> 5;
  const int d = a.d_model;
  TS::put(stg, acc, lc, g);
  wait_lgkm0();
#pragma unroll
  for (int k = 0; k < TS::NI; ++k) {
    const int tok = TS::token(k, lane);
    const int tp = __shfl(tok_pos, tok, 64);
    const int f = TS::feature(lane);
    const u32x4 piece = TS::get(stg, k, lane);
    if (tp >= 0 && f < DH)
      st16((T *)a.dqkv + ((long long)b * a.T + tp) * 3 * d + which * d + h * DH + f, piece);
  }
  wait_lgkm0();
  if (tok_pos < 0) return;
  T *dst;
  long long ld;
  if (tok_pos < a.s) {
    dst = (T *)a.tS[which] + (long long)b * a.s + tok_pos;
    ld = a.tS_ld;
  } else {
    dst = (T *)a.tN[which] + (long long)(tok_pos - a.s) * a.tN_g + b;
    ld = a.tN_ld;
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int c = acc_row(v, g);
    if (c < DH) dst[(long long)(h * DH + c) * ld] = from_f32<T>(acc[v]);
  }
}

template <typename T, int DH>
__global__ __launch_bounds__(ATTB_WAVES * 64) void attn_dkdv_kernel(const AttnBwdArgs a) {
  using M = Mma<T>;
  using frag = typename M::frag;
  using TS = TileStage<T>;
  constexpr int NW = ATTB_WAVES;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int LDQ = DH + EPC;       // padded row of a [32][DH] tile
  constexpr int LDT = 32 + EPC;       // padded row of a [DH][32] transposed tile
  constexpr int CPR = DH / EPC;       // 16-byte pieces per row
  constexpr int NK = DH / M::KSTEP;   // k-steps over the head dimension
  constexpr int MC = 32 / M::KSTEP;   // k-steps over 32 queries
  __shared__ __attribute__((aligned(16))) T sQ[32 * LDQ];
  __shared__ __attribute__((aligned(16))) T sO[32 * LDQ];
  __shared__ __attribute__((aligned(16))) T sQt[DH * LDT];
  __shared__ __attribute__((aligned(16))) T sOt[DH * LDT];
  __shared__ float sL[32], sD[32];
  __shared__ __attribute__((aligned(16))) T stage[NW][TS::SIZE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lc = lane & 31;
  const int H = a.n_heads, n_pairs = a.n_seq * H;
  const int kb = blockIdx.x / n_pairs;             // key blocks of every pair, heaviest (first) first
  const int pair = blockIdx.x - kb * n_pairs;
  const int b = pair / H, h = pair - b * H;
  const int kw0 = kb * 32 * NW + wave * 32;        // this wave's first key
  const int key = kw0 + lc;
  const bool key_ok = key < a.T;

  const T *kbase = (const T *)a.k + (long long)b * a.kv_sb + (long long)h * a.T * DH;
  const T *vbase = (const T *)a.v + (long long)b * a.kv_sb + (long long)h * a.T * DH;
  frag kf[NK], vf[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    kf[kk] = key_ok ? *(const frag *)(kbase + (long long)key * DH + kk * M::KSTEP + g * M::KPL) : M::zero();
    vf[kk] = key_ok ? *(const frag *)(vbase + (long long)key * DH + kk * M::KSTEP + g * M::KPL) : M::zero();
  }
  const T *qbase = (const T *)a.q + (long long)b * a.q_sb + (long long)h * a.R * DH;
  const T *obase = (const T *)a.dout + (long long)b * a.R * a.d_model + h * DH;
  const float *lbase = a.lse + ((long long)b * H + h) * a.R;
  const float *dbase = a.dvec + ((long long)b * H + h) * a.R;

  f32x16 dk = f32x16{}, dv = f32x16{};
  // first query that sees any key of the workgroup: position p0 + i >= kb * 32 * NW
  const int i_lo = max(0, kb * 32 * NW - a.p0);
  for (int qt = (i_lo / 32) * 32; qt < a.R; qt += 32) {
    __syncthreads();
    for (int ch = tid; ch < 2 * 32 * CPR; ch += NW * 64) {
      const int which = ch / (32 * CPR), rem = ch - which * (32 * CPR);
      const int row = rem / CPR, c0 = (rem - row * CPR) * EPC;
      const int i = qt + row;
      u32x4 v = {0, 0, 0, 0};
      if (i < a.R) v = which == 0 ? ld16(qbase + (long long)i * DH + c0) : ld16(obase + (long long)i * a.d_model + c0);
      T *rt = which == 0 ? sQ : sO;
      T *tt = which == 0 ? sQt : sOt;
      st16(&rt[row * LDQ + c0], v);
      const T *ve = (const T *)&v;
#pragma unroll
      for (int e = 0; e < EPC; ++e) tt[(c0 + e) * LDT + row] = ve[e];
    }
    if (tid < 32) {
      const int i = qt + tid;
      sL[tid] = i < a.R ? lbase[i] : __builtin_inff();
      sD[tid] = i < a.R ? dbase[i] : 0.0f;
    }
    __syncthreads();
    // (wave-uniform) no key of the wave exists, or its first key lies past the tile's last query
    if (kw0 >= a.T || kw0 > a.p0 + qt + 31) continue;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const frag qa = *(const frag *)(&sQ[lc * LDQ + kk * M::KSTEP + g * M::KPL]);
      const frag oa = *(const frag *)(&sO[lc * LDQ + kk * M::KSTEP + g * M::KPL]);
      s = M::mma(qa, kf[kk], s);
      dp = M::mma(oa, vf[kk], dp);
    }
    // query qt + acc_row(v, g) sees key iff key <= p0 + qt + acc_row(v, g)
    const int lim = key - a.p0 - qt;
    float p[16], ds[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = acc_row(v, g);
      const bool vis = key_ok && r >= lim;
      p[v] = vis ? __builtin_amdgcn_exp2f(s[v] - sL[r]) : 0.0f;
      ds[v] = p[v] * (dp[v] - sD[r]);
    }
    const T *ot_row = &sOt[(lc < DH ? lc : 0) * LDT];
    const T *qt_row = &sQt[(lc < DH ? lc : 0) * LDT];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
      const frag oa = lc < DH ? TrFrag<T>::load(ot_row, mc, g) : M::zero();
      const frag qa = lc < DH ? TrFrag<T>::load(qt_row, mc, g) : M::zero();
      dv = M::mma(oa, TrFrag<T>::from_acc(p, mc), dv);
      dk = M::mma(qa, TrFrag<T>::from_acc(ds, mc), dk);
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) dk[v] *= LN2;
  store_grad<T, DH>(a, stage[wave], dk, 0, b, h, key_ok ? key : -1, lane);
  store_grad<T, DH>(a, stage[wave], dv, 1, b, h, key_ok ? key : -1, lane);
}

template <typename T, int DH>
__global__ __launch_bounds__(ATTB_WAVES * 64) void attn_dq_kernel(const AttnBwdArgs a) {
  using M = Mma<T>;
  using frag = typename M::frag;
  using TS = TileStage<T>;
  constexpr int NW = ATTB_WAVES;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int KT = 64;              // keys per shared tile
  constexpr int LDK = DH + EPC;
  constexpr int LDT = KT + EPC;
  constexpr int CPR = DH / EPC;
  constexpr int NK = DH / M::KSTEP;
  constexpr int MC = 32 / M::KSTEP;
  __shared__ __attribute__((aligned(16))) T sK[KT * LDK];
  __shared__ __attribute__((aligned(16))) T sV[KT * LDK];
  __shared__ __attribute__((aligned(16))) T sKt[DH * LDT];
  __shared__ __attribute__((aligned(16))) T stage[NW][TS::SIZE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lc = lane & 31;
  const int H = a.n_heads, n_pairs = a.n_seq * H;
  const int qb = a.n_qblocks - 1 - (int)(blockIdx.x / n_pairs);   // longest key ranges first
  const int pair = blockIdx.x - (a.n_qblocks - 1 - qb) * n_pairs;
  const int b = pair / H, h = pair - b * H;
  const int qw0 = qb * 32 * NW + wave * 32;
  const int qi = qw0 + lc;
  const bool q_ok = qi < a.R;
  const int qpos = a.p0 + qi;

  frag qf[NK], of[NK];
  {
    const T *qrow = (const T *)a.q + (long long)b * a.q_sb + (long long)h * a.R * DH + (long long)(q_ok ? qi : 0) * DH;
    const T *orow = (const T *)a.dout + ((long long)b * a.R + (q_ok ? qi : 0)) * a.d_model + h * DH;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      qf[kk] = q_ok ? *(const frag *)(qrow + kk * M::KSTEP + g * M::KPL) : M::zero();
      of[kk] = q_ok ? *(const frag *)(orow + kk * M::KSTEP + g * M::KPL) : M::zero();
    }
  }
  const float lse = q_ok ? a.lse[((long long)b * H + h) * a.R + qi] : __builtin_inff();
  const float dd = q_ok ? a.dvec[((long long)b * H + h) * a.R + qi] : 0.0f;
  const T *kbase = (const T *)a.k + (long long)b * a.kv_sb + (long long)h * a.T * DH;
  const T *vbase = (const T *)a.v + (long long)b * a.kv_sb + (long long)h * a.T * DH;

  // keys up to the workgroup's last query position
  const int wg_last = min(a.R, (qb + 1) * 32 * NW) - 1;
  const int n_keys = min(a.T, a.p0 + wg_last + 1);
  const int wave_last = min(a.R, qw0 + 32) - 1;
  const int wave_max = qw0 < a.R ? a.p0 + wave_last : -1;

  f32x16 dq = f32x16{};
  for (int k0 = 0; k0 < n_keys; k0 += KT) {
    __syncthreads();
    for (int ch = tid; ch < 2 * KT * CPR; ch += NW * 64) {
      const int which = ch / (KT * CPR), rem = ch - which * (KT * CPR);
      const int row = rem / CPR, c0 = (rem - row * CPR) * EPC;
      const int kg = k0 + row;
      u32x4 v = {0, 0, 0, 0};
      if (kg < n_keys) v = ld16((which == 0 ? kbase : vbase) + (long long)kg * DH + c0);
      st16(&(which == 0 ? sK : sV)[row * LDK + c0], v);
      if (which == 0) {
        const T *ve = (const T *)&v;
#pragma unroll
        for (int e = 0; e < EPC; ++e) sKt[(c0 + e) * LDT + row] = ve[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < KT / 32; ++sub) {
      const int kb = k0 + sub * 32;
      if (kb >= n_keys || kb > wave_max) break;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const frag ka = *(const frag *)(&sK[(sub * 32 + lc) * LDK + kk * M::KSTEP + g * M::KPL]);
        const frag va = *(const frag *)(&sV[(sub * 32 + lc) * LDK + kk * M::KSTEP + g * M::KPL]);
        s = M::mma(ka, qf[kk], s);
        dp = M::mma(va, of[kk], dp);
      }
      // key kb + acc_row(v, g) is visible iff it is at most min(qpos, n_keys - 1)
      const int lim = min(qpos, n_keys - 1) - kb;
      float ds[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool vis = q_ok && acc_row(v, g) <= lim;
        const float p = vis ? __builtin_amdgcn_exp2f(s[v] - lse) : 0.0f;
        ds[v] = p * (dp[v] - dd);
      }
      const T *kt_row = &sKt[(lc < DH ? lc : 0) * LDT + sub * 32];
#pragma unroll
      for (int mc = 0; mc < MC; ++mc) {
        const frag ka = lc < DH ? TrFrag<T>::load(kt_row, mc, g) : M::zero();
        dq = M::mma(ka, TrFrag<T>::from_acc(ds, mc), dq);
      }
    }
  }
  const float scale = 1.0f / sqrtf((float)DH);
#pragma unroll
  for (int v = 0; v < 16; ++v) dq[v] *= scale;
  store_grad<T, DH>(a, stage[wave], dq, 2, b, h, q_ok ? qpos : -1, lane);
}

template <typename T, int DH>
hipError_t launch_dh(const AttnBwdArgs &a, hipStream_t s) {
  const int n_pairs = a.n_seq * a.n_heads;
  if (a.n_kblocks > 0)
    hipLaunchKernelGGL((attn_dkdv_kernel<T, DH>), dim3(a.n_kblocks * n_pairs), dim3(ATTB_WAVES * 64), 0, s, a);
  if (a.n_qblocks > 0)
    hipLaunchKernelGGL((attn_dq_kernel<T, DH>), dim3(a.n_qblocks * n_pairs), dim3(ATTB_WAVES * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(int dtype, int d_head, const AttnBwdArgs &a, hipStream_t s) {
  if (a.n_seq * a.n_heads == 0) return hipSuccess;
  if (dtype == 1) return d_head == 16 ? launch_dh<bf16, 16>(a, s) : launch_dh<bf16, 32>(a, s);
  return d_head == 16 ? launch_dh<float, 16>(a, s) : launch_dh<float, 32>(a, s);
}

}  // namespace ot
