// Backward of the causal mixed attention (fun-rec-mdbook 7.5.1 causal mask, 7.5.2 pyramid tail
// queries) for the training step's activation recomputation (7.5.3, closing paragraph).
//
// With the forward's base-2 convention (queries stored as Qs = Q log2(e) / sqrt(dh), lse the base-2
// log-sum-exp of each query's visible scores), per head:
//   P = exp2(Qs K^T - lse),  dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  D = rowsum(dO * O)
//   dK = dS^T Qs / log2(e),  dQ = dS K / sqrt(dh)
// The probabilities are recomputed, never stored. Two kernels, each owning its outputs (no atomics):
//   attn_dkdv_kernel: a workgroup per (sequence, head, 32 * ATTB_WAVES keys); a wave keeps its 32
//     keys' K and V fragments in registers and walks the 64-query tiles that can see them. Scores are
//     formed as S = Qs K^T with queries as accumulator rows, so that P and dS (per lane: 16
//     queries of one key) are already the B operand of dV^T += dO^T P and dK^T += Qs^T dS, whose
//     contraction index is a permutation of the tile's 32 queries; dO^T and Qs^T are read from
//     transposed LDS copies with the same permutation.
//   attn_dq_kernel: a workgroup per (sequence, head, 32 * ATTB_WAVES queries); a wave keeps its 32
//     queries' Qs and dO fragments in registers and walks the 64-key tiles they can see, forming
//     S^T = K Qs^T (keys as rows, one query per lane column, its lse and D in the lane), and
//     dQ^T += K^T dS^T with K^T from a transposed LDS copy.
// bf16 at d_head 32: the transposed operands (dO^T, Qs^T, K^T) are read from the row-major tiles by
// the transposing LDS read, so no transposed copy is written.
// Both stage their shared tiles in two LDS buffers: the next tile's global loads are issued into
// registers before the current tile is computed and written to the other buffer after it, so one
// workgroup barrier per tile separates the two and the loads' latency hides behind the math.

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
  // dK's call also writes the zero dQ^T of S keys before p0 (positions that issue no query): the
  // weight gradient of W_Q contracts over every S token
  if (which == 0 && tok_pos < a.p0) {
    T *dq0 = (T *)a.tS[2] + (long long)b * a.s + tok_pos;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = acc_row(v, g);
      if (c < DH) dq0[(long long)(h * DH + c) * ld] = from_f32<T>(0.0f);
    }
  }
}

template <typename T, int DH>
__global__ __launch_bounds__(ATTB_WAVES * 64) void attn_dkdv_kernel(const AttnBwdArgs a) {
  using M = Mma<T>;
  using frag = typename M::frag;
  using TS = TileStage<T>;
  constexpr int NW = ATTB_WAVES;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int QT = 64;              // queries per shared tile (two 32-query halves)
  constexpr int LDQ = DH + EPC;       // padded row of a [QT][DH] tile
  constexpr int LDT = QT + EPC;       // padded row of a [DH][QT] transposed tile
  constexpr int CPR = DH / EPC;       // 16-byte pieces per row
  constexpr int NPT = (2 * QT * CPR + NW * 64 - 1) / (NW * 64);   // pieces per thread and tile
  constexpr int NK = DH / M::KSTEP;   // k-steps over the head dimension
  constexpr int MC = 32 / M::KSTEP;   // k-steps over 32 queries
  // double-buffered tiles: Q and dO rows, their transposes (bf16 at d_head 32: read from the rows
  // by the transposing LDS read instead), lse and D
  constexpr bool TRB = sizeof(T) == 2 && DH == 32;
  __shared__ __attribute__((aligned(16))) T sQ[2][QT * LDQ];
  __shared__ __attribute__((aligned(16))) T sO[2][QT * LDQ];
  __shared__ __attribute__((aligned(16))) T sQt[2][TRB ? EPC : DH * LDT];
  __shared__ __attribute__((aligned(16))) T sOt[2][TRB ? EPC : DH * LDT];
  __shared__ __attribute__((aligned(16))) float sL[2][QT];
  __shared__ __attribute__((aligned(16))) float sD[2][QT];
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

  // a tile's global loads into registers (rows past R: zeros, lse +inf so that P = 0) ...
  u32x4 reg[NPT];
  float rl = 0.0f, rd = 0.0f;
  auto gload = [&](int qt) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int ch = tid + k * NW * 64;
      const int which = ch / (QT * CPR), rem = ch - which * (QT * CPR);
      const int row = rem / CPR, c0 = (rem - row * CPR) * EPC;
      const int i = qt + row;
      reg[k] = u32x4{0, 0, 0, 0};
      if (ch < 2 * QT * CPR && i < a.R)
        reg[k] = which == 0 ? ld16(qbase + (long long)i * DH + c0) : ld16(obase + (long long)i * a.d_model + c0);
    }
    if (tid < QT) {
      const int i = qt + tid;
      rl = i < a.R ? lbase[i] : __builtin_inff();
      rd = i < a.R ? dbase[i] : 0.0f;
    }
  };
  // ... and from registers into LDS buffer `buf`, rows and transposes
  auto lstore = [&](int buf) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int ch = tid + k * NW * 64;
      if (ch < 2 * QT * CPR) {
        const int which = ch / (QT * CPR), rem = ch - which * (QT * CPR);
        const int row = rem / CPR, c0 = (rem - row * CPR) * EPC;
        T *rt = which == 0 ? sQ[buf] : sO[buf];
        st16(&rt[row * LDQ + c0], reg[k]);
        if constexpr (!TRB) {
          T *tt = which == 0 ? sQt[buf] : sOt[buf];
          const T *ve = (const T *)&reg[k];
#pragma unroll
          for (int e = 0; e < EPC; ++e) tt[(c0 + e) * LDT + row] = ve[e];
        }
      }
    }
    if (tid < QT) {
      sL[buf][tid] = rl;
      sD[buf][tid] = rd;
    }
  };

  f32x16 dk = f32x16{}, dv = f32x16{};
  // first query that sees any key of the workgroup: position p0 + i >= kb * 32 * NW
  const int i_lo = max(0, kb * 32 * NW - a.p0);
  const int qt0 = (i_lo / 32) * 32;
  if (qt0 < a.R) {
    gload(qt0);
    lstore(0);
  }
  __syncthreads();
  for (int qt = qt0, it = 0; qt < a.R; qt += QT, ++it) {
    const int buf = it & 1;
    const bool more = qt + QT < a.R;
    if (more) gload(qt + QT);   // in flight while this tile is computed
#pragma unroll
    for (int sub = 0; sub < QT / 32; ++sub) {
      const int q0 = qt + sub * 32;
      // (wave-uniform) no key of the wave, no query in this half, or every query of the half
      // before the wave's first key
      if (kw0 >= a.T || q0 >= a.R || kw0 > a.p0 + q0 + 31) continue;
      // the accumulators start at -lse and -D of their query rows (acc_row(4 j + e, g) =
      // 8 j + 4 g + e), so the products come out as exp2 arguments and dP - D
      f32x16 s, dp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 l4 = *(const f32x4 *)&sL[buf][sub * 32 + 8 * j + 4 * g];
        const f32x4 d4 = *(const f32x4 *)&sD[buf][sub * 32 + 8 * j + 4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[4 * j + e] = -l4[e];
          dp[4 * j + e] = -d4[e];
        }
      }
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const frag qa = *(const frag *)(&sQ[buf][(sub * 32 + lc) * LDQ + kk * M::KSTEP + g * M::KPL]);
        const frag oa = *(const frag *)(&sO[buf][(sub * 32 + lc) * LDQ + kk * M::KSTEP + g * M::KPL]);
        s = M::mma(qa, kf[kk], s);
        dp = M::mma(oa, vf[kk], dp);
      }
      // query q0 + acc_row(v, g) sees key iff key <= p0 + q0 + acc_row(v, g): only the tiles that
      // cross the diagonal need the mask (rows past R have lse = +inf, so P = 0 there; keys past
      // T have zero K and V and their columns are never stored)
      float p[16], ds[16];
      if (kw0 + 31 <= a.p0 + q0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          p[v] = __builtin_amdgcn_exp2f(s[v]);
          ds[v] = p[v] * dp[v];
        }
      } else {
        const int lim = key - a.p0 - q0;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          p[v] = acc_row(v, g) >= lim ? __builtin_amdgcn_exp2f(s[v]) : 0.0f;
          ds[v] = p[v] * dp[v];
        }
      }
      if constexpr (TRB) {
        const int src = tr_src<LDQ>(sub * 32, lane);
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
          dv = M::mma(tr_frag<LDQ>((const bf16 *)sO[buf] + src, mc), TrFrag<T>::from_acc(p, mc), dv);
          dk = M::mma(tr_frag<LDQ>((const bf16 *)sQ[buf] + src, mc), TrFrag<T>::from_acc(ds, mc), dk);
        }
      } else {
        const T *ot_row = &sOt[buf][(lc < DH ? lc : 0) * LDT + sub * 32];
        const T *qt_row = &sQt[buf][(lc < DH ? lc : 0) * LDT + sub * 32];
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
          const frag oa = lc < DH ? TrFrag<T>::load(ot_row, mc, g) : M::zero();
          const frag qa = lc < DH ? TrFrag<T>::load(qt_row, mc, g) : M::zero();
          dv = M::mma(oa, TrFrag<T>::from_acc(p, mc), dv);
          dk = M::mma(qa, TrFrag<T>::from_acc(ds, mc), dk);
        }
      }
    }
    // the other buffer was last read in the previous iteration, before the barrier below it
    if (more) lstore(buf ^ 1);
    __syncthreads();
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
  constexpr int KT = 64;              // keys per shared tile (two 32-key halves)
  constexpr int LDK = DH + EPC;
  constexpr int LDT = KT + EPC;
  constexpr int CPR = DH / EPC;
  constexpr int NPT = (2 * KT * CPR + NW * 64 - 1) / (NW * 64);
  constexpr int NK = DH / M::KSTEP;
  constexpr int MC = 32 / M::KSTEP;
  __shared__ __attribute__((aligned(16))) T sK[2][KT * LDK];
  __shared__ __attribute__((aligned(16))) T sV[2][KT * LDK];
  constexpr bool TRB = sizeof(T) == 2 && DH == 32;   // K^T read from the K rows by the transposing read
  __shared__ __attribute__((aligned(16))) T sKt[2][TRB ? EPC : DH * LDT];
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

  u32x4 reg[NPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int ch = tid + k * NW * 64;
      const int which = ch / (KT * CPR), rem = ch - which * (KT * CPR);
      const int row = rem / CPR, c0 = (rem - row * CPR) * EPC;
      const int kg = k0 + row;
      reg[k] = u32x4{0, 0, 0, 0};
      if (ch < 2 * KT * CPR && kg < n_keys) reg[k] = ld16((which == 0 ? kbase : vbase) + (long long)kg * DH + c0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int ch = tid + k * NW * 64;
      if (ch < 2 * KT * CPR) {
        const int which = ch / (KT * CPR), rem = ch - which * (KT * CPR);
        const int row = rem / CPR, c0 = (rem - row * CPR) * EPC;
        st16(&(which == 0 ? sK[buf] : sV[buf])[row * LDK + c0], reg[k]);
        if (!TRB && which == 0) {
          const T *ve = (const T *)&reg[k];
#pragma unroll
          for (int e = 0; e < EPC; ++e) sKt[buf][(c0 + e) * LDT + row] = ve[e];
        }
      }
    }
  };

  f32x16 dq = f32x16{};
  if (n_keys > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int k0 = 0, it = 0; k0 < n_keys; k0 += KT, ++it) {
    const int buf = it & 1;
    const bool more = k0 + KT < n_keys;
    if (more) gload(k0 + KT);   // in flight while this tile is computed
#pragma unroll
    for (int sub = 0; sub < KT / 32; ++sub) {
      const int kb = k0 + sub * 32;
      if (kb >= n_keys || kb > wave_max) continue;   // wave-uniform
      // accumulators start at -lse and -D of the lane's query
      f32x16 s, dp;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s[v] = -lse;
        dp[v] = -dd;
      }
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const frag ka = *(const frag *)(&sK[buf][(sub * 32 + lc) * LDK + kk * M::KSTEP + g * M::KPL]);
        const frag va = *(const frag *)(&sV[buf][(sub * 32 + lc) * LDK + kk * M::KSTEP + g * M::KPL]);
        s = M::mma(ka, qf[kk], s);
        dp = M::mma(va, of[kk], dp);
      }
      // key kb + acc_row(v, g) is visible iff it is at most qpos: only tiles that cross the
      // diagonal need the mask (queries past R have lse = +inf, so P = 0; keys past n_keys have
      // zero K rows, so they add nothing to dQ)
      float ds[16];
      if (kb + 31 <= a.p0 + qw0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) ds[v] = __builtin_amdgcn_exp2f(s[v]) * dp[v];
      } else {
        const int lim = qpos - kb;
#pragma unroll
        for (int v = 0; v < 16; ++v) ds[v] = acc_row(v, g) <= lim ? __builtin_amdgcn_exp2f(s[v]) * dp[v] : 0.0f;
      }
      if constexpr (TRB) {
        const bf16 *src = (const bf16 *)sK[buf] + tr_src<LDK>(sub * 32, lane);
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) dq = M::mma(tr_frag<LDK>(src, mc), TrFrag<T>::from_acc(ds, mc), dq);
      } else {
        const T *kt_row = &sKt[buf][(lc < DH ? lc : 0) * LDT + sub * 32];
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
          const frag ka = lc < DH ? TrFrag<T>::load(kt_row, mc, g) : M::zero();
          dq = M::mma(ka, TrFrag<T>::from_acc(ds, mc), dq);
        }
      }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
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
