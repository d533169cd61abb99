// Causal mixed attention with pyramid tail queries and the Stage II two-segment key set.
//
// What is computed (fun-rec-mdbook 7.5.1 causal mask, 7.5.2 Pyramid Stack, 7.5.3 two-stage
// serving): for every head h and query row at position p,
//     o = sum_{key u <= p} softmax_u(q . k_u / sqrt(d_head)) v_u
// Keys span every row of the block input; queries are only the tail rows. In Stage II the keys
// of a candidate's NS query j are the user's cached S rows followed by the candidate's own NS
// rows 0..j, one softmax over both. With ragged cached users every sequence's query positions
// and prefix key count move by that user's own cached length.
//
// Work layout: a workgroup (ATTN_WAVES waves) handles one (sequence or user, head) and up to
// 32 * ATTN_WAVES query rows; a wave owns 32 query rows. Scores are formed transposed,
// S^T = K Q^T, with one MFMA 32x32 tile per 32 keys, so a lane holds 16 of the 32 keys of ONE
// query (its column) and the softmax statistics of that query stay in the lane (one cross-half
// swap per tile). The probabilities are then already laid out as the B operand of
// O^T += V^T P^T: the k index of that product is a permutation of the 32 keys, and the V^T
// operand is read with the same permutation from an LDS copy of V stored transposed
// ([d_head][key]). K/V tiles of 16 * ATTN_WAVES keys are staged in LDS once per workgroup and
// shared by all its waves.
//
// Online softmax in base 2: queries arrive multiplied by log2(e)/sqrt(dh), so a probability is
// exp2 of the score minus the running maximum. For bf16 the row sums are packed bf16 dot products
// of the probabilities as rounded for the P.V product (two per instruction). Fully masked tiles
// are skipped per wave; the accumulator is rescaled only when a tile raises the running maximum
// by more than a fixed headroom.

#include "common.hpp"
#include "launch.hpp"

namespace ot {

namespace {

constexpr float NEG_INF = -__builtin_inff();

template <typename T> struct VtFrag;

// bf16: the 8 k elements of lane-group g in k-chunk mc are keys {16mc + 4g + 0..3, 16mc + 8 + 4g + 0..3}
template <> struct VtFrag<bf16> {
  static __device__ __forceinline__ bf16x8 load(const bf16 *row, int mc, int g) {
    const bf16x4 lo = *(const bf16x4 *)(row + 16 * mc + 4 * g);
    const bf16x4 hi = *(const bf16x4 *)(row + 16 * mc + 8 + 4 * g);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  static __device__ __forceinline__ bf16x8 pfrag(const float *p, int mc) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)p[8 * mc + e];
    return r;
  }
};

template <> struct VtFrag<float> {
  static __device__ __forceinline__ float load(const float *row, int mc, int g) { return row[acc_row(mc, g)]; }
  static __device__ __forceinline__ float pfrag(const float *p, int mc) { return p[mc]; }
};

// The value x of the lane in the other half of the wave (lane ^ 32), by one cross-half swap.
__device__ __forceinline__ float other_half(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // sw[0]: upper lanes now hold the lower lanes' x; sw[1]: lower lanes hold the upper lanes' x
  return __uint_as_float((threadIdx.x & 32) ? sw[0] : sw[1]);
}

// Headroom (in base-2 exponent units) of the running maximum: a tile whose maximum exceeds the
// running one by at most this much is folded in against the stale maximum, so its probabilities
// are at most 2^8 and the accumulator need not be rescaled. The final division by the running
// sum, taken against the same maximum, gives the same softmax.
constexpr float RESCALE_HEADROOM = 8.0f;

// Running softmax state of the lane's query: maximum m (base-2 units), output accumulator o, and
// this lane's partial row sum (its 16 of every 32 keys; the other half sits in lane +- 32).
struct SoftmaxState {
  float m, lsum;
  f32x16 o;
};

// Scores of one 32-key tile against the lane's query: K rows from LDS (krow = this lane's key row
// at its k offset), Q fragments in registers.
template <typename T, int DH>
__device__ __forceinline__ f32x16 score_tile(const T *krow, const typename Mma<T>::frag *qf) {
  using M = Mma<T>;
  f32x16 s = f32x16{};
#pragma unroll
  for (int kk = 0; kk < DH / M::KSTEP; ++kk) s = M::mma(*(const typename M::frag *)(krow + kk * M::KSTEP), qf[kk], s);
  return s;
}

// One 32-key tile: fold the scores s (base-2 units, -inf where invisible) into the running state.
// The probabilities are first taken against the running maximum m as it stands. Any one of them
// above 2^RESCALE_HEADROOM makes the lane's tile sum exceed that bound too, so the tile maximum is
// only searched (and the state rescaled, the probabilities retaken) when some lane's sum does: on
// the first tile (m starts far below every score) and when the scores climb by more than the
// headroom. A tile whose sum crosses the bound with no single probability above it costs one
// needless rescale, which changes nothing in the result.
template <typename T, int DH>
__device__ __forceinline__ void softmax_pv(const f32x16 &s, SoftmaxState &st,
                                           const T *vt_row /* this lane's V^T row, or null if lc >= DH */,
                                           int g) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int MC = 32 / M::KSTEP;
  frag pf[MC];
  float tsum;
  // probabilities of the tile against the current maximum, as the P.V operand, and their sum
  auto take = [&]() {
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(s[v] - st.m);
    tsum = 0.0f;
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
      pf[mc] = VtFrag<T>::pfrag(p, mc);
      if constexpr (sizeof(T) == 2) {
        // sum of the probabilities as rounded for the product: packed bf16 dot products
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t one2 = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          tsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pf[mc][e], pf[mc][e + 1]}, one2, tsum, false);
      } else {
        tsum += pf[mc];
      }
    }
  };
  take();
  constexpr float BOUND = 256.0f;   // 2^RESCALE_HEADROOM
  static_assert(RESCALE_HEADROOM == 8.0f, "bound is 2^headroom");
  if (__any(!(tsum <= BOUND))) {    // wave-uniform; also catches an infinite sum
    float mt = s[0];
#pragma unroll
    for (int v = 1; v < 15; v += 2) mt = fmaxf(fmaxf(mt, s[v]), s[v + 1]);   // three-operand max
    mt = fmaxf(mt, s[15]);
    mt = fmaxf(mt, other_half(mt));
    const float mn = fmaxf(st.m, mt);
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
    st.m = mn;
    st.lsum *= alpha;
#pragma unroll
    for (int v = 0; v < 16; ++v) st.o[v] *= alpha;
    take();
  }
  st.lsum += tsum;
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    frag vf = (DH == 32 || vt_row) ? VtFrag<T>::load(vt_row, mc, g) : M::zero();
    st.o = M::mma(vf, pf[mc], st.o);
  }
}

template <typename T, int DH, bool STAGE2>
__global__ __launch_bounds__(ATTN_WAVES * 64) void attn_kernel(const AttnArgs a) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int NWA = ATTN_WAVES;
  constexpr int KT = 16 * NWA;       // keys per shared tile (one K and one V piece per thread at d_head 32)
  constexpr int LDK = DH + EPC;      // padded K row (elements)
  constexpr int LDV = KT + EPC;      // padded V^T row (keys)
  constexpr int LDW = 32 + EPC;      // padded V^T row of a wave's own-key tile
  constexpr int CPK = DH / EPC;      // 16-byte chunks per key row
  __shared__ __attribute__((aligned(16))) T sK[KT * LDK];
  __shared__ __attribute__((aligned(16))) T sVt[DH * LDV];
  __shared__ __attribute__((aligned(16))) T sKw[STAGE2 ? NWA * 32 * LDK : EPC];
  __shared__ __attribute__((aligned(16))) T sVw[STAGE2 ? NWA * DH * LDW : EPC];
  using TS = TileStage<T>;
  __shared__ __attribute__((aligned(16))) T stage[NWA][TS::SIZE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lc = lane & 31;
  const int H = a.n_heads;
  // Work order. Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD b % 8),
  // and each XCD has its own L2. XCD x takes a contiguous range of logical work items lg, and lg
  // walks groups of ATTN_GROUP (sequence/user, head) pairs: within a group the longest query
  // blocks of all its pairs go first, then the shorter ones. All query blocks of a pair thus run on
  // one XCD close together in time (its K/V rows come from HBM once), and each group still starts
  // with its heaviest workgroups.
  constexpr int ATTN_GROUP = 8;
  const int total = gridDim.x, nq = a.n_qblocks, n_pairs = a.n_seq_grp * H;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int lg = xcd * (total >> 3) + min(xcd, total & 7) + slot;
  const int group = lg / (ATTN_GROUP * nq);
  const int r = lg - group * ATTN_GROUP * nq;
  const int gp = min(ATTN_GROUP, n_pairs - group * ATTN_GROUP);   // pairs in this group
  const int qb = nq - 1 - r / gp;
  const int pair = group * ATTN_GROUP + r % gp;
  const int h = pair % H, grp = pair / H;

  // ---- this lane's query --------------------------------------------------------------------
  int z, qi, cslot = 0, cpw = 0, c_first = 0;
  bool valid;
  if constexpr (!STAGE2) {
    z = grp;
    qi = qb * ATTN_QBLOCK + wave * 32 + lc;
    valid = qi < a.R;
  } else {
    cpw = 32 / a.R;
    cslot = lc / a.R;
    qi = lc - cslot * a.R;
    c_first = qb * NWA * cpw + wave * cpw;
    const int c = c_first + cslot;
    valid = cslot < cpw && c < a.n_cand;
    z = grp * a.n_cand + (valid ? c : 0);
  }
  // ragged cached lengths: this sequence's positions and prefix keys start `shift` rows later
  const int shift = a.seq_shift ? a.seq_shift[grp] : 0;
  const int p0 = a.p0 + shift, n_pre = a.n_pre + shift;
  const int qpos = p0 + qi;

  frag qf[DH / M::KSTEP];
  {
    const T *qrow = (const T *)a.q + z * a.q_sb + h * a.q_sh + (long long)(valid ? qi : 0) * DH + g * M::KPL;
#pragma unroll
    for (int kk = 0; kk < DH / M::KSTEP; ++kk) qf[kk] = valid ? *(const frag *)(qrow + kk * M::KSTEP) : M::zero();
  }

  // ---- key range of the shared (prefix) segment --------------------------------------------
  int n_keys, wave_min = 0, wave_max = 0;
  if constexpr (!STAGE2) {
    const int wg_last = min(a.R, (qb + 1) * ATTN_QBLOCK) - 1;
    n_keys = min(n_pre, p0 + wg_last + 1);
    const int wf = qb * ATTN_QBLOCK + wave * 32;
    const int wl = min(a.R, wf + 32) - 1;
    wave_min = p0 + wf;
    wave_max = wf < a.R ? p0 + wl : -1;
  } else {
    n_keys = n_pre;
  }
  const T *kp = (const T *)a.k_pre + grp * a.pre_sb + h * a.pre_sh;
  const T *vp = (const T *)a.v_pre + grp * a.pre_sb + h * a.pre_sh;

  SoftmaxState st;
  st.m = -1e30f;
  st.lsum = 0.0f;
  st.o = f32x16{};

  for (int k0 = 0; k0 < n_keys; k0 += KT) {
    __syncthreads();
    for (int ch = tid; ch < KT * CPK; ch += NWA * 64) {
      const int key = ch / CPK, c0 = (ch - key * CPK) * EPC;
      const int kg = k0 + key;
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (kg < n_keys) {
        kv = ld16(kp + (long long)kg * DH + c0);
        vv = ld16(vp + (long long)kg * DH + c0);
      }
      st16(&sK[key * LDK + c0], kv);
      const T *ve = (const T *)&vv;
#pragma unroll
      for (int e = 0; e < EPC; ++e) sVt[(c0 + e) * LDV + key] = ve[e];
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < KT / 32; ++sub) {
      const int kb = k0 + sub * 32;
      if (kb >= n_keys) break;
      if (!STAGE2 && kb > wave_max) break;
      f32x16 s = score_tile<T, DH>(&sK[(sub * 32 + lc) * LDK + g * M::KPL], qf);
      const bool need_mask = STAGE2 ? (kb + 32 > n_keys) : (kb + 31 > wave_min || kb + 32 > n_keys);
      if (need_mask) {
        // key kb + acc_row(v, g) is visible iff it is at most min(qpos, n_keys - 1) (Stage II: no
        // causal limit within the prefix); compare element v's constant row offset with one
        // per-lane bound
        const int lim = (STAGE2 ? n_keys - 1 : min(qpos, n_keys - 1)) - kb - 4 * g;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (acc_row(v, 0) > lim) s[v] = NEG_INF;
      }
      softmax_pv<T, DH>(s, st, lc < DH ? &sVt[lc * LDV + sub * 32] : nullptr, g);
    }
  }

  // ---- Stage II: the candidates' own NS keys (block-diagonal causal) -----------------------
  if constexpr (STAGE2) {
    T *kw = sKw + wave * 32 * LDK;
    T *vw = sVw + wave * DH * LDW;
    const int n_own = cpw * a.R;
    for (int ch = lane; ch < 32 * CPK; ch += 64) {
      const int ks = ch / CPK, c0 = (ch - ks * CPK) * EPC;
      const int kc = ks / a.R, j2 = ks - kc * a.R;
      const int c = c_first + kc;
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (ks < n_own && c < a.n_cand) {
        const long long off = (long long)(grp * a.n_cand + c) * a.own_sb + h * a.own_sh + (long long)j2 * DH + c0;
        kv = ld16((const T *)a.k_own + off);
        vv = ld16((const T *)a.v_own + off);
      }
      st16(&kw[ks * LDK + c0], kv);
      const T *ve = (const T *)&vv;
#pragma unroll
      for (int e = 0; e < EPC; ++e) vw[(c0 + e) * LDW + ks] = ve[e];
    }
    __syncthreads();
    f32x16 s = score_tile<T, DH>(&kw[lc * LDK + g * M::KPL], qf);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int ks = acc_row(v, g);
      const int kc = ks / a.R, j2 = ks - kc * a.R;
      const bool vis = ks < n_own && kc == cslot && j2 <= qi && c_first + kc < a.n_cand;
      if (!vis) s[v] = NEG_INF;
    }
    softmax_pv<T, DH>(s, st, lc < DH ? &vw[lc * LDW] : nullptr, g);
  }

  // ---- normalise and store O[b][i][h*dh + c] through the wave's LDS staging tile ---------------
  const float lt = st.lsum + other_half(st.lsum);
  const float inv = valid ? 1.0f / lt : 0.0f;
  f32x16 o = st.o;
#pragma unroll
  for (int v = 0; v < 16; ++v) o[v] *= inv;
  T *stg = stage[wave];
  TS::put(stg, o, lc, g);
#pragma unroll
  for (int k = 0; k < TS::NI; ++k) {
    const int tok = TS::token(k, lane);
    const int tz = __shfl(z, tok, 64), tq = __shfl(qi, tok, 64);
    const bool tv = __shfl((int)valid, tok, 64) != 0;
    const u32x4 piece = TS::get(stg, k, lane);
    const int f = TS::feature(lane);
    if (tv && f < DH) st16((T *)a.o + tz * a.o_sb + (long long)tq * a.d_model + h * DH + f, piece);
  }
}

template <typename T, int DH>
hipError_t launch_dh(int stage2, const AttnArgs &a, hipStream_t s) {
  dim3 gd(a.n_qblocks * a.n_seq_grp * a.n_heads), bd(ATTN_WAVES * 64);
  if (stage2)
    hipLaunchKernelGGL((attn_kernel<T, DH, true>), gd, bd, 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<T, DH, false>), gd, bd, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(int dtype, int d_head, int stage2, const AttnArgs &a, hipStream_t s) {
  if (a.n_qblocks * a.n_seq_grp * a.n_heads == 0) return hipSuccess;
  if (dtype == 1) return d_head == 16 ? launch_dh<bf16, 16>(stage2, a, s) : launch_dh<bf16, 32>(stage2, a, s);
  return d_head == 16 ? launch_dh<float, 16>(stage2, a, s) : launch_dh<float, 32>(stage2, a, s);
}

}  // namespace ot
