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
// operand is read with the same permutation. K/V tiles of 16 * ATTN_WAVES keys are staged in LDS
// once per workgroup and shared by all its waves. bf16 at d_head 32 (the OneTrans shapes): both
// tiles row-major, brought in by direct global->LDS loads into two buffers one tile ahead (one
// barrier per tile, no staging registers), V^T fragments read from the row-major V tile by the
// transposing LDS read. Other storage types and head sizes stage through registers, with V
// stored transposed ([d_head][key]).
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

// P.V operand fragment k-chunk mc of this lane from a transposed V^T tile: vt_row is the lane's
// V^T row (feature lc), or null when lc >= DH (zero rows of the product).
template <typename T, int DH>
struct VtRow {
  const T *vt_row;
  int g;
  __device__ __forceinline__ typename Mma<T>::frag operator()(int mc) const {
    return (DH == 32 || vt_row) ? VtFrag<T>::load(vt_row, mc, g) : Mma<T>::zero();
  }
};

// The same fragment (bf16, d_head 32) from a row-major V tile [key][32] by the transposing LDS
// read (tr_frag); v = tile + tr_src<32>(first key of the subtile, lane).
struct VRowTr {
  const bf16 *v;
  __device__ __forceinline__ bf16x8 operator()(int mc) const { return tr_frag<32>(v, mc); }
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

// One 32-key tile: fold the scores (base-2 units, -inf where invisible) into the running state.
// `scores()` forms the tile's masked scores from LDS; it is called once on the common path, and
// once more on the rare rescale path instead of keeping the 16 score registers alive across the
// tile (which lets the kernel fit 64 registers and eight waves per SIMD).
// The probabilities are first taken against the running maximum m as it stands. Any one of them
// above 2^RESCALE_HEADROOM makes the lane's tile sum exceed that bound too, so the tile maximum is
// only searched (and the state rescaled, the probabilities retaken) when some lane's sum does: on
// the first tile (m starts far below every score) and when the scores climb by more than the
// headroom. A tile whose sum crosses the bound with no single probability above it costs one
// needless rescale, which changes nothing in the result.
template <typename T, int DH, typename Scores, typename VFrag>
__device__ __forceinline__ void softmax_pv(const Scores &scores, SoftmaxState &st, const VFrag &vfrag) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int MC = 32 / M::KSTEP;
  frag pf[MC];
  float tsum;
  // probabilities of the tile against the current maximum, as the P.V operand, and their sum
  auto take = [&](const f32x16 &s, bool again) {
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
    // distinct (empty) markers keep the two uses of this block apart: otherwise the compiler merges
    // their common tail after the branch and keeps the fp32 probabilities alive across it
    if (again) asm volatile("; retake" ::); else asm volatile("; take" ::);
  };
  take(scores(), false);
  constexpr float BOUND = 256.0f;   // 2^RESCALE_HEADROOM
  static_assert(RESCALE_HEADROOM == 8.0f, "bound is 2^headroom");
  if (__any(!(tsum <= BOUND))) {    // wave-uniform; also catches an infinite sum
    // rare: the scores are formed again from LDS rather than kept in registers through the
    // common path
    asm volatile("" ::: "memory");
    const f32x16 s = scores();
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
    take(s, true);
  }
  st.lsum += tsum;
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    st.o = M::mma(vfrag(mc), pf[mc], st.o);
  }
}

// bf16: a register budget of eight waves per SIMD (64 registers, no spills), so that four 8-wave
// workgroups per CU hide each other's barrier and LDS waits (measured 6 % faster than six waves).
// fp32 storage (the parity mode) keeps the compiler's own budget.
template <typename T, int DH, bool STAGE2>
__global__ __launch_bounds__(ATTN_WAVES * 64, sizeof(T) == 2 ? 8 : 1) void attn_kernel(const AttnArgs a) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int NWA = ATTN_WAVES;
  constexpr int KT = 16 * NWA;       // keys per shared tile (one K and one V piece per thread at d_head 32)
  constexpr int LDK = DH + EPC;      // padded K row (elements)
  constexpr int LDV = KT + EPC;      // padded V^T row (keys)
  constexpr int LDW = 32 + EPC;      // padded V^T row of a wave's own-key tile
  constexpr int CPK = DH / EPC;      // 16-byte chunks per key row
  // bf16 at d_head 32: K and V tiles row-major ([key][32], K's 16-byte pieces XOR-swizzled) in two
  // buffers filled by direct global->LDS loads one tile ahead; V read by the transposing LDS read.
  // Otherwise one buffer filled through registers: K row-major with padded rows, V transposed
  // ([d_head][key], padded rows). After the key loop the same bytes hold the output staging tiles.
  constexpr bool TRV = sizeof(T) == 2 && DH == 32;
  using TS = TileStage<T>;
  constexpr int KBUF = TRV ? KT * DH : KT * LDK, VBUF = TRV ? KT * DH : DH * LDV, NBUF = TRV ? 2 : 1;
  constexpr int TILE_BYTES = NBUF * (KBUF + VBUF) * (int)sizeof(T);
  constexpr int STAGE_BYTES = NWA * TS::SIZE * (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) unsigned char smem[TILE_BYTES > STAGE_BYTES ? TILE_BYTES : STAGE_BYTES];
  T *const sK = (T *)smem;                 // [NBUF][KBUF]
  T *const sVt = sK + NBUF * KBUF;         // [NBUF][VBUF]
  T (*stage)[TS::SIZE] = (T (*)[TS::SIZE])smem;
  __shared__ __attribute__((aligned(16))) T sKw[STAGE2 ? NWA * 32 * LDK : EPC];
  __shared__ __attribute__((aligned(16))) T sVw[STAGE2 ? NWA * DH * LDW : EPC];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  if constexpr (TRV) {
    // thread tid loads piece tid % 4 of key row tid / 4 of a tile, K's piece into slot
    // piece ^ ((key >> 2) & 3) (the 32 rows of a score fragment read then touch every bank once)
    const int dkey = tid >> 2, dslot = tid & 3;
    const uint32_t kpiece = (uint32_t)((dslot ^ ((dkey >> 2) & 3)) * 16), vpiece = (uint32_t)(dslot * 16);
    const uint32_t kl = lds_addr(sK), vl = lds_addr(sVt);
    auto issue = [&](int k0, int b) {
      const uint32_t row = (uint32_t)min(k0 + dkey, n_keys - 1) * (uint32_t)(DH * sizeof(T));   // rows past the end repeat the last (masked)
      const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(b * KBUF * (int)sizeof(T)) + (uint32_t)wave * 1024u);
      dma16s(kp, row + kpiece, kl + dst);
      dma16s(vp, row + vpiece, vl + dst);
    };
    if (n_keys > 0) issue(0, 0);
    int buf = 0;
    for (int k0 = 0; k0 < n_keys; k0 += KT, buf ^= 1) {
      wait_vm<0>();     // this wave's loads of tile k0 have landed
      wait_lgkm0();     // and its reads of the other buffer are done
      bare_barrier();
      if (k0 + KT < n_keys) issue(k0 + KT, buf ^ 1);
      const T *kt = sK + buf * KBUF, *vt = sVt + buf * VBUF;
#pragma unroll
      for (int sub = 0; sub < KT / 32; ++sub) {
        const int kb = k0 + sub * 32;
        if (kb >= n_keys) break;
        if (!STAGE2 && kb > wave_max) break;
        const bool need_mask = STAGE2 ? (kb + 32 > n_keys) : (kb + 31 > wave_min || kb + 32 > n_keys);
        auto scores = [&]() {
          const int key = sub * 32 + lc, sw = (key >> 2) & 3;
          f32x16 s = f32x16{};
#pragma unroll
          for (int kk = 0; kk < DH / M::KSTEP; ++kk)
            s = M::mma(*(const frag *)(kt + key * DH + 8 * ((2 * kk + g) ^ sw)), qf[kk], s);
          if (need_mask) {
            const int lim = (STAGE2 ? n_keys - 1 : min(qpos, n_keys - 1)) - kb - 4 * g;
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (acc_row(v, 0) > lim) s[v] = NEG_INF;
          }
          return s;
        };
        softmax_pv<T, DH>(scores, st, VRowTr{(const bf16 *)vt + tr_src<32>(sub * 32, lane)});
      }
    }
  } else {
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
        const bool need_mask = STAGE2 ? (kb + 32 > n_keys) : (kb + 31 > wave_min || kb + 32 > n_keys);
        auto scores = [&]() {
          f32x16 s = score_tile<T, DH>(&sK[(sub * 32 + lc) * LDK + g * M::KPL], qf);
          if (need_mask) {
            // key kb + acc_row(v, g) is visible iff it is at most min(qpos, n_keys - 1) (Stage II:
            // no causal limit within the prefix); compare element v's constant row offset with one
            // per-lane bound
            const int lim = (STAGE2 ? n_keys - 1 : min(qpos, n_keys - 1)) - kb - 4 * g;
  #pragma unroll
            for (int v = 0; v < 16; ++v)
              if (acc_row(v, 0) > lim) s[v] = NEG_INF;
          }
          return s;
        };
        softmax_pv<T, DH>(scores, st, VtRow<T, DH>{lc < DH ? &sVt[lc * LDV + sub * 32] : nullptr, g});
      }
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
    auto scores = [&]() {
      f32x16 s = score_tile<T, DH>(&kw[lc * LDK + g * M::KPL], qf);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ks = acc_row(v, g);
        const int kc = ks / a.R, j2 = ks - kc * a.R;
        const bool vis = ks < n_own && kc == cslot && j2 <= qi && c_first + kc < a.n_cand;
        if (!vis) s[v] = NEG_INF;
      }
      return s;
    };
    softmax_pv<T, DH>(scores, st, VtRow<T, DH>{lc < DH ? &vw[lc * LDW] : nullptr, g});
  }

  // ---- normalise and store O[b][i][h*dh + c] through the wave's LDS staging tile ---------------
  const float lt = st.lsum + other_half(st.lsum);
  const float inv = valid ? 1.0f / lt : 0.0f;
  if (a.lse && valid && g == 0) a.lse[((long long)z * H + h) * a.R + qi] = st.m + log2f(lt);
  f32x16 o = st.o;
#pragma unroll
  for (int v = 0; v < 16; ++v) o[v] *= inv;
  __syncthreads();   // every wave is done with the K / V tiles the staging tiles overlay
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

// Launches with at most 32 query rows per (sequence or user, head): an append's new rows, the
// last pyramid blocks, Stage II of one or two candidates per user. One workgroup per (sequence or
// user, head) whose waves split the KEYS: wave w takes a contiguous range of 32-key subtiles of the
// prefix for the same 32 query lanes, streams them through its own LDS tile (loads of subtile i + 1
// in flight while subtile i is computed; no workgroup barrier in the key loop); in Stage II the last
// wave also folds in the candidates' own NS keys. The eight partial softmax states (m, l, o) are
// merged exactly at the end:
//   o = sum_w 2^(m_w - M) o_w / sum_w 2^(m_w - M) l_w,   M = max_w m_w.
template <typename T, int DH, bool STAGE2>
__global__ __launch_bounds__(ATTN_WAVES * 64) void attn_split_kernel(const AttnArgs a) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int NWA = ATTN_WAVES;
  constexpr int LDK = DH + EPC;      // padded K row (elements)
  constexpr int LDW = 32 + EPC;      // padded V^T row (keys)
  constexpr int CPK = DH / EPC;      // 16-byte pieces per key row
  constexpr int NPL = (32 * CPK + 63) / 64;   // K (and V) pieces per lane per subtile
  using TS = TileStage<T>;
  // LDS: per-wave K / V^T tiles during the key loop; after a barrier the same bytes hold the merge
  // (every wave's m, l and o) and the output staging tile
  // bf16 at d_head 32: V row-major ([key][32], read by the transposing LDS read); else transposed
  constexpr bool TRV = sizeof(T) == 2 && DH == 32;
  constexpr int VW = TRV ? 32 * DH : DH * LDW;   // elements of a wave's V tile
  constexpr int TILE_BYTES = NWA * (32 * LDK + VW) * (int)sizeof(T);
  constexpr int MERGE_BYTES = NWA * (2 * 32 + 16 * 64) * 4 + TS::SIZE * (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) unsigned char smem[TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES];
  T (*sK)[32 * LDK] = (T (*)[32 * LDK])smem;
  T (*sV)[VW] = (T (*)[VW])(smem + NWA * 32 * LDK * sizeof(T));
  float (*s_o)[16][64] = (float (*)[16][64])smem;
  float (*s_m)[32] = (float (*)[32])(smem + NWA * 16 * 64 * 4);
  float (*s_l)[32] = (float (*)[32])(smem + NWA * (16 * 64 + 32) * 4);
  T *stage = (T *)(smem + NWA * (16 * 64 + 64) * 4);

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lc = lane & 31;
  const int H = a.n_heads;
  const int pair = blockIdx.x;
  const int h = pair % H, grp = pair / H;
  // this lane's query: forward, row lc of sequence grp; Stage II, NS row qi of candidate cslot
  int z, qi, cslot = 0, cpw = 0;
  bool valid;
  if constexpr (!STAGE2) {
    z = grp;
    qi = lc;
    valid = qi < a.R;
  } else {
    cpw = 32 / a.R;
    cslot = lc / a.R;
    qi = lc - cslot * a.R;
    valid = cslot < cpw && cslot < a.n_cand;
    z = grp * a.n_cand + (valid ? cslot : 0);
  }
  const int shift = a.seq_shift ? a.seq_shift[grp] : 0;
  const int p0 = a.p0 + shift, n_pre = a.n_pre + shift;
  const int qpos = p0 + qi;

  frag qf[DH / M::KSTEP];
  {
    const T *qrow = (const T *)a.q + z * a.q_sb + h * a.q_sh + (long long)(valid ? qi : 0) * DH + g * M::KPL;
#pragma unroll
    for (int kk = 0; kk < DH / M::KSTEP; ++kk) qf[kk] = valid ? *(const frag *)(qrow + kk * M::KSTEP) : M::zero();
  }
  // prefix keys 0..n_keys-1 (forward: up to the last query's position), split in whole subtiles
  const int n_keys = STAGE2 ? n_pre : min(n_pre, p0 + a.R);
  const int n_sub = (n_keys + 31) / 32;
  const int per = (n_sub + NWA - 1) / NWA;
  const int sub0 = min(n_sub, wave * per), sub1 = min(n_sub, sub0 + per);
  const T *kp = (const T *)a.k_pre + grp * a.pre_sb + h * a.pre_sh;
  const T *vp = (const T *)a.v_pre + grp * a.pre_sb + h * a.pre_sh;

  SoftmaxState st;
  st.m = -1e30f;
  st.lsum = 0.0f;
  st.o = f32x16{};
  T *kw = sK[wave];
  T *vw = sV[wave];
  u32x4 pk[NPL], pv[NPL];
  auto load = [&](int sub) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int ch = lane + 64 * i;
      const int key = ch / CPK, c0 = (ch - key * CPK) * EPC;
      const int kg = sub * 32 + key;
      pk[i] = u32x4{0, 0, 0, 0};
      pv[i] = u32x4{0, 0, 0, 0};
      if (ch < 32 * CPK && kg < n_keys) {
        pk[i] = ld16(kp + (long long)kg * DH + c0);
        pv[i] = ld16(vp + (long long)kg * DH + c0);
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int ch = lane + 64 * i;
      if (ch < 32 * CPK) {
        const int key = ch / CPK, c0 = (ch - key * CPK) * EPC;
        st16(&kw[key * LDK + c0], pk[i]);
        if constexpr (TRV) {
          st16(&vw[key * DH + c0], pv[i]);
        } else {
          const T *ve = (const T *)&pv[i];
#pragma unroll
          for (int e = 0; e < EPC; ++e) vw[(c0 + e) * LDW + key] = ve[e];
        }
      }
    }
  };
  if (sub0 < sub1) load(sub0);
  for (int sub = sub0; sub < sub1; ++sub) {
    wait_lgkm0();                              // this wave's reads of the previous subtile are done
    store();
    if (sub + 1 < sub1) load(sub + 1);
    wait_lgkm0();                              // the tile is in LDS (only this wave reads it)
    const int kb = sub * 32;
    auto scores = [&]() {
      f32x16 s = score_tile<T, DH>(&kw[lc * LDK + g * M::KPL], qf);
      if ((!STAGE2 && kb + 31 > p0) || kb + 32 > n_keys) {
        const int lim = (STAGE2 ? n_keys - 1 : min(qpos, n_keys - 1)) - kb - 4 * g;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (acc_row(v, 0) > lim) s[v] = NEG_INF;
      }
      return s;
    };
    if constexpr (TRV) softmax_pv<T, DH>(scores, st, VRowTr{(const bf16 *)vw + tr_src<32>(0, lane)});
    else softmax_pv<T, DH>(scores, st, VtRow<T, DH>{lc < DH ? &vw[lc * LDW] : nullptr, g});
  }

  // ---- Stage II: the candidates' own NS keys (block-diagonal causal), on the last wave --------
  if constexpr (STAGE2) {
    if (wave == NWA - 1) {
      const int n_own = min(cpw, a.n_cand) * a.R;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int ch = lane + 64 * i;
        const int ks = ch / CPK, c0 = (ch - ks * CPK) * EPC;
        const int kc = ks / a.R, j2 = ks - kc * a.R;
        pk[i] = u32x4{0, 0, 0, 0};
        pv[i] = u32x4{0, 0, 0, 0};
        if (ch < 32 * CPK && ks < n_own) {
          const long long off = (long long)(grp * a.n_cand + kc) * a.own_sb + h * a.own_sh + (long long)j2 * DH + c0;
          pk[i] = ld16((const T *)a.k_own + off);
          pv[i] = ld16((const T *)a.v_own + off);
        }
      }
      wait_lgkm0();
      store();
      wait_lgkm0();
      auto scores = [&]() {
        f32x16 s = score_tile<T, DH>(&kw[lc * LDK + g * M::KPL], qf);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ks = acc_row(v, g);
          const int kc = ks / a.R, j2 = ks - kc * a.R;
          if (!(ks < n_own && kc == cslot && j2 <= qi)) s[v] = NEG_INF;
        }
        return s;
      };
      if constexpr (TRV) softmax_pv<T, DH>(scores, st, VRowTr{(const bf16 *)vw + tr_src<32>(0, lane)});
      else softmax_pv<T, DH>(scores, st, VtRow<T, DH>{lc < DH ? &vw[lc * LDW] : nullptr, g});
    }
  }

  // ---- merge the waves' partial states ------------------------------------------------------
  const float lt = st.lsum + other_half(st.lsum);
  __syncthreads();                             // every wave is done with its tiles
  if (g == 0) {
    s_m[wave][lc] = st.m;
    s_l[wave][lc] = lt;
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) s_o[wave][v][lane] = st.o[v];
  __syncthreads();
  if (wave != 0) return;
  float mx = s_m[0][lc];
#pragma unroll
  for (int w = 1; w < NWA; ++w) mx = fmaxf(mx, s_m[w][lc]);
  float l = 0.0f;
  f32x16 o = f32x16{};
#pragma unroll
  for (int w = 0; w < NWA; ++w) {
    const float sc = __builtin_amdgcn_exp2f(s_m[w][lc] - mx);
    l += sc * s_l[w][lc];
#pragma unroll
    for (int v = 0; v < 16; ++v) o[v] += sc * s_o[w][v][lane];
  }
  const float inv = valid ? 1.0f / l : 0.0f;
  if (a.lse && valid && g == 0) a.lse[((long long)z * a.n_heads + h) * a.R + qi] = mx + log2f(l);
#pragma unroll
  for (int v = 0; v < 16; ++v) o[v] *= inv;
  TS::put(stage, o, lc, g);
#pragma unroll
  for (int k = 0; k < TS::NI; ++k) {
    const int tok = TS::token(k, lane);
    const int tz = __shfl(z, tok, 64), tq = __shfl(qi, tok, 64);
    const bool tv = __shfl((int)valid, tok, 64) != 0;
    const u32x4 piece = TS::get(stage, k, lane);
    const int f = TS::feature(lane);
    if (tv && f < DH) st16((T *)a.o + tz * a.o_sb + (long long)tq * a.d_model + h * DH + f, piece);
  }
}

// Append and Stage II together (a cross-request append followed by the scoring of the user's
// candidates): one workgroup per (user, head) streams the user's prefix keys once, as
// attn_split_kernel does, and folds every subtile into two query groups per wave:
//   group A (args a): the appended rows, R <= 32 per user at positions p0 + i, causal;
//   group B (args b): the candidates' NS rows, n_cand * R <= 32 per user, Stage II: every prefix
//   key visible, then (last wave) the candidates' own NS keys, block-diagonal causal.
// Both groups see the same prefix keys (the cache after the append: n_pre rows, shifted by the
// user's own length when ragged), so the K/V tiles are loaded and staged once for both. Each
// group's eight partial states merge exactly as in attn_split_kernel (wave 0 merges group A,
// wave 1 group B).
template <typename T, int DH>
struct QGroup {
  typename Mma<T>::frag qf[DH / Mma<T>::KSTEP];
  SoftmaxState st;
  int z, qi, cslot;
  bool valid;
};

template <typename T, int DH>
__global__ __launch_bounds__(ATTN_WAVES * 64) void attn_pair_kernel(const AttnArgs a, const AttnArgs b) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int NWA = ATTN_WAVES;
  constexpr int LDK = DH + EPC;
  constexpr int LDW = 32 + EPC;
  constexpr int CPK = DH / EPC;
  constexpr int NPL = (32 * CPK + 63) / 64;
  using TS = TileStage<T>;
  constexpr bool TRV = sizeof(T) == 2 && DH == 32;
  constexpr int VW = TRV ? 32 * DH : DH * LDW;
  constexpr int TILE_BYTES = NWA * (32 * LDK + VW) * (int)sizeof(T);
  constexpr int GROUP_BYTES = NWA * (2 * 32 + 16 * 64) * 4;          // one group's m, l and o of every wave
  constexpr int MERGE_BYTES = 2 * GROUP_BYTES + 2 * TS::SIZE * (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) unsigned char smem[TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES];
  T (*sK)[32 * LDK] = (T (*)[32 * LDK])smem;
  T (*sV)[VW] = (T (*)[VW])(smem + NWA * 32 * LDK * sizeof(T));

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lc = lane & 31;
  const int H = a.n_heads;
  const int pair = blockIdx.x;
  const int h = pair % H, grp = pair / H;

  QGroup<T, DH> A, B;
  A.z = grp;
  A.qi = lc;
  A.cslot = 0;
  A.valid = lc < a.R;
  const int cpw = 32 / b.R;
  B.cslot = lc / b.R;
  B.qi = lc - B.cslot * b.R;
  B.valid = B.cslot < cpw && B.cslot < b.n_cand;
  B.z = grp * b.n_cand + (B.valid ? B.cslot : 0);
  const int shift = a.seq_shift ? a.seq_shift[grp] : 0;
  const int p0 = a.p0 + shift, n_keys = a.n_pre + shift;
  const int qpos = p0 + A.qi;
  {
    const T *qa = (const T *)a.q + A.z * a.q_sb + h * a.q_sh + (long long)(A.valid ? A.qi : 0) * DH + g * M::KPL;
    const T *qb = (const T *)b.q + B.z * b.q_sb + h * b.q_sh + (long long)(B.valid ? B.qi : 0) * DH + g * M::KPL;
#pragma unroll
    for (int kk = 0; kk < DH / M::KSTEP; ++kk) {
      A.qf[kk] = A.valid ? *(const frag *)(qa + kk * M::KSTEP) : M::zero();
      B.qf[kk] = B.valid ? *(const frag *)(qb + kk * M::KSTEP) : M::zero();
    }
  }
  for (QGroup<T, DH> *q : {&A, &B}) {
    q->st.m = -1e30f;   // below every score (as in the other kernels)
    q->st.lsum = 0.0f;
    q->st.o = f32x16{};
  }
  const int n_sub = (n_keys + 31) / 32;
  const int per = (n_sub + NWA - 1) / NWA;
  const int sub0 = min(n_sub, wave * per), sub1 = min(n_sub, sub0 + per);
  const T *kp = (const T *)a.k_pre + grp * a.pre_sb + h * a.pre_sh;
  const T *vp = (const T *)a.v_pre + grp * a.pre_sb + h * a.pre_sh;

  T *kw = sK[wave];
  T *vw = sV[wave];
  u32x4 pk[NPL], pv[NPL];
  auto load = [&](int sub) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int ch = lane + 64 * i;
      const int key = ch / CPK, c0 = (ch - key * CPK) * EPC;
      const int kg = sub * 32 + key;
      pk[i] = u32x4{0, 0, 0, 0};
      pv[i] = u32x4{0, 0, 0, 0};
      if (ch < 32 * CPK && kg < n_keys) {
        pk[i] = ld16(kp + (long long)kg * DH + c0);
        pv[i] = ld16(vp + (long long)kg * DH + c0);
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int ch = lane + 64 * i;
      if (ch < 32 * CPK) {
        const int key = ch / CPK, c0 = (ch - key * CPK) * EPC;
        st16(&kw[key * LDK + c0], pk[i]);
        if constexpr (TRV) {
          st16(&vw[key * DH + c0], pv[i]);
        } else {
          const T *ve = (const T *)&pv[i];
#pragma unroll
          for (int e = 0; e < EPC; ++e) vw[(c0 + e) * LDW + key] = ve[e];
        }
      }
    }
  };
  // one group's softmax over the wave's current tile: masked scores past `lim0` (relative to the
  // tile's first key and lane half), when `mask`
  auto fold = [&](QGroup<T, DH> &q, bool mask, int lim0) {
    auto scores = [&]() {
      f32x16 s = score_tile<T, DH>(&kw[lc * LDK + g * M::KPL], q.qf);
      if (mask) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (acc_row(v, 0) > lim0) s[v] = NEG_INF;
      }
      return s;
    };
    if constexpr (TRV) softmax_pv<T, DH>(scores, q.st, VRowTr{(const bf16 *)vw + tr_src<32>(0, lane)});
    else softmax_pv<T, DH>(scores, q.st, VtRow<T, DH>{lc < DH ? &vw[lc * LDW] : nullptr, g});
  };
  if (sub0 < sub1) load(sub0);
  for (int sub = sub0; sub < sub1; ++sub) {
    wait_lgkm0();
    store();
    if (sub + 1 < sub1) load(sub + 1);
    wait_lgkm0();
    const int kb = sub * 32;
    fold(A, kb + 31 > p0 || kb + 32 > n_keys, min(qpos, n_keys - 1) - kb - 4 * g);
    fold(B, kb + 32 > n_keys, n_keys - 1 - kb - 4 * g);
  }

  // ---- group B: the candidates' own NS keys (block-diagonal causal), on the last wave ---------
  if (wave == NWA - 1) {
    const int n_own = min(cpw, b.n_cand) * b.R;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int ch = lane + 64 * i;
      const int ks = ch / CPK, c0 = (ch - ks * CPK) * EPC;
      const int kc = ks / b.R, j2 = ks - kc * b.R;
      pk[i] = u32x4{0, 0, 0, 0};
      pv[i] = u32x4{0, 0, 0, 0};
      if (ch < 32 * CPK && ks < n_own) {
        const long long off = (long long)(grp * b.n_cand + kc) * b.own_sb + h * b.own_sh + (long long)j2 * DH + c0;
        pk[i] = ld16((const T *)b.k_own + off);
        pv[i] = ld16((const T *)b.v_own + off);
      }
    }
    wait_lgkm0();
    store();
    wait_lgkm0();
    auto scores = [&]() {
      f32x16 s = score_tile<T, DH>(&kw[lc * LDK + g * M::KPL], B.qf);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ks = acc_row(v, g);
        const int kc = ks / b.R, j2 = ks - kc * b.R;
        if (!(ks < n_own && kc == B.cslot && j2 <= B.qi)) s[v] = NEG_INF;
      }
      return s;
    };
    if constexpr (TRV) softmax_pv<T, DH>(scores, B.st, VRowTr{(const bf16 *)vw + tr_src<32>(0, lane)});
    else softmax_pv<T, DH>(scores, B.st, VtRow<T, DH>{lc < DH ? &vw[lc * LDW] : nullptr, g});
  }

  // ---- merge each group's partial states: wave 0 group A, wave 1 group B ----------------------
  const float ltA = A.st.lsum + other_half(A.st.lsum), ltB = B.st.lsum + other_half(B.st.lsum);
  __syncthreads();   // every wave is done with its tiles
  for (int gi = 0; gi < 2; ++gi) {
    const QGroup<T, DH> &q = gi ? B : A;
    unsigned char *gb = smem + gi * GROUP_BYTES;
    float (*s_o)[16][64] = (float (*)[16][64])gb;
    float (*s_m)[32] = (float (*)[32])(gb + NWA * 16 * 64 * 4);
    float (*s_l)[32] = (float (*)[32])(gb + NWA * (16 * 64 + 32) * 4);
    if (g == 0) {
      s_m[wave][lc] = q.st.m;
      s_l[wave][lc] = gi ? ltB : ltA;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) s_o[wave][v][lane] = q.st.o[v];
  }
  __syncthreads();
  if (wave > 1) return;
  const QGroup<T, DH> &q = wave ? B : A;
  const AttnArgs &ar = wave ? b : a;
  unsigned char *gb = smem + wave * GROUP_BYTES;
  float (*s_o)[16][64] = (float (*)[16][64])gb;
  float (*s_m)[32] = (float (*)[32])(gb + NWA * 16 * 64 * 4);
  float (*s_l)[32] = (float (*)[32])(gb + NWA * (16 * 64 + 32) * 4);
  T *stage = (T *)(smem + 2 * GROUP_BYTES) + wave * TS::SIZE;
  float mx = s_m[0][lc];
#pragma unroll
  for (int w = 1; w < NWA; ++w) mx = fmaxf(mx, s_m[w][lc]);
  float l = 0.0f;
  f32x16 o = f32x16{};
#pragma unroll
  for (int w = 0; w < NWA; ++w) {
    const float sc = __builtin_amdgcn_exp2f(s_m[w][lc] - mx);
    l += sc * s_l[w][lc];
#pragma unroll
    for (int v = 0; v < 16; ++v) o[v] += sc * s_o[w][v][lane];
  }
  const float inv = q.valid ? 1.0f / l : 0.0f;
  if (ar.lse && q.valid && g == 0) ar.lse[((long long)q.z * ar.n_heads + h) * ar.R + q.qi] = mx + log2f(l);
#pragma unroll
  for (int v = 0; v < 16; ++v) o[v] *= inv;
  TS::put(stage, o, lc, g);
#pragma unroll
  for (int k = 0; k < TS::NI; ++k) {
    const int tok = TS::token(k, lane);
    const int tz = __shfl(q.z, tok, 64), tq = __shfl(q.qi, tok, 64);
    const bool tv = __shfl((int)q.valid, tok, 64) != 0;
    const u32x4 piece = TS::get(stage, k, lane);
    const int f = TS::feature(lane);
    if (tv && f < DH) st16((T *)ar.o + tz * ar.o_sb + (long long)tq * ar.d_model + h * DH + f, piece);
  }
}

template <typename T, int DH>
hipError_t launch_dh(int stage2, const AttnArgs &a, hipStream_t s) {
  dim3 bd(ATTN_WAVES * 64);
  const dim3 split_grid(a.n_seq_grp * a.n_heads);
  if (stage2) {
    if (a.n_cand * a.R <= 32)   // every candidate of a user in the 32 query lanes of one wave
      hipLaunchKernelGGL((attn_split_kernel<T, DH, true>), split_grid, bd, 0, s, a);
    else
      hipLaunchKernelGGL((attn_kernel<T, DH, true>), dim3(a.n_qblocks * a.n_seq_grp * a.n_heads), bd, 0, s, a);
  } else if (a.R <= 32) {
    hipLaunchKernelGGL((attn_split_kernel<T, DH, false>), split_grid, bd, 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_kernel<T, DH, false>), dim3(a.n_qblocks * a.n_seq_grp * a.n_heads), bd, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_pair(int dtype, int d_head, const AttnArgs &a, const AttnArgs &b, hipStream_t s) {
  if (a.n_seq_grp * a.n_heads == 0) return hipSuccess;
  const dim3 grid(a.n_seq_grp * a.n_heads), bd(ATTN_WAVES * 64);
  if (dtype == 1) {
    if (d_head == 16) hipLaunchKernelGGL((attn_pair_kernel<bf16, 16>), grid, bd, 0, s, a, b);
    else hipLaunchKernelGGL((attn_pair_kernel<bf16, 32>), grid, bd, 0, s, a, b);
  } else {
    if (d_head == 16) hipLaunchKernelGGL((attn_pair_kernel<float, 16>), grid, bd, 0, s, a, b);
    else hipLaunchKernelGGL((attn_pair_kernel<float, 32>), grid, bd, 0, s, a, b);
  }
  return hipGetLastError();
}

hipError_t launch_attn(int dtype, int d_head, int stage2, const AttnArgs &a, hipStream_t s) {
  if (a.n_qblocks * a.n_seq_grp * a.n_heads == 0) return hipSuccess;
  if (dtype == 1) return d_head == 16 ? launch_dh<bf16, 16>(stage2, a, s) : launch_dh<bf16, 32>(stage2, a, s);
  return d_head == 16 ? launch_dh<float, 16>(stage2, a, s) : launch_dh<float, 32>(stage2, a, s);
}

}  // namespace ot
