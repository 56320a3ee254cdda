// online_attn.hip -- fused online-softmax attention for head dims 32, 64, 128.
//
// Method: the streaming softmax of the cuDNN Blackwell FMHA example
// (native_sparse_attention fmha.py, softmax_step and correction_epilog): keep a
// running row maximum m and row sum l per query, and for each block of keys
// rescale the output accumulator by 2^(m_old - m_new) before adding P V; divide
// by l at the end.  The exponent is taken base 2 with the scale folded in
// (scale * log2 e), as that page does; exp2 is the hardware v_exp_f32.
//
// gfx950 mapping (one workgroup = 8 waves = 128 queries of one head):
//   * Waves 0-3 and 4-7 form two groups over the same 128 queries; group g takes
//     the key blocks t = g, g + 2, ... with its own double-buffered K/V tiles,
//     so every SIMD runs two waves and one wave's softmax overlaps the other's
//     MFMAs.  At the end group 1 hands its (m, l, O) to group 0 through LDS and
//     group 0 merges the two exactly: O = (2^(m0-M) O0 + 2^(m1-M) O1) /
//     (2^(m0-M) l0 + 2^(m1-M) l1), M = max(m0, m1).
//   * Each wave owns 32 queries.  It computes S^T = K Q^T for a 64-key block
//     with v_mfma_f32_32x32x16_bf16, keys on the M side and queries on the N
//     side, so that every lane owns one query: the row max and row sum are
//     in-lane reductions plus one swap between the two lane halves.
//   * The S^T accumulator layout is, register for register, the B operand of
//     O^T += V^T P^T once the 32 keys of a block are relabelled; so P goes from
//     the softmax to the second MFMA without touching LDS.
//   * K and V tiles both go global -> LDS with direct buffer loads (XOR-swizzled
//     16-byte chunks) and stay row-major; the V^T fragments of the second MFMA
//     come from the gfx950 LDS transpose read (ds_read_b64_tr_b16), so no
//     register passes through V on its way in.
//   * K/V tiles are double-buffered: the next tile's loads are in flight while
//     the current one is consumed.
//   * Unmasked, the block maximum is a one-sided max3 chain on the raw scores
//     (the maximum, or for a negative scale the minimum) scaled once.
//   * Keys past L, and outside the query's band (after it when causal, or
//     beyond a sliding window), are masked to -inf; a workgroup visits only
//     the key blocks its queries' bands meet, a wave skips blocks its own
//     queries do not see, and loads past the end of a head return zero
//     through the buffer resource bounds.
//   * Heads are found through a HeadMap (any batch, head and row strides with
//     contiguous channels; one key/value head per `group` query heads), or,
//     for a batch of sequences of different lengths packed along the tokens,
//     through the sequence offsets (fmha.py's cum_seqlen); the merged (m, l)
//     give each row's log-sum-exp when it is asked for.
#include <algorithm>

#include "device.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int kBN = 64;           // keys per step
constexpr int kBM = 128;          // queries per workgroup with 4 query waves per group
constexpr float kLazy = 8.f;      // reference slack (log2 units) before O is rescaled

template <int D, int G>
struct OnlineSmem {
  static constexpr int TILE = kBN * D * 2;  // one 64-key K or V tile
  char k[G][2][TILE];                      // per group, double-buffered
  char v[G][2][TILE];
};

// LAYOUT: where head bh's rows are.  kPlain: q, k, v and out contiguous
// [B, H, L, D] with one key/value head per query head, so head bh starts at
// bh * L * D (no division by H, whose expansion would sit ahead of the first
// load of this short kernel).  kStrided: through the head map.  kVarlen:
// sequences of different lengths packed along the token dimension; sequence
// b = bh / H holds query tokens [vs.cu_q[b], vs.cu_q[b + 1]) and key/value
// tokens [vs.cu_k[b], vs.cu_k[b + 1]) (cu_k null: the same), clamped to the
// views and to the longest lengths; rows are hm.*.ld apart and heads hm.*.h
// apart.  Query i of a sequence stands at key position i + Lk - Lq.
enum { kPlain = 0, kStrided = 1, kVarlen = 2 };
// MASK: which keys below L each query i may see -- kAllKeys: all of them;
// kCausal: j <= i; kWindow: i - left <= j <= i + right (band.left, band.right,
// either side possibly unbounded); kCompressed (token-packed sequences only):
// j <= (i + 1) / cf - 1 with cf = max(1, Lq / Lk), the compressed causal mask
// of fmha.py's softmax, each key standing for cf consecutive queries.  Causal
// has its own instantiation so that it carries no left-side tests.
enum { kAllKeys = 0, kCausal = 1, kWindow = 2, kCompressed = 3 };
// QW: query waves per group (32 queries each); G: key-block groups, each
// taking every G-th key block of the workgroup's band with its own tiles.
template <int D, int MASK, int LAYOUT, int QW, int G>
__global__ __launch_bounds__(64 * QW * G) void online_attn_kernel(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse, HeadMap hm, int Lmax,
                                                    int nqb, float sl2, Band band, VarSeqs vs,
                                                    KeySplit ks) {
  constexpr int BM = 32 * QW;                      // queries per workgroup
  constexpr int GT = 64 * QW;                      // threads per group
  constexpr int CPR = D / 8;                       // 16-byte chunks per K or V row
  // K chunk c of row r sits at c ^ kswz(r): a 16-lane cycle of a 16-byte
  // fragment read covers 16 consecutive rows, and kswz makes their chunks land
  // in 16 distinct 16-byte bank groups (row r starts at bank group CPR r mod 16).
  constexpr int KSH = CPR == 4 ? 2 : CPR == 8 ? 1 : 0;
  constexpr int LOADS = kBN * CPR / GT;            // direct loads per thread per K (and V) tile
  constexpr int NS = D / 16;                       // k16 steps for S
  constexpr int NCB = D / 32;                      // 32-channel blocks of O
  constexpr int TILE = OnlineSmem<D, G>::TILE;
  static_assert(LOADS >= 1 && LOADS * GT == kBN * CPR, "tile shape");

  // One LDS object (two would make the compiler wait on every direct load in
  // flight before each LDS read).
  __shared__ OnlineSmem<D, G> smem;

  const int lane = threadIdx.x & 63;
  // Wave-uniform, read from lane 0 so that the branches on them are scalar.
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x / GT);              // key-block group
  const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) % QW);  // query wave in the group
  const int c32 = lane & 31, h = lane >> 5;
  char* const ktiles = &smem.k[g][0][0];
  char* const vtiles = &smem.v[g][0][0];

  // Workgroup = (head, query block, key split); the splits of one block are
  // neighbours, so they run on one XCD and share its L2.
  const uint32_t lid0 = xcd_logical_id(blockIdx.x, gridDim.x);
  const int split = ks.n > 1 ? (int)(lid0 % (uint32_t)ks.n) : 0;
  const uint32_t lid = ks.n > 1 ? lid0 / (uint32_t)ks.n : lid0;
  const int bh = lid / nqb;
  int qb = lid % nqb;
  if (MASK == kCausal || MASK == kCompressed) qb = nqb - 1 - qb;  // the longest rows start first
  constexpr bool BANDED = MASK != kAllKeys, HAS_LEFT = MASK == kWindow;
  int left = HAS_LEFT ? band.left : kNoLimit;
  int right = MASK == kCausal ? 0 : band.right;
  int cf = 1;  // kCompressed: queries per key

  constexpr bool PLAIN = LAYOUT == kPlain;
  const int ldq = PLAIN ? D : hm.q.ld, ldk = PLAIN ? D : hm.k.ld, ldv = PLAIN ? D : hm.v.ld;
  const int ldo = PLAIN ? D : hm.o.ld;
  // This head's row 0 in each operand (elements), its query and key lengths,
  // and where its log-sum-exp values go (lse_base + lse_step * query).
  int L = Lmax, Lk = Lmax;
  int64_t qoff, koff, voff, ooff, lse_base;
  int lse_step = 1;
  if constexpr (LAYOUT == kVarlen) {
    const int b = bh / hm.H, h = bh - b * hm.H;
    const int qs = min(max(vs.cu_q[b], 0), vs.total_q);
    const int qe = min(max(vs.cu_q[b + 1], qs), vs.total_q);
    L = min(qe - qs, Lmax);
    if (qb * BM >= L) return;  // the whole workgroup, before any barrier
    const int* cuk = vs.cu_k != nullptr ? vs.cu_k : vs.cu_q;
    const int tk = vs.cu_k != nullptr ? vs.total_k : vs.total_q;
    const int ks0 = min(max(cuk[b], 0), tk);
    const int ke = min(max(cuk[b + 1], ks0), tk);
    Lk = min(ke - ks0, vs.max_k);
    if constexpr (MASK == kCompressed) {
      cf = Lk > 0 && L / Lk > 1 ? L / Lk : 1;
    } else {
      // Query i stands at key position i + Lk - L: shift the band by that.
      const int shift = Lk - L;
      if (left < kNoLimit) left -= shift;
      if (right < kNoLimit) right += shift;
    }
    qoff = (int64_t)qs * ldq + (int64_t)h * hm.q.h;
    koff = (int64_t)ks0 * ldk + (int64_t)(h / hm.group) * hm.k.h;
    voff = (int64_t)ks0 * ldv + (int64_t)(h / hm.group) * hm.v.h;
    ooff = (int64_t)qs * ldo + (int64_t)h * hm.o.h;
    lse_base = (int64_t)qs * hm.H + h;  // lse is [total_q, H]
    lse_step = hm.H;
  } else if constexpr (PLAIN) {
    qoff = koff = voff = ooff = (int64_t)(hm.bh0 + bh) * L * D;
    lse_base = (int64_t)(hm.bh0 + bh) * L;
  } else {
    qoff = hm.q_off(bh);
    koff = hm.k_off(bh);
    voff = hm.v_off(bh);
    ooff = hm.o_off(bh);
    lse_base = (int64_t)(hm.bh0 + bh) * L;
  }
  // Rows past the end of each head read as zero: the resources end after its
  // last row (and are empty for a sequence without keys).
  const auto rq = make_rsrc(q + qoff, ((uint32_t)(L - 1) * ldq + D) * 2);
  const u32x4 rk = rsrc_words(k + koff, Lk > 0 ? ((uint32_t)(Lk - 1) * ldk + D) * 2 : 0u);
  const u32x4 rv = rsrc_words(v + voff, Lk > 0 ? ((uint32_t)(Lk - 1) * ldv + D) * 2 : 0u);

  const int q0 = qb * BM + wave * 32;  // first query of this wave
  const int myq = q0 + c32;             // this lane's query
  // The last key query i may see (kNoLimit-sized when unbounded).
  auto last_key = [&](int i) { return MASK == kCompressed ? (i + 1) / cf - 1 : i + right; };
  const int my_last = last_key(myq);

  // Q fragments: B operand of S^T, lane holds Q[myq][16 s + 8 h .. + 8].
  bf16x8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, load16(rq, (uint32_t)(myq * ldq + 16 * s + 8 * h) * 2));

  // Key blocks t0 .. t0 + ntiles - 1 meet the band of this workgroup's queries.
  const int kstart = HAS_LEFT ? max(0, qb * BM - left) : 0;
  const int kend = BANDED ? min(Lk, last_key(qb * BM + BM - 1) + 1) : Lk;
  int t0 = kstart / kBN;
  int ntiles = max(0, (kend + kBN - 1) / kBN - t0);
  if (ks.n > 1) {  // this split's share of those blocks (possibly none)
    const int a = t0 + ntiles * split / ks.n, b = t0 + ntiles * (split + 1) / ks.n;
    t0 = a;
    ntiles = b - a;
  }

  // Both tiles are [64 keys][D channels] rows of 16-byte chunks, filled by
  // direct loads (one 1 KB run of 64 chunks per load and wave), issued
  // untracked: the wait for them is the explicit one before each barrier.  K
  // chunk c of row r sits at c ^ kswz(r) (above); V chunk c at c ^ vswz(r), so
  // that the four rows one transpose read gathers fall in distinct banks.
  auto kswz = [](int r) { return (r >> KSH) & (CPR - 1); };
  auto vswz = [](int r) { return CPR >= 8 ? 2 * (r & 3) : 2 * ((r >> 1) & 1); };
  auto issue = [&](int t, int slot) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int P = (j * QW + wave) * 64 + lane;
      const int row = P / CPR, lc = P % CPR;
      const uint32_t key = (uint32_t)(t * kBN + row);
      load16_to_lds_untracked(rk, ktiles + slot * TILE + (j * QW + wave) * 1024,
                              (key * ldk + (uint32_t)(lc ^ kswz(row)) * 8) * 2);
      load16_to_lds_untracked(rv, vtiles + slot * TILE + (j * QW + wave) * 1024,
                              (key * ldv + (uint32_t)(lc ^ vswz(row)) * 8) * 2);
    }
  };

  // S^T block of 64 keys x 32 queries (two 32-key halves) from a K tile.  Every
  // K fragment read is issued before the first MFMA, so that the MFMAs do not
  // each wait out one read's latency.
  auto compute_s = [&](const char* kt, f32x16 (&s)[2]) {
    bf16x8 ka[NS][2];
#pragma unroll
    for (int ss = 0; ss < NS; ++ss)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = kb * 32 + c32;
        const int pc = (2 * ss + h) ^ kswz(row);
        ka[ss][kb] = *(const bf16x8*)&kt[(row * CPR + pc) * 16];
      }
    __builtin_amdgcn_sched_barrier(0);
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ss = 0; ss < NS; ++ss)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(ka[ss][kb], qf[ss], s[kb]);
  };

  // V^T fragment of MFMA (c, kb, u) for O^T += V^T P^T: lane half h of channel
  // 32c + c32 takes keys kb*32 + 16u + {4h..4h+3, 8+4h..8+4h+3}, the order in
  // which the S^T registers hold them.  Two gfx950 transpose reads: in each
  // 16-lane group, lane L addresses the 4 channels 4(L % 4).. of key row
  // r0 + L / 4, and lane i receives the 4 keys r0.. of the group's channel i.
  auto vfrag = [&](const char* vt, int c, int kb, int u) {
    const int g16 = lane >> 4, L4 = lane & 15;
    const int m = c * 32 + 16 * (g16 & 1) + 4 * (L4 & 3);
    const int r0 = kb * 32 + 16 * u + 4 * (g16 >> 1) + (L4 >> 2);
    const int off = r0 * (D * 2) + ((((m >> 3) ^ vswz(r0)) << 4) | ((m & 7) * 2));
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((short4_lds*)(vt + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((short4_lds*)(vt + off + 8 * D * 2));
    const s16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
  };

  f32x16 o[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) o[c] = f32x16{};
  float m = -INFINITY, lsum = 0.f;

  // Softmax update of key block t from its S^T, then O^T += V^T P^T.
  auto softmax_pv = [&](int t, f32x16 (&s)[2], const char* vt) {
    const int kbase = t * kBN;
    // At D = 128 the V^T fragments are all read here, before the softmax (they
    // do not depend on P), so that they have arrived when the MFMAs issue.
    constexpr bool V_EARLY = D >= 128;
    bf16x8 vf[V_EARLY ? NCB : 1][2][2];
    if constexpr (V_EARLY) {
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u) vf[c][kb][u] = vfrag(vt, c, kb, u);
    }
    // This lane's query over its 32 of the 64 keys.  Unmasked, the maximum is
    // taken on the raw scores and scaled afterwards (the maximum when sl2 >= 0,
    // else the minimum), and y - m is one FMA: p = 2^(s * sl2 - m).
    const bool need_mask = (kbase + kBN > Lk) || (BANDED && kbase + kBN - 1 > last_key(q0)) ||
                           (HAS_LEFT && kbase < q0 + 31 - left);
    float tmax;
    if (need_mask) {
      tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kbase + kb * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
          const bool off = key >= Lk || (BANDED && key > my_last) || (HAS_LEFT && key < myq - left);
          s[kb][j] = off ? -INFINITY : s[kb][j] * sl2;
          tmax = fmaxf(tmax, s[kb][j]);
        }
      }
    } else if (sl2 >= 0.f) {
      float hi = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) hi = fmaxf(hi, s[kb][j]);
      tmax = hi * sl2;
    } else {
      float lo = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) lo = fminf(lo, s[kb][j]);
      tmax = lo * sl2;
    }
    tmax = wave_swap32_max(tmax);
    // Lazy reference: m moves only when this block's maximum exceeds it by more
    // than kLazy (log2 units), so most blocks skip the rescale of O.  P and l
    // always use the same reference, so the result is unchanged; p <= 2^kLazy.
    const bool grow = tmax > m + kLazy;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = grow ? tmax : m;
      const float alpha = m == -INFINITY ? 0.f : exp2_fast(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[c][j] *= alpha;
    }
    const float muse = m == -INFINITY ? 0.f : m;
    const float mul = need_mask ? 1.f : sl2;
    unsigned pk[2][8];
    float ps[2] = {0.f, 0.f};  // two partial sums of the rounded P, to shorten the chain
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        const float p0 = exp2_fast(fmaf(s[kb][j], mul, -muse));
        const float p1 = exp2_fast(fmaf(s[kb][j + 1], mul, -muse));
        pk[kb][j >> 1] = pack_bf16x2(p0, p1);
        ps[kb] = add_bf16x2(pk[kb][j >> 1], ps[kb]);  // sum of the rounded P actually used
      }
    }
    lsum += ps[0] + ps[1];
    // The P of MFMA (kb, u) is exactly the S^T registers 8u..8u+7 of block kb.
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4 bv = {pk[kb][4 * u], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]};
          const bf16x8 av = V_EARLY ? vf[V_EARLY ? c : 0][kb][u] : vfrag(vt, c, kb, u);
          o[c] = mfma32x32x16(av, __builtin_bit_cast(bf16x8, bv), o[c]);
        }
      }
    }
  };

  // Group g takes key blocks t = t0 + g + G * it, double-buffered: the loads
  // of its next block are in flight while it works on this one.  All groups
  // run the same number of iterations (so that every wave meets every
  // barrier); a block past the end, or one this wave's queries do not see, is
  // skipped.
  const int niter = (ntiles + G - 1) / G;
  const int tend = t0 + ntiles;
  auto active = [&](int t) {
    const int kbase = t * kBN;
    return t < tend && (!BANDED || kbase <= last_key(q0 + 31)) &&
           (!HAS_LEFT || kbase + kBN - 1 >= q0 - left);
  };
  if (g < ntiles) issue(t0 + g, 0);
  // A wait the compiler sees (not an asm one), so that it knows the Q
  // fragments have arrived: otherwise it waits for them again before each
  // block's first MFMAs, and that wait also holds for the next block's loads,
  // which are counted alongside.
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  __syncthreads();
  for (int it = 0; it < niter; ++it) {
    const int t = t0 + g + G * it;
    const int slot = it & 1;
    if (t + G < tend) issue(t + G, slot ^ 1);
    if (active(t)) {
      f32x16 s[2];
      compute_s(ktiles + slot * TILE, s);
      softmax_pv(t, s, vtiles + slot * TILE);
    }
    wait_vmem();
    __syncthreads();
  }

  // Merge the groups' partial results.  Groups 1 .. G-1 leave O (fp32), m
  // and l in the tiles, which no wave reads any more; group 0 combines them
  // exactly: O = sum_g 2^(m_g - M) O_g / sum_g 2^(m_g - M) l_g, M = max_g m_g.
  // Lane holds channels 32c + 8i + 4h + r (r = 0..3) of query myq in o[c][4i + r].
  lsum = wave_swap32_sum(lsum);
  constexpr int XO = QW * NCB * 16 * 64;          // floats of O per group
  float* xo = (float*)&smem;                       // [G-1][QW waves][NCB][16][64 lanes]
  float* xm = xo + (G - 1) * XO;                   // [G-1][QW waves][64 lanes]
  float* xl = xm + (G - 1) * QW * 64;
  static_assert(((G - 1) * XO + 2 * (G - 1) * QW * 64) * 4 <= (int)sizeof(OnlineSmem<D, G>),
                "exchange fits in the tiles");
  if (g > 0) {
    float* po = xo + (g - 1) * XO;
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j) po[((wave * NCB + c) * 16 + j) * 64 + lane] = o[c][j];
    xm[((g - 1) * QW + wave) * 64 + lane] = m;
    xl[((g - 1) * QW + wave) * 64 + lane] = lsum;
  }
  __syncthreads();
  if (g > 0) return;
  {
    float mg[G], lg[G];
    mg[0] = m;
    lg[0] = lsum;
    float M = m;
#pragma unroll
    for (int gi = 1; gi < G; ++gi) {
      mg[gi] = xm[((gi - 1) * QW + wave) * 64 + lane];
      lg[gi] = xl[((gi - 1) * QW + wave) * 64 + lane];
      M = fmaxf(M, mg[gi]);
    }
    float a[G];
    lsum = 0.f;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      a[gi] = mg[gi] == -INFINITY ? 0.f : exp2_fast(mg[gi] - M);
      lsum += a[gi] * lg[gi];
    }
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float acc = a[0] * o[c][j];
#pragma unroll
        for (int gi = 1; gi < G; ++gi)
          acc += a[gi] * xo[(gi - 1) * XO + ((wave * NCB + c) * 16 + j) * 64 + lane];
        o[c][j] = acc;
      }
    m = M;
  }
  if (ks.n > 1) {
    // A key split: this share's unnormalised O, m and l for the combine kernel
    // (m = -inf, l = 0 where the share holds no key the query sees).
    if (myq < L) {
      const size_t row = ((size_t)split * ks.heads + bh) * Lmax + myq;  // [split][head][Lmax]
      float* po = ks.part + row * D;
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *(f32x4*)(po + c * 32 + 8 * i + 4 * h) =
              f32x4{o[c][4 * i], o[c][4 * i + 1], o[c][4 * i + 2], o[c][4 * i + 3]};
      if (h == 0) *(f32x2*)(ks.stats + 2 * row) = f32x2{m, lsum};
    }
    return;
  }
  // The row's softmax denominator is sum_j 2^(y_j) = 2^m * lsum (y in log2 units).
  if (lse != nullptr && myq < L && h == 0)
    lse[lse_base + (int64_t)lse_step * myq] = (m + log2f(lsum)) * 0.6931471805599453f;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;  // a row that sees no key gives 0
  if (myq < L) {
    uint16_t* orow = out + ooff + (int64_t)myq * ldo;
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w = {pack_bf16x2(o[c][4 * i] * inv, o[c][4 * i + 1] * inv),
                   pack_bf16x2(o[c][4 * i + 2] * inv, o[c][4 * i + 3] * inv)};
        *(u32x2*)(orow + c * 32 + 8 * i + 4 * h) = w;
      }
    }
  }
}

// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the key splits
// (M = max_s m_s), rounded once to bf16; one thread per (head, row, 8 channels)
// of the shares' [head][L] rows.  Token-packed sequences (vs.cu_q non-null)
// place row `row` of head bh = b * H + h at token cu_q[b] + row, up to that
// sequence's length.  A row that saw no key gives 0 and an LSE of -inf.
template <int D>
__global__ __launch_bounds__(256) void online_combine_kernel(KeySplit ks, uint16_t* __restrict__ out,
                                                             float* __restrict__ lse, HeadMap hm,
                                                             int L, VarSeqs vs) {
  constexpr int C8 = D / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)ks.heads * L * C8) return;
  const int chunk = (int)(i % C8);
  const int64_t rowall = i / C8;  // head * L + row
  const int bh = (int)(rowall / L), row = (int)(rowall - (int64_t)bh * L);
  int64_t orow, lrow;  // out element offset of the row, lse index
  if (vs.cu_q != nullptr) {
    const int b = bh / hm.H, h = bh - b * hm.H;
    const int qs = min(max(vs.cu_q[b], 0), vs.total_q);
    const int qe = min(max(vs.cu_q[b + 1], qs), vs.total_q);
    if (row >= min(qe - qs, L)) return;  // past this sequence's queries
    orow = (int64_t)(qs + row) * hm.o.ld + (int64_t)h * hm.o.h;
    lrow = (int64_t)(qs + row) * hm.H + h;
  } else {
    orow = hm.o_off(bh) + (int64_t)row * hm.o.ld;
    lrow = (int64_t)(hm.bh0 + bh) * L + row;
  }
  const size_t plane = (size_t)ks.heads * L;  // rows per split
  float M = -INFINITY;
  for (int sp = 0; sp < ks.n; ++sp) M = fmaxf(M, ks.stats[2 * (sp * plane + rowall)]);
  float den = 0.f;
  f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < ks.n; ++sp) {
    const size_t r = sp * plane + rowall;
    const f32x2 ml = *(const f32x2*)(ks.stats + 2 * r);
    const float w = ml[0] == -INFINITY ? 0.f : exp2_fast(ml[0] - M);
    den += w * ml[1];
    const f32x4* p = (const f32x4*)(ks.part + r * D + 8 * chunk);
    a += w * p[0];
    b += w * p[1];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const u32x4 wds = {pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv),
                     pack_bf16x2(b[0] * inv, b[1] * inv), pack_bf16x2(b[2] * inv, b[3] * inv)};
  *(u32x4*)(out + orow + 8 * chunk) = wds;
  if (lse != nullptr && chunk == 0) lse[lrow] = (M + log2f(den)) * 0.6931471805599453f;
}

template <int D, int MASK, int LAYOUT, int QW, int G>
hipError_t launch_one(const void* q, const void* k, const void* v, void* out, float* lse,
                      HeadMap hm, int BH, int L, float sl2, Band band, VarSeqs vs,
                      KeySplit ks, hipStream_t s) {
  const int nqb = (L + 32 * QW - 1) / (32 * QW);
  const dim3 grid((unsigned)(nqb * BH * (ks.n > 1 ? ks.n : 1))), block(64 * QW * G);
  const uint16_t* qp = (const uint16_t*)q;
  const uint16_t* kp = (const uint16_t*)k;
  const uint16_t* vp = (const uint16_t*)v;
  uint16_t* op = (uint16_t*)out;
  void* args[] = {&qp, &kp, &vp, &op, &lse, &hm, &L, (void*)&nqb, &sl2, &band, &vs, &ks};
  return hipLaunchKernel((const void*)&online_attn_kernel<D, MASK, LAYOUT, QW, G>, grid, block,
                         args, 0, s);
}

// Four query waves by two key-block groups: 8 waves, 128 queries.  (Four
// groups, and 64-query workgroups for causal masks, measured no faster.)
template <int D, int MASK, int LAYOUT>
hipError_t launch_l(const void* q, const void* k, const void* v, void* out, float* lse,
                    HeadMap hm, int BH, int L, float sl2, Band band, VarSeqs vs,
                    KeySplit ks, hipStream_t s) {
  return launch_one<D, MASK, LAYOUT, 4, 2>(q, k, v, out, lse, hm, BH, L, sl2, band, vs, ks, s);
}

template <int D, int MASK>
hipError_t launch_m(const void* q, const void* k, const void* v, void* out, float* lse,
                    const HeadMap& hm, int BH, int L, float sl2, Band band,
                    const VarSeqs& vs, KeySplit ks, hipStream_t s) {
  if (vs.cu_q != nullptr)
    return launch_l<D, MASK, kVarlen>(q, k, v, out, lse, hm, BH, L, sl2, band, vs, ks, s);
  if constexpr (MASK == kCompressed) {
    return hipErrorInvalidValue;  // token-packed sequences only
  } else {
    if (is_plain(hm, L, D))
      return launch_l<D, MASK, kPlain>(q, k, v, out, lse, hm, BH, L, sl2, band, vs, ks, s);
    return launch_l<D, MASK, kStrided>(q, k, v, out, lse, hm, BH, L, sl2, band, vs, ks, s);
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* out, float* lse,
                    const HeadMap& hm, int BH, int L, float sl2, Band band,
                    const VarSeqs& vs, KeySplit ks, hipStream_t s) {
  if (band.compressed)
    return launch_m<D, kCompressed>(q, k, v, out, lse, hm, BH, L, sl2, band, vs, ks, s);
  if (band_is_full(band))
    return launch_m<D, kAllKeys>(q, k, v, out, lse, hm, BH, L, sl2, band, vs, ks, s);
  if (band_is_causal(band))
    return launch_m<D, kCausal>(q, k, v, out, lse, hm, BH, L, sl2, band, vs, ks, s);
  return launch_m<D, kWindow>(q, k, v, out, lse, hm, BH, L, sl2, band, vs, ks, s);
}

}  // namespace

hipError_t launch_online(const void* q, const void* k, const void* v, void* out, float* lse,
                         const HeadMap& hm, int BH, int L, int d, float sl2, const Band& band,
                         const VarSeqs& vs, const KeySplit& ks, hipStream_t s) {
  switch (d) {
    case 32: return launch_d<32>(q, k, v, out, lse, hm, BH, L, sl2, band, vs, ks, s);
    case 64: return launch_d<64>(q, k, v, out, lse, hm, BH, L, sl2, band, vs, ks, s);
    case 128: return launch_d<128>(q, k, v, out, lse, hm, BH, L, sl2, band, vs, ks, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_online_combine(const KeySplit& ks, void* out, float* lse, const HeadMap& hm,
                                 int L, int d, const VarSeqs& vs, hipStream_t s) {
  const int64_t n = (int64_t)ks.heads * L * (d / 8);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  KeySplit k = ks;
  HeadMap m = hm;
  VarSeqs v = vs;
  uint16_t* op = (uint16_t*)out;
  void* args[] = {&k, &op, &lse, &m, &L, &v};
  switch (d) {
    case 32: return hipLaunchKernel((const void*)&online_combine_kernel<32>, grid, block, args, 0, s);
    case 64: return hipLaunchKernel((const void*)&online_combine_kernel<64>, grid, block, args, 0, s);
    case 128: return hipLaunchKernel((const void*)&online_combine_kernel<128>, grid, block, args, 0, s);
    default: return hipErrorInvalidValue;
  }
}

int online_split(int64_t BH, int64_t Lq, int64_t Lk) {
  const int64_t wgs = BH * ((Lq + kBM - 1) / kBM);  // workgroups without a split
  if (wgs * 2 > kValuesTargetWorkgroups) return 1;
  int64_t s = std::min<int64_t>(kValuesTargetWorkgroups / wgs, kOnlineMaxSplit);
  // Each share keeps at least two key blocks per group.
  s = std::min<int64_t>(s, (Lk + kBN - 1) / kBN / (2 * 2));
  return s >= 2 ? (int)s : 1;
}

}  // namespace attn
