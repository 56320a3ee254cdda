// two_pass_attn.hip -- exact attention for large head dims (128 < d <= 1024).
//
// The pages' design for the Wan2.2 mid-block attention (FastVideo
// wan22_vae_decode attn.cu, header comment: S = q k^T with fp32 accumulation,
// a row softmax, then O = p v) materialises S in fp32 and P in bf16.  On
// MI355X the per-frame O tile (rows x 1024 fp32) does not fit a CU's register
// file next to a useful query block, so the path stays two-pass like the
// pages', but moves the softmax into the two GEMMs:
//
//   scores pass  for each 256-key x 256-query tile of S^T = K Q^T (fp32):
//                y = scale*log2(e) * s; per query and 128-key half t of the
//                tile m_t = ceil(max over those keys of y) (an integer);
//                E = bf16(2^(y - m_t)); store E, m_t and psum_t = sum of the
//                stored E over those keys.
//   values pass  per query M = max_t m_t, l = sum_t 2^(m_t - M) psum_t, and
//                O = (sum_t 2^(m_t - M) E_t V_t) / l, with the factor applied
//                to E exactly: m_t - M is an integer, so scaling bf16 E by it
//                is a saturating subtract on the exponent bits.
//
// So S never leaves the registers in fp32, E is written once in bf16 (the
// pages' P rounding point), the normaliser sums exactly the values the second
// contraction uses, and there is no extra pass over S or P.  V is read in place:
// the values pass stages V rows in LDS and builds its MFMA operand with the
// gfx950 transpose read (ds_read_b64_tr_b16), so no V^T copy is made.  The subtraction of
// a per-tile reference before the exponential is the stable softmax of the
// attn.cu row_softmax_kernel and of the FMHA example's softmax_step; the
// rescale by 2^(m_t - M) is that example's correction step, done once per
// tile with exact factors.
//
// Masks are bands of keys per query (causal, or a sliding window): both passes
// visit only the tiles a query tile's band meets.  Operands are found through
// a head map (strides, key/value head groups), so packed and strided layouts
// are read in place.  For few heads the values pass runs on 128 x 128 tiles,
// or splits the keys and sums fp32 shares in a third kernel.
#include <algorithm>
#include <atomic>
#include <cstddef>
#include <type_traits>

#include "device.h"
#include "gemm_core.h"
#include "internal.h"

namespace attn {

TwoPassDims two_pass_dims(int64_t L, int64_t d) {
  TwoPassDims t;
  t.L = (int)L;
  t.d = (int)d;
  t.T = (int)((L + kTile - 1) / kTile);
  t.TK = (int)((L + 127) / 128);
  t.QB = (int)((L + 31) / 32);
  t.EB = 16 * t.T;
  t.Lk = (int)((L + 63) / 64 * 64);
  return t;
}

static int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

int64_t two_pass_head_bytes(const TwoPassDims& t) {
  return round256((int64_t)t.QB * t.EB * 1024) + 2 * round256((int64_t)t.TK * t.L * 4);
}

namespace {

// A staged 16-byte chunk of tile row r holds its 8-byte halves swapped when
// r % 32 >= 16; put them back in order.
__device__ __forceinline__ u32x4 unswap_halves(u32x4 x, int r) {
  return (r & 16) ? u32x4{x[2], x[3], x[0], x[1]} : x;
}

// ---------------------------------------------------------------------------
// Scores pass.  Tile (kt, qt) of head bh: keys [256 kt, +256) on the M side,
// queries [256 qt, +256) on the N side, so each lane of the accumulator owns a
// query and holds 4 runs of 4 consecutive keys per 32x32 block.
//
// E layout (internal.h): 1 KB blocks of 32 queries x 16 key positions.  Inside
// each 32-key block of a tile, key c sits at position kperm(c) (bits 2 and 3 of
// c exchanged), so that a lane's 16 values of one 32x32 accumulator block are
// two runs of 8 consecutive positions, i.e. 16 bytes in each of two blocks: one
// register-direct store instruction writes one whole block (8 full cache lines;
// row-major E took 32 scattered 32-byte pieces per instruction and cost a fifth
// of this pass).  The values pass reads V rows in the same key order.
//
// Statistics per 128-key half of a tile (the keys one wave holds), so that
// each wave's epilogue needs nothing from the others: per query,
// m = ceil(max over the half's keys of y), y = sl2 * s; E = bf16(2^(y - m))
// (so 1/2 < max E <= 1); psum = sum of the stored E.  Half h of tile kt is
// statistics tile 2 kt + h.  MASK selects the edge-tile version (keys past L,
// keys outside the band); it is a template flag so that the per-element test
// compiles to selects, not branches.
constexpr int kSK = 128;  // keys per statistics tile
// Three K stages and two Q stages (160 KB, all of a CU's LDS): the K loads of a
// step go out two steps ahead, the Q loads a step and a quarter ahead.
struct alignas(16) ScoresSmem {
  char a[3][kStageBytes];  // K
  char b[2][kStageBytes];  // Q
};

struct ScoresTile {
  int bh, qt, kt;
};

// 8 waves, two per SIMD: wave w owns keys [128 wm, +128) x queries
// [128 wn + 64 hf, +64) of the tile, as 4 x 2 accumulator blocks.  Two waves
// per SIMD keep the matrix cores busier than one wave with twice the
// accumulators (measured 68-72% against 55-57% of cycles on this GEMM shape),
// at 1.5x the LDS fragment reads.
//
// Waves w and w + 4 share a SIMD; with p = w % 4 and g = w / 4 the roles are
// wm = p / 2 ^ g, wn = p % 2 ^ g, hf = p / 2, so the two waves of a SIMD differ
// in both key half and query half.  On the last key tile or query tile of a
// head, whose far half lies past L, every SIMD then keeps one wave of real work
// while its partner (see scores_wave_idle) skips its MFMAs.
constexpr int kScoresWaves = 8;
constexpr int kScoresNJ = 2;
__device__ __forceinline__ int scores_key_half(int wave) { return ((wave >> 1) ^ (wave >> 2)) & 1; }
__device__ __forceinline__ int scores_query_base(int wave) {
  return ((wave ^ (wave >> 2)) & 1) * 128 + ((wave >> 1) & 1) * 64;
}

// Tile idx of the pass: heads in order, then the tiles of a head.  No mask:
// key tiles in blocks of kKeyBlock, and within a block query tiles, then key
// tiles, so that the 32 tiles an XCD runs at a time share 4 key tiles and
// about 8 query tiles (fewer K and Q slices fetched into its L2 per step than
// with all of a query tile's key tiles in a row: -1.7% on this pass at 31
// frames).  Causal (kt <= qt): query tiles, then their key tiles (closed
// form).  A sliding window: query tiles, then the key tiles each one's band
// meets (band_tiles), found by a walk.  per_head tiles per head.
constexpr int kKeyBlock = 4;
__device__ __forceinline__ ScoresTile scores_tile(int idx, int T, const Band& band, int per_head) {
  ScoresTile t;
  t.bh = idx / per_head;
  int r = idx - t.bh * per_head;
  if (band_is_full(band)) {
    const int b = r / (kKeyBlock * T), rb = r - b * kKeyBlock * T;
    const int w = min(kKeyBlock, T - kKeyBlock * b);  // key tiles in this block
    t.qt = rb / w;
    t.kt = kKeyBlock * b + (rb - t.qt * w);
  } else if (band_is_causal(band)) {
    int qt = (int)((sqrtf(8.f * (float)r + 1.f) - 1.f) * 0.5f);
    while ((qt + 1) * (qt + 2) / 2 <= r) ++qt;
    while (qt * (qt + 1) / 2 > r) --qt;
    t.qt = qt;
    t.kt = r - qt * (qt + 1) / 2;
  } else {
    int qt = 0, lo = 0, hi = 0;
    for (;; ++qt) {  // r < per_head: ends at a query tile below T
      band_tiles(band, qt, kTile, T, kTile, &lo, &hi);
      if (r <= hi - lo) break;
      r -= hi - lo + 1;
    }
    t.qt = qt;
    t.kt = lo + r;
  }
  return t;
}

// Every (query, key) pair of the tile lies inside the band and below L.
__device__ __forceinline__ bool scores_tile_unmasked(const ScoresTile& t, const Band& band, int L) {
  const int k0 = t.kt * kTile, q0 = t.qt * kTile;
  return k0 + kTile <= L && k0 >= q0 + kTile - 1 - band.left && k0 + kTile - 1 <= q0 + band.right;
}

// True when every score of this wave's block in the tile is discarded: its keys
// or its queries all lie past L, or all its keys lie outside all its queries'
// bands (e.g. causal: all its keys follow all its queries).  Such a wave issues
// its share of the loads and meets every barrier but skips its fragment reads
// and MFMAs, and enters the epilogue with zero accumulators, none of which
// reach memory: keys past L or outside the band are selected away, and rows
// past L are not stored (their maxima and sums are exchanged only with the
// partner wave holding the same rows).
__device__ __forceinline__ bool scores_wave_idle(const ScoresTile& t, int wave, int L,
                                                 const Band& band) {
  const int key0 = t.kt * kTile + scores_key_half(wave) * 128;
  const int q0 = t.qt * kTile + scores_query_base(wave);
  return key0 >= L || q0 >= L || key0 > q0 + 63 + band.right || key0 + 127 < q0 - band.left;
}

template <bool MASK>
__device__ __forceinline__ void scores_epilogue(f32x16 (&acc)[4][kScoresNJ],
                                                uint16_t* __restrict__ E,
                                                float* __restrict__ mref,
                                                float* __restrict__ psum, const ScoresTile& t,
                                                int L, int QB, int EB, int TK, float sl2,
                                                const Band& band) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = scores_key_half(wave), c32 = lane & 31, h = lane >> 5;
  const int qbase = scores_query_base(wave);  // this wave's first query column in the tile
  const int key0 = t.kt * kTile + wm * kSK;
  uint16_t* Eh = E + (size_t)t.bh * QB * EB * 512;
  // This half's statistics (none for a half wholly past L: no such tile).
  const bool stats = key0 < L;
  float* mref_t = mref + ((size_t)t.bh * TK + (key0 / kSK)) * L;
  float* psum_t = psum + ((size_t)t.bh * TK + (key0 / kSK)) * L;

#pragma unroll
  for (int bj = 0; bj < kScoresNJ; ++bj) {
    const int ql = qbase + bj * 32 + c32;
    const int query = t.qt * kTile + ql;
    // Key key0 + 4h + c (c = 32 bi + 8 (j / 4) + j % 4, a constant) is allowed
    // for this query iff lo <= c < lim.
    const int lim = min(L, query + band.right + 1) - (key0 + 4 * h);
    const int lo = query - band.left - (key0 + 4 * h);
    auto masked = [&](int bi, int j) {
      const int c = bi * 32 + 8 * (j >> 2) + (j & 3);
      return c >= lim || c < lo;
    };

    // Maximum of y (interior tiles: on the raw accumulator, then scaled; the
    // sign of sl2 picks max or min).
    float tmax;
    if (!MASK && sl2 >= 0.f) {
      float hi = acc[0][bj][0];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int j = 0; j < 16; ++j) hi = fmaxf(hi, acc[bi][bj][j]);
      tmax = hi * sl2;
    } else if (!MASK) {
      float lo2 = acc[0][bj][0];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int j = 0; j < 16; ++j) lo2 = fminf(lo2, acc[bi][bj][j]);
      tmax = lo2 * sl2;
    } else {
      float mx = -INFINITY;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, masked(bi, j) ? -INFINITY : acc[bi][bj][j] * sl2);
      tmax = mx;
    }
    tmax = wave_swap32_max(tmax);
    const float m2 = tmax == -INFINITY ? -INFINITY : ceilf(tmax);
    const float add = tmax == -INFINITY ? 0.f : -m2;
    float s = 0.f;
    // This column's 32 queries are one query block; blocks 2 bi and 2 bi + 1 of
    // the half's 16-key blocks take w[0] and w[1].
    uint16_t* blk = Eh + ((size_t)(min(query, L - 1) >> 5) * EB + (key0 >> 4)) * 512 + lane * 8;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      u32x4 w[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = exp2_fast(fmaf(acc[bi][bj][4 * i + r], sl2, add));
          if (MASK) e[r] = masked(bi, 4 * i + r) ? 0.f : e[r];
        }
        const unsigned w0 = pack_bf16x2(e[0], e[1]), w1 = pack_bf16x2(e[2], e[3]);
        // the normaliser sums exactly the rounded values the values pass multiplies
        s = add_bf16x2(w1, add_bf16x2(w0, s));
        // keys 8 i + 4 h + 0..3 of the block sit at positions 16 (i / 2) + 8 h + 4 (i % 2) + 0..3
        w[i >> 1][2 * (i & 1)] = w0;
        w[i >> 1][2 * (i & 1) + 1] = w1;
      }
      if (query < L) {
        *(u32x4*)(blk + (2 * bi) * 512) = w[0];
        *(u32x4*)(blk + (2 * bi + 1) * 512) = w[1];
      }
    }
    s = wave_swap32_sum(s);
    if (h == 0 && query < L && stats) {
      mref_t[query] = m2;
      psum_t[query] = s;
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the next column's copies after this one's
  }
}

// Persistent: workgroup g takes tiles g, g + G, g + 2G, ... (G = grid size; g
// after the XCD renumbering, so each XCD works through a contiguous range).
// The K steps of all its tiles form one stream through the LDS stages: the
// loads run two steps ahead across tile boundaries, so the next tile's first
// stages arrive while this tile's epilogue computes and stores E.  Step s reads
// K stage s % 3 and Q stage s % 2.  During step s the wave issues its K loads
// of step s + 2 (in the first sub-step, into the K stage step s - 1 read) and,
// after the barrier that ends step s, its Q loads of step s + 2 (into the Q
// stage step s read).  So before that barrier it waits for everything but the
// last four loads it issued (loads complete in order; a store issued between
// them, such as the epilogue's, only makes the wait longer).
// One LDS object, so that the compiler puts no wait for the direct loads in
// flight before the fragment reads (gemm_core.h, header).
__global__ __launch_bounds__(64 * kScoresWaves) void scores_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, uint16_t* __restrict__ E,
    float* __restrict__ mref, float* __restrict__ psum, HeadMap hm, int L, int d, int T, int TK,
    int QB, int EB, float sl2, Band band, int per_head, int ntiles) {
  __shared__ ScoresSmem sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: stage addresses in scalar registers
  const int abase = scores_key_half(wave) * 128;  // key rows of this wave
  const int bbase = scores_query_base(wave);  // query rows of this wave
  const int G = (int)gridDim.x;
  const int first = (int)xcd_logical_id(blockIdx.x, gridDim.x);
  const int my_tiles = (ntiles - 1 - first) / G + 1;  // first < ntiles
  const int nk = d / kStepK;                          // >= 3 on this path
  const int ldk = hm.k.ld, ldq = hm.q.ld;
  constexpr int kLoads = KContiguousT<kScoresWaves>::kLoads;  // per wave and operand
  static_assert(kLoads == 4, "one load per MFMA pair; the waits below count 4 loads");

  KContiguousT<kScoresWaves> la, lb;  // per-lane offsets within a tile; resources start at its first row
  la.init((uint32_t)ldk, 0, wave, lane);
  lb.init((uint32_t)ldq, 0, wave, lane);

  // Load cursor: the step (tile li, K step lk) whose loads go out next.
  int li = 0, lk = 0;
  __amdgpu_buffer_rsrc_t rk, rq;
  auto set_load_tile = [&](int i) {
    const ScoresTile t = scores_tile(first + i * G, T, band, per_head);
    const int k0 = t.kt * kTile, q0 = t.qt * kTile;
    // Each resource ends after the head's row L - 1: rows past L read as zero.
    rk = make_rsrc(k + hm.k_off(t.bh) + (size_t)k0 * ldk, ((uint32_t)(L - 1 - k0) * ldk + d) * 2u);
    rq = make_rsrc(q + hm.q_off(t.bh) + (size_t)q0 * ldq, ((uint32_t)(L - 1 - q0) * ldq + d) * 2u);
  };
  // Past the last step the cursor stays there: the loads of steps beyond the
  // end reload it into stages no longer read.
  auto advance = [&]() {
    if (li == my_tiles - 1 && lk == nk - 1) return;
    if (++lk == nk) {
      lk = 0;
      set_load_tile(++li);
    }
  };
  // Before the barrier ending a step: this wave's loads of the next step have
  // landed (only the K loads of the step after it may still be in flight).
  auto wait_next = [&]() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); };

  set_load_tile(0);
  la.issue_from(rk, 0, sm.a[0], wave);
  lb.issue_from(rq, 0, sm.b[0], wave);
  advance();
  wait_vmem();
  block_sync();
  la.issue_from(rk, lk * kStepK, sm.a[1], wave);  // nk >= 3: a step of the first tile
  lb.issue_from(rq, lk * kStepK, sm.b[1], wave);
  advance();  // the cursor is on step 2

  f32x16 acc[4][kScoresNJ];
  NoTransform nx;
  FragsT<kScoresNJ> cur, nxt;
  read_frags(cur, la, lb, sm.a[0], sm.b[0], abase, bbase, lane, 0);

  // One K step s (K stage ka = s % 3): sub-step 0 starts the accumulators
  // when FIRST (the first step of a tile).
  auto step = [&](auto first_step, int s, int ka) {
    constexpr bool FIRST = decltype(first_step)::value;
    const int kn = ka == 2 ? 0 : ka + 1, kf = kn == 2 ? 0 : kn + 1;  // stages of steps s + 1, s + 2
    const int st = s & 1;
    const char* sa = sm.a[ka];
    const char* sb = sm.b[st];
    // Issue priority 1 while the wave runs the step's MFMAs, 0 at the barrier
    // and in the epilogue (measured: the pass 687.7 -> 652.4 us on 31 frames;
    // kept at 1 across the barrier it gains nothing).
    // Sub-step 0: its MFMAs in pairs, each followed by one K load of step s + 2.
    __builtin_amdgcn_s_setprio(1);
    read_frags(nxt, la, lb, sa, sb, abase, bbase, lane, 1);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      __builtin_amdgcn_sched_barrier(0);
      acc[p][0] = mfma32x32x16(cur.a[p], cur.b[0], FIRST ? f32x16{} : acc[p][0]);
      acc[p][1] = mfma32x32x16(cur.a[p], cur.b[1], FIRST ? f32x16{} : acc[p][1]);
      la.issue_one(rk, lk * kStepK, sm.a[kf], wave, p);
    }
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
#pragma unroll
    for (int ss = 1; ss < 3; ++ss) {
      read_frags(nxt, la, lb, sa, sb, abase, bbase, lane, ss + 1);
      mma_substep(acc, cur, nx);
      sched_substep<kScoresNJ>();
      cur = nxt;
    }
    // Last sub-step: next stage complete everywhere, this stage drained.
    __builtin_amdgcn_s_setprio(0);
    wait_next();
    block_sync();
    __builtin_amdgcn_s_setprio(1);
    // This sub-step's MFMAs in pairs, each pair followed by one Q load of step
    // s + 2, with the next step's first fragments read before the last pair.
    // Measured: loads as a burst right after the barrier, or those reads right
    // after it, both cost a few percent.
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p == 3) {
        __builtin_amdgcn_sched_barrier(0);
        read_frags(nxt, la, lb, sm.a[kn], sm.b[st ^ 1], abase, bbase, lane, 0);  // past the end: unused
      }
      __builtin_amdgcn_sched_barrier(0);
      acc[p][0] = mfma32x32x16(cur.a[p], cur.b[0], acc[p][0]);
      acc[p][1] = mfma32x32x16(cur.a[p], cur.b[1], acc[p][1]);
      lb.issue_one(rq, lk * kStepK, sm.b[st], wave, p);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    cur = nxt;
    advance();
  };

  // A step of a wave whose block of the tile is discarded: its loads and the
  // barrier only.
  auto idle_step = [&](int s, int ka) {
    const int kf = ka == 0 ? 2 : ka - 1;  // (s + 2) % 3
#pragma unroll
    for (int p = 0; p < 4; ++p) la.issue_one(rk, lk * kStepK, sm.a[kf], wave, p);
    wait_next();
    block_sync();
#pragma unroll
    for (int p = 0; p < 4; ++p) lb.issue_one(rq, lk * kStepK, sm.b[s & 1], wave, p);
    advance();
  };

  int s = 0, ka = 0;  // ka = s % 3
  auto next_ka = [&]() { ka = ka == 2 ? 0 : ka + 1; };
  for (int i = 0; i < my_tiles; ++i) {
    const ScoresTile t = scores_tile(first + i * G, T, band, per_head);
    if (__builtin_amdgcn_readfirstlane((int)scores_wave_idle(t, wave, L, band))) {
      // Fresh (zero) accumulators: nothing stays live across tiles.
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < kScoresNJ; ++bj) acc[bi][bj] = f32x16{};
      for (int kk = 0; kk < nk; ++kk) {
        idle_step(s++, ka);
        next_ka();
      }
    } else {
      step(std::true_type{}, s++, ka);
      next_ka();
      for (int kk = 1; kk < nk; ++kk) {
        step(std::false_type{}, s++, ka);
        next_ka();
      }
    }
    if (!scores_tile_unmasked(t, band, L))
      scores_epilogue<true>(acc, E, mref, psum, t, L, QB, EB, TK, sl2, band);
    else
      scores_epilogue<false>(acc, E, mref, psum, t, L, QB, EB, TK, sl2, band);
    // The next step's first fragments: read again (its stage is not refilled
    // before that step's end) instead of holding them through the epilogue.
    read_frags(cur, la, lb, sm.a[ka], sm.b[s & 1], abase, bbase, lane, 0);
  }
  wait_vmem();
}

// ---------------------------------------------------------------------------
// Values pass.  Tile (ct, qt): channels [256 ct, +256) on the M side (A = V^T),
// queries [256 qt, +256) on the N side (B = E), K = keys in 64-wide steps.
// Each lane owns four queries (one per 32-column block j); before each pair
// of steps (one 128-key score tile t) it turns M - m_t into the exponent
// shift for those queries.
constexpr int kMaxTiles = kTwoPassMaxTiles;

// NQ: query columns per lane (one per 32-query block of the wave).
template <int NQ>
struct PowerOfTwoShift {
  int col[NQ];      // this lane's query columns in the tile
  unsigned sw[NQ];  // shift words (s << 7 | s << 23) of the current 128-key tile

  // The shifts of 128-key tile t (from [t][query in tile]: M - m_t), and the
  // shift words made from them.
  template <int QT>
  __device__ __forceinline__ void load(const uint8_t (*tab)[QT], int t, unsigned (&s)[NQ]) const {
#pragma unroll
    for (int j = 0; j < NQ; ++j) s[j] = tab[t][col[j]];
  }
  __device__ __forceinline__ void set(const unsigned (&s)[NQ]) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) sw[j] = (s[j] << 7) | (s[j] << 23);
  }
  __device__ __forceinline__ bf16x8 operator()(bf16x8 f, int j) const {
    u32x4 w = __builtin_bit_cast(u32x4, f);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = scale_pow2_down(w[e], sw[j]);
    return __builtin_bit_cast(bf16x8, w);
  }
};

// The statistics of query q0 + tid of head bh over score tiles [tlo, thi]:
// M = max_t m_t, l = sum_t 2^(m_t - M) psum_t, the shift M - m_t of each tile
// (a nonnegative integer; -inf tiles -> 255) into shift_tab[t][tid], 1/l into
// inv_l[tid], and when write_lse the log-sum-exp into lse.
// The stats of up to 32 tiles are read at once, so that their latencies
// overlap and, for query tiles that meet at most 32 score tiles (L <= 4096
// without a band), the shifts come from the same registers: one round of
// loads instead of four (batches of 16 and a second pass).
template <int QT>
__device__ __forceinline__ void values_stats(const float* __restrict__ mref,
                                             const float* __restrict__ psum,
                                             float* __restrict__ lse, bool write_lse, int bh,
                                             int bh0, int TK, int L, int q0, int tlo, int thi,
                                             uint8_t (*shift_tab)[QT], float* inv_l, int tid) {
  const float* mh = mref + (size_t)bh * TK * L;
  const float* ph = psum + (size_t)bh * TK * L;
  const int qc = min(q0 + tid, L - 1);
  constexpr int kB = 32;
  float M = -INFINITY, l = 0.f;
  float mt[kB];
  for (int t0 = tlo; t0 <= thi; t0 += kB) {
    float pt[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int t = min(t0 + u, thi);
      mt[u] = mh[(size_t)t * L + qc];
      pt[u] = ph[(size_t)t * L + qc];
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < kB; ++u) Mn = fmaxf(Mn, mt[u]);
    l = M == -INFINITY ? 0.f : l * exp2_fast(M - Mn);
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (t0 + u <= thi && mt[u] != -INFINITY) l += pt[u] * exp2_fast(mt[u] - Mn);
    M = Mn;
  }
  // The shifts need the final M: from the registers when one batch held
  // every tile, else a second pass over the (now cached) stats.
  if (thi - tlo < kB) {
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (tlo + u <= thi) shift_tab[tlo + u][tid] = (uint8_t)fminf(M - mt[u], 255.f);
  } else {
    // Every load is consumed (entries past thi rewrite thi's), so that none
    // is left in flight for the compiler to wait on later.
    for (int t0 = tlo; t0 <= thi; t0 += kB) {
#pragma unroll
      for (int u = 0; u < kB; ++u) mt[u] = mh[(size_t)min(t0 + u, thi) * L + qc];
#pragma unroll
      for (int u = 0; u < kB; ++u) shift_tab[min(t0 + u, thi)][tid] = (uint8_t)fminf(M - mt[u], 255.f);
    }
  }
  inv_l[tid] = 1.f / l;
  // The row's softmax denominator is sum_j 2^(y_j) = 2^M l (y in log2 units).
  const int query = q0 + tid;
  if (lse != nullptr && write_lse && query < L)
    lse[(size_t)(bh0 + bh) * L + query] = (M + log2f(l)) * 0.6931471805599453f;
}

// The values pass walks the keys in steps of 32 through four LDS stages of
// 32 KB (V 16 KB, E 16 KB): the loads of step kt + 3 go out during step kt,
// so a load has three steps to arrive (two 64-key stages gave it about half
// of one 64-key step).
constexpr int kVK = 32;      // keys per values step
constexpr int kVStages = 4;  // stages in flight
constexpr int kVStageBytes = kVK * kTile * 2;

struct alignas(16) ValuesSmem {
  char v[kVStages][kVStageBytes];  // V rows [32 keys][256 channels]
  char e[kVStages][kVStageBytes];  // E blocks [8 query blocks][2 key blocks]
  uint8_t shift_tab[kMaxTiles][kTile];
  float inv_l[kTile];
};
static_assert(sizeof(ValuesSmem) <= 160 * 1024, "a CU's LDS");

// Staging of the values pass, 8 waves: V read as V^T (32 key rows x 256
// channels per stage, 512 bytes per row, 16-byte chunk c of row r at
// c ^ 4 (r % 4), stage row r holding key k0 + kperm(r): the order the scores
// pass gives the keys of each 32-key block of E) and E (the 8 x 2 blocks of
// 32 queries x 16 keys the step covers, copied as they are: block (i, j) at
// 1 KB x (2 i + j); a lane's MFMA operand is 16 contiguous bytes of a block).
// Each wave issues 2 loads of each per step, through untracked direct loads:
// the transpose reads of V carry no alias information, and the compiler would
// otherwise wait for every load in flight before each of them.
constexpr int kValuesWaves = 8;
struct ValuesV {
  uint32_t off[2];
  uint32_t ld2;  // bytes per key row
  __device__ __forceinline__ void init(uint32_t ld, int m0, int wave, int lane) {
    ld2 = ld * 2u;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int P = (wave * 2 + j) * 64 + lane;  // 16-byte chunk slot in the stage
      const int row = P >> 5, pc = P & 31, lc = pc ^ ((row & 3) << 2);
      off[j] = (uint32_t)kperm(row) * ld2 + (uint32_t)(m0 + lc * 8) * 2u;
    }
  }
  __device__ __forceinline__ void issue(const u32x4& r, int k0, char* stage, int wave, int j) const {
    load16_to_lds_untracked(r, stage + (wave * 2 + j) * 1024, off[j] + (uint32_t)k0 * ld2);
  }
};
// Wave w copies query block w of the tile's 8, key blocks k0 / 16 and k0 / 16 + 1.
struct ValuesE {
  uint32_t off;
  __device__ __forceinline__ void init(int EB, int wave, int lane) {
    off = (uint32_t)wave * (uint32_t)EB * 1024u + (uint32_t)lane * 16u;
  }
  __device__ __forceinline__ void issue(const u32x4& r, int k0, char* stage, int wave, int j) const {
    load16_to_lds_untracked(r, stage + (wave * 2 + j) * 1024, off + (uint32_t)((k0 >> 4) + j) * 1024u);
  }
};

// One k16 sub-step's fragments of a values wave: 2 V^T blocks of 32 channels,
// 4 E blocks of 32 queries.
struct ValuesFrags {
  bf16x8 a[2], b[4];
};

// SPLIT: the keys of each query tile are divided among `split` workgroups that
// write fp32 shares of O to `part` (a separate instantiation, so that the
// unsplit kernel carries none of it).
//
// 8 waves, two per SIMD: wave w owns channels [64 (w % 4), +64) x queries
// [128 (w / 4), +128) of the tile, as 2 x 4 accumulator blocks.  Per k16
// sub-step it reads 2 V^T fragments (two transpose reads each) and 4 E
// fragments for 8 MFMAs; the next sub-step's fragments are read while the
// current MFMAs run.  Step kt (32 keys, two sub-steps): the loads of step
// kt + 3 go out one per MFMA pair in the first sub-step (into the stage step
// kt - 1 read); the wave then waits for its loads of step kt + 1, meets the
// others at the barrier, and runs the second sub-step's MFMAs (fragments
// already in registers) while it reads the first fragments of step kt + 1.
template <bool SPLIT>
__global__ __launch_bounds__(64 * kValuesWaves) void values_kernel(const uint16_t* __restrict__ v,
                                                     const uint16_t* __restrict__ E,
                                                     const float* __restrict__ mref,
                                                     const float* __restrict__ psum,
                                                     uint16_t* __restrict__ out,
                                                     float* __restrict__ lse,
                                                     float* __restrict__ part, HeadMap hm, int L,
                                                     int d, int T, int TK, int QB, int EB,
                                                     int Lk, Band band, int ncb, int split,
                                                     int nheads) {
  __shared__ ValuesSmem sm;
  uint8_t(&shift_tab)[kMaxTiles][kTile] = sm.shift_tab;
  float(&inv_l)[kTile] = sm.inv_l;

  if (!SPLIT) split = 1;
  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int per_head = T * ncb * split;
  const int bh = lid / per_head;
  const int r = lid % per_head;
  const int qt = r / (ncb * split), ct = (r / split) % ncb, sp = SPLIT ? r % split : 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cq = wave & 3, qh = wave >> 2, c32 = lane & 31, h = lane >> 5;

  // Score tiles [tlo, thi] (128 keys each) meet this query tile's band: keys
  // [kbeg, kend).
  int tlo, thi;
  band_tiles(band, qt, kTile, TK, kSK, &tlo, &thi);
  const int kbeg = tlo * kSK, kend = min(Lk, (thi + 1) * kSK);
  // Split sp of `split` takes steps [k_first, k_first + nk) (never empty: the
  // host keeps split <= the fewest 64-key steps of any query tile).
  const int nk_all = (kend - kbeg) / kVK;
  const int k_first = kbeg / kVK + (SPLIT ? nk_all * sp / split : 0);
  const int nk = SPLIT ? kbeg / kVK + nk_all * (sp + 1) / split - k_first : nk_all;

  // V's resource ends after the head's row L - 1 (keys past L read as zero).
  // Channels past d of a 256-channel tile read whatever lies there (zero past
  // the end) and only feed accumulator rows that are never stored.
  const int ldv = hm.v.ld;
  const u32x4 rv = rsrc_words(v + hm.v_off(bh), ((uint32_t)(L - 1) * ldv + d) * 2u);
  // E from the tile's first query block; blocks past the head's last read as zero.
  const u32x4 re = rsrc_words(E + ((size_t)bh * QB + (size_t)qt * 8) * EB * 512,
                              (uint32_t)(QB - qt * 8) * (uint32_t)EB * 1024u);
  ValuesV la;
  ValuesE lb;
  la.init((uint32_t)ldv, ct * kTile, wave, lane);
  lb.init(EB, wave, lane);
  // Load j (0..3) of step u into its stage; steps past the last reload the
  // last (into a stage no longer read), so every step issues 4 loads.
  const int kb = k_first * kVK;
  auto issue = [&](int u, int j) {
    const int k0 = kb + min(u, nk - 1) * kVK;
    if (j < 2)
      la.issue(rv, k0, sm.v[u & 3], wave, j);
    else
      lb.issue(re, k0, sm.e[u & 3], wave, j - 2);
  };
  // Steps 0, 1 and 2 go out first, and arrive while the statistics are read.
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) issue(u, j);

  // Thread tid < 256 owns query qt*256 + tid.
  if (tid < kTile)
    values_stats<kTile>(mref, psum, lse, ct == 0 && sp == 0, bh, hm.bh0, TK, L, qt * kTile, tlo,
                        thi, shift_tab, inv_l, tid);
  // Step 0 staged (only steps 1 and 2 may be in flight); the shift table and
  // 1/l complete.
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  block_sync();

  PowerOfTwoShift<4> sh;
  float invl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sh.col[j] = qh * 128 + j * 32 + c32;
    invl[j] = inv_l[sh.col[j]];
  }

  KOuter ka;  // fragment reads only (the loads go through ValuesV)
  auto read = [&](ValuesFrags& f, int st, int ss) {
#pragma unroll
    for (int i = 0; i < 2; ++i) f.a[i] = ka.frag(sm.v[st], cq * 64 + i * 32, ss, lane);
    // E block (query block 4 qh + j, key block ss): 16 contiguous bytes per lane.
#pragma unroll
    for (int j = 0; j < 4; ++j)
      f.b[j] = *(const bf16x8*)(sm.e[st] + ((qh * 4 + j) * 2 + ss) * 1024 + lane * 16);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // The E fragments are scaled as soon as they arrive, in the second half of
  // the sub-step that reads them, so that the MFMAs after a barrier start at
  // once.  The shift words of a step are read during the step before.
  // 8 MFMAs of one sub-step in pairs; after pair p, load p of step kt + 3
  // (LOADS) and, in pairs 2 and 3, the scaling of two fragments of `f`.
  auto mfma_pairs = [&](const ValuesFrags& c, ValuesFrags& f, int kt, bool loads) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      __builtin_amdgcn_sched_barrier(0);
      const int i = p >> 1, j0 = 2 * (p & 1);
      acc[i][j0] = mfma32x32x16(c.a[i], c.b[j0], acc[i][j0]);
      acc[i][j0 + 1] = mfma32x32x16(c.a[i], c.b[j0 + 1], acc[i][j0 + 1]);
      if (loads) issue(kt + 3, p);
      if (p >= 2) {
        // Scaled here (the empty asm keeps the compiler from sinking the
        // scaling past the barrier to its first use).
        const int j = 2 * (p - 2);
        f.b[j] = sh(f.b[j], j);
        f.b[j + 1] = sh(f.b[j + 1], j + 1);
        asm volatile("" : "+v"(f.b[j]), "+v"(f.b[j + 1]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // A wave whose 128 queries all lie past L (the far half of a head's last
  // query tile when L mod 256 <= 128) only issues its loads and meets the
  // barriers: its accumulators stay zero and none of its rows is stored.
  if (__builtin_amdgcn_readfirstlane((int)(qt * kTile + qh * 128 >= L))) {
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int p = 0; p < 4; ++p) issue(kt + 3, p);
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      block_sync();
    }
  } else {
    ValuesFrags cur, nxt;
    {
      unsigned s0[4];
      sh.load(shift_tab, k_first >> 2, s0);
      sh.set(s0);
    }
    read(cur, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) cur.b[j] = sh(cur.b[j], j);
    // Issue priority 1 through each step but 0 across its wait and barrier, as
    // in the scores pass (measured: 731.9 -> 723.8 us on 31 frames, 97.5 ->
    // 95.9 us on 4).
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_s_setprio(1);
      const int st = kt & 3;
      // The shifts of step kt + 1 (past the end: unused), turned into shift
      // words after this sub-step's MFMAs.
      unsigned sn[4];
      sh.load(shift_tab, min((k_first + kt + 1) >> 2, thi), sn);
      // Sub-step 0, with the loads of step kt + 3.
      read(nxt, st, 1);
      mfma_pairs(cur, nxt, kt, true);
      cur = nxt;
      // Step kt + 1 staged everywhere (this wave's loads of steps kt + 2 and
      // kt + 3 may still be in flight); stage st is read no more after this
      // barrier (sub-step 1's fragments are in registers).
      __builtin_amdgcn_s_setprio(0);
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      block_sync();
      __builtin_amdgcn_s_setprio(1);
      read(nxt, (kt + 1) & 3, 0);  // past the last step: unused
      sh.set(sn);
      mfma_pairs(cur, nxt, kt, false);
      cur = nxt;
      __builtin_amdgcn_s_setprio(0);
    }
  }
  // No load in flight into the stages (the O tile below reuses them).
  wait_vmem();
  block_sync();

  if constexpr (SPLIT) {
    // This split's share of O = (its part of the sum) / l, in fp32, for the
    // reduction kernel: lane (query) stores 4 consecutive channels at a time.
    float* ph = part + ((size_t)sp * nheads + bh) * L * d;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int query = qt * kTile + qh * 128 + bj * 32 + c32;
      if (query >= L) continue;
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = ct * kTile + cq * 64 + bi * 32 + 8 * i + 4 * h;
          if (ch < d) {
            const f32x16& a = acc[bi][bj];
            f32x4 o = {a[4 * i] * invl[bj], a[4 * i + 1] * invl[bj], a[4 * i + 2] * invl[bj],
                       a[4 * i + 3] * invl[bj]};
            *(f32x4*)(ph + (size_t)query * d + ch) = o;
          }
        }
    }
    return;
  }

  // O[query][ch] = acc / l, rounded once to bf16.  The tile goes through the
  // drained stages (128 KB from sm.v[0] on) as [query][256 channels] rows
  // (laid out like the E tile of the scores pass) so that the global stores
  // write whole row segments.
  static_assert(offsetof(ValuesSmem, e) == kVStages * kVStageBytes &&
                    2 * kVStages * kVStageBytes >= kTile * kTile * 2,
                "the O tile fits the stages");
  char* stage = sm.v[0];
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    const int ql = qh * 128 + bj * 32 + c32;
    char* row = stage + ql * 512 + 8 * (h ^ (c32 >> 4));
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x16& a = acc[bi][bj];
        const u32x2 w = {pack_bf16x2(a[4 * i] * invl[bj], a[4 * i + 1] * invl[bj]),
                         pack_bf16x2(a[4 * i + 2] * invl[bj], a[4 * i + 3] * invl[bj])};
        const int chunk = cq * 8 + bi * 4 + i;
        *(u32x2*)(row + ((chunk ^ c32) << 4)) = w;
      }
    }
  }
  __syncthreads();
  {
    const int c = tid & 31;
    const int ch = ct * kTile + 8 * c;
    if (ch < d) {
      const int ldo = hm.o.ld;
      uint16_t* oh = out + hm.o_off(bh) + (size_t)(qt * kTile) * ldo + ch;
#pragma unroll 8
      for (int j = 0; j < 16; ++j) {
        const int rr = (tid >> 5) + 16 * j;
        if (qt * kTile + rr < L)
          *(u32x4*)(oh + (size_t)rr * ldo) = unswap_halves(*(const u32x4*)(stage + rr * 512 + ((c ^ (rr & 31)) << 4)), rr);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Values pass on 128 x 128 tiles, for calls whose 256 x 256 tiles would fill
// at most half of the compute units (one head at L = 3432: 56 of them against
// 216 narrow ones).  It needs no key split, so no fp32 partial outputs and no
// reduction pass.  Tile (ct, qt): channels [128 ct, +128) on the M side,
// queries [128 qt, +128) on the N side, keys in steps of 64 through four LDS
// stages of 32 KB (V 16 KB, E 16 KB); the loads of step kt + 3 go out during
// step kt, as in the wide kernel.
constexpr int kNT = 128;                     // narrow tile edge
constexpr int kNK = 64;                      // keys per step
constexpr int kNStages = 4;
constexpr int kNStageBytes = kNK * kNT * 2;  // per operand

struct alignas(16) NarrowSmem {
  char v[kNStages][kNStageBytes];  // V rows [64 keys][128 channels], 256 bytes each
  char e[kNStages][kNStageBytes];  // E blocks [4 query blocks][4 key blocks]
  uint8_t shift_tab[kMaxTiles][kNT];
  float inv_l[kNT];
};
static_assert(sizeof(NarrowSmem) <= 160 * 1024, "a CU's LDS");

// V rows as V^T: 64 key rows x 128 channels per stage, 16-byte chunk c of row
// r at c ^ 4 (r % 4), stage row r holding key k0 + kperm(r) (as in ValuesV).
// Each of the 8 waves issues 2 of the 16 loads of 1 KB.
struct NarrowV {
  uint32_t off[2];
  uint32_t ld2;  // bytes per key row
  __device__ __forceinline__ void init(uint32_t ld, int m0, int wave, int lane) {
    ld2 = ld * 2u;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int P = (wave * 2 + j) * 64 + lane;  // 16-byte chunk slot in the stage
      const int row = P >> 4, pc = P & 15, lc = pc ^ ((row & 3) << 2);
      off[j] = (uint32_t)kperm(row) * ld2 + (uint32_t)(m0 + lc * 8) * 2u;
    }
  }
  __device__ __forceinline__ void issue(const u32x4& r, int k0, char* stage, int wave, int j) const {
    load16_to_lds_untracked(r, stage + (wave * 2 + j) * 1024, off[j] + (uint32_t)k0 * ld2);
  }
};
// E: the 4 x 4 blocks of 32 queries x 16 keys a step covers, block (i, j) at
// 1 KB x (4 i + j); wave w copies query block w / 2, key blocks 2 (w % 2) and
// 2 (w % 2) + 1 of the step.
struct NarrowE {
  uint32_t off;
  int kb0;  // first key block of this wave within a step
  __device__ __forceinline__ void init(int EB, int wave, int lane) {
    off = (uint32_t)(wave >> 1) * (uint32_t)EB * 1024u + (uint32_t)lane * 16u;
    kb0 = 2 * (wave & 1);
  }
  __device__ __forceinline__ void issue(const u32x4& r, int k0, char* stage, int wave, int j) const {
    load16_to_lds_untracked(r, stage + (wave * 2 + j) * 1024,
                            off + (uint32_t)((k0 >> 4) + kb0 + j) * 1024u);
  }
};

struct NarrowFrags {
  bf16x8 a, b[2];
};

// 8 waves, two per SIMD: wave w owns channels [32 (w % 4), +32) x queries
// [64 (w / 4), +64) of the tile, as 1 x 2 accumulator blocks.  Per k16
// sub-step it reads one V^T fragment (two transpose reads) and two E
// fragments for 2 MFMAs, two sub-steps ahead (one sub-step's 128 cycles of
// MFMAs per SIMD do not cover an LDS read).  Step kt (64 keys, four
// sub-steps): the loads of step kt + 3 go out one per MFMA in the first two
// sub-steps, whose reads finish the stage; the wave then waits for its loads
// of step kt + 1 and meets the others at the barrier, and runs the last two
// sub-steps' MFMAs while it reads the first two of step kt + 1.
__global__ __launch_bounds__(64 * kValuesWaves) void values_narrow_kernel(
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ E, const float* __restrict__ mref,
    const float* __restrict__ psum, uint16_t* __restrict__ out, float* __restrict__ lse,
    HeadMap hm, int L, int d, int T2, int TK, int QB, int EB, int Lk, Band band, int ncb2) {
  __shared__ NarrowSmem sm;

  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int per_head = T2 * ncb2;
  const int bh = lid / per_head;
  const int r = lid % per_head;
  const int qt = r / ncb2, ct = r % ncb2;  // a query tile's channel tiles are neighbours (one XCD)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cq = wave & 3, qh = wave >> 2, c32 = lane & 31, h = lane >> 5;

  // Score tiles [tlo, thi] (128 keys each) meet this query tile's band: keys
  // [kbeg, kend), a whole number of steps (Lk is a multiple of 64), at least
  // one (the tile holds a query below L, whose band keeps its diagonal).
  int tlo, thi;
  band_tiles(band, qt, kNT, TK, kSK, &tlo, &thi);
  const int kbeg = tlo * kSK, kend = min(Lk, (thi + 1) * kSK);
  const int nk = (kend - kbeg) / kNK;
  const int k_first = kbeg / kNK;

  const int ldv = hm.v.ld;
  const u32x4 rv = rsrc_words(v + hm.v_off(bh), ((uint32_t)(L - 1) * ldv + d) * 2u);
  const u32x4 re = rsrc_words(E + ((size_t)bh * QB + (size_t)qt * 4) * EB * 512,
                              (uint32_t)(QB - qt * 4) * (uint32_t)EB * 1024u);
  NarrowV la;
  NarrowE lb;
  la.init((uint32_t)ldv, ct * kNT, wave, lane);
  lb.init(EB, wave, lane);
  // Load j (0..3) of step u; steps past the last reload the last.
  auto issue = [&](int u, int j) {
    const int k0 = kbeg + min(u, nk - 1) * kNK;
    if (j < 2)
      la.issue(rv, k0, sm.v[u & 3], wave, j);
    else
      lb.issue(re, k0, sm.e[u & 3], wave, j - 2);
  };
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) issue(u, j);

  // Thread tid < 128 owns query qt*128 + tid.
  if (tid < kNT)
    values_stats<kNT>(mref, psum, lse, ct == 0, bh, hm.bh0, TK, L, qt * kNT, tlo, thi,
                      sm.shift_tab, sm.inv_l, tid);
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  block_sync();

  PowerOfTwoShift<2> sh;
  float invl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    sh.col[j] = qh * 64 + j * 32 + c32;
    invl[j] = sm.inv_l[sh.col[j]];
  }
  KOuterT<kNT * 2> ka;
  auto read = [&](NarrowFrags& f, int st, int ss) {
    f.a = ka.frag(sm.v[st], cq * 32, ss, lane);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      f.b[j] = *(const bf16x8*)(sm.e[st] + ((qh * 2 + j) * 4 + ss) * 1024 + lane * 16);
  };
  // E fragments are scaled once read (the empty asm keeps the compiler from
  // sinking the scaling to their first use after the barrier).
  auto scale = [&](NarrowFrags& f) {
    f.b[0] = sh(f.b[0], 0);
    f.b[1] = sh(f.b[1], 1);
    asm volatile("" : "+v"(f.b[0]), "+v"(f.b[1]));
  };

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  // A wave whose 64 queries all lie past L only issues its loads and meets
  // the barriers.
  if (__builtin_amdgcn_readfirstlane((int)(qt * kNT + qh * 64 >= L))) {
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int p = 0; p < 4; ++p) issue(kt + 3, p);
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      block_sync();
    }
  } else {
    // f0: this sub-step's fragments (scaled), f1: the next (read, to be
    // scaled), f2: the one after (being read).
    NarrowFrags f0, f1, f2;
    auto mfmas = [&](const NarrowFrags& f, int kt, int ss) {
      __builtin_amdgcn_sched_barrier(0);
      acc[0] = mfma32x32x16(f.a, f.b[0], acc[0]);
      if (ss < 2) issue(kt + 3, 2 * ss);
      acc[1] = mfma32x32x16(f.a, f.b[1], acc[1]);
      if (ss < 2) issue(kt + 3, 2 * ss + 1);
      __builtin_amdgcn_sched_barrier(0);
    };
    {
      unsigned s0[2];
      sh.load(sm.shift_tab, k_first >> 1, s0);
      sh.set(s0);
    }
    read(f0, 0, 0);
    read(f1, 0, 1);
    scale(f0);
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 3;
      unsigned sn[2];  // shifts of step kt + 1 (past the end: unused)
      sh.load(sm.shift_tab, min((k_first + kt + 1) >> 1, thi), sn);
      // Sub-steps 0 and 1, each with two loads of step kt + 3.
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        read(f2, st, ss + 2);
        mfmas(f0, kt, ss);
        scale(f1);
        f0 = f1;
        f1 = f2;
      }
      // Step kt + 1 staged everywhere (steps kt + 2 and kt + 3 may be in
      // flight); every read of stage st issued (and done at the barrier).
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      block_sync();
      // Sub-steps 2 and 3, reading the first two of step kt + 1.
      read(f2, (kt + 1) & 3, 0);
      mfmas(f0, kt, 2);
      scale(f1);  // sub-step 3: this step's shifts
      sh.set(sn);
      f0 = f1;
      f1 = f2;
      read(f2, (kt + 1) & 3, 1);
      mfmas(f0, kt, 3);
      scale(f1);  // step kt + 1, sub-step 0
      f0 = f1;
      f1 = f2;
    }
  }
  // No load in flight into the stages (the O tile below reuses them).
  wait_vmem();
  block_sync();

  // O[query][ch] = acc / l, rounded once to bf16, staged as [query][128
  // channels] rows of 256 bytes (chunk c of row r at c ^ (r % 16), 8-byte
  // halves swapped when r % 32 >= 16) so that the stores write whole rows.
  static_assert(offsetof(NarrowSmem, e) == kNStages * kNStageBytes &&
                    kNStages * kNStageBytes >= kNT * kNT * 2,
                "the O tile fits the V stages");
  char* stage = sm.v[0];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ql = qh * 64 + j * 32 + c32;
    char* row = stage + ql * 256 + 8 * (h ^ (c32 >> 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x16& a = acc[j];
      const u32x2 w = {pack_bf16x2(a[4 * i] * invl[j], a[4 * i + 1] * invl[j]),
                       pack_bf16x2(a[4 * i + 2] * invl[j], a[4 * i + 3] * invl[j])};
      const int chunk = cq * 4 + i;
      *(u32x2*)(row + ((chunk ^ (c32 & 15)) << 4)) = w;
    }
  }
  __syncthreads();
  {
    const int c = tid & 15;
    const int ch = ct * kNT + 8 * c;
    if (ch < d) {
      const int ldo = hm.o.ld;
      uint16_t* oh = out + hm.o_off(bh) + (size_t)(qt * kNT) * ldo + ch;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = (tid >> 4) + 32 * j;
        if (qt * kNT + rr < L)
          *(u32x4*)(oh + (size_t)rr * ldo) =
              unswap_halves(*(const u32x4*)(stage + rr * 256 + ((c ^ (rr & 15)) << 4)), rr);
      }
    }
  }
}

// out = bf16(sum over the splits of part), 8 elements per thread.  part is
// [split][head][L][d] contiguous; out is addressed through the head map.
__global__ __launch_bounds__(256) void values_reduce_kernel(const float* __restrict__ part,
                                                            uint16_t* __restrict__ out, HeadMap hm,
                                                            int L, int d, int64_t n8,
                                                            int64_t stride, int split) {
  const int c8n = d / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const f32x4* p = (const f32x4*)part + 2 * i;
    f32x4 lo = p[0], hi = p[1];
    for (int s = 1; s < split; ++s) {
      lo += p[(size_t)s * (stride / 4)];
      hi += p[(size_t)s * (stride / 4) + 1];
    }
    const u32x4 w = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                     pack_bf16x2(hi[2], hi[3])};
    const int64_t row_all = i / c8n;  // head * L + row
    const int c8 = (int)(i - row_all * c8n);
    const int bh = (int)(row_all / L), row = (int)(row_all - (int64_t)bh * L);
    *(u32x4*)(out + hm.o_off(bh) + (size_t)row * hm.o.ld + 8 * c8) = w;
  }
}

}  // namespace

// Compute units of the current device (cached per device).
static int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Score tiles of one head: the key tiles each query tile's band meets.
int band_tiles_per_head(const Band& band, int T) {
  int n = 0;
  for (int qt = 0; qt < T; ++qt) {
    int lo, hi;
    band_tiles(band, qt, kTile, T, kTile, &lo, &hi);
    n += hi - lo + 1;
  }
  return n;
}

hipError_t launch_scores(const void* q, const void* k, void* E, float* mref, float* psum,
                         const HeadMap& hm, int BH, const TwoPassDims& t, float sl2,
                         const Band& band, hipStream_t s) {
  const uint16_t* qp = (const uint16_t*)q;
  const uint16_t* kp = (const uint16_t*)k;
  uint16_t* ep = (uint16_t*)E;
  int L = t.L, d = t.d, T = t.T, TK = t.TK, QB = t.QB, EB = t.EB;
  int per_head = band_tiles_per_head(band, T);
  int ntiles = BH * per_head;
  const int grid = std::min(ntiles, device_cu_count());  // one workgroup per CU (LDS-bound)
  HeadMap m = hm;
  Band b = band;
  void* args[] = {&qp, &kp, &ep, &mref, &psum, &m, &L, &d, &T, &TK, &QB, &EB, &sl2, &b, &per_head,
                  &ntiles};
  return hipLaunchKernel((const void*)&scores_kernel, dim3((unsigned)grid),
                         dim3(64 * kScoresWaves), args, 0, s);
}

bool values_narrow(int64_t BH, const TwoPassDims& t) {
  const int64_t wide = BH * t.T * ((t.d + kTile - 1) / kTile);
  const int64_t narrow = BH * ((t.L + kNT - 1) / kNT) * ((t.d + kNT - 1) / kNT);
  return wide * 2 <= kValuesTargetWorkgroups && narrow <= kValuesTargetWorkgroups;
}

int values_split(int64_t BH, const TwoPassDims& t, const Band& band) {
  const int64_t base = BH * t.T * ((t.d + kTile - 1) / kTile);  // workgroups without a split
  if (base * 2 > kValuesTargetWorkgroups || values_narrow(BH, t)) return 1;
  int64_t fewest = t.Lk / kStepK;  // K steps of the narrowest query tile's band
  for (int qt = 0; qt < t.T; ++qt) {
    int lo, hi;
    band_tiles(band, qt, kTile, t.TK, kSK, &lo, &hi);
    fewest = std::min<int64_t>(fewest, (std::min(t.Lk, (hi + 1) * kSK) - lo * kSK) / kStepK);
  }
  // Each split keeps at least kValuesMinSplitSteps K steps: shorter loops are
  // dominated by the fixed cost of a workgroup, and the partials cost a pass.
  int64_t s = std::min<int64_t>(kValuesTargetWorkgroups / base, kValuesMaxSplit);
  s = std::min(s, fewest / kValuesMinSplitSteps);
  return s >= 2 ? (int)s : 1;
}

hipError_t launch_values(const void* v, const void* E, const float* mref, const float* psum,
                         void* out, float* lse, float* part, int split, const HeadMap& hm, int BH,
                         const TwoPassDims& t, const Band& band, hipStream_t s) {
  const uint16_t* vtp = (const uint16_t*)v;
  const uint16_t* ep = (const uint16_t*)E;
  uint16_t* op = (uint16_t*)out;
  int L = t.L, d = t.d, T = t.T, TK = t.TK, QB = t.QB, EB = t.EB, Lk = t.Lk;
  int ncb = (t.d + kTile - 1) / kTile;
  int nheads = BH;
  HeadMap m = hm;
  Band b = band;
  void* args[] = {&vtp, &ep, &mref, &psum, &op, &lse, &part, &m, &L, &d, &T, &TK, &QB, &EB, &Lk, &b,
                  &ncb, &split, &nheads};
  if (split == 1 && values_narrow(BH, t)) {
    int T2 = (t.L + kNT - 1) / kNT, ncb2 = (t.d + kNT - 1) / kNT;
    void* nargs[] = {&vtp, &ep, &mref, &psum, &op, &lse, &m, &L, &d, &T2, &TK, &QB, &EB, &Lk, &b,
                     &ncb2};
    return hipLaunchKernel((const void*)&values_narrow_kernel, dim3((unsigned)(BH * T2 * ncb2)),
                           dim3(64 * kValuesWaves), nargs, 0, s);
  }
  const void* kern = split > 1 ? (const void*)&values_kernel<true> : (const void*)&values_kernel<false>;
  return hipLaunchKernel(kern, dim3((unsigned)(BH * T * ncb * split)), dim3(64 * kValuesWaves), args,
                         0, s);
}

hipError_t launch_values_reduce(const float* part, void* out, int split, const HeadMap& hm,
                                int BH, const TwoPassDims& t, hipStream_t s) {
  int64_t stride = (int64_t)BH * t.L * t.d;  // floats per split
  int64_t n8 = stride / 8;                   // d is a multiple of 64
  const int blocks = (int)std::min<int64_t>((n8 + 255) / 256, 2048);
  uint16_t* op = (uint16_t*)out;
  HeadMap m = hm;
  int L = t.L, d = t.d;
  void* args[] = {&part, &op, &m, &L, &d, &n8, &stride, &split};
  return hipLaunchKernel((const void*)&values_reduce_kernel, dim3((unsigned)blocks), dim3(256),
                         args, 0, s);
}

}  // namespace attn
