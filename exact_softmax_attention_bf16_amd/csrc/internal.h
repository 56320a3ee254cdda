// internal.h -- launchers the C ABI dispatches to (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Element strides of one bf16 operand viewed as [B, heads, L, d] with
// contiguous channels: rows of a head are `ld` elements apart.
struct Strides {
  int64_t b, h;  // batch and head strides
  int ld;        // row stride, >= d, a multiple of 8 (16-byte rows)
};

// Where the heads of one launch live.  Launch head i is global head
// bh = bh0 + i = b * H + h; query head h reads key/value head h / group.
struct HeadMap {
  int H;      // query heads per batch entry
  int group;  // query heads per key/value head
  int bh0;    // global index of the launch's first head
  Strides q, k, v, o;

  __host__ __device__ int64_t q_off(int i) const { return off(q, i, 1); }
  __host__ __device__ int64_t k_off(int i) const { return off(k, i, group); }
  __host__ __device__ int64_t v_off(int i) const { return off(v, i, group); }
  __host__ __device__ int64_t o_off(int i) const { return off(o, i, 1); }
  __host__ __device__ int64_t off(const Strides& s, int i, int g) const {
    const int bh = bh0 + i, b = bh / H, h = bh - b * H;
    return (int64_t)b * s.b + (int64_t)(h / g) * s.h;
  }
};

// Contiguous [B, H, L, d] operands, H query and key/value heads.
inline HeadMap contiguous_heads(int H, int L, int d) {
  const Strides s{(int64_t)H * L * d, (int64_t)L * d, d};
  return HeadMap{H, 1, 0, s, s, s, s};
}

// True when the map is contiguous_heads(H, L, d): head bh of every operand
// starts at bh * L * d.
inline bool is_plain(const HeadMap& m, int L, int d) {
  auto dense = [&](const Strides& s) {
    return s.ld == d && s.h == (int64_t)L * d && s.b == (int64_t)m.H * L * d;
  };
  return m.group == 1 && dense(m.q) && dense(m.k) && dense(m.v) && dense(m.o);
}

// Keys each query sees: key j is allowed for query i iff
// i - left <= j <= i + right (and j < L).  An unbounded side holds kNoLimit;
// causal attention is {kNoLimit, 0}.
// compressed != 0 selects the compressed causal mask instead (token-packed
// sequences only): with cf = max(1, Lq / Lk), key j is allowed for query i iff
// j <= (i + 1) / cf - 1, positions counted from 0 within the sequence.
constexpr int kNoLimit = 1 << 30;
struct Band {
  int left, right;
  int compressed;
};
inline Band make_band(int64_t left, int64_t right, bool causal, int64_t L) {
  Band b;
  b.left = (left < 0 || left >= L) ? kNoLimit : (int)left;
  b.right = (right < 0 || right >= L) ? kNoLimit : (int)right;
  if (causal) b.right = 0;
  b.compressed = 0;
  return b;
}
__host__ __device__ inline bool band_is_full(const Band& b) {
  return b.left >= kNoLimit && b.right >= kNoLimit;
}
__host__ __device__ inline bool band_is_causal(const Band& b) {
  return b.left >= kNoLimit && b.right == 0;
}
// Key tiles (`ktile` keys each, TK of them) that the queries
// [qt * qtile, qt * qtile + qtile) meet: [*lo, *hi] within [0, TK).
__host__ __device__ inline void band_tiles(const Band& b, int qt, int qtile, int TK, int ktile,
                                           int* lo, int* hi) {
  const int first_key = qt * qtile - b.left;  // the tile's first query, leftmost key
  *lo = (b.left >= kNoLimit || first_key <= 0) ? 0 : first_key / ktile;
  const int64_t last_key = (int64_t)qt * qtile + qtile - 1 + b.right;
  *hi = (b.right >= kNoLimit || last_key >= (int64_t)TK * ktile) ? TK - 1 : (int)(last_key / ktile);
  if (*hi < *lo) *hi = *lo - 1;  // no key tile (cannot happen for bands that keep the diagonal)
}

// Sizes of the two-pass path's per-head staging, all in elements.
struct TwoPassDims {
  int L;   // sequence length
  int d;   // head dimension
  int T;   // number of 256-query tiles: ceil(L / 256)
  int TK;  // number of 128-key score tiles (the statistics' granularity): ceil(L / 128)
  int QB;  // 32-query blocks of E: ceil(L / 32)
  int EB;  // 16-key blocks of E per query block: 16 T (keys padded to 256 T)
  int Lk;  // keys the values pass iterates over: ceil(L / 64) * 64 (<= 256 T)
};
// E, the bf16 exponentials, is stored in 1 KB blocks of 32 queries x 16 keys:
// block (qb, kb) of a head holds, at element 8 * lane, keys 16 kb + 8 (lane / 32)
// .. + 8 (in the scores pass's key order) of query 32 qb + lane % 32 -- the 16
// bytes one lane of a register-direct store holds, and the 16 bytes one lane
// of the values pass's MFMA operand needs.  Blocks are ordered [qb][kb].

TwoPassDims two_pass_dims(int64_t L, int64_t d);

// The values pass keeps one byte per (128-key score tile, query) of its query
// tile in LDS next to the 128 KB GEMM stages, which caps L at 124 * 128 = 15872.
constexpr int kTwoPassMaxTiles = 124;

// Bytes of workspace one head needs on the two-pass path: E and the
// per-(128-key tile, query) exponent reference and partial sum.
int64_t two_pass_head_bytes(const TwoPassDims& t);

// A split of each query block's keys among n workgroups (n > 1): share s of
// head h writes its unnormalised O to part[s][h][L][d] and its (m, l) to
// stats[s][h][L][2] (fp32); the combine kernel merges the shares.
struct KeySplit {
  float* part;
  float* stats;
  int n;      // shares per query block (<= 1: no split)
  int heads;  // heads of the launch
};
constexpr int kOnlineMaxSplit = 8;

// Sequences of different lengths packed along the tokens (cu_q null: none).
// Sequence b holds query tokens [cu_q[b], cu_q[b + 1]) and key/value tokens
// [cu_k[b], cu_k[b + 1]) (cu_k null: the query offsets), clamped to
// [0, total_q] / [0, total_k] and to L / max_k tokens.
struct VarSeqs {
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  int max_k;
};

// Fused online-softmax kernel, d in {32, 64, 128}.  sl2 = scale * log2(e).
// lse (may be null): fp32 [global head][L], the natural log of each row's
// softmax denominator.  With vs.cu_q non-null the heads are the sequences of
// vs (L: the longest query length), rows hm.*.ld and heads hm.*.h elements
// apart, and lse is [total_q][H]; query i of a sequence stands at key
// position i + Lk - Lq for the band.
// With ks.n > 1 it writes the shares ([split][head][L] rows, L the longest
// query length) instead of out and lse, and launch_online_combine finishes the
// call.
hipError_t launch_online(const void* q, const void* k, const void* v, void* out, float* lse,
                         const HeadMap& hm, int BH, int L, int d, float sl2, const Band& band,
                         const VarSeqs& vs, const KeySplit& ks, hipStream_t s);
hipError_t launch_online_combine(const KeySplit& ks, void* out, float* lse, const HeadMap& hm,
                                 int L, int d, const VarSeqs& vs, hipStream_t s);
// Shares per query block for BH heads of (longest) query length Lq and key
// length Lk: 1 unless the unsplit grid would leave at least half of the
// compute units idle.  Shape only.
int online_split(int64_t BH, int64_t Lq, int64_t Lk);

// Scores pass: per 128-key x 256-query tile, E = bf16(2^(y - m)) with
// y = sl2 * q.k, m = ceil(max over the tile's keys of y) per query, plus m and
// the sum of the stored E per (tile, query).
hipError_t launch_scores(const void* q, const void* k, void* E, float* mref, float* psum,
                         const HeadMap& hm, int BH, const TwoPassDims& t, float sl2,
                         const Band& band, hipStream_t s);

// Values pass: O = (sum over tiles of 2^(m_t - M) E_t V_t) / (sum_t 2^(m_t - M) psum_t).
// With split > 1 the keys of each query tile are divided among `split`
// workgroups, each writing its share of O in fp32 to part[split][BH][L][d];
// launch_values_reduce then sums the shares into bf16 `out`.
constexpr int kValuesTargetWorkgroups = 256;  // MI355X compute units
constexpr int kValuesMaxSplit = 4;
constexpr int kValuesMinSplitSteps = 8;  // K steps (64 keys each) per split at least
// Whether the values pass runs on 128 x 128 tiles (no split): when the
// 256 x 256 grid would leave at least half of the compute units idle and the
// narrow grid fits on them in one round.  Depends on the shape only.
bool values_narrow(int64_t BH, const TwoPassDims& t);
// Splits used for BH heads: 1 unless the unsplit grid would leave at least half
// of the compute units idle and the narrow tiles do not apply.  Depends on the
// shape only.
int values_split(int64_t BH, const TwoPassDims& t, const Band& band);
// lse as for launch_online.
hipError_t launch_values(const void* v, const void* E, const float* mref, const float* psum,
                         void* out, float* lse, float* part, int split, const HeadMap& hm, int BH,
                         const TwoPassDims& t, const Band& band, hipStream_t s);
hipError_t launch_values_reduce(const float* part, void* out, int split, const HeadMap& hm,
                                int BH, const TwoPassDims& t, hipStream_t s);

}  // namespace attn
