// internal.h -- launchers the C ABI dispatches to (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Sizes of the two-pass path's per-head staging, all in elements.
struct TwoPassDims {
  int L;   // sequence length
  int d;   // head dimension
  int T;   // number of 256-key score tiles: ceil(L / 256)
  int Ls;  // row stride of E: 256 T + 128 (an odd multiple of 256 bytes, which
           // spreads a tile's rows over the memory channels)
  int Lk;  // keys the values pass iterates over: ceil(L / 64) * 64 (<= Ls)
};

TwoPassDims two_pass_dims(int64_t L, int64_t d);

// The values pass keeps one byte per (score tile, query) of its query tile in
// LDS next to the 128 KB GEMM stages, which caps L at 124 * 256 = 31744 there.
constexpr int kTwoPassMaxTiles = 124;

// Bytes of workspace one head needs on the two-pass path: E and the
// per-(tile, query) exponent reference and partial sum.
int64_t two_pass_head_bytes(const TwoPassDims& t);

// Fused online-softmax kernel, d in {32, 64, 128}.  sl2 = scale * log2(e).
hipError_t launch_online(const void* q, const void* k, const void* v, void* out, int BH, int L,
                         int d, float sl2, bool causal, hipStream_t s);

// Scores pass: per 256x256 (key, query) tile, E = bf16(2^(y - m)) with
// y = sl2 * q.k, m = ceil(max over the tile's keys of y) per query, plus m and
// the sum of the stored E per (tile, query).
hipError_t launch_scores(const void* q, const void* k, void* E, float* mref, float* psum, int BH,
                         const TwoPassDims& t, float sl2, bool causal, hipStream_t s);

// Values pass: O = (sum over tiles of 2^(m_t - M) E_t V_t) / (sum_t 2^(m_t - M) psum_t).
// With split > 1 the keys of each query tile are divided among `split`
// workgroups, each writing its share of O in fp32 to part[split][BH][L][d];
// launch_values_reduce then sums the shares into bf16 `out`.
constexpr int kValuesTargetWorkgroups = 256;  // MI355X compute units
constexpr int kValuesMaxSplit = 4;
constexpr int kValuesMinSplitSteps = 8;  // K steps (64 keys each) per split at least
// Splits used for BH heads: 1 unless the unsplit grid would leave at least half
// of the compute units idle.  Depends on the shape only.
int values_split(int64_t BH, const TwoPassDims& t, bool causal);
hipError_t launch_values(const void* v, const void* E, const float* mref, const float* psum,
                         void* out, float* part, int split, int BH, const TwoPassDims& t,
                         bool causal, hipStream_t s);
hipError_t launch_values_reduce(const float* part, void* out, int split, int BH,
                                const TwoPassDims& t, hipStream_t s);

}  // namespace attn
