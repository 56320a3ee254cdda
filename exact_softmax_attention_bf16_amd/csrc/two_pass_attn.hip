// two_pass_attn.hip -- exact attention for large head dims (128 < d <= 1024).
//
// The pages' design for the Wan2.2 mid-block attention (FastVideo
// wan22_vae_decode attn.cu, header comment: S = q k^T with fp32 accumulation,
// a row softmax, then O = p v) materialises S in fp32 and P in bf16.  On
// MI355X the per-frame O tile (rows x 1024 fp32) does not fit a CU's register
// file next to a useful query block, so the path stays two-pass like the
// pages', but moves the softmax into the two GEMMs:
//
//   scores pass  for each 256-key x 256-query tile t of S^T = K Q^T (fp32):
//                y = scale*log2(e) * s; per query m_t = ceil(max_keys y) (an
//                integer); E = bf16(2^(y - m_t)); store E, m_t and
//                psum_t = sum of the stored E over the tile's keys.
//   values pass  per query M = max_t m_t, l = sum_t 2^(m_t - M) psum_t, and
//                O = (sum_t 2^(m_t - M) E_t V_t) / l, with the factor applied
//                to E exactly: m_t - M is an integer, so scaling bf16 E by it
//                is a saturating subtract on the exponent bits.
//
// So S never leaves the registers in fp32, E is written once in bf16 (the
// pages' P rounding point), the normaliser sums exactly the values the second
// contraction uses, and there is no extra pass over S or P.  The subtraction of
// a per-tile reference before the exponential is the stable softmax of the
// attn.cu row_softmax_kernel and of the FMHA example's softmax_step; the
// rescale by 2^(m_t - M) is that example's correction step, done once per
// tile with exact factors.
#include "device.h"
#include "gemm_core.h"
#include "internal.h"

namespace attn {

TwoPassDims two_pass_dims(int64_t L, int64_t d) {
  TwoPassDims t;
  t.L = (int)L;
  t.d = (int)d;
  t.T = (int)((L + kTile - 1) / kTile);
  t.Ls = t.T * kTile;
  t.Lk = (int)((L + 63) / 64 * 64);
  return t;
}

static int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

int64_t two_pass_head_bytes(const TwoPassDims& t) {
  return round256((int64_t)t.L * t.Ls * 2) + round256((int64_t)t.d * t.Lk * 2) +
         2 * round256((int64_t)t.T * t.L * 4);
}

namespace {

// ---------------------------------------------------------------------------
// V [BH, L, d] -> V^T [BH, d, Lk] through a 64x64 LDS tile; keys >= L read as 0.
__global__ __launch_bounds__(256) void v_transpose_kernel(const uint16_t* __restrict__ v,
                                                          uint16_t* __restrict__ vt, int L, int d,
                                                          int Lk, int nkb, int ncb) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int tid = threadIdx.x;
  const int per_head = nkb * ncb;
  const int bh = blockIdx.x / per_head;
  const int r = blockIdx.x % per_head;
  const int kb = r / ncb, cb = r % ncb;
  const auto rv = make_rsrc(v + (size_t)bh * L * d, (uint32_t)L * d * 2);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 3, col8 = c & 7;
    const u32x4 x = load16(rv, (uint32_t)((kb * 64 + row) * d + cb * 64 + col8 * 8) * 2);
    *(u32x4*)&tile[row][col8 * 8] = x;
  }
  __syncthreads();
  uint16_t* dst = vt + (size_t)bh * d * Lk;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    const int ch = c >> 3, g = c & 7;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (unsigned)tile[8 * g + 2 * e][ch] | ((unsigned)tile[8 * g + 2 * e + 1][ch] << 16);
    *(u32x4*)(dst + (size_t)(cb * 64 + ch) * Lk + kb * 64 + 8 * g) = w;
  }
}

// ---------------------------------------------------------------------------
// Scores pass.  Tile (kt, qt) of head bh: keys [256 kt, +256) on the M side,
// queries [256 qt, +256) on the N side, so each lane of the accumulator owns a
// query and holds 4 runs of 4 consecutive keys per 32x32 block.
__global__ __launch_bounds__(256) void scores_kernel(const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k,
                                                     uint16_t* __restrict__ E,
                                                     float* __restrict__ mref,
                                                     float* __restrict__ psum, int L, int d, int T,
                                                     int Ls, float sl2, int causal) {
  __shared__ GemmSmem sm;
  __shared__ float red[2][kTile];

  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int per_head = T * T;
  const int bh = lid / per_head;
  const int r = lid % per_head;
  const int qt = r / T, kt = r % T;
  if (causal && kt > qt) return;  // every key after every query of the tile

  const uint32_t head_bytes = (uint32_t)L * d * 2;
  const auto rq = make_rsrc(q + (size_t)bh * L * d, head_bytes);
  const auto rk = make_rsrc(k + (size_t)bh * L * d, head_bytes);

  f32x16 acc[4][4];
  NoTransform nx;
  gemm_tile(acc, rk, (uint32_t)d, kt * kTile, rq, (uint32_t)d, qt * kTile, d / kStepK, sm, nx);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, c32 = lane & 31, h = lane >> 5;
  const int key0 = kt * kTile + wm * 128;

  // Per-query maximum of y = sl2 * s over this wave's 128 keys.  Interior tiles
  // (no key past L, no key after a query) take it on the raw accumulator; edge
  // tiles scale and mask each element.  The accumulator is only read here.
  const bool need_mask = (kt + 1) * kTile > L || (causal && kt >= qt);
  auto masked = [&](int bi, int bj, int j) {
    const int key = key0 + bi * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
    const int query = qt * kTile + wn * 128 + bj * 32 + c32;
    return key >= L || (causal && key > query);
  };
  float wmax[4];
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    float mx = -INFINITY;
    if (!need_mask) {
      float hi = -INFINITY, lo = INFINITY;
      if (sl2 >= 0.f) {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
          for (int j = 0; j < 16; ++j) hi = fmaxf(hi, acc[bi][bj][j]);
        mx = hi * sl2;
      } else {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
          for (int j = 0; j < 16; ++j) lo = fminf(lo, acc[bi][bj][j]);
        mx = lo * sl2;
      }
    } else {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          mx = fmaxf(mx, masked(bi, bj, j) ? -INFINITY : acc[bi][bj][j] * sl2);
    }
    wmax[bj] = wave_swap32_max(mx);
  }
#pragma unroll
  for (int bj = 0; bj < 4; ++bj)
    if (h == 0) red[wm][wn * 128 + bj * 32 + c32] = wmax[bj];
  __syncthreads();

  // E = bf16(2^(y - m)) with m = ceil(tile max of y): at most 1, at least 1/2 at the max.
  float mt[4], ps[4];
  uint16_t* Eh = E + (size_t)bh * L * Ls;
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    const int ql = wn * 128 + bj * 32 + c32;
    const int query = qt * kTile + ql;
    const float tmax = fmaxf(red[0][ql], red[1][ql]);
    const float m2 = tmax == -INFINITY ? -INFINITY : ceilf(tmax);
    const float add = tmax == -INFINITY ? 0.f : -m2;
    float s = 0.f;
    uint16_t* erow = Eh + (size_t)query * Ls + key0 + 4 * h;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = exp2_fast(fmaf(acc[bi][bj][4 * i + r], sl2, add));
          if (need_mask && masked(bi, bj, 4 * i + r)) e[r] = 0.f;
        }
        const unsigned w0 = pack_bf16x2(e[0], e[1]);
        const unsigned w1 = pack_bf16x2(e[2], e[3]);
        s += (bf16_lo(w0) + bf16_hi(w0)) + (bf16_lo(w1) + bf16_hi(w1));
        if (query < L) *(u32x2*)(erow + bi * 32 + 8 * i) = u32x2{w0, w1};
      }
    }
    mt[bj] = m2;
    ps[bj] = wave_swap32_sum(s);
  }
  __syncthreads();
  if (h == 0) {
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) red[wm][wn * 128 + bj * 32 + c32] = ps[bj];
  }
  __syncthreads();
  if (wm == 0 && h == 0) {
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int ql = wn * 128 + bj * 32 + c32;
      const int query = qt * kTile + ql;
      if (query < L) {
        const size_t at = ((size_t)bh * T + kt) * L + query;
        mref[at] = mt[bj];
        psum[at] = red[0][ql] + red[1][ql];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Values pass.  Tile (ct, qt): channels [256 ct, +256) on the M side (A = V^T),
// queries [256 qt, +256) on the N side (B = E), K = keys in 64-wide steps.
// Each lane owns four queries (one per 32-column block j); before each group
// of four steps (one 256-key score tile t) it turns M - m_t into the exponent
// shift for those queries, fetched one tile ahead.
constexpr int kMaxTiles = kTwoPassMaxTiles;

struct PowerOfTwoShift {
  const uint8_t (*tab)[kTile];  // [t][query in tile]: M - m_t, capped at 255
  int col[4];                   // this lane's four query columns in the tile
  unsigned sw[4];               // current shift words (s << 7 | s << 23)

  __device__ __forceinline__ void step(int kt) {
    if ((kt & 3) == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned s = tab[kt >> 2][col[j]];
        sw[j] = (s << 7) | (s << 23);
      }
    }
  }
  __device__ __forceinline__ bf16x8 operator()(bf16x8 f, int j) const {
    u32x4 w = __builtin_bit_cast(u32x4, f);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = scale_pow2_down(w[e], sw[j]);
    return __builtin_bit_cast(bf16x8, w);
  }
};

__global__ __launch_bounds__(256) void values_kernel(const uint16_t* __restrict__ vt,
                                                     const uint16_t* __restrict__ E,
                                                     const float* __restrict__ mref,
                                                     const float* __restrict__ psum,
                                                     uint16_t* __restrict__ out, int L, int d,
                                                     int T, int Ls, int Lk, int causal, int ncb) {
  __shared__ GemmSmem sm;
  __shared__ uint8_t shift_tab[kMaxTiles][kTile];
  __shared__ float inv_l[kTile];

  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int per_head = T * ncb;
  const int bh = lid / per_head;
  const int r = lid % per_head;
  const int qt = r / ncb, ct = r % ncb;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, c32 = lane & 31, h = lane >> 5;

  const int tiles = causal ? qt + 1 : T;
  const int kend = causal ? min(Lk, (qt + 1) * kTile) : Lk;
  const int nk = kend / kStepK;

  // Thread tid owns query qt*256 + tid: M = max_t m_t, l = sum_t 2^(m_t - M) psum_t,
  // and the shift M - m_t of each tile (a nonnegative integer; -inf tiles -> 255).
  {
    const float* mh = mref + (size_t)bh * T * L;
    const float* ph = psum + (size_t)bh * T * L;
    const int qc = min(qt * kTile + tid, L - 1);
    float M = -INFINITY;
    for (int t = 0; t < tiles; ++t) M = fmaxf(M, mh[(size_t)t * L + qc]);
    float l = 0.f;
    for (int t = 0; t < tiles; ++t) {
      const float mt = mh[(size_t)t * L + qc];
      l += ph[(size_t)t * L + qc] * exp2_fast(mt - M);
      shift_tab[t][tid] = (uint8_t)fminf(M - mt, 255.f);
    }
    inv_l[tid] = 1.f / l;
  }
  __syncthreads();

  PowerOfTwoShift sh;
  sh.tab = shift_tab;
  float invl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sh.col[j] = wn * 128 + j * 32 + c32;
    invl[j] = inv_l[sh.col[j]];
  }

  const auto ra = make_rsrc(vt + (size_t)bh * d * Lk, (uint32_t)d * Lk * 2);
  const auto rb = make_rsrc(E + (size_t)bh * L * Ls, (uint32_t)L * Ls * 2);
  f32x16 acc[4][4];
  gemm_tile(acc, ra, (uint32_t)Lk, ct * kTile, rb, (uint32_t)Ls, qt * kTile, nk, sm, sh);

  // O[query][ch] = acc / l, rounded once to bf16; lane holds 4 consecutive channels per run.
  uint16_t* oh = out + (size_t)bh * L * d;
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    const int query = qt * kTile + wn * 128 + bj * 32 + c32;
    if (query >= L) continue;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = ct * kTile + wm * 128 + bi * 32 + 8 * i + 4 * h;
        if (ch < d) {
          const f32x16& a = acc[bi][bj];
          u32x2 w = {pack_bf16x2(a[4 * i] * invl[bj], a[4 * i + 1] * invl[bj]),
                     pack_bf16x2(a[4 * i + 2] * invl[bj], a[4 * i + 3] * invl[bj])};
          *(u32x2*)(oh + (size_t)query * d + ch) = w;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_v_transpose(const void* v, void* vt, int BH, const TwoPassDims& t,
                              hipStream_t s) {
  const int nkb = t.Lk / 64, ncb = t.d / 64;
  const uint16_t* vp = (const uint16_t*)v;
  uint16_t* vtp = (uint16_t*)vt;
  int L = t.L, d = t.d, Lk = t.Lk;
  void* args[] = {&vp, &vtp, &L, &d, &Lk, (void*)&nkb, (void*)&ncb};
  return hipLaunchKernel((const void*)&v_transpose_kernel, dim3((unsigned)(BH * nkb * ncb)),
                         dim3(256), args, 0, s);
}

hipError_t launch_scores(const void* q, const void* k, void* E, float* mref, float* psum, int BH,
                         const TwoPassDims& t, float sl2, bool causal, hipStream_t s) {
  const uint16_t* qp = (const uint16_t*)q;
  const uint16_t* kp = (const uint16_t*)k;
  uint16_t* ep = (uint16_t*)E;
  int L = t.L, d = t.d, T = t.T, Ls = t.Ls, c = causal ? 1 : 0;
  void* args[] = {&qp, &kp, &ep, &mref, &psum, &L, &d, &T, &Ls, &sl2, &c};
  return hipLaunchKernel((const void*)&scores_kernel, dim3((unsigned)(BH * T * T)), dim3(256),
                         args, 0, s);
}

hipError_t launch_values(const void* vt, const void* E, const float* mref, const float* psum,
                         void* out, int BH, const TwoPassDims& t, bool causal, hipStream_t s) {
  const uint16_t* vtp = (const uint16_t*)vt;
  const uint16_t* ep = (const uint16_t*)E;
  uint16_t* op = (uint16_t*)out;
  int L = t.L, d = t.d, T = t.T, Ls = t.Ls, Lk = t.Lk, c = causal ? 1 : 0;
  int ncb = (t.d + kTile - 1) / kTile;
  void* args[] = {&vtp, &ep, &mref, &psum, &op, &L, &d, &T, &Ls, &Lk, &c, &ncb};
  return hipLaunchKernel((const void*)&values_kernel, dim3((unsigned)(BH * T * ncb)), dim3(256),
                         args, 0, s);
}

}  // namespace attn
