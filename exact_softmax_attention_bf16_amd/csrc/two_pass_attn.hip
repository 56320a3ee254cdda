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
// contraction uses, and there is no extra pass over S or P.  V is read in place:
// the values pass stages V rows in LDS and builds its MFMA operand with the
// gfx950 transpose read (ds_read_b64_tr_b16), so no V^T copy is made.  The subtraction of
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
  t.Ls = t.T * kTile + kTile / 2;
  t.Lk = (int)((L + 63) / 64 * 64);
  return t;
}

static int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

int64_t two_pass_head_bytes(const TwoPassDims& t) {
  return round256((int64_t)t.L * t.Ls * 2) + 2 * round256((int64_t)t.T * t.L * 4);
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
// Epilogue, per query: m = ceil(max over the tile's keys of y), y = sl2 * s;
// E = bf16(2^(y - m)) (so 1/2 < max E <= 1); psum = sum of the stored E.
// MASK selects the edge-tile version (keys past L, keys after the query); it is
// a template flag so that the per-element test compiles to selects, not branches.
// The E tile (256 queries x 256 keys) is staged through the drained GEMM stages
// in LDS so that the global stores write whole 512-byte row segments.
template <bool MASK>
__device__ __forceinline__ void scores_epilogue(const f32x16 (&acc)[4][4], float (&red)[2][kTile],
                                                char* __restrict__ stage,
                                                uint16_t* __restrict__ Eh,
                                                float* __restrict__ mref_t,
                                                float* __restrict__ psum_t, int L, int Ls,
                                                int kt, int qt, float sl2, int causal) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, c32 = lane & 31, h = lane >> 5;
  const int key0 = kt * kTile + wm * 128;
  // Key key0 + 4h + c (c = 32 bi + 8 (j / 4) + j % 4, a constant) is allowed for
  // query column bj iff c < lim[bj].
  int lim[4];
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    const int query = qt * kTile + wn * 128 + bj * 32 + c32;
    lim[bj] = (causal ? min(L, query + 1) : L) - (key0 + 4 * h);
  }
  auto masked = [&](int bi, int bj, int j) { return bi * 32 + 8 * (j >> 2) + (j & 3) >= lim[bj]; };

  // Per-query maximum of y over this wave's 128 keys (interior tiles: on the
  // raw accumulator, then scaled; the sign of sl2 picks max or min).
  float wmax[4];
  if (!MASK && sl2 >= 0.f) {
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      float hi = acc[0][bj][0];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int j = 0; j < 16; ++j) hi = fmaxf(hi, acc[bi][bj][j]);
      wmax[bj] = hi * sl2;
    }
  } else if (!MASK) {
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      float lo = acc[0][bj][0];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int j = 0; j < 16; ++j) lo = fminf(lo, acc[bi][bj][j]);
      wmax[bj] = lo * sl2;
    }
  } else {
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      float mx = -INFINITY;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          mx = fmaxf(mx, masked(bi, bj, j) ? -INFINITY : acc[bi][bj][j] * sl2);
      wmax[bj] = mx;
    }
  }
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    const float m = wave_swap32_max(wmax[bj]);
    if (h == 0) red[wm][wn * 128 + bj * 32 + c32] = m;
  }
  __syncthreads();  // red complete; every wave is past its GEMM (the stages are free)
  // Recompute the mask below instead of keeping 256 mask bits alive across the
  // barrier (the compiler would otherwise hold them in scalar registers).
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) asm volatile("" : "+v"(lim[bj]));

  // E into LDS as [query][key] rows of 512 bytes; 16-byte chunk c of row r is
  // stored at chunk c ^ (r % 32), with its two 8-byte halves swapped when
  // r % 32 >= 16 (the 32 rows one write instruction touches then fill 32
  // different bank pairs).
  float mt[4], ps[4];
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    const int ql = wn * 128 + bj * 32 + c32;
    const float tmax = fmaxf(red[0][ql], red[1][ql]);
    const float m2 = tmax == -INFINITY ? -INFINITY : ceilf(tmax);
    const float add = tmax == -INFINITY ? 0.f : -m2;
    float s = 0.f;
    char* row = stage + ql * 512 + 8 * (h ^ (c32 >> 4));
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = exp2_fast(fmaf(acc[bi][bj][4 * i + r], sl2, add));
          if (MASK) e[r] = masked(bi, bj, 4 * i + r) ? 0.f : e[r];
        }
        const unsigned w0 = pack_bf16x2(e[0], e[1]), w1 = pack_bf16x2(e[2], e[3]);
        // the normaliser sums exactly the rounded values the values pass multiplies
        s = add_bf16x2(w1, add_bf16x2(w0, s));
        const int chunk = wm * 16 + bi * 4 + i;
        *(u32x2*)(row + ((chunk ^ c32) << 4)) = u32x2{w0, w1};
      }
    }
    mt[bj] = m2;
    ps[bj] = wave_swap32_sum(s);
  }
  __syncthreads();  // E tile complete in LDS; red no longer read
  if (h == 0) {
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) red[wm][wn * 128 + bj * 32 + c32] = ps[bj];
  }
  // Whole-row stores: thread t writes chunk t % 32 of rows t / 32 + 8 j.
  {
    const int c = tid & 31;
    uint16_t* base = Eh + (size_t)(qt * kTile) * Ls + kt * kTile + 8 * c;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
      const int r = (tid >> 5) + 8 * j;
      if (qt * kTile + r < L)
        *(u32x4*)(base + (size_t)r * Ls) = unswap_halves(*(const u32x4*)(stage + r * 512 + ((c ^ (r & 31)) << 4)), r);
    }
  }
  __syncthreads();  // partial sums complete
  if (wm == 0 && h == 0) {
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int ql = wn * 128 + bj * 32 + c32;
      const int query = qt * kTile + ql;
      if (query < L) {
        mref_t[query] = mt[bj];
        psum_t[query] = red[0][ql] + red[1][ql];
      }
    }
  }
}

// One LDS object per kernel: with a single object the compiler attaches no
// alias scopes, and its LDS-DMA wait tracking then does not make the fragment
// reads of one stage wait for the loads just issued into the other (with
// several objects it does, and every K step stalls on the whole memory latency).
// The stage protocol itself (wait for this wave's loads, then a barrier) is
// explicit in the GEMM loop.
struct ScoresSmem {
  GemmSmem g;
  float red[2][kTile];
};

__global__ __launch_bounds__(256) void scores_kernel(const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k,
                                                     uint16_t* __restrict__ E,
                                                     float* __restrict__ mref,
                                                     float* __restrict__ psum, int L, int d, int T,
                                                     int Ls, float sl2, int causal) {
  __shared__ ScoresSmem smem;
  GemmSmem& sm = smem.g;
  float(&red)[2][kTile] = smem.red;

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
  gemm_tile<KContiguous>(acc, rk, (uint32_t)d, kt * kTile, rq, (uint32_t)d, qt * kTile, d / kStepK,
                         sm, nx);

  uint16_t* Eh = E + (size_t)bh * L * Ls;
  float* mref_t = mref + ((size_t)bh * T + kt) * L;
  float* psum_t = psum + ((size_t)bh * T + kt) * L;
  const bool need_mask = (kt + 1) * kTile > L || (causal && kt >= qt);
  char* stage = sm.a[0];  // 128 KB of drained GEMM stages hold the E tile
  if (need_mask)
    scores_epilogue<true>(acc, red, stage, Eh, mref_t, psum_t, L, Ls, kt, qt, sl2, causal);
  else
    scores_epilogue<false>(acc, red, stage, Eh, mref_t, psum_t, L, Ls, kt, qt, sl2, causal);
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

struct ValuesSmem {
  GemmSmem g;
  uint8_t shift_tab[kMaxTiles][kTile];
  float inv_l[kTile];
};

__global__ __launch_bounds__(256) void values_kernel(const uint16_t* __restrict__ v,
                                                     const uint16_t* __restrict__ E,
                                                     const float* __restrict__ mref,
                                                     const float* __restrict__ psum,
                                                     uint16_t* __restrict__ out, int L, int d,
                                                     int T, int Ls, int Lk, int causal, int ncb) {
  __shared__ ValuesSmem smem;
  GemmSmem& sm = smem.g;
  uint8_t(&shift_tab)[kMaxTiles][kTile] = smem.shift_tab;
  float(&inv_l)[kTile] = smem.inv_l;

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
  // The stats are read in batches of 16 tiles so their latencies overlap.
  {
    const float* mh = mref + (size_t)bh * T * L;
    const float* ph = psum + (size_t)bh * T * L;
    const int qc = min(qt * kTile + tid, L - 1);
    float M = -INFINITY, l = 0.f;
    for (int t0 = 0; t0 < tiles; t0 += 16) {
      float mt[16], pt[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int t = min(t0 + u, tiles - 1);
        mt[u] = mh[(size_t)t * L + qc];
        pt[u] = ph[(size_t)t * L + qc];
      }
      float Mn = M;
#pragma unroll
      for (int u = 0; u < 16; ++u) Mn = fmaxf(Mn, mt[u]);
      l = M == -INFINITY ? 0.f : l * exp2_fast(M - Mn);
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (t0 + u < tiles) l += pt[u] * exp2_fast(mt[u] - Mn);
      M = Mn;
    }
    // The shifts need the final M: a second pass over the (now cached) stats.
    for (int t0 = 0; t0 < tiles; t0 += 16) {
      float mt[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) mt[u] = mh[(size_t)min(t0 + u, tiles - 1) * L + qc];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (t0 + u < tiles) shift_tab[t0 + u][tid] = (uint8_t)fminf(M - mt[u], 255.f);
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

  const auto ra = make_rsrc(v + (size_t)bh * L * d, (uint32_t)L * d * 2);
  const auto rb = make_rsrc(E + (size_t)bh * L * Ls, (uint32_t)L * Ls * 2);
  f32x16 acc[4][4];
  gemm_tile<KOuter>(acc, ra, (uint32_t)d, ct * kTile, rb, (uint32_t)Ls, qt * kTile, nk, sm, sh);

  // O[query][ch] = acc / l, rounded once to bf16.  The tile goes through the
  // drained GEMM stages as [query][256 channels] rows (laid out like the E tile
  // of the scores pass) so that the global stores write whole row segments.
  __syncthreads();  // every wave is past its GEMM: the stages are free
  char* stage = sm.a[0];
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    const int ql = wn * 128 + bj * 32 + c32;
    char* row = stage + ql * 512 + 8 * (h ^ (c32 >> 4));
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x16& a = acc[bi][bj];
        const u32x2 w = {pack_bf16x2(a[4 * i] * invl[bj], a[4 * i + 1] * invl[bj]),
                         pack_bf16x2(a[4 * i + 2] * invl[bj], a[4 * i + 3] * invl[bj])};
        const int chunk = wm * 16 + bi * 4 + i;
        *(u32x2*)(row + ((chunk ^ c32) << 4)) = w;
      }
    }
  }
  __syncthreads();
  {
    const int c = tid & 31;
    const int ch = ct * kTile + 8 * c;
    if (ch < d) {
      uint16_t* oh = out + (size_t)bh * L * d + (size_t)(qt * kTile) * d + ch;
#pragma unroll 8
      for (int j = 0; j < 32; ++j) {
        const int r = (tid >> 5) + 8 * j;
        if (qt * kTile + r < L)
          *(u32x4*)(oh + (size_t)r * d) = unswap_halves(*(const u32x4*)(stage + r * 512 + ((c ^ (r & 31)) << 4)), r);
      }
    }
  }
}

}  // namespace

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

hipError_t launch_values(const void* v, const void* E, const float* mref, const float* psum,
                         void* out, int BH, const TwoPassDims& t, bool causal, hipStream_t s) {
  const uint16_t* vtp = (const uint16_t*)v;
  const uint16_t* ep = (const uint16_t*)E;
  uint16_t* op = (uint16_t*)out;
  int L = t.L, d = t.d, T = t.T, Ls = t.Ls, Lk = t.Lk, c = causal ? 1 : 0;
  int ncb = (t.d + kTile - 1) / kTile;
  void* args[] = {&vtp, &ep, &mref, &psum, &op, &L, &d, &T, &Ls, &Lk, &c, &ncb};
  return hipLaunchKernel((const void*)&values_kernel, dim3((unsigned)(BH * T * ncb)), dim3(256),
                         args, 0, s);
}

}  // namespace attn
