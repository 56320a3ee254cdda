// online_attn.hip -- fused online-softmax attention for head dims 32, 64, 128.
//
// Method: the streaming softmax of the cuDNN Blackwell FMHA example
// (native_sparse_attention fmha.py, softmax_step and correction_epilog): keep a
// running row maximum m and row sum l per query, and for each block of keys
// rescale the output accumulator by 2^(m_old - m_new) before adding P V; divide
// by l at the end.  The exponent is taken base 2 with the scale folded in
// (scale * log2 e), as that page does; exp2 is the hardware v_exp_f32.
//
// gfx950 mapping (one workgroup = 4 waves = 128 queries of one head):
//   * Each wave owns 32 queries.  It computes S^T = K Q^T for a 64-key block
//     with v_mfma_f32_32x32x16_bf16, keys on the M side and queries on the N
//     side, so that every lane owns one query: the row max and row sum are
//     in-lane reductions plus one swap between the two lane halves.
//   * The S^T accumulator layout is, register for register, the B operand of
//     O^T += V^T P^T once the 32 keys of a block are relabelled; so P goes from
//     the softmax to the second MFMA without touching LDS.
//   * K tiles go global -> LDS with direct buffer loads (XOR-swizzled 16-byte
//     chunks, conflict-free fragment reads); V tiles are transposed in
//     registers on the way into LDS so that V^T rows hold consecutive keys.
//   * K/V tiles are double-buffered: the next tile's loads are in flight while
//     the current one is consumed.
//   * Keys past L (and, when causal, past the query) are masked to -inf; loads
//     past the end of a head return zero through the buffer resource bounds.
#include "device.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // queries per workgroup
constexpr int kBN = 64;           // keys per step
constexpr float kLazy = 8.f;      // reference slack (log2 units) before O is rescaled

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void online_attn_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          uint16_t* __restrict__ out, int L,
                                                          int nqb, float sl2) {
  constexpr int CPR = D / 8;                       // 16-byte chunks per K row
  constexpr int SWZ = (CPR >= 8 ? 8 : CPR) - 1;    // chunk-index bits that are swizzled
  constexpr int KT_BYTES = kBN * D * 2;
  constexpr int VROW = kBN * 2 + 8;                // bytes per V^T row: 64 keys + pad
  constexpr int VT_BYTES = D * VROW;
  constexpr int K_LOADS = kBN * CPR / 256;         // direct loads per thread per K tile
  constexpr int V_BLOCKS = 16 * CPR;               // 4-key x 8-channel blocks per V tile
  constexpr int NS = D / 16;                       // k16 steps for S
  constexpr int NCB = D / 32;                      // 32-channel blocks of O
  static_assert(K_LOADS >= 1 && V_BLOCKS <= 256, "tile shape");

  __shared__ __attribute__((aligned(16))) char kbuf[2][KT_BYTES];
  __shared__ __attribute__((aligned(16))) char vbuf[2][VT_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, h = lane >> 5;

  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int bh = lid / nqb;
  int qb = lid % nqb;
  if (CAUSAL) qb = nqb - 1 - qb;  // the longest rows start first

  const size_t head = (size_t)bh * L * D;
  const uint32_t head_bytes = (uint32_t)L * D * 2;
  const auto rq = make_rsrc(q + head, head_bytes);
  const auto rk = make_rsrc(k + head, head_bytes);
  const auto rv = make_rsrc(v + head, head_bytes);

  const int q0 = qb * kBM + wave * 32;  // first query of this wave
  const int myq = q0 + c32;             // this lane's query

  // Q fragments: B operand of S^T, lane holds Q[myq][16 s + 8 h .. + 8].
  bf16x8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, load16(rq, (uint32_t)(myq * D + 16 * s + 8 * h) * 2));

  const int kend = CAUSAL ? min(L, qb * kBM + kBM) : L;
  const int ntiles = (kend + kBN - 1) / kBN;

  auto issue_k = [&](int t, int buf) {
#pragma unroll
    for (int j = 0; j < K_LOADS; ++j) {
      const int P = (j * kWaves + wave) * 64 + lane;
      const int row = P / CPR, pc = P % CPR;
      const int lc = pc ^ (row & SWZ);
      const uint32_t voff = (uint32_t)((t * kBN + row) * D + lc * 8) * 2;
      load16_to_lds(rk, &kbuf[buf][(j * kWaves + wave) * 64 * 16], voff);
    }
  };
  // Thread tid owns V block (g = tid % 16 -> keys 4g..4g+3, c8 = tid / 16 -> channels 8c8..+7).
  const bool vblk = tid < V_BLOCKS;
  const int vg = tid & 15, vc8 = tid >> 4;
  auto load_v = [&](int t, u32x4 (&vr)[4]) {
    if (vblk) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        vr[kk] = load16(rv, (uint32_t)((t * kBN + 4 * vg + kk) * D + 8 * vc8) * 2);
    }
  };
  auto store_vt = [&](int buf, const u32x4 (&vr)[4]) {
    if (vblk) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const unsigned a0 = vr[0][w], a1 = vr[1][w], a2 = vr[2][w], a3 = vr[3][w];
        u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        *(u32x2*)&vbuf[buf][(8 * vc8 + 2 * w) * VROW + 8 * vg] = lo;
        *(u32x2*)&vbuf[buf][(8 * vc8 + 2 * w + 1) * VROW + 8 * vg] = hi;
      }
    }
  };

  f32x16 o[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) o[c] = f32x16{};
  float m = -INFINITY, lsum = 0.f;

  u32x4 vr[4];
  issue_k(0, 0);
  load_v(0, vr);
  wait_vmem();
  store_vt(0, vr);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool has_next = t + 1 < ntiles;
    if (has_next) {
      issue_k(t + 1, buf ^ 1);
      load_v(t + 1, vr);
    }
    const int kbase = t * kBN;
    const bool active = !CAUSAL || kbase <= q0 + 31;
    if (active) {
      // S^T block: 64 keys x 32 queries, two 32-key halves.
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ss = 0; ss < NS; ++ss) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = kb * 32 + c32;
          const int pc = (2 * ss + h) ^ (row & SWZ);
          const bf16x8 a = *(const bf16x8*)&kbuf[buf][(row * CPR + pc) * 16];
          s[kb] = mfma32x32x16(a, qf[ss], s[kb]);
        }
      }
      // Softmax update for this lane's query over its 32 of the 64 keys.  The
      // maximum is taken on the raw scores (scaled afterwards; the sign of sl2
      // picks max or min), and y - m is one FMA: p = 2^(s * sl2 - m).
      const bool need_mask = (kbase + kBN > L) || (CAUSAL && kbase + kBN - 1 > q0);
      float tmax;
      if (need_mask) {
        tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = kbase + kb * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
            const bool off = key >= L || (CAUSAL && key > myq);
            s[kb][j] = off ? -INFINITY : s[kb][j] * sl2;
            tmax = fmaxf(tmax, s[kb][j]);
          }
        }
      } else {
        float hi = s[0][0], lo = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            hi = fmaxf(hi, s[kb][j]);
            lo = fminf(lo, s[kb][j]);
          }
        tmax = sl2 >= 0.f ? hi * sl2 : lo * sl2;
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
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          const float p0 = exp2_fast(fmaf(s[kb][j], mul, -muse));
          const float p1 = exp2_fast(fmaf(s[kb][j + 1], mul, -muse));
          pk[kb][j >> 1] = pack_bf16x2(p0, p1);
          lsum = add_bf16x2(pk[kb][j >> 1], lsum);  // sum of the rounded P actually used
        }
      }
      // O^T += V^T P^T.  MFMA (kb, u) covers keys kb*32 + 16u + {4h..4h+3, 8+4h..8+4h+3}
      // in lane half h: exactly the S^T registers 8u..8u+7 of block kb.
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const int ch = c * 32 + c32;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const char* base = &vbuf[buf][ch * VROW + (kb * 32 + 16 * u + 4 * h) * 2];
            const u32x2 lo = *(const u32x2*)base;
            const u32x2 hi = *(const u32x2*)(base + 16);
            const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
            const u32x4 bv = {pk[kb][4 * u], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]};
            o[c] = mfma32x32x16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), o[c]);
          }
        }
      }
    }
    if (has_next) {
      wait_vmem();
      store_vt(buf ^ 1, vr);
    }
    __syncthreads();
  }

  // Epilogue: O = O / l, rounded once to bf16.  Lane holds channels
  // 32c + 8i + 4h + r (r = 0..3) of query myq in o[c][4i + r].
  const float inv = 1.f / wave_swap32_sum(lsum);
  if (myq < L) {
    uint16_t* orow = out + head + (size_t)myq * D;
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

template <int D, bool C>
hipError_t launch_one(const void* q, const void* k, const void* v, void* out, int BH, int L,
                      float sl2, hipStream_t s) {
  const int nqb = (L + kBM - 1) / kBM;
  const dim3 grid((unsigned)(nqb * BH)), block(256);
  const uint16_t* qp = (const uint16_t*)q;
  const uint16_t* kp = (const uint16_t*)k;
  const uint16_t* vp = (const uint16_t*)v;
  uint16_t* op = (uint16_t*)out;
  void* args[] = {&qp, &kp, &vp, &op, &L, (void*)&nqb, &sl2};
  return hipLaunchKernel((const void*)&online_attn_kernel<D, C>, grid, block, args, 0, s);
}

}  // namespace

hipError_t launch_online(const void* q, const void* k, const void* v, void* out, int BH, int L,
                         int d, float sl2, bool causal, hipStream_t s) {
  switch (d) {
    case 32: return causal ? launch_one<32, true>(q, k, v, out, BH, L, sl2, s)
                           : launch_one<32, false>(q, k, v, out, BH, L, sl2, s);
    case 64: return causal ? launch_one<64, true>(q, k, v, out, BH, L, sl2, s)
                           : launch_one<64, false>(q, k, v, out, BH, L, sl2, s);
    case 128: return causal ? launch_one<128, true>(q, k, v, out, BH, L, sl2, s)
                            : launch_one<128, false>(q, k, v, out, BH, L, sl2, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
