// split_columns.hip -- design probe for head dim 1024, not part of the
// attention path: the one-kernel alternative to the two-pass design that
// splits the OUTPUT COLUMNS across the waves of a workgroup.
//
// One workgroup = 8 waves = 64 query rows of one head.  Wave w owns the 128
// channels [128 w, 128 w + 128) of d = 1024: its share of every dot product
// q . k and its 64 x 128 block of O (fp32, 128 registers a lane).  Per block
// of 32 keys:
//   1. each wave forms the partial S^T (32 keys x 64 queries) over its 128
//      channels with v_mfma_f32_32x32x16_bf16, K and Q fragments loaded from
//      global memory (Q is re-read every block: with O resident, a 64 x 128
//      Q share does not also fit in the 256 registers a lane has at two waves
//      per SIMD);
//   2. the 8 partials go through LDS and are summed, 8 threads per query, which
//      then run the online softmax of the page's streaming method (running row
//      maximum and sum; p = 2^(s log2e scale - m)); P (bf16) and each row's
//      rescale factor go back through LDS;
//   3. each wave rescales its O and adds P V over its 128 channels, V staged
//      in LDS by direct loads and read with the gfx950 transpose read.
// K and V are streamed once per workgroup (each wave its own 128 columns), so
// every 32-key block moves 64 KB of K, 64 KB of V and 128 KB of Q into the CU.
#include <hip/hip_runtime.h>

#include "../device.h"
#include "attn_probe.h"

namespace attn_probe {
namespace {
using namespace attn;

constexpr int kD = 1024;     // head dim this probe is written for
constexpr int kBM = 64;      // query rows per workgroup
constexpr int kBK = 32;      // keys per block
constexpr int kWaves = 8;    // 8 x 128 channels
constexpr int kCols = 128;   // channels per wave

struct Smem {
  float part[kWaves][2][64][16];          // 64 KB: S^T partials [wave][query half][lane][acc reg]
  char vt[kWaves][kBK * kCols * 2];       // 64 KB: each wave's V rows [32 keys][128 channels]
  unsigned short p[kBM][kBK];             // P (bf16) [query][key]
  float alpha[kBM];                       // this block's rescale factor per query
  float lrow[kBM];                        // final row sums
};

// V rows are 256 bytes (16 chunks of 16 bytes); chunk c of row r sits at
// c ^ 2 (r % 4), so that the 4 rows one transpose read gathers fall in
// distinct banks.
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 3); }

__global__ __launch_bounds__(64 * kWaves) void split_columns_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, int L, int nqb, float sl2) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int bh = lid / nqb, qb = lid % nqb;
  const size_t hoff = (size_t)bh * L * kD;
  const uint32_t hbytes = (uint32_t)L * kD * 2;
  const auto rq = make_rsrc(q + hoff, hbytes);
  const auto rk = make_rsrc(k + hoff, hbytes);
  const u32x4 rv = rsrc_words(v + hoff, hbytes);
  const int q0 = qb * kBM, c0 = w * kCols;

  f32x16 o[2][4];  // O^T blocks [query half][32-channel block]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) o[a][c] = f32x16{};

  // Reduction threads: 8 per query; thread t takes query rq = t / 8 and the
  // accumulator registers 4 jq .. 4 jq + 3 of lane rl of each partial, i.e.
  // keys 8 jq + 4 hh + 0..3 of the block.
  const int rqq = tid >> 3, sub = tid & 7, rqh = rqq >> 5, hh = sub >> 2, jq = sub & 3;
  const int rl = (rqq & 31) + 32 * hh;
  float m_run = -INFINITY, l_run = 0.f;

  const int nkb = (L + kBK - 1) / kBK;
  for (int kb = 0; kb < nkb; ++kb) {
    const int key0 = kb * kBK;
    // V rows of this block, this wave's channels, into its own LDS region
    // (read last by this wave in the previous block's P V).
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int P = j * 64 + lane, row = P >> 4, lc = P & 15;
      load16_to_lds_untracked(rv, sm.vt[w] + j * 1024,
                              (uint32_t)((key0 + row) * kD + c0 + (lc ^ vswz(row)) * 8) * 2);
    }
    // 1. Partial S^T over this wave's channels.  Step s, lane half h takes
    // channels c0 + 16 s + 8 h .. + 8 for both K and Q: the two lane halves of
    // one row read 32 contiguous bytes in each load.
    f32x16 st[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t ch = (uint32_t)(c0 + 16 * s + 8 * h);
      const bf16x8 kf = __builtin_bit_cast(bf16x8, load16(rk, ((uint32_t)(key0 + n) * kD + ch) * 2));
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const bf16x8 qf =
            __builtin_bit_cast(bf16x8, load16(rq, ((uint32_t)(q0 + 32 * a + n) * kD + ch) * 2));
        st[a] = mfma32x32x16(kf, qf, st[a]);
      }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(f32x4*)&sm.part[w][a][lane][4 * i] =
            f32x4{st[a][4 * i], st[a][4 * i + 1], st[a][4 * i + 2], st[a][4 * i + 3]};
    __syncthreads();

    // 2. Sum the partials and run the online softmax for query rqq.
    f32x4 sacc = *(const f32x4*)&sm.part[0][rqh][rl][4 * jq];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) sacc += *(const f32x4*)&sm.part[ww][rqh][rl][4 * jq];
    float sc[4], bmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + 8 * jq + 4 * hh + i;
      sc[i] = key < L ? sacc[i] * sl2 : -INFINITY;
      bmax = fmaxf(bmax, sc[i]);
    }
#pragma unroll
    for (int x = 1; x < 8; x <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, x, 64));
    const float m_new = fmaxf(m_run, bmax);
    const float alpha = m_run == -INFINITY ? 0.f : exp2_fast(m_run - m_new);
    const unsigned p01 = pack_bf16x2(exp2_fast(sc[0] - m_new), exp2_fast(sc[1] - m_new));
    const unsigned p23 = pack_bf16x2(exp2_fast(sc[2] - m_new), exp2_fast(sc[3] - m_new));
    float psum = add_bf16x2(p23, add_bf16x2(p01, 0.f));  // sum of the rounded P used
#pragma unroll
    for (int x = 1; x < 8; x <<= 1) psum += __shfl_xor(psum, x, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    *(u32x2*)&sm.p[rqq][8 * jq + 4 * hh] = u32x2{p01, p23};
    if (sub == 0) sm.alpha[rqq] = alpha;
    wait_vmem();  // this wave's V rows have landed
    __syncthreads();

    // 3. O^T = alpha O^T + V^T P^T over this wave's channels.
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const float al = sm.alpha[32 * a + n];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[a][c] *= al;
    }
    const int g16 = lane >> 4, L4 = lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 pf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) pf[a] = *(const bf16x8*)&sm.p[32 * a + n][16 * u + 8 * h];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // A operand V^T: lane (channel 32c + n, half h) takes keys 16u + 8h .. + 8;
        // in each 16-lane group lane L4 addresses row r0 + L4 / 4, channels m.. .
        const int m = 32 * c + 16 * (g16 & 1) + 4 * (L4 & 3);
        const int r0 = 16 * u + 8 * (g16 >> 1) + (L4 >> 2);
        const int off = r0 * (kCols * 2) + ((((m >> 3) ^ vswz(r0)) << 4) | ((m & 7) * 2));
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((short4_lds*)(sm.vt[w] + off));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (short4_lds*)(sm.vt[w] + off + 4 * kCols * 2));
        const s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int a = 0; a < 2; ++a)
          o[a][c] = mfma32x32x16(__builtin_bit_cast(bf16x8, vv), pf[a], o[a][c]);
      }
    }
  }

  // O = O / l, rounded once to bf16.  Lane holds channels c0 + 32c + 8i + 4h
  // + r of query 32a + n in o[a][c][4i + r].
  if (sub == 0) sm.lrow[rqq] = l_run;
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int qr = q0 + 32 * a + n;
    if (qr >= L) continue;
    const float lr = sm.lrow[32 * a + n];
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    uint16_t* orow = out + hoff + (size_t)qr * kD + c0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(u32x2*)(orow + 32 * c + 8 * i + 4 * h) =
            u32x2{pack_bf16x2(o[a][c][4 * i] * inv, o[a][c][4 * i + 1] * inv),
                  pack_bf16x2(o[a][c][4 * i + 2] * inv, o[a][c][4 * i + 3] * inv)};
  }
}

}  // namespace
}  // namespace attn_probe

extern "C" int attn_probe_split_columns(const void* q, const void* k, const void* v, void* out,
                                        int64_t B, int64_t H, int64_t L, int64_t d, float scale,
                                        void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return 1;
  if (d != attn_probe::kD || B < 1 || H < 1 || L < 1) return 2;
  // One head is addressed with 32-bit byte offsets.
  if (L * attn_probe::kD * 2 >= ((int64_t)1 << 31) || B * H >= ((int64_t)1 << 20)) return 2;
  const int Li = (int)L;
  int nqb = (Li + attn_probe::kBM - 1) / attn_probe::kBM;
  float sl2 = scale * 1.4426950408889634f;
  const uint16_t* qp = (const uint16_t*)q;
  const uint16_t* kp = (const uint16_t*)k;
  const uint16_t* vp = (const uint16_t*)v;
  uint16_t* op = (uint16_t*)out;
  int Lv = Li;
  void* args[] = {&qp, &kp, &vp, &op, &Lv, &nqb, &sl2};
  const hipError_t e =
      hipLaunchKernel((const void*)&attn_probe::split_columns_kernel,
                      dim3((unsigned)(B * H * nqb)), dim3(64 * attn_probe::kWaves), args, 0,
                      (hipStream_t)stream);
  return e == hipSuccess ? 0 : 8;
}
