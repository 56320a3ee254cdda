// gemm_core.h -- 256x256 bf16 MFMA tile, C = A B^T with both operands K-contiguous.
//
// Used by both passes of the large-head-dim path: the scores pass (A = K rows,
// B = Q rows, K = d) and the values pass (A = V^T rows, B = E rows, K = keys).
//
// Workgroup: 4 waves in a 2x2 grid, each wave owning a 128x128 block of C as
// 4x4 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 registers per lane).
// The K loop runs in 64-wide steps through two LDS stages (2 x 64 KB); the next
// step's A and B tiles are fetched straight into LDS with buffer loads while
// the current stage feeds the MFMAs.  Each 128-byte LDS row holds eight
// 16-byte chunks stored at chunk ^ (row % 8), so the eight lanes that read one
// column of chunks in a fragment load hit eight different bank groups.
#pragma once

#include "device.h"

namespace attn {

constexpr int kTile = 256;  // C tile edge
constexpr int kStepK = 64;  // K elements per step
constexpr int kStageBytes = kTile * kStepK * 2;

struct GemmSmem {
  char a[2][kStageBytes];
  char b[2][kStageBytes];
};

// Copy rows [r0, r0 + 256) x columns [k0, k0 + 64) of a row-major bf16 matrix
// (row stride `ld` elements) into one LDS stage; 8 direct loads per lane.
__device__ __forceinline__ void gemm_load_tile(__amdgpu_buffer_rsrc_t r, uint32_t ld, int r0,
                                               int k0, char* stage, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int P = (wave * 8 + j) * 64 + lane;  // 16-byte chunk slot in the stage
    const int row = P >> 3, pc = P & 7, lc = pc ^ (row & 7);
    const uint32_t voff = ((uint32_t)(r0 + row) * ld + (uint32_t)(k0 + lc * 8)) * 2u;
    load16_to_lds(r, stage + (wave * 8 + j) * 1024, voff);
  }
}

__device__ __forceinline__ bf16x8 gemm_frag(const char* stage, int row, int lc) {
  return *(const bf16x8*)(stage + row * 128 + ((lc ^ (row & 7)) << 4));
}

struct NoTransform {
  __device__ __forceinline__ void step(int) {}
  __device__ __forceinline__ bf16x8 operator()(bf16x8 f, int) const { return f; }
};

// acc[i][j] += A[m0 + 128 wm + 32 i + .., :] . B[n0 + 128 wn + 32 j + .., :] over nk steps.
// `bx.step(kt)` runs at the top of step kt; `bx(frag, j)` may rewrite each B fragment.
template <class BX>
__device__ __forceinline__ void gemm_tile(f32x16 (&acc)[4][4], __amdgpu_buffer_rsrc_t ra,
                                          uint32_t lda, int m0, __amdgpu_buffer_rsrc_t rb,
                                          uint32_t ldb, int n0, int nk, GemmSmem& sm, BX& bx) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, c32 = lane & 31, h = lane >> 5;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  gemm_load_tile(ra, lda, m0, 0, sm.a[0], wave, lane);
  gemm_load_tile(rb, ldb, n0, 0, sm.b[0], wave, lane);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    wait_vmem();
    __syncthreads();  // stage st landed; every wave is done reading stage st ^ 1
    if (kt + 1 < nk) {
      gemm_load_tile(ra, lda, m0, (kt + 1) * kStepK, sm.a[st ^ 1], wave, lane);
      gemm_load_tile(rb, ldb, n0, (kt + 1) * kStepK, sm.b[st ^ 1], wave, lane);
    }
    bx.step(kt);
    const char* sa = sm.a[st];
    const char* sb = sm.b[st];
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = gemm_frag(sa, wm * 128 + i * 32 + c32, 2 * ss + h);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = bx(gemm_frag(sb, wn * 128 + j * 32 + c32, 2 * ss + h), j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
    }
  }
}

}  // namespace attn
