// gemm_core.h -- 256x256 bf16 MFMA tile pieces of the large-head-dim path.
//
// Shared by its two passes: the scores pass (A = K rows, B = Q rows, both
// K-contiguous, contraction over the head dim in 64-wide steps) and the values
// pass (A = V read as V^T through the transpose read, B = E blocks,
// contraction over keys).  Each kernel owns its stage layout and K loop; this
// file holds the operand staging of K-contiguous tiles, the fragment reads,
// the MFMA sub-step and its interleaving with the reads of the next.
//
// The compiler guards LDS reads against direct-to-LDS loads still in flight:
// a read it cannot prove disjoint from them gets a wait for all of them.
// Ordinary reads of a kernel whose LDS is one object pass; the transpose
// reads never do, so the kernels that use them issue their direct loads from
// inline assembly (untracked) and wait for them explicitly.
#pragma once

#include "device.h"

namespace attn {

constexpr int kTile = 256;  // C tile edge
constexpr int kStepK = 64;  // K elements per step of a K-contiguous stage
constexpr int kStageBytes = kTile * kStepK * 2;

// Operand stored K-contiguous in global memory (row r, K index k at r * ld + k).
// Its stage holds 256 rows x 64 K values; each 128-byte LDS row keeps eight
// 16-byte chunks at chunk ^ swz(row), swz(row) = (row % 8) ^ ((row / 8) % 2):
// the 8 or 16 consecutive rows one fragment read serves per LDS cycle then hit
// distinct banks.  Per-lane byte offsets of the chunks this lane copies, at k = 0.
__device__ __forceinline__ int kc_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// NW waves share the stage's 2048 chunks: each issues 32 / NW loads of 1 KB.
template <int NW>
struct KContiguousT {
  static constexpr int kLoads = 32 / NW;
  uint32_t off[kLoads];

  __device__ __forceinline__ void init(uint32_t ld, int r0, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int P = (wave * kLoads + j) * 64 + lane;  // 16-byte chunk slot in the stage
      const int row = P >> 3, pc = P & 7, lc = pc ^ kc_swz(row);
      off[j] = ((uint32_t)(r0 + row) * ld + (uint32_t)(lc * 8)) * 2u;
    }
  }
  // Rows [r0, r0 + 256) x columns [k0, k0 + 64) of the tensor behind `rs` into
  // `stage` (r0 = 0 when the resource starts at the tile's first row).
  __device__ __forceinline__ void issue_from(__amdgpu_buffer_rsrc_t rs, int k0, char* stage,
                                             int wave) const {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) issue_one(rs, k0, stage, wave, j);
  }
  // Load j of this wave's kLoads.
  __device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t rs, int k0, char* stage,
                                            int wave, int j) const {
    load16_to_lds(rs, stage + (wave * kLoads + j) * 1024, off[j], (uint32_t)k0 * 2u);
  }
  // MFMA fragment: lane supplies row rbase + lane % 32, K values 16 ss + 8 (lane / 32) .. + 8.
  __device__ __forceinline__ bf16x8 frag(const char* stage, int rbase, int ss, int lane) const {
    const int row = rbase + (lane & 31), lc = 2 * ss + (lane >> 5);
    return *(const bf16x8*)(stage + row * 128 + ((lc ^ kc_swz(row)) << 4));
  }
};

// Operand A stored with K as the outer index (A[m][k] at k * ld + m), e.g. V read
// as the A operand of O^T = V^T E^T.  Its stage holds K rows of 256 or 128 m
// values (512 or 256 bytes per row, 16-byte chunk c at c ^ 4 (row % 4)).  Stage row r holds K
// row k0 + kperm(r), kperm exchanging bits 2 and 3 of the index: the order the
// scores pass gives the keys of each 32-key block of E, so that the B operand
// (E, K-contiguous) and this one agree.  Fragments are built with two
// ds_read_b64_tr_b16: in each 16-lane group, lane L reads the 4 values
// A[m0 + 4 (L % 4) ..][k0 + L / 4] and the hardware hands lane i the 4 K values
// of column m0 + i.
__device__ __forceinline__ int kperm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// PITCH: bytes per stage row.  In either width the 32 lanes of a half-wave
// read 4 rows x 4 chunks that the swizzle puts on distinct banks.
template <int PITCH>
struct KOuterT {
  // Sub-step ss (K rows 16 ss .. 16 ss + 15 of the stage), columns mbase ..
  // mbase + 31.
  __device__ __forceinline__ bf16x8 frag(const char* stage, int mbase, int ss, int lane) const {
    const int g = lane >> 4, L = lane & 15;
    const int m = mbase + (g & 1) * 16 + 4 * (L & 3);
    const int row = 16 * ss + 8 * (g >> 1) + (L >> 2);
    auto at = [&](int rr) {
      return (short4_lds*)(stage + rr * PITCH + (((m >> 3) ^ ((rr & 3) << 2)) << 4) + (m & 7) * 2);
    };
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(row));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(row + 4));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};
using KOuter = KOuterT<512>;

struct NoTransform {
  __device__ __forceinline__ void step(int, bool) {}
  __device__ __forceinline__ bf16x8 operator()(bf16x8 f, int) const { return f; }
};

// One k16 sub-step's fragments of a wave: 4 A blocks of 32 rows, NJ B blocks.
template <int NJ>
struct FragsT {
  bf16x8 a[4], b[NJ];
};

// A rows abase + 32 i, B rows bbase + 32 j.
template <class LA, class LB, int NJ>
__device__ __forceinline__ void read_frags(FragsT<NJ>& f, const LA& la, const LB& lb,
                                           const char* sa, const char* sb, int abase, int bbase,
                                           int lane, int ss) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = la.frag(sa, abase + i * 32, ss, lane);
#pragma unroll
  for (int j = 0; j < NJ; ++j) f.b[j] = lb.frag(sb, bbase + j * 32, ss, lane);
}

template <int NJ, class BX>
__device__ __forceinline__ void mma_substep(f32x16 (&acc)[4][NJ], const FragsT<NJ>& f,
                                            const BX& bx) {
  bf16x8 b[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) b[j] = bx(f.b[j], j);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32x32x16(f.a[i], b[j], acc[i][j]);
}

// Interleave a sub-step's 4 NJ MFMAs with the 4 + NJ LDS reads of the next.
template <int NJ>
__device__ __forceinline__ void sched_substep() {
  if constexpr (NJ == 4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
    }
  } else {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMAs
  }
}

__device__ __forceinline__ void block_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS reads are done
  __builtin_amdgcn_s_barrier();
}

}  // namespace attn
