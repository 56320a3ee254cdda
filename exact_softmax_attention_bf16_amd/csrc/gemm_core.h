// gemm_core.h -- 256x256 bf16 MFMA tiles for the large-head-dim path.
//
// Building blocks of both passes -- the scores pass (A = K rows, B = Q rows,
// K = d; its own persistent loop) and the values pass (A = V read as V^T,
// B = E rows, K = keys; gemm_tile below).
//
// Workgroup: 4 waves in a 2x2 grid, each wave owning a 128x128 block of C as
// 4x4 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 registers per lane, held
// in AGPRs).  The K loop runs in 64-wide steps through two LDS stages
// (2 x 64 KB) filled by direct buffer->LDS loads, XOR-swizzled so that the
// lanes that read one column of chunks in a fragment load hit different banks.
//
// Schedule per 64-wide step (4 sub-steps of k = 16, 16 MFMAs each): the
// fragments of sub-step s + 1 are read from LDS while the MFMAs of sub-step s
// run.  In the last sub-step the wave waits for its own loads of the next
// stage, the workgroup meets at one barrier (next stage complete everywhere,
// current stage no longer read), the first fragments of the next step are
// read, and the B loads two steps ahead go into the stage just drained, one
// after each pair of the sub-step's MFMAs; the matching A loads follow the
// same way in the next step's first sub-step (issued as one burst they hold
// up the MFMAs behind them while the address queue drains).  Measured on the
// values pass, 31 frames: all 16 loads in the last sub-step 789 us; A there
// and B in the next first sub-step 771 us; B there and A in the next first
// sub-step 747 us (E, read by fewer workgroups than V, gets the longer lead);
// loads spread into the second sub-step 808 us (too little of the step left
// to cover their latency).
//
// The compiler guards LDS reads against direct-to-LDS loads still in flight:
// a read it cannot prove disjoint from them gets a wait for all of them.
// Ordinary reads of a kernel whose LDS is one object pass; the transpose
// reads of the K-outer layout never do.  So for that layout all A fragments of
// the next step are read before its loads are issued (held in registers for the
// whole step), and no read after them is one the compiler would stall.
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
  __amdgpu_buffer_rsrc_t r;
  uint32_t off[kLoads];

  __device__ __forceinline__ void init(__amdgpu_buffer_rsrc_t rsrc, uint32_t ld, int r0, int wave,
                                       int lane) {
    r = rsrc;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int P = (wave * kLoads + j) * 64 + lane;  // 16-byte chunk slot in the stage
      const int row = P >> 3, pc = P & 7, lc = pc ^ kc_swz(row);
      off[j] = ((uint32_t)(r0 + row) * ld + (uint32_t)(lc * 8)) * 2u;
    }
  }
  // Rows [r0, r0 + 256) x columns [k0, k0 + 64) into `stage`.
  __device__ __forceinline__ void issue(int k0, char* stage, int wave) const {
    issue_from(r, k0, stage, wave);
  }
  // The same from another tensor of the same row stride (offsets as for r0 = 0
  // when the resource starts at the tile's first row).
  __device__ __forceinline__ void issue_from(__amdgpu_buffer_rsrc_t rs, int k0, char* stage,
                                             int wave) const {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) issue_one(rs, k0, stage, wave, j);
  }
  // Load j of this wave's kLoads.
  __device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t rs, int k0, char* stage,
                                            int wave, int j) const {
    load16_to_lds(rs, stage + (wave * kLoads + j) * 1024, off[j] + (uint32_t)k0 * 2u);
  }
  // MFMA fragment: lane supplies row rbase + lane % 32, K values 16 ss + 8 (lane / 32) .. + 8.
  __device__ __forceinline__ bf16x8 frag(const char* stage, int rbase, int ss, int lane) const {
    const int row = rbase + (lane & 31), lc = 2 * ss + (lane >> 5);
    return *(const bf16x8*)(stage + row * 128 + ((lc ^ kc_swz(row)) << 4));
  }
};

// Operand A stored with K as the outer index (A[m][k] at k * ld + m), e.g. V read
// as the A operand of O^T = V^T E^T.  Its stage holds 64 K rows x 256 m values
// (512 bytes per row, 16-byte chunk c at c ^ 4 (row % 4)).  Stage row r holds K
// row k0 + kperm(r), kperm exchanging bits 2 and 3 of the index: the order the
// scores pass gives the keys of each 32-key block of E, so that the B operand
// (E, K-contiguous) and this one agree.  Fragments are built with two
// ds_read_b64_tr_b16: in each 16-lane group, lane L reads the 4 values
// A[m0 + 4 (L % 4) ..][k0 + L / 4] and the hardware hands lane i the 4 K values
// of column m0 + i.
__device__ __forceinline__ int kperm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

struct KOuter {
  static constexpr bool kWholeStepA = true;  // fragments come from transpose reads
  __amdgpu_buffer_rsrc_t r;
  uint32_t off[8];
  uint32_t ld2;  // bytes per K row

  __device__ __forceinline__ void init(__amdgpu_buffer_rsrc_t rsrc, uint32_t ld, int m0, int wave,
                                       int lane) {
    r = rsrc;
    ld2 = ld * 2u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int P = (wave * 8 + j) * 64 + lane;  // 16-byte chunk slot in the stage
      const int row = P >> 5, pc = P & 31, lc = pc ^ ((row & 3) << 2);
      off[j] = (uint32_t)kperm(row) * ld2 + (uint32_t)(m0 + lc * 8) * 2u;
    }
  }
  __device__ __forceinline__ void issue(int k0, char* stage, int wave) const {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      load16_to_lds(r, stage + (wave * 8 + j) * 1024, off[j] + (uint32_t)k0 * ld2);
  }
  __device__ __forceinline__ void issue_one(int k0, char* stage, int wave, int j) const {
    load16_to_lds(r, stage + (wave * 8 + j) * 1024, off[j] + (uint32_t)k0 * ld2);
  }
  __device__ __forceinline__ bf16x8 frag(const char* stage, int mbase, int ss, int lane) const {
    const int g = lane >> 4, L = lane & 15;
    const int m = mbase + (g & 1) * 16 + 4 * (L & 3);
    const int row = 16 * ss + 8 * (g >> 1) + (L >> 2);
    auto at = [&](int rr) {
      return (short4_lds*)(stage + rr * 512 + (((m >> 3) ^ ((rr & 3) << 2)) << 4) + (m & 7) * 2);
    };
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(row));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(row + 4));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

using KContiguous = KContiguousT<4>;

struct NoTransform {
  __device__ __forceinline__ void step(int, bool) {}
  __device__ __forceinline__ bf16x8 operator()(bf16x8 f, int) const { return f; }
};

// One k16 sub-step's fragments of a wave: 4 A blocks of 32 rows, NJ B blocks.
template <int NJ>
struct FragsT {
  bf16x8 a[4], b[NJ];
};
using Frags = FragsT<4>;

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

// 16 MFMAs with 4 LDS reads early among them (the reads feed the next sub-step's
// first MFMAs).
__device__ __forceinline__ void sched_substep_b_only() {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);  // 12 MFMAs
}

// acc[i][j] = A[m0 + 128 wm + 32 i + .., K] . B[n0 + 128 wn + 32 j + .., K] over the
// K steps [k_first, k_first + nk) (64 wide each), with A in the K-outer layout
// (LA = KOuter) and B K-contiguous.  All A fragments of a step are read right
// after the barrier, before that step's loads go out (the transpose reads
// would otherwise wait for them).  `bx.step(kt, first)` runs before step kt's
// MFMAs (kt absolute); `bx(frag, j)` may rewrite each B fragment.
template <class LA, class BX>
__device__ __forceinline__ void gemm_tile(f32x16 (&acc)[4][4], __amdgpu_buffer_rsrc_t ra,
                                          uint32_t lda, int m0, __amdgpu_buffer_rsrc_t rb,
                                          uint32_t ldb, int n0, int k_first, int nk,
                                          GemmSmem& sm, BX& bx) {
  static_assert(LA::kWholeStepA, "the K loop below reads A a whole step at a time");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  LA la;
  KContiguous lb;
  la.init(ra, lda, m0, wave, lane);
  lb.init(rb, ldb, n0, wave, lane);

  // Stage 0 <- the first step; stage 1 <- the second (a harmless reload of the
  // first when nk == 1).
  const int kb = k_first * kStepK;
  la.issue(kb, sm.a[0], wave);
  lb.issue(kb, sm.b[0], wave);
  wait_vmem();
  block_sync();
  const int k1 = kb + (nk > 1 ? kStepK : 0);

  Frags f[4];  // f[ss].a: A of sub-step ss; f[ss].b: B of sub-step ss (as it arrives)
  auto read_a_step = [&](Frags (&g)[4], const char* sa) {
#pragma unroll
    for (int ss = 0; ss < 4; ++ss)
#pragma unroll
      for (int i = 0; i < 4; ++i) g[ss].a[i] = la.frag(sa, wm * 128 + i * 32, ss, lane);
  };
  auto read_b = [&](bf16x8 (&b)[4], const char* sb, int ss) {
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = lb.frag(sb, wn * 128 + j * 32, ss, lane);
  };
  read_a_step(f, sm.a[0]);
  read_b(f[0].b, sm.b[0], 0);
  lb.issue(k1, sm.b[1], wave);
  // The A loads of step kt + 1 are issued during step kt's first sub-step
  // (into the stage step kt does not read; step 1's from step 0), so that each
  // sub-step carries at most 8 loads per wave: 16 at once, from all four waves
  // right after the barrier, back up the address queue and hold the MFMAs
  // behind them.
  int kb_pend = k1;  // K offset of the A loads the next first sub-step issues
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const char* sb = sm.b[st];
    bx.step(k_first + kt, kt == 0);
    read_b(f[1].b, sb, 1);
    {
      bf16x8 b0[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b0[j] = bx(f[0].b[j], j);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        __builtin_amdgcn_sched_barrier(0);
        const int i = p >> 1, j0 = 2 * (p & 1);
        acc[i][j0] = mfma32x32x16(f[0].a[i], b0[j0], acc[i][j0]);
        acc[i][j0 + 1] = mfma32x32x16(f[0].a[i], b0[j0 + 1], acc[i][j0 + 1]);
        la.issue_one(kb_pend, sm.a[st ^ 1], wave, p);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ss = 1; ss < 3; ++ss) {
      read_b(f[ss + 1].b, sb, ss + 1);
      mma_substep(acc, f[ss], bx);
      sched_substep_b_only();
    }
    // Last sub-step: next stage complete everywhere, this stage drained.
    const Frags last = f[3];
    wait_vmem();
    block_sync();
    read_a_step(f, sm.a[st ^ 1]);
    read_b(f[0].b, sm.b[st ^ 1], 0);
    const int k2 = kb + (kt + 2 < nk ? kt + 2 : nk - 1) * kStepK;  // past the end: reload, unused
    // The reads above, then the sub-step's MFMAs in pairs with one B load
    // after each pair; the A loads follow in the next step's first sub-step
    // (none after the last step).
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 lbf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) lbf[j] = bx(last.b[j], j);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      __builtin_amdgcn_sched_barrier(0);
      const int i = p >> 1, j0 = 2 * (p & 1);
      acc[i][j0] = mfma32x32x16(last.a[i], lbf[j0], acc[i][j0]);
      acc[i][j0 + 1] = mfma32x32x16(last.a[i], lbf[j0 + 1], acc[i][j0 + 1]);
      lb.issue_one(lb.r, k2, sm.b[st], wave, p);
    }
    __builtin_amdgcn_sched_barrier(0);
    kb_pend = k2;
  }
  wait_vmem();  // no LDS writes in flight past the loop
}

}  // namespace attn
