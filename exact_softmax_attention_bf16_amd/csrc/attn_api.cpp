// attn_api.cpp -- the C ABI: argument checks, path choice, workspace, timing.
//
// The pages' host entry points (FastVideo wan22_vae_decode attn.cu,
// attn_forward; cuDNN fmha.py, __call__) check shapes and raise; this library
// returns status codes instead and makes every check before any HIP call, so
// each error path can be exercised without a GPU.
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <utility>
#include <mutex>
#include <vector>

#include "internal.h"
#include "workspace.h"

namespace {

bool head_dim_supported(int64_t d) {
  return d == 32 || d == 64 || d == 128 || (d > 128 && d <= 1024 && d % 64 == 0);
}

// Heads per two-pass chunk: enough to fill the chip, capped near 2 GiB of workspace.
constexpr int64_t kChunkBudget = int64_t(2) << 30;

int64_t heads_per_chunk(int64_t BH, int64_t head_bytes, int64_t budget = kChunkBudget) {
  int64_t n = budget / (head_bytes > 0 ? head_bytes : 1);
  if (n < 1) n = 1;
  return n < BH ? n : BH;
}

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

// Two-pass workspace for a chunk of n heads: per head E and the two statistics
// tables, plus the values pass's fp32 partial outputs when it splits the keys.
int64_t chunk_workspace_bytes(int64_t n, const attn::TwoPassDims& t, const attn::Band& band) {
  const int split = attn::values_split(n, t, band);
  const int64_t part = split > 1 ? round256((int64_t)split * n * t.L * t.d * 4) : 0;
  return n * attn::two_pass_head_bytes(t) + part;
}

// Bytes attn_forward draws for BH heads: the largest of its chunks.
int64_t two_pass_workspace_bytes(int64_t BH, const attn::TwoPassDims& t, const attn::Band& band) {
  const int64_t chunk = heads_per_chunk(BH, attn::two_pass_head_bytes(t));
  const int64_t last = BH - (BH - 1) / chunk * chunk;
  return std::max(chunk_workspace_bytes(chunk, t, band), chunk_workspace_bytes(last, t, band));
}

// Online path: fp32 shares of O and their (m, l) when the keys are split.
int64_t online_workspace_bytes(int64_t BH, int64_t L, int64_t d) {
  const int n = attn::online_split(BH, L, L);
  return n > 1 ? round256((int64_t)n * BH * L * (d + 2) * 4) : 0;
}

bool overlaps(const void* a, int64_t an, const void* b, int64_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bn && b0 < a0 + (uintptr_t)an;
}

// ---- workspace: one buffer per (device, stream), kept between calls and
// leased for the whole of a call (csrc/workspace.h states the invariants).
struct HipBackend {
  using Stream = hipStream_t;
  using Event = hipEvent_t;
  // Only this device's streams wait on the event (hipStreamWaitEvent), so a
  // device-scope release is enough; the default system-scope fence would write
  // back and invalidate L2 at the end of every call.
  int create_event(hipEvent_t* e) {
    return hipEventCreateWithFlags(e, hipEventDisableTiming | hipEventReleaseToDevice);
  }
  int record(hipEvent_t e, hipStream_t s) { return hipEventRecord(e, s); }
  int stream_wait(hipStream_t s, hipEvent_t e) { return hipStreamWaitEvent(s, e, 0); }
  int malloc_async(void** p, size_t n, hipStream_t s) { return hipMallocAsync(p, n, s); }
  int free_async(void* p, hipStream_t s) { return hipFreeAsync(p, s); }
};
HipBackend g_hip_backend;
attn::WorkspaceCache<HipBackend> g_ws(g_hip_backend);

// A lease of the calling stream's buffer for one call: acquire() before the
// first launch, release() after the last (also on every error path).
class WorkspaceLease {
 public:
  explicit WorkspaceLease(hipStream_t s) : s_(s) {}
  ~WorkspaceLease() { (void)release(); }
  hipError_t acquire(size_t bytes) {
    int dev = 0;
    hipError_t e = s_ ? hipStreamGetDevice(s_, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    return (hipError_t)g_ws.acquire(dev, s_, bytes, &l_);
  }
  void* ptr() const { return l_.ptr; }
  hipError_t release() { return (hipError_t)g_ws.release(s_, &l_); }

 private:
  hipStream_t s_;
  attn::WorkspaceCache<HipBackend>::Lease l_;
};

// ---- the no-allocation entry point's scratch memory: one array per device,
// held from the library's first use on that device until the process ends.
// Host code reaches it only through the address hipGetSymbolAddress gives for
// the current device (the array's name is a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of `scratch` on device `dev`, looked up once per device with
// that device current.
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& sl = g_scratch[dev];
  std::call_once(sl.once, [&] {
    int cur = -1;
    sl.err = hipGetDevice(&cur);
    if (sl.err == hipSuccess && cur != dev) sl.err = hipSetDevice(dev);
    if (sl.err == hipSuccess) sl.err = hipGetSymbolAddress(&sl.ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t e = hipSetDevice(cur);
      if (sl.err == hipSuccess) sl.err = e;
    }
    if (sl.err != hipSuccess) sl.ptr = nullptr;
  });
  *out = sl.ptr;
  return sl.err;
}

// Where one call's scratch memory comes from: the stream's leased workspace
// (grown as needed), or -- for the no-allocation entry point -- the device's
// fixed `scratch` array, whose capacity bounds what the call may use.  get()
// is the first HIP call a forward call makes, after every host check.
class Scratch {
 public:
  Scratch(hipStream_t s, bool fixed) : s_(s), fixed_(fixed), lease_(s) {}
  bool fixed() const { return fixed_; }
  static constexpr int64_t capacity() { return ATTN_NOALLOC_SCRATCH_BYTES; }
  hipError_t get(size_t bytes, void** p) {
    if (!fixed_) {
      const hipError_t e = lease_.acquire(bytes);
      *p = lease_.ptr();
      return e;
    }
    if ((int64_t)bytes > capacity()) return hipErrorInvalidValue;  // callers size to capacity()
    int dev = 0;
    const hipError_t e = s_ ? hipStreamGetDevice(s_, &dev) : hipGetDevice(&dev);
    return e != hipSuccess ? e : scratch_address(dev, p);
  }
  hipError_t release() { return fixed_ ? hipSuccess : lease_.release(); }

 private:
  hipStream_t s_;
  bool fixed_;
  WorkspaceLease lease_;
};

// ---- kernel timing (benchmarks only).
struct TimingRecord {
  int id;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing = false;
std::vector<TimingRecord> g_records;
std::vector<hipEvent_t> g_free_events;  // reused across calls (creating events is slow)

hipError_t take_event(hipEvent_t* ev) {
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (!g_free_events.empty()) {
      *ev = g_free_events.back();
      g_free_events.pop_back();
      return hipSuccess;
    }
  }
  // Timestamps only, read after the caller synchronises: no system-scope
  // fence, which would write back and invalidate L2 between the kernels timed.
  return hipEventCreateWithFlags(ev, hipEventDisableSystemFence);
}

void give_event(hipEvent_t ev) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_free_events.push_back(ev);
}

bool timing_on() {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  return g_timing;
}

template <class F>
hipError_t timed(int id, hipStream_t s, bool on, F&& launch) {
  if (!on) return launch();
  TimingRecord r{id, nullptr, nullptr};
  hipError_t e = take_event(&r.start);
  if (e == hipSuccess) e = take_event(&r.stop);
  if (e == hipSuccess) e = hipEventRecord(r.start, s);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(r.stop, s);
  if (e != hipSuccess) {
    if (r.start) give_event(r.start);
    if (r.stop) give_event(r.stop);
    return e;
  }
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_records.push_back(r);
  return hipSuccess;
}

int run_two_pass(const void* q, const void* k, const void* v, void* out, float* lse,
                 attn::HeadMap hm, int64_t BH, int64_t L, int64_t d, float sl2,
                 const attn::Band& band, hipStream_t stream, Scratch& sc, bool on) {
  const attn::TwoPassDims t = attn::two_pass_dims(L, d);
  const int64_t per_head = attn::two_pass_head_bytes(t);
  // A fixed scratch array holds the chunk's staging (checked by the caller to
  // fit one head); the values pass's key split is dropped for a chunk whose
  // partial outputs would not fit next to it.
  const int64_t chunk = sc.fixed() ? heads_per_chunk(BH, per_head, Scratch::capacity())
                                   : heads_per_chunk(BH, per_head);
  const int64_t need = sc.fixed() ? Scratch::capacity() : two_pass_workspace_bytes(BH, t, band);

  void* ws = nullptr;
  if (sc.get((size_t)need, &ws) != hipSuccess) return ATTN_ERR_WORKSPACE;
  char* base = (char*)ws;

  hipError_t err = hipSuccess;
  for (int64_t h0 = 0; h0 < BH && err == hipSuccess; h0 += chunk) {
    const int n = (int)((BH - h0) < chunk ? (BH - h0) : chunk);
    hm.bh0 = (int)h0;  // the kernels find the chunk's heads through the map
    // This chunk's layout: E, the two statistics tables, the partial outputs.
    const int64_t e_bytes = round256((int64_t)t.QB * t.EB * 1024) * n;
    const int64_t st_bytes = round256((int64_t)t.TK * t.L * 4) * n;
    void* E = base;
    float* mref = (float*)(base + e_bytes);
    float* psum = (float*)(base + e_bytes + st_bytes);
    float* part = (float*)(base + e_bytes + 2 * st_bytes);
    int split = attn::values_split(n, t, band);
    if (split > 1 && chunk_workspace_bytes(n, t, band) > need) split = 1;
    err = timed(ATTN_KERNEL_SCORES, stream, on, [&] {
      return attn::launch_scores(q, k, E, mref, psum, hm, n, t, sl2, band, stream);
    });
    if (err == hipSuccess)
      err = timed(ATTN_KERNEL_VALUES, stream, on, [&] {
        return attn::launch_values(v, E, mref, psum, out, lse, part, split, hm, n, t, band,
                                   stream);
      });
    if (err == hipSuccess && split > 1)
      err = timed(ATTN_KERNEL_VALUES_REDUCE, stream, on, [&] {
        return attn::launch_values_reduce(part, out, split, hm, n, t, stream);
      });
  }
  const hipError_t rerr = sc.release();
  if (err != hipSuccess || rerr != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

// Checks shared by both forward entry points, after the shape and pointer
// checks: the kernels' 32-bit offsets and int head counts, then the launches.
// ld_max: the largest row stride of q, k and v (elements).
int forward(const void* q, const void* k, const void* v, void* out, float* lse,
            const attn::HeadMap& hm, int64_t bh, int64_t L, int64_t d, int64_t ld_max,
            float scale, const attn::Band& band, hipStream_t stream, bool fixed_scratch = false) {
  // Kernels address one head with 32-bit byte offsets (rows up to L + 255 are
  // formed, past-the-end ones read as zero) and count heads in int.
  if ((L + 256) * ld_max * 2 >= ((int64_t)1 << 31) || bh >= ((int64_t)1 << 31) / 1024)
    return ATTN_ERR_TOO_LARGE;
  const float sl2 = scale * 1.4426950408889634f;

  if (attn_path_for_head_dim(d) == ATTN_PATH_ONLINE) {
    const int64_t nqb = (L + 127) / 128;
    int nsplit = attn::online_split(bh, L, L);
    // A fixed scratch array: as many shares as fit (one share needs none).
    auto share_bytes = [&](int n) { return round256((int64_t)n * bh * L * (d + 2) * 4); };
    while (fixed_scratch && nsplit > 1 && share_bytes(nsplit) > Scratch::capacity()) --nsplit;
    if (nqb * bh * nsplit >= ((int64_t)1 << 31)) return ATTN_ERR_TOO_LARGE;
    const bool on = !fixed_scratch && timing_on();
    attn::KeySplit ks{nullptr, nullptr, 1, (int)bh};
    Scratch ws(stream, fixed_scratch);
    if (nsplit > 1) {  // few heads: the keys of each query block are split
      void* p = nullptr;
      if (ws.get((size_t)share_bytes(nsplit), &p) != hipSuccess) return ATTN_ERR_WORKSPACE;
      ks.part = (float*)p;
      ks.stats = ks.part + (size_t)nsplit * bh * L * d;
      ks.n = nsplit;
    }
    hipError_t e = timed(ATTN_KERNEL_ONLINE, stream, on, [&] {
      return attn::launch_online(q, k, v, out, lse, hm, (int)bh, (int)L, (int)d, sl2, band,
                                 attn::VarSeqs{nullptr, nullptr, 0, 0, 0}, ks, stream);
    });
    if (e == hipSuccess && nsplit > 1)
      e = timed(ATTN_KERNEL_ONLINE_COMBINE, stream, on, [&] {
        return attn::launch_online_combine(ks, out, lse, hm, (int)L, (int)d,
                                           attn::VarSeqs{nullptr, nullptr, 0, 0, 0}, stream);
      });
    const hipError_t rerr = ws.release();
    return e == hipSuccess && rerr == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  }
  const attn::TwoPassDims t = attn::two_pass_dims(L, d);
  // One head's E is addressed with 32-bit byte offsets.
  if (t.TK > attn::kTwoPassMaxTiles || (int64_t)t.QB * t.EB * 1024 >= ((int64_t)1 << 32) - 1 ||
      (int64_t)t.T * t.TK * bh >= ((int64_t)1 << 31))
    return ATTN_ERR_TOO_LARGE;
  if (fixed_scratch && attn::two_pass_head_bytes(t) > Scratch::capacity())
    return ATTN_ERR_SCRATCH_TOO_SMALL;
  Scratch sc(stream, fixed_scratch);
  return run_two_pass(q, k, v, out, lse, hm, bh, L, d, sl2, band, stream, sc,
                      !fixed_scratch && timing_on());
}

// One operand of attn_forward_ex: dims [B, heads, L, d] with element strides
// st[0..2] (batch, head, row) and unit channel stride.
struct View {
  int64_t n[3];
  int64_t st[3];
  int64_t d;
  // Elements from the first to one past the last addressed element.
  int64_t span() const {
    int64_t e = d;
    for (int i = 0; i < 3; ++i) e += (n[i] - 1) * st[i];
    return e;
  }
  bool strides_valid() const {
    for (int i = 0; i < 3; ++i)
      if (st[i] < 0 || st[i] % 8 != 0) return false;
    return st[2] >= d;
  }
  // No two elements share an address: with the dims of extent > 1 sorted by
  // stride, each stride is at least the span of the smaller ones.
  bool one_to_one() const {
    int idx[3] = {0, 1, 2};
    std::sort(idx, idx + 3, [&](int a, int b) { return st[a] < st[b]; });
    int64_t span_below = d;
    for (int i : idx) {
      if (n[i] <= 1) continue;
      if (st[i] < span_below) return false;
      span_below += (n[i] - 1) * st[i];
    }
    return true;
  }
};

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL_PTR: return "a tensor pointer is NULL";
    case ATTN_ERR_BAD_SHAPE: return "a size is negative or the byte sizes overflow";
    case ATTN_ERR_UNSUPPORTED_HEAD_DIM:
      return "unsupported head dimension: need 32, 64, 128, or a multiple of 64 in (128, 1024]";
    case ATTN_ERR_BAD_SCALE: return "scale is not finite";
    case ATTN_ERR_MISALIGNED: return "a tensor pointer is not 16-byte aligned";
    case ATTN_ERR_ALIAS: return "out overlaps q, k or v";
    case ATTN_ERR_WORKSPACE: return "workspace allocation failed";
    case ATTN_ERR_HIP: return "a HIP launch or runtime call failed";
    case ATTN_ERR_TOO_LARGE: return "problem too large: one head exceeds 32-bit byte offsets, or L > 15872 with d > 128";
    case ATTN_ERR_BAD_MASK: return "the compressed causal mask takes no window";
    case ATTN_ERR_SCRATCH_TOO_SMALL:
      return "attn_forward_noalloc: one head needs more scratch memory than its fixed "
             "per-device array holds (ATTN_NOALLOC_SCRATCH_BYTES)";
    case ATTN_ERR_BAD_STRIDE:
      return "bad strides: negative, not a multiple of 8 elements, a row stride below d, or an "
             "output layout whose elements overlap";
    default: return "unknown status";
  }
}

int attn_path_for_head_dim(int64_t d) {
  if (d == 32 || d == 64 || d == 128) return ATTN_PATH_ONLINE;
  if (head_dim_supported(d)) return ATTN_PATH_TWO_PASS;
  return ATTN_PATH_NONE;
}

int64_t attn_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t d, int causal) {
  if (B < 0 || H < 0 || L < 0 || attn_path_for_head_dim(d) == ATTN_PATH_NONE) return 0;
  if (B == 0 || H == 0 || L == 0) return 0;
  if (L > (int64_t)1 << 20) return 0;
  if (attn_path_for_head_dim(d) == ATTN_PATH_ONLINE) return online_workspace_bytes(B * H, L, d);
  const attn::TwoPassDims t = attn::two_pass_dims(L, d);
  return two_pass_workspace_bytes(B * H, t, attn::make_band(-1, -1, causal != 0, L));
}

// attn_forward's and attn_forward_noalloc's argument checks; *bh = B * H.
// Returns -1 when every check passed and there is work to do.
static int check_forward_args(const void* q, const void* k, const void* v, const void* out, int64_t B,
                       int64_t H, int64_t L, int64_t d, float scale, int64_t* bh_out) {
  if (B < 0 || H < 0 || L < 0 || d < 0) return ATTN_ERR_BAD_SHAPE;
  int64_t bh = 0, rows = 0, elems = 0, bytes = 0;
  if (__builtin_mul_overflow(B, H, &bh) || __builtin_mul_overflow(bh, L, &rows) ||
      __builtin_mul_overflow(rows, d, &elems) || __builtin_mul_overflow(elems, (int64_t)2, &bytes))
    return ATTN_ERR_BAD_SHAPE;
  if (!head_dim_supported(d)) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  if (rows == 0) return ATTN_OK;
  if (!q || !k || !v || !out) return ATTN_ERR_NULL_PTR;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return ATTN_ERR_MISALIGNED;
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
    return ATTN_ERR_ALIAS;
  if (L > ((int64_t)1 << 30) || H > ((int64_t)1 << 30)) return ATTN_ERR_TOO_LARGE;
  *bh_out = bh;
  return -1;
}

int attn_forward(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t H,
                 int64_t L, int64_t d, float scale, int causal, hipStream_t stream) {
  int64_t bh = 0;
  const int st = check_forward_args(q, k, v, out, B, H, L, d, scale, &bh);
  if (st >= 0) return st;
  return forward(q, k, v, out, nullptr, attn::contiguous_heads((int)H, (int)L, (int)d), bh, L, d,
                 d, scale, attn::make_band(-1, -1, causal != 0, L), stream);
}

int attn_forward_noalloc(const void* q, const void* k, const void* v, void* out, int64_t B,
                         int64_t H, int64_t L, int64_t d, float scale, int causal,
                         hipStream_t stream) {
  int64_t bh = 0;
  const int st = check_forward_args(q, k, v, out, B, H, L, d, scale, &bh);
  if (st >= 0) return st;
  return forward(q, k, v, out, nullptr, attn::contiguous_heads((int)H, (int)L, (int)d), bh, L, d,
                 d, scale, attn::make_band(-1, -1, causal != 0, L), stream, true);
}

int attn_forward_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                    int64_t B, int64_t H, int64_t H_kv, int64_t L, int64_t d,
                    const int64_t* q_strides, const int64_t* k_strides,
                    const int64_t* v_strides, const int64_t* o_strides, float scale, int causal,
                    int64_t window_left, int64_t window_right, hipStream_t stream) {
  if (B < 0 || H < 0 || H_kv < 0 || L < 0 || d < 0) return ATTN_ERR_BAD_SHAPE;
  if (window_left < -1 || window_right < -1) return ATTN_ERR_BAD_SHAPE;
  int64_t bh = 0, rows = 0, elems = 0, bytes = 0;
  if (__builtin_mul_overflow(B, H, &bh) || __builtin_mul_overflow(bh, L, &rows) ||
      __builtin_mul_overflow(rows, d, &elems) || __builtin_mul_overflow(elems, (int64_t)2, &bytes))
    return ATTN_ERR_BAD_SHAPE;
  if (H > 0 && (H_kv < 1 || H % H_kv != 0)) return ATTN_ERR_BAD_SHAPE;
  if (!head_dim_supported(d)) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  if (rows == 0) return ATTN_OK;
  if (!q || !k || !v || !out) return ATTN_ERR_NULL_PTR;
  if (L > ((int64_t)1 << 30) || H > ((int64_t)1 << 30)) return ATTN_ERR_TOO_LARGE;

  // Views with the default (contiguous) strides where none are given.
  auto make = [&](const int64_t* st, int64_t heads) {
    View w{{B, heads, L}, {heads * L * d, L * d, d}, d};
    if (st)
      for (int i = 0; i < 3; ++i) w.st[i] = st[i];
    return w;
  };
  const View vq = make(q_strides, H), vk = make(k_strides, H_kv), vv = make(v_strides, H_kv),
             vo = make(o_strides, H);
  for (const View* w : {&vq, &vk, &vv, &vo}) {
    if (!w->strides_valid()) return ATTN_ERR_BAD_STRIDE;
    // Spans beyond int64 bytes cannot describe memory.
    if (w->st[0] > (INT64_MAX / 8) / std::max<int64_t>(B, 1) ||
        w->st[1] > (INT64_MAX / 8) / std::max<int64_t>(H, 1) ||
        w->st[2] > (INT64_MAX / 8) / std::max<int64_t>(L, 1))
      return ATTN_ERR_BAD_STRIDE;
  }
  if (!vo.one_to_one()) return ATTN_ERR_BAD_STRIDE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15 || ((uintptr_t)lse & 3))
    return ATTN_ERR_MISALIGNED;
  const int64_t ob = vo.span() * 2;
  if (overlaps(out, ob, q, vq.span() * 2) || overlaps(out, ob, k, vk.span() * 2) ||
      overlaps(out, ob, v, vv.span() * 2))
    return ATTN_ERR_ALIAS;
  if (lse) {
    const int64_t lb = rows * 4;
    if (overlaps(lse, lb, out, ob) || overlaps(lse, lb, q, vq.span() * 2) ||
        overlaps(lse, lb, k, vk.span() * 2) || overlaps(lse, lb, v, vv.span() * 2))
      return ATTN_ERR_ALIAS;
  }
  for (const View* w : {&vq, &vk, &vv, &vo})
    if (w->st[2] >= ((int64_t)1 << 30)) return ATTN_ERR_TOO_LARGE;

  attn::HeadMap hm;
  hm.H = (int)H;
  hm.group = (int)(H / H_kv);
  hm.bh0 = 0;
  hm.q = {vq.st[0], vq.st[1], (int)vq.st[2]};
  hm.k = {vk.st[0], vk.st[1], (int)vk.st[2]};
  hm.v = {vv.st[0], vv.st[1], (int)vv.st[2]};
  hm.o = {vo.st[0], vo.st[1], (int)vo.st[2]};
  const int64_t ld_max = std::max(vq.st[2], std::max(vk.st[2], vv.st[2]));
  return forward(q, k, v, out, lse, hm, bh, L, d, ld_max, scale,
                 attn::make_band(window_left, window_right, causal != 0, L), stream);
}

int attn_forward_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                        const int32_t* cu_seqlens, int64_t B, int64_t max_seqlen, int64_t total,
                        const int32_t* cu_seqlens_k, int64_t max_seqlen_k, int64_t total_k,
                        int64_t H, int64_t H_kv, int64_t d, const int64_t* q_strides,
                        const int64_t* k_strides, const int64_t* v_strides,
                        const int64_t* o_strides, float scale, int causal, int64_t window_left,
                        int64_t window_right, hipStream_t stream) {
  if (!cu_seqlens_k) {  // keys share the query offsets and lengths
    max_seqlen_k = max_seqlen;
    total_k = total;
  }
  if (B < 0 || max_seqlen < 0 || total < 0 || H < 0 || H_kv < 0 || d < 0 || max_seqlen_k < 0 ||
      total_k < 0)
    return ATTN_ERR_BAD_SHAPE;
  if (window_left < -1 || window_right < -1) return ATTN_ERR_BAD_SHAPE;
  const bool compressed = causal == ATTN_MASK_COMPRESSED_CAUSAL;
  if (compressed && (window_left != -1 || window_right != -1)) return ATTN_ERR_BAD_MASK;
  int64_t rows = 0, elems = 0, bytes = 0, bh = 0, slots = 0;
  if (__builtin_mul_overflow(total, H, &rows) || __builtin_mul_overflow(rows, d, &elems) ||
      __builtin_mul_overflow(elems, (int64_t)2, &bytes) || __builtin_mul_overflow(B, H, &bh) ||
      __builtin_mul_overflow(bh, max_seqlen, &slots))
    return ATTN_ERR_BAD_SHAPE;
  if (H > 0 && (H_kv < 1 || H % H_kv != 0)) return ATTN_ERR_BAD_SHAPE;
  if (attn_path_for_head_dim(d) != ATTN_PATH_ONLINE) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  if (rows == 0 || slots == 0) return ATTN_OK;
  // With no key tokens at all, k and v are never read and may be NULL.
  if (!q || !out || !cu_seqlens || (total_k > 0 && (!k || !v))) return ATTN_ERR_NULL_PTR;

  // Operands as [1, heads, tokens] views: strides {token, head} given, channels contiguous.
  auto make = [&](const int64_t* st, int64_t heads, int64_t tokens) {
    View w{{1, heads, tokens}, {0, d, heads * d}, d};
    if (st) {
      w.st[2] = st[0];
      w.st[1] = st[1];
    }
    return w;
  };
  const View vq = make(q_strides, H, total), vk = make(k_strides, H_kv, total_k),
             vv = make(v_strides, H_kv, total_k), vo = make(o_strides, H, total);
  for (const View* w : {&vq, &vk, &vv, &vo}) {
    if (!w->strides_valid()) return ATTN_ERR_BAD_STRIDE;
    if (w->st[1] > (INT64_MAX / 8) / std::max<int64_t>(H, 1) ||
        w->st[2] > (INT64_MAX / 8) / std::max<int64_t>(std::max(total, total_k), 1))
      return ATTN_ERR_BAD_STRIDE;
  }
  if (!vo.one_to_one()) return ATTN_ERR_BAD_STRIDE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15 ||
      ((uintptr_t)lse & 3) || ((uintptr_t)cu_seqlens & 3) || ((uintptr_t)cu_seqlens_k & 3))
    return ATTN_ERR_MISALIGNED;
  const int64_t ob = vo.span() * 2, cb = (B + 1) * 4;
  // Empty key views (total_k == 0) address nothing.
  const int64_t kb = total_k > 0 ? vk.span() * 2 : 0, vb = total_k > 0 ? vv.span() * 2 : 0;
  const int64_t ckb = cu_seqlens_k ? cb : 0;
  if (overlaps(out, ob, q, vq.span() * 2) || overlaps(out, ob, k, kb) || overlaps(out, ob, v, vb) ||
      overlaps(out, ob, cu_seqlens, cb) || overlaps(out, ob, cu_seqlens_k, ckb))
    return ATTN_ERR_ALIAS;
  if (lse) {
    const int64_t lb = rows * 4;
    if (overlaps(lse, lb, out, ob) || overlaps(lse, lb, q, vq.span() * 2) ||
        overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, vb) ||
        overlaps(lse, lb, cu_seqlens, cb) || overlaps(lse, lb, cu_seqlens_k, ckb))
      return ATTN_ERR_ALIAS;
  }
  // One sequence per 32-bit offsets (rows up to max_seqlen + 255 are formed),
  // token indices and workgroup counts in int.
  const int64_t ld_kv = std::max(vk.st[2], vv.st[2]);
  for (const View* w : {&vq, &vk, &vv, &vo})
    if (w->st[2] >= ((int64_t)1 << 30) || w->st[1] >= ((int64_t)1 << 30)) return ATTN_ERR_TOO_LARGE;
  if (max_seqlen > ((int64_t)1 << 30) || max_seqlen_k > ((int64_t)1 << 30) ||
      total >= ((int64_t)1 << 31) - 1 || total_k >= ((int64_t)1 << 31) - 1 ||
      (max_seqlen + 256) * vq.st[2] * 2 >= ((int64_t)1 << 31) ||
      (max_seqlen_k + 256) * ld_kv * 2 >= ((int64_t)1 << 31) || H >= ((int64_t)1 << 30) ||
      (max_seqlen + 127) / 128 * bh >= ((int64_t)1 << 31))
    return ATTN_ERR_TOO_LARGE;

  attn::HeadMap hm;
  hm.H = (int)H;
  hm.group = (int)(H / H_kv);
  hm.bh0 = 0;
  hm.q = {0, vq.st[1], (int)vq.st[2]};
  hm.k = {0, vk.st[1], (int)vk.st[2]};
  hm.v = {0, vv.st[1], (int)vv.st[2]};
  hm.o = {0, vo.st[1], (int)vo.st[2]};
  attn::Band band =
      attn::make_band(window_left, window_right, causal != 0, std::max(max_seqlen, max_seqlen_k) + 1);
  band.compressed = compressed ? 1 : 0;
  const float sl2 = scale * 1.4426950408889634f;
  const attn::VarSeqs vs{cu_seqlens, cu_seqlens_k, (int)total, (int)total_k, (int)max_seqlen_k};
  // Few (sequence, head) pairs -- e.g. decoding against long caches: split the keys.
  const int nsplit = attn::online_split(bh, max_seqlen, max_seqlen_k);
  if ((max_seqlen + 127) / 128 * bh * nsplit >= ((int64_t)1 << 31)) return ATTN_ERR_TOO_LARGE;
  const bool on = timing_on();
  attn::KeySplit ks{nullptr, nullptr, 1, (int)bh};
  WorkspaceLease ws(stream);
  if (nsplit > 1) {
    const int64_t bytes = round256((int64_t)nsplit * bh * max_seqlen * (d + 2) * 4);
    if (ws.acquire((size_t)bytes) != hipSuccess) return ATTN_ERR_WORKSPACE;
    ks.part = (float*)ws.ptr();
    ks.stats = ks.part + (size_t)nsplit * bh * max_seqlen * d;
    ks.n = nsplit;
  }
  hipError_t e = timed(ATTN_KERNEL_ONLINE, stream, on, [&] {
    return attn::launch_online(q, k, v, out, lse, hm, (int)bh, (int)max_seqlen, (int)d, sl2, band,
                               vs, ks, stream);
  });
  if (e == hipSuccess && nsplit > 1)
    e = timed(ATTN_KERNEL_ONLINE_COMBINE, stream, on, [&] {
      return attn::launch_online_combine(ks, out, lse, hm, (int)max_seqlen, (int)d, vs, stream);
    });
  const hipError_t rerr = ws.release();
  return e == hipSuccess && rerr == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing = enable != 0;
  return ATTN_OK;
}

int attn_timing_collect(double* sum_ms, int64_t* launches, int n) {
  std::vector<TimingRecord> recs;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    recs.swap(g_records);
  }
  int status = ATTN_OK;
  for (const TimingRecord& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      status = ATTN_ERR_HIP;
    else if (r.id >= 0 && r.id < n) {
      if (sum_ms) sum_ms[r.id] += ms;
      if (launches) launches[r.id] += 1;
    }
    give_event(r.start);
    give_event(r.stop);
  }
  return status;
}

}  // extern "C"
