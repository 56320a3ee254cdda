/*
 * attn.h -- C ABI of the MI355X (gfx950) exact softmax attention library.
 *
 * The operation (FastVideo wan22_vae_decode attn.cu, header comment and
 * row_softmax_kernel; cuDNN native_sparse_attention fmha.py, module docstring
 * and softmax_step): for every batch b and head h,
 *
 *     O[b,h] = softmax( scale * Q[b,h] K[b,h]^T ) V[b,h]
 *
 * where the softmax runs over keys with the row maximum subtracted first, and,
 * when causal is nonzero, key j is allowed for query i only if j <= i.  Both
 * contractions accumulate in fp32; the result is rounded once to bf16.
 *
 * Conventions shared by every entry point:
 *   - q, k, v, out are device pointers to bf16 values (raw 16-bit patterns),
 *     each a row-major contiguous [B, H, L, d] tensor; q, k, v share L and d.
 *   - The caller owns all four buffers and keeps them alive until the work
 *     queued on `stream` has finished.  `out` is written, never read, and must
 *     not overlap q, k or v.  The library keeps no reference to them.
 *   - Work is queued asynchronously on `stream` (0 = the null stream); no
 *     entry point synchronises the device.
 *   - Every argument is checked on the host before any HIP call; a failed check
 *     returns its status code and queues nothing.  No exception crosses the ABI.
 *   - Thread safety: any number of host threads may call concurrently, on the
 *     same stream or on different ones.  A call that needs scratch memory leases
 *     the workspace buffer the library keeps for (device, stream) from before
 *     its first launch until after its last, under that buffer's lock: calls on
 *     one stream queue their kernels one call after another (never interleaved
 *     over the buffer), calls on different streams never wait for each other.
 *     A buffer grows stream-ordered (hipFreeAsync of the old one and
 *     hipMallocAsync of the new one on the caller's stream), so no call
 *     synchronises the device or waits on the host for the GPU.  The buffers
 *     live until the process ends.
 */
#ifndef ATTN_MI355X_ATTN_H
#define ATTN_MI355X_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (the pages' host code throws on bad shapes -- attn.cu's
 * attn_forward checks, fmha.py's __call__ type errors; here they are returns). */
enum {
  ATTN_OK = 0,                       /* success; also B*H*L == 0 (nothing queued) */
  ATTN_ERR_NULL_PTR = 1,             /* q, k, v or out is NULL (with B*H*L > 0)   */
  ATTN_ERR_BAD_SHAPE = 2,            /* a negative size, or byte sizes overflow   */
  ATTN_ERR_UNSUPPORTED_HEAD_DIM = 3, /* d not in {32,64,128} nor 128<d<=1024, d%64==0 */
  ATTN_ERR_BAD_SCALE = 4,            /* scale is NaN or infinite                  */
  ATTN_ERR_MISALIGNED = 5,           /* a pointer is not 16-byte aligned          */
  ATTN_ERR_ALIAS = 6,                /* out overlaps q, k or v                    */
  ATTN_ERR_WORKSPACE = 7,            /* the stream-ordered workspace allocation failed */
  ATTN_ERR_HIP = 8,                  /* a HIP launch or runtime call failed       */
  ATTN_ERR_TOO_LARGE = 9,            /* one head exceeds the kernels' 32-bit byte offsets,
                                        or L > 15872 with d > 128 (the values pass keeps a
                                        byte per 128 keys and query of its tile in LDS) */
  ATTN_ERR_BAD_STRIDE = 10,          /* attn_forward_ex: a stride is negative or not a multiple
                                        of 8, a row stride is below d, or out's elements overlap */
  ATTN_ERR_BAD_MASK = 11,            /* attn_forward_varlen: the compressed causal mask
                                        combined with a window                   */
  ATTN_ERR_SCRATCH_TOO_SMALL = 12    /* attn_forward_noalloc: one head needs more scratch
                                        than ATTN_NOALLOC_SCRATCH_BYTES          */
};

/* Values of the `causal` argument.  attn_forward and attn_forward_ex treat
 * every nonzero value as ATTN_MASK_CAUSAL (with equal query and key lengths the
 * compressed causal mask is the causal mask); attn_forward_varlen also takes
 * ATTN_MASK_COMPRESSED_CAUSAL. */
enum {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_CAUSAL = 1,
  ATTN_MASK_COMPRESSED_CAUSAL = 2
};

/* Kernel paths chosen by head dimension. */
enum {
  ATTN_PATH_NONE = -1,
  ATTN_PATH_ONLINE = 0,   /* d in {32, 64, 128}: one fused online-softmax kernel  */
  ATTN_PATH_TWO_PASS = 1  /* 128 < d <= 1024, d % 64 == 0: scores pass + values pass */
};

/*
 * attn_forward -- O = softmax(scale * Q K^T) V on bf16 [B,H,L,d] tensors.
 *
 *   q, k, v : const device pointers, bf16 [B,H,L,d] contiguous, 16-byte aligned.
 *   out     : device pointer, bf16 [B,H,L,d] contiguous, 16-byte aligned.
 *   B, H, L : batch, heads, sequence length (>= 0; B*H*L == 0 queues nothing).
 *   d       : head dimension: 32, 64, 128, or a multiple of 64 in (128, 1024].
 *   scale   : finite logit scale (any sign, 0 allowed); callers usually pass 1/sqrt(d).
 *   causal  : 0 = no mask; nonzero = key j allowed for query i iff j <= i.
 *   stream  : HIP stream the kernels are queued on.
 *
 * Returns ATTN_OK or one of the codes above.  For d <= 128 with so few heads
 * that most compute units would idle, the keys of each 128-query block are
 * split among up to 8 workgroups whose fp32 shares of O and (max, sum) pairs
 * are merged by a second kernel (a split over keys with a log-sum-exp style
 * combine); that uses the workspace buffer below too (attn_workspace_bytes
 * gives its size).  For d > 128 the call uses the
 * workspace buffer the library keeps for (current device, stream), growing it
 * when needed (about 16384*ceil(L/32)*ceil(L/256) + 8*L*ceil(L/128) bytes per
 * head, heads processed in chunks of at most 2 GiB).  When so few heads would
 * leave most compute units idle, the values pass runs on 128 x 128 tiles if
 * they fit the compute units in one round, and otherwise splits the keys,
 * adding up to 3 fp32 copies of the output to the workspace
 * (attn_workspace_bytes gives the exact figure).
 * Neither growing nor reusing the buffer waits on the host (see the thread
 * safety note above).
 */
int attn_forward(const void* q, const void* k, const void* v, void* out,
                 int64_t B, int64_t H, int64_t L, int64_t d,
                 float scale, int causal, hipStream_t stream);

/*
 * attn_forward_noalloc -- attn_forward for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, checks, results and
 * status codes as attn_forward; it calls no hipMalloc, hipFree, stream-ordered
 * allocator or other allocating routine, and records no timing events.
 *
 * Scratch memory (the large-head-dim path's staged exponentials and
 * statistics, the few-heads key splits' partial outputs) comes from one
 * statically sized device array per GPU, ATTN_NOALLOC_SCRATCH_BYTES long, which
 * each GPU the library runs on holds from the first such call until the
 * process ends.  Heads are processed in chunks that fit it, and a key split is
 * narrowed (or dropped) when its shares would not fit.  When one head of the
 * large-head-dim path alone needs more than the array holds (about
 * 16384 * ceil(L / 32) * ceil(L / 256) + 8 * L * ceil(L / 128) bytes for
 * d > 128, i.e. L above 7936) the call returns ATTN_ERR_SCRATCH_TOO_SMALL
 * before any HIP call and queues nothing.  Nothing in the array has to start
 * at zero: every call writes the scratch it reads.
 *
 * All calls on one GPU share that GPU's array: calls whose work may overlap on
 * the device (different streams, or different host threads without ordering)
 * race on it and give undefined results.  Serialise them (one stream, calls
 * made in order) or use attn_forward.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (128u << 20)
int attn_forward_noalloc(const void* q, const void* k, const void* v, void* out,
                         int64_t B, int64_t H, int64_t L, int64_t d,
                         float scale, int causal, hipStream_t stream);

/*
 * attn_forward_ex -- the same operation on strided operands, with key/value
 * heads shared by groups of query heads and an optional log-sum-exp output.
 *
 * What it adds, and where it comes from: FastVideo wan22_vae_decode attn.cu,
 * attn_forward, takes one packed [T, 1, HW, 3C] qkv tensor (frames T,
 * positions HW, channels C) and reads q and k in place with a position stride
 * of 3C; q, k and v are the channel ranges [0, C), [C, 2C), [2C, 3C).  Here:
 * q = qkv, k = qkv + C, v = qkv + 2C (element offsets), B = T, H = H_kv = 1,
 * L = HW, d = C and strides {HW*3C, HW*3C, 3C} for all three; nothing is
 * copied.  cuDNN native_sparse_attention fmha.py, __call__, takes per-tensor
 * strides, lets the query heads be a multiple of the key/value heads (each
 * key/value head broadcast over its group of consecutive query heads) and
 * optionally writes each row's log-sum-exp (log of the row sum plus the
 * scaled row maximum, stored in its epilogue); it also takes a sliding window
 * (window_size_left / window_size_right).
 *
 *   q, out        : [B, H, L, d] views; k, v : [B, H_kv, L, d] views.  Each is a
 *                   device pointer to its element [0,0,0,0] plus three element
 *                   strides (batch, head, row) in a host array of 3 int64_t;
 *                   NULL means contiguous ({heads*L*d, L*d, d}).  Channels are
 *                   always contiguous.  Strides must be >= 0 and multiples of 8
 *                   (16-byte rows), row strides >= d; zero batch or head
 *                   strides broadcast an input.  out's strides must map every
 *                   element to its own address.  Pointers 16-byte aligned.
 *   lse           : NULL, or a device pointer to fp32 [B, H, L] contiguous
 *                   (4-byte aligned) that receives, per query row i, the
 *                   natural log of its softmax denominator:
 *                   lse[i] = log(sum over allowed j of exp(scale * q_i . k_j)).
 *   H_kv          : key/value heads, >= 1 and dividing H; query head h reads
 *                   key/value head h / (H / H_kv) of the same batch entry.
 *   window_left,  : a sliding window (fmha.py's window_size_left / _right):
 *   window_right    key j is allowed for query i only if
 *                   i - window_left <= j <= i + window_right; -1 leaves that
 *                   side unbounded (-1, -1: no window).  causal additionally
 *                   caps the right side at 0.  Every row keeps key i, so no
 *                   row is empty.  Values below -1 return ATTN_ERR_BAD_SHAPE.
 *   B, H, L, d, scale, causal, stream : as for attn_forward.
 *
 * out must not overlap q, k, v (compared as the address ranges each view
 * spans), nor lse any of them; q, k and v may overlap each other (they are
 * only read).  Returns ATTN_OK or a status code; strides are checked before
 * any HIP call like everything else.  Workspace as for attn_forward.
 */
int attn_forward_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                    int64_t B, int64_t H, int64_t H_kv, int64_t L, int64_t d,
                    const int64_t* q_strides, const int64_t* k_strides,
                    const int64_t* v_strides, const int64_t* o_strides,
                    float scale, int causal, int64_t window_left, int64_t window_right,
                    hipStream_t stream);

/*
 * attn_forward_varlen -- a batch of sequences of different lengths packed
 * along one token dimension (cuDNN native_sparse_attention fmha.py, __call__:
 * cum_seqlen_q / cum_seqlen_k, and the epilogue's LSE store at
 * row + cum_seqlen).  Sequence b's queries attend to its own keys only; the
 * two may differ in number (cross-attention, or decoding a few queries against
 * a cache), query i standing at key position i + Lk - Lq (bottom-right
 * alignment, so the last query sees the last key) for the causal and window
 * masks.  A query left with no key (possible when Lq > Lk) gives 0 and an LSE
 * of -inf.
 *
 * causal == ATTN_MASK_COMPRESSED_CAUSAL selects the compressed causal mask of
 * fmha.py's softmax (its compressed-causal mask type), where the keys compress
 * the queries: with cf = Lq / Lk (integer division, at least 1) per sequence,
 * key j is allowed for query i iff j <= (i + 1) / cf - 1, positions counted
 * from 0 within the sequence (no bottom-right shift).  The first cf - 1
 * queries see no key and give 0 (LSE -inf).  It takes no window
 * (ATTN_ERR_BAD_MASK otherwise).  Any other nonzero value is the causal mask.
 *
 *   q, out        : [total, H, d] views; k, v : [total_k, H_kv, d] views.  Each is
 *                   a device pointer to element [0,0,0] plus two element strides
 *                   (token, head) in a host array of 2 int64_t; NULL means packed
 *                   ({heads*d, d}).  Channels contiguous; strides >= 0 and
 *                   multiples of 8, token strides >= d; out one to one.
 *   lse           : NULL, or a device pointer to fp32 [total, H] contiguous, as
 *                   for attn_forward_ex (per token and head).
 *   cu_seqlens    : device pointer to B + 1 int32 offsets: sequence b is tokens
 *                   [cu_seqlens[b], cu_seqlens[b + 1]).  The caller guarantees
 *                   0 <= cu_seqlens[b] <= cu_seqlens[b + 1] <= total and that no
 *                   sequence is longer than max_seqlen; the kernels clamp every
 *                   sequence to [0, total] and max_seqlen tokens, so accesses
 *                   stay inside the views whatever the array holds.  Tokens in
 *                   no sequence are neither read as queries nor written.
 *   B, max_seqlen : sequences, and the longest one's query length (sizes the grid).
 *   total         : query tokens in the q and out views.
 *   cu_seqlens_k, : key/value offsets (device int32 [B + 1], same contract as
 *   max_seqlen_k,   cu_seqlens), the longest key length and the key tokens in
 *   total_k         the k and v views; cu_seqlens_k NULL: keys use cu_seqlens,
 *                   max_seqlen and total (self-attention), the other two ignored.
 *                   With total_k == 0, k and v may be NULL (never read): every
 *                   query sees no key and gives 0.
 *   H, H_kv, d, scale, causal, window_left, window_right, stream : as for
 *                   attn_forward_ex, positions counted within each sequence;
 *                   d must be 32, 64 or 128 (the head dims fmha.py's interface
 *                   takes), else ATTN_ERR_UNSUPPORTED_HEAD_DIM.
 *
 * When B * H * ceil(max_seqlen / 128) workgroups would leave most compute
 * units idle (e.g. decoding a few sequences against long caches) the keys are
 * split as for attn_forward, using the per-stream workspace buffer:
 * splits * B * H * max_seqlen * (d + 2) * 4 bytes, splits <= 8.  out must not
 * overlap q, k, v or either offsets array (address ranges), nor lse any of
 * them.  Returns ATTN_OK (also when nothing is to be done:
 * B, H, max_seqlen or total zero) or a status code.
 */
int attn_forward_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                        const int32_t* cu_seqlens, int64_t B, int64_t max_seqlen, int64_t total,
                        const int32_t* cu_seqlens_k, int64_t max_seqlen_k, int64_t total_k,
                        int64_t H, int64_t H_kv, int64_t d,
                        const int64_t* q_strides, const int64_t* k_strides,
                        const int64_t* v_strides, const int64_t* o_strides,
                        float scale, int causal, int64_t window_left, int64_t window_right,
                        hipStream_t stream);

/* Static English text for a status code (never NULL). */
const char* attn_status_string(int status);

/* The kernel path attn_forward uses for head dimension d, or ATTN_PATH_NONE.
 * Host-only; makes no HIP call. */
int attn_path_for_head_dim(int64_t d);

/* Workspace bytes attn_forward draws for one chunk of this problem: the
 * two-pass path's staging (d > 128), or the online path's key-split shares
 * when few heads split (d <= 128); 0 when none is needed or for an invalid
 * shape.  attn_forward_ex draws at most this for the same B, H, L, d and
 * causal flag (a window can only narrow the key split); attn_forward_varlen
 * draws what its own comment states.  Host-only; makes no HIP call. */
int64_t attn_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t d, int causal);

/*
 * Kernel timing, for benchmarks.  While enabled, attn_forward records a pair of
 * HIP events around every kernel it queues (on the caller's stream).
 * attn_timing_collect waits for those events, adds each kernel's elapsed
 * milliseconds and launch count into sum_ms[id] / launches[id] for
 * id < n (ids below), and forgets the records.  Returns a status code.
 */
enum {
  ATTN_KERNEL_ONLINE = 0,  /* fused online-softmax kernel (d <= 128)              */
  ATTN_KERNEL_SCORES = 1,  /* two-pass path: S = QK^T tiles -> bf16 exp + stats   */
  ATTN_KERNEL_VALUES = 2,  /* two-pass path: O = P V with the row normalisation   */
  ATTN_KERNEL_VALUES_REDUCE = 3, /* two-pass path, few heads: sum of the key splits */
  ATTN_KERNEL_ONLINE_COMBINE = 4, /* online path, few heads: merge of the key splits  */
  ATTN_KERNEL_COUNT = 5
};
int attn_timing_enable(int enable);
int attn_timing_collect(double* sum_ms, int64_t* launches, int n);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_ATTN_H */
