/*
 * invattn.h -- C ABI of the batch-invariant attention forward library
 * (libinvattn.so, HIP for gfx950 / MI355X).
 *
 * Contract followed throughout ("RFC: Gemma-4-31B-it train/rollout
 * consistency", section 4 "Numerical contract"): every reduction has a
 * declared fp32 accumulator and an order that does not depend on batch
 * size, batch position, packing, launch geometry, CU count or occupancy;
 * no Split-K, Stream-K or cross-workgroup atomics (decode uses a split-KV
 * whose chunk size and merge order are fixed constants, declared below);
 * no fast-math; casts only at the three declared points; unsupported
 * geometry fails closed with an error and never falls back to another path.
 *
 * Arithmetic, for each query row i with allowed key set A_i, keys visited
 * in one ascending order of 32-key tiles (prefill) or 16-key cache blocks
 * (decode), c = fl32(scale * log2(e)):
 *   s_j  = fp32 MFMA dot product of bf16 q_i and bf16 k_j, head dim in
 *          ascending MFMA steps of 32
 *   m    = reference max (scaled units), -inf before the first allowed key;
 *          it moves to the tile's scaled max at the first allowed key, and
 *          after that only when the row would otherwise see large p (head
 *          dims 256 and 512: one of the row's four lanes' sums of the
 *          tile's p exceeds 2^8; head dim 64 and decode: tile max > m + 8)
 *   p_j  = exp2(fma(s_j, c, -m))          (hardware exp2, fp32; m -> 0
 *          while m = -inf)
 *   l    = l * alpha + (sum of the tile's p in a fixed order); head dims
 *          256 and 512 keep one such sum per lane and combine a row's four
 *          lanes once, after the last tile, in a fixed order
 *   acc  = acc * alpha + bf16(p) . v      (bf16 MFMA, fp32 accumulate)
 *          with alpha = exp2(m_old - m_new) on a move, else 1 (no multiply)
 *   o    = bf16_rne(acc / l)              (IEEE fp32 division)
 * The rules are fixed per (head dim, group size); a row's bytes depend
 * only on its own sequence.  Declared casts: inputs are bf16 as given;
 * p -> bf16 (round to nearest even) before the PV product; o -> bf16 (round
 * to nearest even).
 *
 * Threading: stateless apart from the thread-local error text and
 * provenance record; calls from several host threads are safe.
 * Memory: the library allocates nothing; every buffer is caller-owned
 * device memory.  Calls enqueue on the caller's stream and return without
 * synchronising (except when INVATTN_VALIDATE=1, see below).
 */
#ifndef INVATTN_H
#define INVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream handle, declared as HIP's runtime header declares it, so
 * this header needs no HIP include (the same typedef may appear twice). */
typedef struct ihipStream_t* hipStream_t;

/* Window value meaning "no window": a global (full causal) layer. */
#define ATTN_WINDOW_NONE (-1)

/* Decode split: keys are cut into chunks of this many positions, aligned to
 * position 0, whatever the batch; partial results merge in ascending chunk
 * order.  A fixed constant of the library. */
#define ATTN_DECODE_CHUNK 512

/* Return codes. */
enum {
  ATTN_OK = 0,
  ATTN_E_NULL = 1,        /* a required pointer is NULL */
  ATTN_E_SHAPE = 2,       /* non-positive or inconsistent sizes */
  ATTN_E_UNSUPPORTED = 3, /* geometry outside the strict contract */
  ATTN_E_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  ATTN_E_WORKSPACE = 5,   /* decode workspace too small */
  ATTN_E_HIP = 6,         /* a HIP runtime call or launch failed */
  ATTN_E_VALIDATE = 7     /* device-side index content failed validation */
};

/*
 * attn_prefill_varlen -- attention forward over packed variable-length
 * sequences (sliding-window or global layer, GQA, optional bidirectional
 * spans).
 *
 * Passages: sliding and global attention cores as separate layer types
 * ("RFC: Gemma-4-31B-it train/rollout consistency", section 3 "Architecture
 * map" and section 6, items sliding_attention_core / global_attention_core);
 * bidirectional vision-token spans (same page, section 1, Phase B; contiguous
 * soft-token runs per "Gemma-4-E4B-it multimodal baseline", commit log);
 * per-row invariance to unrelated rows and packing (section 4, items 2 and 6).
 *
 * Arguments (all device pointers caller-owned, bf16 = 16-bit bfloat):
 *   q          bf16 [T, num_q_heads, head_dim], contiguous, 16-byte aligned
 *   k, v       bf16 [T, num_kv_heads, head_dim], contiguous, 16-byte aligned
 *   o          bf16 [T, num_q_heads, head_dim] output; rows of tokens outside
 *              every sequence (T beyond cu_seqlens[batch]) are not written
 *   lse_opt    fp32 [T, num_q_heads] natural-log sum of exp(scale*q.k) over
 *              each row's allowed keys, or NULL
 *   cu_seqlens int32 [batch+1] on the device; sequence b holds packed tokens
 *              [cu_seqlens[b], cu_seqlens[b+1]); non-decreasing, starting at 0
 *   batch      number of sequences (0 -> nothing enqueued, returns ATTN_OK)
 *   max_seqlen host upper bound on every sequence length; sizes the grid only
 *              (any bound >= the true maximum gives identical output bytes)
 *   num_q_heads, num_kv_heads: GQA with contiguous groups, query head h reads
 *              KV head h / (num_q_heads / num_kv_heads)
 *   head_dim   64, 256 or 512
 *   window     ATTN_WINDOW_NONE, or W >= 1: key j is allowed for query i of
 *              the same sequence when 0 <= i - j < W
 *   softmax_scale  finite and > 0 (normally 1/sqrt(head_dim))
 *   spans_opt  int32 [num_spans][2] on the device: packed [start, end) ranges,
 *              each inside one sequence, sorted and disjoint; every query of a
 *              span also sees every key of the span (whatever the window).
 *              NULL when num_spans == 0.  Malformed spans cannot make
 *              the kernel read out of bounds (ranges are clamped to the
 *              sequence) but give unspecified masks; INVATTN_VALIDATE=1
 *              rejects them.
 *   stream     HIP stream the work is enqueued on; NULL = the default stream
 *
 * Supported: group size num_q_heads/num_kv_heads in {1, 2, 4, 8}.
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE, ATTN_E_UNSUPPORTED, ATTN_E_ALIGN,
 * ATTN_E_HIP, ATTN_E_VALIDATE; nothing is enqueued on error and
 * attn_last_error() names the argument.
 */
int attn_prefill_varlen(const void* q, const void* k, const void* v, void* o,
                        float* lse_opt, const int32_t* cu_seqlens,
                        int32_t batch, int32_t max_seqlen,
                        int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t window, float softmax_scale,
                        const int32_t* spans_opt, int32_t num_spans,
                        hipStream_t stream);

/*
 * attn_prefill_paged -- chunked prefill: each sequence's new query tokens
 * attend to its keys already in a paged KV cache (the cached prefix plus the
 * chunk itself), read in place through the block table.
 *
 * Passages: a row is invariant to chunking ("RFC: Gemma-4-31B-it
 * train/rollout consistency", section 4, item 6); strict calls consume the
 * paged KV cache directly ("Vime ROCm Attention operator ablation", section
 * "Prerequisites"); layer types as attn_prefill_varlen.
 *
 * Sequence b has n_b = cu_seqlens[b+1] - cu_seqlens[b] new tokens, at
 * positions [q_start[b], q_start[b] + n_b); its keys are positions
 * [0, q_start[b] + n_b), all already written to the cache (the chunk's own
 * K/V included).  Query i attends to key j when 0 <= i - j (< window).
 * Every output row is bitwise identical to the row of the same position
 * from attn_prefill_varlen over the whole sequence with the same K/V
 * (positions are tiled from 0 in both), whatever the chunk boundaries.
 *
 * Arguments (device pointers caller-owned):
 *   q          bf16 [T, num_q_heads, head_dim], packed new tokens, contiguous
 *   k_cache, v_cache  bf16 [num_blocks, block_size, num_kv_heads, head_dim]
 *   o          bf16 [T, num_q_heads, head_dim]; rows beyond cu_seqlens[batch]
 *              are not written
 *   lse_opt    fp32 [T, num_q_heads] as attn_prefill_varlen, or NULL
 *   cu_seqlens int32 [batch+1]: packed ranges of the new tokens, as
 *              attn_prefill_varlen (an empty range is allowed)
 *   q_start    int32 [batch], >= 0: position of each sequence's first new
 *              token (the length of its cached prefix)
 *   block_table int32 [batch, max_blocks_per_seq]; key j of sequence b is in
 *              block block_table[b][j / block_size], slot j % block_size.
 *              Cache blocks are read only for keys in [first attended key of
 *              the first new token, q_start[b] + n_b); entries of other blocks
 *              may be read from the table but may hold anything.  An entry
 *              used outside [0, num_blocks) is clamped into it
 *              (INVATTN_VALIDATE=1 rejects it)
 *   batch      >= 0 (0 -> nothing enqueued)
 *   max_query_len    host bound on every n_b (sizes the grid only)
 *   max_context_len  host bound on every q_start[b] + n_b; at most
 *              max_blocks_per_seq * block_size
 *   num_blocks, block_size (must be 16), num_q_heads, num_kv_heads,
 *   head_dim, window, softmax_scale: as attn_decode_paged / attn_prefill_varlen
 *   stream     HIP stream
 * No bidirectional spans in this layout.
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE, ATTN_E_UNSUPPORTED, ATTN_E_ALIGN,
 * ATTN_E_HIP, ATTN_E_VALIDATE; nothing is enqueued on error.
 */
int attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                       void* o, float* lse_opt, const int32_t* cu_seqlens,
                       const int32_t* q_start, const int32_t* block_table,
                       int32_t max_blocks_per_seq, int32_t batch,
                       int32_t max_query_len, int32_t max_context_len,
                       int32_t num_blocks, int32_t block_size,
                       int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t window, float softmax_scale,
                       hipStream_t stream);

/*
 * attn_prefill_varlen_backward -- gradients dq, dk, dv of
 * attn_prefill_varlen for an upstream gradient dout = dL/do, with every sum
 * in a fixed order and no atomics.
 *
 * Passages: the train/rollout goal includes the training step ("RFC:
 * Gemma-4-31B-it train/rollout consistency", section 1); fixed fp32
 * accumulators and orders, no split-K or cross-workgroup atomics (section 4,
 * items 1 and 3).  Masks, spans and the GQA map are those of the forward.
 *
 * Arithmetic (c = fl32(scale * log2 e); lse2 = fl32(lse * log2 e)):
 *   s_ij, dp_ij, delta_i: bf16 MFMA dot products with fp32 accumulation of
 *           q_i.k_j, v_j.dout_i and o_i.dout_i (delta by the same MFMA
 *           sequence as dp, so dp_ij = delta_i exactly when v_j = o_i)
 *   p_ij    = exp2(fma(s_ij, c, -lse2_i))         (0 off the mask)
 *   ds_ij   = p_ij (dp_ij - delta_i)
 *   dq_i    = scale * sum_j bf16(ds_ij) k_j       MFMAs over 32 keys, key
 *                                                  tiles [32m, 32m + 32) of
 *                                                  the sequence, ascending
 *   dk_j    = scale * sum_(i,h) bf16(ds_ij) q_ih  MFMAs over 32 (row, head)
 *   dv_j    =         sum_(i,h) bf16(p_ij) dout_ih pairs: rows ascending, then
 *                                                  the group's heads
 * Two kernels run on the stream: dq (and delta into the workspace), then dk
 * and dv.  Each output element is written once; no atomics.
 *
 * Arguments (device pointers caller-owned):
 *   q, k, v, o  bf16 as for attn_prefill_varlen (o = its output)
 *   lse         fp32 [T, num_q_heads]: the forward's lse_opt output
 *   dout        bf16 [T, num_q_heads, head_dim]
 *   dq          fp32 [T, num_q_heads, head_dim] output
 *   dk, dv      fp32 [T, num_kv_heads, head_dim] outputs
 *   workspace   fp32 [total_tokens, num_q_heads] scratch (delta), 16-byte
 *               aligned, contents need no initialisation
 *   total_tokens  host value >= cu_seqlens[batch]
 *   the rest as attn_prefill_varlen.
 * Rows of tokens outside every sequence are not written.
 * Errors: as attn_prefill_varlen.
 */
int attn_prefill_varlen_backward(const void* q, const void* k, const void* v,
                                 const void* o, const float* lse,
                                 const void* dout, float* dq, float* dk,
                                 float* dv, float* workspace,
                                 int32_t total_tokens,
                                 const int32_t* cu_seqlens, int32_t batch,
                                 int32_t max_seqlen, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t window, float softmax_scale,
                                 const int32_t* spans_opt, int32_t num_spans,
                                 hipStream_t stream);

/*
 * attn_qk_prologue -- the attention prologue of a layer, in place on Q and
 * K: RMSNorm of every (token, head) vector over the head dim, then rotary
 * position embedding on its first rotary_dims dims.
 *
 * Passage: the layer prologue names a Q/K RMSNorm for head dims 256 and 512,
 * a RoPE on the sliding layers and a proportional RoPE on the global layers
 * ("RFC: Gemma-4-31B-it train/rollout consistency", section 6, items 4 and
 * 6); the norm's fp32 math, its (offset + weight) scale and its single
 * store cast follow "Gated RMSNorm CUDA kernel for the GDN block" (Summary),
 * without the gate.  The pages fix no epsilon, offset, rotary width,
 * frequency base or pairing: all are arguments, and dims i and i + R/2 form
 * a pair (R = rotary_dims).
 *
 * Arithmetic (fp32 unless stated), per vector x of head_dim bf16 values at
 * position pos:
 *   ss   = sum of x_d^2: each of 64 lanes adds its head_dim/64 consecutive
 *          elements in ascending order, then the lanes combine by the
 *          exchange tree xor 32, 16, 8, 4, 2, 1
 *   y_d  = (x_d * (1 / sqrt(ss / head_dim + eps))) * (weight_offset + w_d)
 *          (IEEE division and square root; skipped when w is NULL)
 *   a_i  = pos * 2^(-2i / freq_dims * log2 rope_theta) in fp64 (i < R/2),
 *          reduced in fp64 by the nearest multiple k of pi/2; c_i, s_i = fp32
 *          cosine and sine of the reduced angle, placed by quadrant k mod 4
 *   out_i = y_i c_i - y_{i+R/2} s_i,  out_{i+R/2} = y_i s_i + y_{i+R/2} c_i,
 *          dims R .. head_dim-1 unchanged; bf16 round to nearest even.
 * freq_dims = rotary_dims is the plain partial RoPE; freq_dims = head_dim
 * with rotary_dims < head_dim keeps the turned dims at the frequencies of a
 * full RoPE (the proportional reading).  A vector's bytes depend only on its
 * values, its position and the arguments.
 *
 * Arguments (device pointers caller-owned; q and k are read and overwritten):
 *   q           bf16 [num_tokens, num_q_heads, head_dim], 16-byte aligned
 *   k           bf16 [num_tokens, num_kv_heads, head_dim] or NULL (Q only)
 *   positions   int32 [num_tokens]: the position of each row in its sequence
 *   q_weight, k_weight  fp32 [head_dim] or NULL (no norm on that tensor)
 *   eps >= 0, weight_offset finite
 *   rotary_dims  0 (no RoPE) .. head_dim, a multiple of head_dim / 32
 *   freq_dims    > 0 when rotary_dims > 0; rope_theta > 0
 *   head_dim     64, 256 or 512
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE, ATTN_E_UNSUPPORTED, ATTN_E_ALIGN,
 * ATTN_E_HIP; nothing is enqueued on error.  num_tokens = 0 does nothing.
 */
int attn_qk_prologue(void* q, void* k, const int32_t* positions, int32_t num_tokens,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     const float* q_weight, const float* k_weight, float eps,
                     float weight_offset, int32_t rotary_dims, int32_t freq_dims,
                     double rope_theta, hipStream_t stream);

/*
 * attn_decode_workspace_size -- bytes of fp32 workspace attn_decode_paged
 * needs for this batch: [batch, num_q_heads, ceil(max_seq_len /
 * ATTN_DECODE_CHUNK), head_dim + 4] fp32 (per chunk record: the unnormalised
 * accumulator, the running max, the running sum, one pad word keeping records
 * 16-byte aligned).  Pure function; returns 0 for non-positive arguments.
 *
 * Passage: a split-KV is allowed when its split and merge tree are fixed
 * ("RFC: Gemma-4-31B-it train/rollout consistency", section 4, item 3); the
 * chunk records are that split's partial results, and the caller owns their
 * memory (the library allocates nothing).
 */
size_t attn_decode_workspace_size(int32_t batch, int32_t max_seq_len,
                                  int32_t num_q_heads, int32_t head_dim);

/*
 * attn_decode_paged -- one query token per sequence against a paged KV
 * cache, read in place through the block table.
 *
 * Passages: strict decode consumes the paged KV cache directly, with a fixed
 * schedule ("Vime ROCm Attention operator ablation", sections "Prerequisites"
 * and "Runtime artifacts and validation"); split-KV only with a fixed split
 * and merge tree ("RFC: Gemma-4-31B-it train/rollout consistency", section 4,
 * item 3); hybrid_kv_cache_contract (same page, section 6).
 *
 * Arguments (device pointers caller-owned):
 *   q            bf16 [batch, num_q_heads, head_dim], contiguous
 *   k_cache, v_cache  bf16 [num_blocks, block_size, num_kv_heads, head_dim].
 *                v_cache may be the same pointer as k_cache (V = K, the
 *                global layers whose K and V share one projection: same
 *                RFC, section 6, global_k_eq_v_projection); each block is
 *                then read once, and the output bytes equal those of a
 *                separate V cache holding the same values.
 *   block_table  int32 [batch, max_blocks_per_seq]; key j of sequence b is in
 *                block block_table[b][j / block_size], slot j % block_size.
 *                Entries for blocks outside the attended key range are never
 *                read.
 *   seq_lens     int32 [batch], each in [1, max_seq_len]; counts the current
 *                token, whose K/V is already in the cache; the query is
 *                position seq_lens[b] - 1
 *   batch        >= 0 (0 -> nothing enqueued)
 *   max_seq_len  host bound on every seq_lens entry (sizes grid/workspace)
 *   num_blocks   number of physical blocks in each cache
 *   block_size   must be 16
 *   num_q_heads, num_kv_heads, head_dim, window, softmax_scale: as prefill
 *   workspace    fp32 scratch of at least attn_decode_workspace_size(...)
 *                bytes, 16-byte aligned; its contents need no initialisation
 *                and are overwritten
 *   o            bf16 [batch, num_q_heads, head_dim] output
 *   stream       HIP stream
 * Two kernels run on the stream: a chunk kernel (one workgroup per
 * ATTN_DECODE_CHUNK keys of one KV head of one sequence) writes partial
 * (max, sum, acc) records, then a merge kernel folds the chunks of each
 * (sequence, head) in ascending chunk order.  No atomics.
 * Errors: as prefill, plus ATTN_E_WORKSPACE.
 */
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* seq_lens, int32_t batch,
                      int32_t max_seq_len, int32_t num_blocks,
                      int32_t block_size, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t window,
                      float softmax_scale, void* workspace,
                      size_t workspace_bytes, void* o, hipStream_t stream);

/* Bytes of the static scratch array attn_decode_paged_noalloc keeps its
 * chunk records in (held on each GPU the library runs on until the process
 * ends). */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * attn_decode_paged_noalloc -- attn_decode_paged for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It takes no workspace: the chunk
 * records go to a static device array of ATTN_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU, so the call allocates nothing (no hipMalloc,
 * no hipFree).  The caller still passes every input and the output.
 *
 * Arguments, layouts, kernels and output bytes are those of
 * attn_decode_paged (without workspace and workspace_bytes).
 * Limit: attn_decode_workspace_size(batch, max_seq_len, num_q_heads,
 * head_dim) must not exceed ATTN_NOALLOC_SCRATCH_BYTES (64 MiB: at 32 query
 * heads and head dim 512, batch x ceil(max_seq_len / ATTN_DECODE_CHUNK) <=
 * 1016), else ATTN_E_WORKSPACE and nothing is enqueued.
 * Sharing: every call on one GPU uses that GPU's one array and leaves its
 * records there; calls that overlap on one GPU (on two streams, or from two
 * host threads before the first has finished on the device) race and must be
 * serialised by the caller.  Nothing in the array needs to start at zero.
 * The first call on a device looks up the array's device address, with that
 * device current.  INVATTN_VALIDATE=1 copies the index tensors to the host
 * and synchronises the stream (not for use under capture).
 * Errors: as attn_decode_paged.
 */
int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, int32_t batch,
                              int32_t max_seq_len, int32_t num_blocks,
                              int32_t block_size, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t window,
                              float softmax_scale, void* o, hipStream_t stream);

/* Text of the last failure on this thread ("" if none).  The pointer stays
 * valid until the next call on this thread.  Unsupported input fails closed
 * with a named reason instead of falling back ("RFC: Gemma-4-31B-it
 * train/rollout consistency", section 4, item 7). */
const char* attn_last_error(void);

/*
 * Provenance record of the last successful call on this thread
 * ("RFC: Gemma-4-31B-it train/rollout consistency", section 4, item 8), as
 * one JSON object with the keys op, requested_backend, actual_backend,
 * kernel_id (the kernel instances launched, with their template parameters),
 * schedule_id (tile geometry), split_policy, accumulator_dtype, layer_type
 * ("sliding" or "global"), device, arch, dtype, shape {batch, max_len,
 * tokens (null unless INVATTN_VALIDATE=1 read it), num_q_heads,
 * num_kv_heads, head_dim, window}, casts, exp, fallback ("none") and
 * version.  With INVATTN_TRACE=1 every successful call also prints its
 * record to stderr.  Writes at most n bytes including the terminating NUL;
 * returns the full length, or -1 if no call succeeded yet.
 */
int attn_last_provenance(char* buf, size_t n);

/* Library version string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* INVATTN_H */
