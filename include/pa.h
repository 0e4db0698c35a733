/*
 * pa.h -- C ABI of the paged-KV attention library for AMD MI355X (gfx950).
 *
 * The operations follow the statement of the problem on three pages about
 * vLLM:
 *   [A] "vLLM 架构概述" (blog.chen3feng.top/vllm-analysis), §2 (the block pool
 *       and per-request int32 block tables: a table lookup plus address
 *       arithmetic inside the kernel) and §3 (the kernel layer: a paged
 *       attention kernel and the reshape_and_cache KV write);
 *   [B] "vLLM：从 KV Cache 到高吞吐推理服务" (liujiyu20000308.github.io/vllm),
 *       tutorial 3 (logical block, physical block, offset, slot, slot
 *       mapping), tutorial 1 (MHA/GQA/MQA head sharing), tutorial 6 (FP8 E4M3
 *       KV with a scale), tutorial 7 (tiling, online softmax, LSE);
 *   [C] reading note on "Inside vLLM" (kb.wilsonhandbook.online), core point
 *       1 (16-token blocks) and core point 2 (decode and chunked prefill in
 *       one step, flattened into one super-sequence, each sequence masked to
 *       its own tokens).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pool layout: key_cache and value_cache are two separate device arrays,
 *    each [num_blocks][block_size][num_kv_heads][head_dim], row-major.
 *  - block_tables: device int32 [num_seqs][bt_stride]; entry j of row s is the
 *    physical block holding positions j*block_size .. j*block_size+block_size-1
 *    of sequence s.  Only the first ceil(seq_len/block_size) entries are read.
 *  - seq_lens[s]: tokens of sequence s INCLUDING the new tokens of this step
 *    (they must have been written into the pool first; the *_write decode
 *    entry points store them themselves).
 *  - query_start_loc: device int32 [num_seqs+1], prefix sums of the new-token
 *    counts; the new tokens of all sequences form one flattened array of
 *    num_tokens = query_start_loc[num_seqs] rows.  Sequence s has
 *    q_len = query_start_loc[s+1]-query_start_loc[s] >= 1 new rows at
 *    positions seq_len-q_len .. seq_len-1; row i attends to positions
 *    0 .. seq_len-q_len+i of its own sequence (causal, bottom-right aligned).
 *  - GQA: q head h reads kv head h / (num_q_heads / num_kv_heads).
 *  - Supported: head_dim 64 or 128; block_size 16; num_q_heads a multiple of
 *    num_kv_heads, at most 256 q heads per kv head (the cascade decode: at
 *    most 16).  The decode takes a kv head's q heads 16 at a time, so above 16
 *    per kv head the K/V of a block are read once per group of 16.
 *  - dtypes: PA_F32, PA_BF16 for activations and pools; PA_FP8_E4M3 pools
 *    hold OCP E4M3FN codes (bias 7, max 448, no infinities).  The output has
 *    the query's dtype; fp32 accumulation throughout; bf16 results are rounded
 *    to nearest even.
 *  - All pointers not marked "host" are device pointers owned by the caller.
 *    The library keeps no pointer after a call returns and allocates no
 *    device memory; scratch space comes from the caller's workspace.
 *  - stream is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it and returns; nothing synchronises.
 *  - Errors: a non-zero pa_status_t.  Argument errors are found on the host
 *    before anything is enqueued and leave device memory untouched.
 *    pa_last_error() returns a thread-local message for the last failure.
 *    The contents of device arrays are trusted, except that block ids are
 *    clamped to [0, num_blocks) and positions past max_seq_len are not read;
 *    setting the environment variable PA_VALIDATE=1 makes every call copy the
 *    metadata to the host (it first waits for all work on the device, then
 *    copies) and reject inconsistent contents with PA_ERR_SHAPE.  Such calls
 *    synchronise, so they cannot be captured in a graph.
 *  - Thread safety: calls are independent; calls on different streams may run
 *    concurrently as long as they do not share output or workspace memory.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* inconsistent sizes or metadata */
  PA_ERR_DTYPE = 3,       /* dtype not valid for this entry point */
  PA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  PA_ERR_UNSUPPORTED = 5, /* valid but not implemented (e.g. head_dim 96) */
  PA_ERR_HIP = 6,         /* the HIP runtime reported an error */
  PA_ERR_NO_SPACE = 7,    /* block pool: not enough free blocks (nothing was changed) */
  PA_ERR_STATE = 8        /* block pool: unknown request, or a call out of order */
} pa_status_t;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype_t;

/* ABI version (PA_ABI_VERSION of the built library). */
int pa_abi_version(void);

/*
 * Metadata validation for every later call on any thread: on = 1 checks the
 * device metadata on the host before each call (the checks PA_VALIDATE=1
 * enables), 0 trusts it, -1 returns to the PA_VALIDATE environment setting.
 */
pa_status_t pa_set_validate(int on);

/* Static text for a status code. */
const char* pa_status_string(pa_status_t status);

/* Thread-local message describing the last failed call on this thread ("" if none). */
const char* pa_last_error(void);

/*
 * pa_slot_mapping -- where each new token's K/V goes.  [B] tutorial 3, [A] §2.
 * For new row i of sequence s (position p = seq_lens[s] - q_len_s + i):
 *   slot_mapping[query_start_loc[s] + i] =
 *       block_tables[s][p / block_size] * block_size + p % block_size.
 * slot_mapping: device int32 [query_start_loc[num_seqs]] (output).
 * Bit-exact integer work.
 */
pa_status_t pa_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, int32_t bt_stride,
                            const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                            int32_t num_tokens, int32_t block_size, void* stream);

/*
 * pa_reshape_and_cache -- write new K/V into the pool through slot_mapping.  [A] §3, [B] tutorial 3.
 * For t < num_tokens with slot = slot_mapping[t] >= 0:
 *   key_cache[slot / block_size][slot % block_size][h][:] = key[t*key_tok_stride + h*head_dim + :]
 * (same for value).  Negative slots are skipped; duplicate slots within one
 * call are undefined.  key/value: [num_tokens][.. token stride in elements ..]
 * with heads contiguous inside a token (so K and V may be slices of a fused
 * QKV output).  dtype: PA_F32 or PA_BF16 for inputs and pools alike; a plain
 * copy, bit-exact.  Slots >= num_blocks*block_size are skipped.
 */
pa_status_t pa_reshape_and_cache(const void* key, const void* value, int64_t key_tok_stride,
                                 int64_t value_tok_stride, void* key_cache, void* value_cache,
                                 const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 pa_dtype_t dtype, void* stream);

/*
 * pa_reshape_and_cache_fp8 -- the same scatter into fp8 pools.  [B] tutorial 6.
 * Stored code = E4M3FN(fl32(x / scale)) with x the fp32 value of the input
 * element, one correctly rounded fp32 division, round to nearest even,
 * finite overflow and infinity saturating to +-448, NaN kept as NaN (0x7F
 * with the input's sign).  k_scale, v_scale: positive per-tensor scales.
 * src_dtype: PA_F32 or PA_BF16.  key_cache/value_cache: uint8 codes.
 */
pa_status_t pa_reshape_and_cache_fp8(const void* key, const void* value, int64_t key_tok_stride,
                                     int64_t value_tok_stride, uint8_t* key_cache, uint8_t* value_cache,
                                     const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     pa_dtype_t src_dtype, float k_scale, float v_scale, void* stream);

/*
 * pa_write_kv -- pa_slot_mapping and pa_reshape_and_cache in one launch
 * ([B] tutorial 3, [A] §2-§3): for new row i of sequence s, slot =
 * block_tables[s][p / block_size] * block_size + p % block_size with p =
 * seq_lens[s] - q_len_s + i (-1 past the table), and the row's K/V (all kv
 * heads) is copied to cache[slot / block_size][slot % block_size] when 0 <=
 * slot < num_blocks * block_size.  Bit-identical to the two calls; the
 * device slot array is not needed.  slot_mapping: optional device int32
 * [num_tokens] output (NULL: not stored).  max_q_len: a host estimate of the
 * longest q_len that sizes the launch (a sequence with more rows still gets
 * all of them written, by fewer work-groups; 0 writes nothing).
 * key/value strides, dtype and pools as pa_reshape_and_cache.
 */
pa_status_t pa_write_kv(const void* key, const void* value, int64_t key_tok_stride, int64_t value_tok_stride,
                        void* key_cache, void* value_cache, int32_t* slot_mapping, const int32_t* block_tables,
                        int32_t bt_stride, const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                        int32_t num_tokens, int32_t max_q_len, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t num_blocks, pa_dtype_t dtype, void* stream);

/* pa_write_kv into E4M3FN pools: the codes of pa_reshape_and_cache_fp8 ([B] tutorial 6). */
pa_status_t pa_write_kv_fp8(const void* key, const void* value, int64_t key_tok_stride, int64_t value_tok_stride,
                            uint8_t* key_cache, uint8_t* value_cache, int32_t* slot_mapping,
                            const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                            const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t max_q_len,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            pa_dtype_t src_dtype, float k_scale, float v_scale, void* stream);

/*
 * pa_decode_workspace_bytes -- scratch pa_decode / pa_decode_fp8 need.
 * The blocks of all sequences, laid end to end, are cut into num_splits
 * equal shares per kv head (0 = automatic: about one wave per SIMD of the
 * current device for every pool type; PA_DECODE_WAVES_PER_SIMD overrides it;
 * the size returned covers twice that count, the share count of the decode
 * part of a fused decode + prefill launch of pa_prefill_varlen*); a sequence
 * split across shares gets partial results that are merged with the
 * log-sum-exp rule ([B] tutorial 7).  The count is capped at
 * num_seqs * ceil(max_seq_len / 16).  Returns 0 when a single share is used
 * (no scratch needed), and 0 for invalid arguments.  The size depends on
 * num_seqs, num_q_heads, head_dim and the share count, not on the contents
 * of seq_lens.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t num_splits);

/*
 * pa_decode -- paged attention for one new token per sequence.  [A] §2-§3,
 * [B] tutorials 1, 3 and 7, [C] core point 2.
 * out[s][h][:] = sum_j softmax_j(scale * q[s][h] . K_j) V_j over positions
 * j = 0 .. seq_lens[s]-1, K_j/V_j read through block_tables.
 * query/out: [num_seqs][num_q_heads][head_dim], dtype; pools: dtype.
 * dtype: PA_F32 or PA_BF16.  max_seq_len: host bound on every seq_lens[s]
 * (longer sequences are cut to it; ceil(max_seq_len/block_size) <=
 * bt_stride).  num_splits: see pa_decode_workspace_bytes (0 = automatic).
 * workspace: at least pa_decode_workspace_bytes(...) bytes of device memory
 * (may be NULL when that is 0), 256-byte aligned; its contents need no
 * initialisation.  The result of a sequence does not depend on where its
 * blocks sit in the pool; it may differ in the last bits between split
 * counts (a different summation order).
 */
pa_status_t pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                      pa_dtype_t dtype, int32_t num_splits, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * pa_decode_window -- pa_decode with sliding-window attention: the query of
 * sequence s (at position L-1, L = seq_lens[s]) attends to positions
 * max(0, L-sliding_window) .. L-1 only.  The pages name sliding-window
 * attention ([A] §5.1, a manager that keeps only the blocks inside the
 * window; [B] tutorial 1, among the cases that bound KV capacity) without
 * fixing where the window starts; this library takes the W most recent
 * positions, the current one included.  Table entries wholly before the
 * window are not read (a caller may have given those blocks up; PA_VALIDATE=1
 * still checks every entry).  dtype: PA_BF16, or PA_F32 (fp32 pools and
 * queries, the vector-ALU kernel).  sliding_window >= 1 (a window of at
 * least seq_lens[s] is pa_decode).
 * workspace: pa_decode_workspace_bytes(...) with the same max_seq_len.
 * Other arguments as pa_decode.
 */
pa_status_t pa_decode_window(void* out, const void* query, const void* key_cache, const void* value_cache,
                             const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                             pa_dtype_t dtype, int32_t sliding_window, int32_t num_splits, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * pa_decode_local -- pa_decode with chunked local attention ([A] §5.1 lists
 * a chunked-local attention manager beside the sliding-window one, without
 * its boundary; this library's reading: positions are cut into chunks of
 * chunk_size tokens, 0 .. C-1, C .. 2C-1, ..., and a row sees the keys of its
 * own chunk up to itself).  The query of sequence s (at position L-1) attends
 * to positions C*((L-1) div C) .. L-1.  Table entries wholly before that
 * chunk are not read.  dtype: PA_BF16 or PA_F32; chunk_size >= 1.  workspace:
 * pa_decode_workspace_bytes(...) with the same max_seq_len.  Other arguments
 * as pa_decode.
 */
pa_status_t pa_decode_local(void* out, const void* query, const void* key_cache, const void* value_cache,
                            const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                            pa_dtype_t dtype, int32_t chunk_size, int32_t num_splits, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * pa_decode_static -- pa_decode that allocates nothing and takes no
 * workspace, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments, result and errors as pa_decode (without workspace and
 * workspace_bytes).  Its scratch is a file-scope device array of the library,
 * 32 MiB (33554432 bytes) per GPU, held from the first call on that GPU until
 * the process ends; a batch whose pa_decode_workspace_bytes(...) exceeds it is
 * refused with PA_ERR_WORKSPACE before anything is enqueued.  Every call on
 * one GPU shares that array, which keeps the last call's contents (nothing in
 * it needs to start at zero): calls that overlap on one GPU (on different
 * streams, or from different threads) race and must not be issued.
 */
pa_status_t pa_decode_static(void* out, const void* query, const void* key_cache, const void* value_cache,
                             const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                             pa_dtype_t dtype, int32_t num_splits, void* stream);

/*
 * pa_decode_fp8 -- pa_decode over E4M3FN pools.  [B] tutorial 6.
 * K_j = decode(code) * k_scale, V_j = decode(code) * v_scale (exact values);
 * q_dtype (= out dtype): PA_BF16 or PA_F32 (fp32 queries are rounded to
 * bf16 for the matrix cores).  Other arguments as pa_decode.
 */
pa_status_t pa_decode_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                          const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                          pa_dtype_t q_dtype, float k_scale, float v_scale, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_write -- one decode step's KV write and attention in one call:
 * the result, and every byte of both pools, are those of pa_write_kv (one
 * new row per sequence: query_start_loc = 0, 1, ..., num_seqs, max_q_len 1)
 * followed by pa_decode.  [A] §3 (the new token's K/V are stored into its
 * slot, then attention reads the cache through the block table), [B]
 * tutorial 3 (slot of position p: block_tables[s][p / block_size] *
 * block_size + p % block_size).  key/value: [num_seqs][num_kv_heads]
 * [head_dim] rows of dtype, row s the K/V of sequence s's position
 * seq_lens[s] - 1, heads and head_dim contiguous, key_tok_stride /
 * value_tok_stride elements between rows.  With bf16 pools and every
 * kv-head slice 16-byte aligned (key, value and both strides in bytes
 * multiples of 16), the decode launch stores the rows itself and attends
 * them from registers; otherwise (fp32 pools, other alignments) the write
 * runs as its own launch first.  Conditions on the batch, beyond
 * pa_decode's: the block holding a sequence's new row is read by no other
 * sequence of the batch (a block manager shares only full blocks); a
 * sequence with seq_lens[s] > max_seq_len is cut as in pa_decode and its row
 * is not stored; a row whose table entry lies outside the pool is not stored
 * (as pa_write_kv) but still attended.  dtype: PA_F32 or PA_BF16, for the
 * pools, query/out and key/value.  Other arguments, workspace and errors as
 * pa_decode.
 */
pa_status_t pa_decode_write(void* out, const void* query, const void* key, const void* value,
                            int64_t key_tok_stride, int64_t value_tok_stride, void* key_cache, void* value_cache,
                            const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                            pa_dtype_t dtype, int32_t num_splits, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * pa_decode_write_fp8 -- pa_decode_write over E4M3FN pools ([B] tutorial 6):
 * the stored codes are pa_write_kv_fp8's (of x / k_scale and x / v_scale),
 * the attention pa_decode_fp8's.  dtype (PA_F32 or PA_BF16) is that of
 * query/out and of key/value; the decode launch stores the rows itself when
 * every kv-head slice is 16-byte aligned.  Other arguments as
 * pa_decode_write and pa_decode_fp8.
 */
pa_status_t pa_decode_write_fp8(void* out, const void* query, const void* key, const void* value,
                                int64_t key_tok_stride, int64_t value_tok_stride, uint8_t* key_cache,
                                uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_seq_len, float scale, pa_dtype_t dtype, float k_scale, float v_scale,
                                int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_window_write, pa_decode_window_write_fp8, pa_decode_local_write,
 * pa_decode_local_write_fp8 -- the decode step that stores its new K/V
 * (pa_decode_write, pa_decode_write_fp8) with the mask of pa_decode_window
 * (sliding_window >= 1) or pa_decode_local (chunk_size >= 1): the bytes of
 * pa_write_kv (pa_write_kv_fp8) followed by the masked decode.  The new row,
 * at position seq_lens[s] - 1, is always visible.  Arguments, conditions,
 * workspace and errors as pa_decode_write and the masked decode.
 */
pa_status_t pa_decode_window_write(void* out, const void* query, const void* key, const void* value,
                                   int64_t key_tok_stride, int64_t value_tok_stride, void* key_cache,
                                   void* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                   const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_seq_len, float scale, pa_dtype_t dtype, int32_t sliding_window,
                                   int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);
pa_status_t pa_decode_window_write_fp8(void* out, const void* query, const void* key, const void* value,
                                       int64_t key_tok_stride, int64_t value_tok_stride, uint8_t* key_cache,
                                       uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                       const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_seq_len, float scale, pa_dtype_t dtype, float k_scale,
                                       float v_scale, int32_t sliding_window, int32_t num_splits, void* workspace,
                                       size_t workspace_bytes, void* stream);
pa_status_t pa_decode_local_write(void* out, const void* query, const void* key, const void* value,
                                  int64_t key_tok_stride, int64_t value_tok_stride, void* key_cache, void* value_cache,
                                  const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                                  pa_dtype_t dtype, int32_t chunk_size, int32_t num_splits, void* workspace,
                                  size_t workspace_bytes, void* stream);
pa_status_t pa_decode_local_write_fp8(void* out, const void* query, const void* key, const void* value,
                                      int64_t key_tok_stride, int64_t value_tok_stride, uint8_t* key_cache,
                                      uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                      const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      int32_t max_seq_len, float scale, pa_dtype_t dtype, float k_scale,
                                      float v_scale, int32_t chunk_size, int32_t num_splits, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * pa_decode_cascade -- pa_decode for a batch whose sequences all begin with
 * the same prefix_blocks physical blocks (prefix sharing: [A] §2, two
 * requests' tables pointing at the same blocks; cascade attention is named in
 * [A]'s attention-backend table).  The result is pa_decode's: the keys of the
 * shared prefix and of each sequence's own suffix are attended separately
 * and combined with the log-sum-exp rule ([B] tutorial 7), so only the order
 * of fp32 sums differs.  The prefix is attended as dense matrix-core tiles:
 * for each kv head, all num_seqs x G query rows (G = num_q_heads /
 * num_kv_heads <= 16) against the prefix blocks, each block read once per 256
 * rows, in one launch with the suffixes' shares (fp8 pools: the tiles convert
 * the codes to bf16 themselves).  With fp32 queries (pa_decode_cascade_fp8)
 * the prefix is read once per group of 16/G sequences by decode waves instead.
 * Requirements: prefix_blocks >= 1; every seq_lens[s] >= prefix_blocks *
 * block_size; block_tables[s][j] the same for every s and j < prefix_blocks
 * (checked under PA_VALIDATE=1, trusted otherwise).  dtype: PA_BF16, or
 * PA_F32 (fp32 pools and queries: the plain fp32 decode over each whole
 * sequence, the same attention without the shared grouping).
 * workspace: pa_decode_cascade_workspace_bytes(...) bytes (needed for every
 * non-empty batch; 0 when num_seqs is 0, and for invalid arguments).
 * num_splits: waves per kv head for the suffixes, as in pa_decode.  Other
 * arguments as pa_decode.
 */
size_t pa_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_seq_len, int32_t prefix_blocks,
                                         int32_t num_splits);
pa_status_t pa_decode_cascade(void* out, const void* query, const void* key_cache, const void* value_cache,
                              const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                              pa_dtype_t dtype, int32_t prefix_blocks, int32_t num_splits, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * pa_decode_cascade_fp8 -- pa_decode_cascade over E4M3FN pools, with the
 * scales and q_dtype of pa_decode_fp8.  [A] §2, [B] tutorials 6 and 7.
 */
pa_status_t pa_decode_cascade_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                                  const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                                  pa_dtype_t q_dtype, float k_scale, float v_scale, int32_t prefix_blocks,
                                  int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_cascade_write -- one decode step of a prefix-shared batch: the
 * result, and every byte of both pools, are those of pa_write_kv (one new row
 * per sequence) followed by pa_decode_cascade.  [A] §2-§3, [B] tutorial 3.
 * key/value, strides, dtype and the conditions on the new rows as
 * pa_decode_write; besides, every new row lies after the shared prefix
 * (seq_lens[s] > prefix_blocks * block_size, checked under PA_VALIDATE=1): the
 * shared blocks are never written.  When the prefix is attended as tiles and
 * every kv-head slice is 16-byte aligned, the suffix waves of the tiles'
 * launch store the rows and attend them from registers; otherwise the write
 * runs as its own launch first.  Workspace: pa_decode_cascade_workspace_bytes.
 * Other arguments and errors as pa_decode_cascade.
 */
pa_status_t pa_decode_cascade_write(void* out, const void* query, const void* key, const void* value,
                                    int64_t key_tok_stride, int64_t value_tok_stride, void* key_cache,
                                    void* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    int32_t max_seq_len, float scale, pa_dtype_t dtype, int32_t prefix_blocks,
                                    int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_cascade_write_fp8 -- pa_decode_cascade_write over E4M3FN pools:
 * the codes of pa_write_kv_fp8, the attention of pa_decode_cascade_fp8.
 * dtype (PA_F32 or PA_BF16): query/out and key/value.  [B] tutorial 6.
 */
pa_status_t pa_decode_cascade_write_fp8(void* out, const void* query, const void* key, const void* value,
                                        int64_t key_tok_stride, int64_t value_tok_stride, uint8_t* key_cache,
                                        uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, int32_t max_seq_len, float scale, pa_dtype_t dtype,
                                        float k_scale, float v_scale, int32_t prefix_blocks, int32_t num_splits,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill_varlen_workspace_bytes -- scratch pa_prefill_varlen needs for
 * this batch.  query_start_loc_host / seq_lens_host: host copies of the
 * metadata (num_seqs+1 and num_seqs entries).  Returns 0 on invalid input.
 */
size_t pa_prefill_varlen_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim);

/*
 * pa_prefill_varlen -- causal paged attention over a flattened batch of any
 * mix of decode rows and chunked-prefill chunks.  [C] core point 2, [A] §2,
 * [B] tutorials 5 (chunked prefill) and 7.
 * For row t of sequence s (new row i, c = seq_lens[s]-q_len cached tokens):
 * out[t][h][:] = sum_{j <= c+i} softmax_j(scale * q[t][h] . K_j) V_j.
 * query/out: [num_tokens][num_q_heads][head_dim]; dtype PA_BF16 (the
 * matrix-core kernel) or PA_F32 (fp32 pools and activations: decode rows on
 * the vector-ALU decode kernel, and a batch with chunks runs every token as a
 * decode row of its own, which sees exactly the keys of its position -- one
 * decode launch, no matrix cores; the workspace sizes below count it).  The
 * host copies of
 * query_start_loc and seq_lens plan the work (the control plane is on the
 * CPU) and must equal the device arrays.  scale must be positive and finite
 * (PA_ERR_SHAPE otherwise; the same holds for every pa_prefill_varlen*
 * entry point): the kernel keeps the running maximum of raw scores and
 * applies the scale inside the exponential.
 */
pa_status_t pa_prefill_varlen(void* out, const void* query, const void* key_cache, const void* value_cache,
                              const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                              const int32_t* query_start_loc, const int32_t* seq_lens_host,
                              const int32_t* query_start_loc_host, int32_t num_seqs, int32_t num_tokens,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, float scale, pa_dtype_t dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * pa_prefill_varlen_write -- one step of a flattened batch that also stores
 * its new K/V: the result, and every byte of both pools, are those of
 * pa_write_kv (max_q_len: the longest q_len) followed by pa_prefill_varlen.
 * [A] §3 (the new tokens' K/V go into their slots, then attention reads the
 * cache), [C] core point 2.  key/value: [num_tokens][num_kv_heads][head_dim]
 * of dtype, row t the K/V of the batch's new row t, heads and head_dim
 * contiguous, key_tok_stride / value_tok_stride elements between rows.  When
 * the step runs as one fused launch of decode rows and chunks (bf16, every
 * kv-head slice 16-byte aligned), that launch stores the rows: the decode
 * waves as pa_decode_write does, and the chunks' tiles read their new keys
 * from key/value while one work item per row tile stores them.  Otherwise
 * the write runs as its own launch first.  Condition beyond
 * pa_prefill_varlen's: a block that holds new rows of one sequence is read by
 * no other sequence of the batch.  Workspace: pa_prefill_varlen_workspace_bytes.
 * Other arguments and errors as pa_prefill_varlen.
 */
pa_status_t pa_prefill_varlen_write(void* out, const void* query, const void* key, const void* value,
                                    int64_t key_tok_stride, int64_t value_tok_stride, void* key_cache,
                                    void* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                    const int32_t* seq_lens, const int32_t* query_start_loc,
                                    const int32_t* seq_lens_host, const int32_t* query_start_loc_host,
                                    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                    pa_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill_varlen_window -- pa_prefill_varlen with sliding-window
 * attention ([A] §5.1, [B] tutorial 1; the window's start is this library's
 * reading, as in pa_decode_window): the row at position p attends to
 * positions max(0, p-sliding_window+1) .. p.  No pool data is read from the
 * blocks wholly before the window of a sequence's first new row (their table
 * entries may name any block; PA_VALIDATE=1 still checks them), and 64-key
 * tiles wholly before it are not computed.  dtype: PA_BF16 or PA_F32 (as
 * pa_prefill_varlen); sliding_window >= 1.  workspace:
 * pa_prefill_varlen_window_workspace_bytes(...) with the same window (the
 * work split depends on it; returns 0 on invalid input).  Other arguments as
 * pa_prefill_varlen.
 */
size_t pa_prefill_varlen_window_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t sliding_window);
pa_status_t pa_prefill_varlen_window(void* out, const void* query, const void* key_cache, const void* value_cache,
                                     const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                     const int32_t* query_start_loc, const int32_t* seq_lens_host,
                                     const int32_t* query_start_loc_host, int32_t num_seqs, int32_t num_tokens,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, float scale, pa_dtype_t dtype, int32_t sliding_window,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill_varlen_local -- pa_prefill_varlen with chunked local attention
 * (the reading of pa_decode_local): the row at position p attends to
 * positions C*(p div C) .. p, C = chunk_size >= 1.  No pool data is read from
 * the blocks wholly before the chunk of a sequence's first new row.  dtype:
 * PA_BF16 or PA_F32.  workspace: pa_prefill_varlen_local_workspace_bytes(...) with the
 * same chunk_size (0 on invalid input).  Other arguments as
 * pa_prefill_varlen.
 */
size_t pa_prefill_varlen_local_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t chunk_size);
pa_status_t pa_prefill_varlen_local(void* out, const void* query, const void* key_cache, const void* value_cache,
                                    const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                    const int32_t* query_start_loc, const int32_t* seq_lens_host,
                                    const int32_t* query_start_loc_host, int32_t num_seqs, int32_t num_tokens,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, float scale, pa_dtype_t dtype, int32_t chunk_size,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill_varlen_fp8 -- pa_prefill_varlen over E4M3FN pools (uint8 codes)
 * with per-tensor scales.  [B] tutorials 5 and 6, [C] core point 2.
 * K_j = decode(code) * k_scale, V_j = decode(code) * v_scale.  Decode rows
 * (q_len == 1) read the codes directly as in pa_decode_fp8; the chunks'
 * K/V tiles are copied as codes and converted to their exact bf16 values
 * inside the matrix-core kernel, with k_scale folded into the score scale
 * and v_scale into the output (nothing is staged: the workspace is the
 * plan's, as for pa_prefill_varlen; bt_stride is checked, >= 1, and does not
 * change the size).  q_dtype (= out dtype): PA_BF16, or PA_F32 (decode rows
 * as pa_decode_fp8 with fp32 queries; a batch with chunks runs every token as
 * a decode row of its own on the fp8 decode kernel, as pa_prefill_varlen does
 * for PA_F32).  Other arguments as pa_prefill_varlen.
 */
size_t pa_prefill_varlen_fp8_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t bt_stride);
pa_status_t pa_prefill_varlen_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                                  const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                  const int32_t* query_start_loc, const int32_t* seq_lens_host,
                                  const int32_t* query_start_loc_host, int32_t num_seqs, int32_t num_tokens,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float scale, pa_dtype_t q_dtype, float k_scale, float v_scale,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_window_fp8, pa_decode_local_fp8 -- pa_decode_window and
 * pa_decode_local over E4M3FN pools, with the scales and q_dtype of
 * pa_decode_fp8 ([A] §5.1; [B] tutorial 6).  workspace:
 * pa_decode_workspace_bytes(...) with the same max_seq_len.  Other arguments
 * as pa_decode_fp8 and pa_decode_window / pa_decode_local.
 */
pa_status_t pa_decode_window_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                                 const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                                 pa_dtype_t q_dtype, float k_scale, float v_scale, int32_t sliding_window,
                                 int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);
pa_status_t pa_decode_local_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                                const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                                pa_dtype_t q_dtype, float k_scale, float v_scale, int32_t chunk_size,
                                int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill_varlen_window_fp8, pa_prefill_varlen_local_fp8 --
 * pa_prefill_varlen_window and pa_prefill_varlen_local over E4M3FN pools,
 * with the scales, q_dtype and in-kernel conversion of pa_prefill_varlen_fp8 ([A] §5.1;
 * [B] tutorials 5 and 6).  workspace: the matching *_workspace_bytes(...)
 * with the same bt_stride and window or chunk size (0 on invalid input).
 */
size_t pa_prefill_varlen_window_fp8_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                    int32_t head_dim, int32_t bt_stride, int32_t sliding_window);
pa_status_t pa_prefill_varlen_window_fp8(void* out, const void* query, const uint8_t* key_cache,
                                         const uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                         const int32_t* seq_lens, const int32_t* query_start_loc,
                                         const int32_t* seq_lens_host, const int32_t* query_start_loc_host,
                                         int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                         int32_t num_blocks, float scale, pa_dtype_t q_dtype, float k_scale,
                                         float v_scale, int32_t sliding_window, void* workspace,
                                         size_t workspace_bytes, void* stream);
size_t pa_prefill_varlen_local_fp8_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                                   int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                   int32_t head_dim, int32_t bt_stride, int32_t chunk_size);
pa_status_t pa_prefill_varlen_local_fp8(void* out, const void* query, const uint8_t* key_cache,
                                        const uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                        const int32_t* seq_lens, const int32_t* query_start_loc,
                                        const int32_t* seq_lens_host, const int32_t* query_start_loc_host,
                                        int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, float scale, pa_dtype_t q_dtype, float k_scale,
                                        float v_scale, int32_t chunk_size, void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * Host block pool -- the control plane that hands out the physical blocks
 * whose ids fill block_tables.  Host memory only; no device call.
 * [A] §5.1: a doubly linked free list with O(1) allocation and release, a
 * prefix-cache map from block hash to block, per-block reference counts and
 * hashes.  [C] core point 1: allocate_slots takes ceil(tokens / block_size)
 * blocks from the head of the free list after checking that enough are free,
 * and records them per request (17 tokens of 16-token blocks: 2 blocks).
 * [C] core point 3: each full block's hash chains the previous block's hash,
 * the block's tokens and extra identity (salt, adapter, ...), and
 * find_longest_cache_hit returns the longest run of cached leading blocks.
 * [B] tutorials 3-4: the null block, eviction of cached free blocks, several
 * physical copies of one hash.
 *
 * Conventions: block 0 is the null block.  It is never handed out and never
 * counted as free; pa_pool_release_before puts it in the table entries it
 * releases (the kernels never read those entries' data with a sliding window
 * that excludes them).  A block whose reference count drops to 0 goes to the
 * tail of the free list and keeps its hash: it can still be hit (and leaves
 * the free list again when it is) until it is handed out from the head, which
 * evicts its hash.  Releases go from a request's last block to its first, so
 * tail blocks are evicted first.  A pool is not thread-safe: one thread at a
 * time.  Failures return a status (pa_last_error has the message) and leave
 * the pool unchanged.
 */
typedef struct pa_block_pool pa_block_pool_t;

/* A pool of num_blocks blocks (>= 2; ids 1 .. num_blocks-1 start free, in order). */
pa_status_t pa_pool_create(int32_t num_blocks, int32_t block_size, pa_block_pool_t** pool);
void pa_pool_destroy(pa_block_pool_t* pool);
/* Blocks in the free list (cached or not); -1 for a NULL pool. */
int32_t pa_pool_num_free(const pa_block_pool_t* pool);

/*
 * Hashes of the num_tokens / block_size full blocks of a token sequence
 * (host int32 tokens), written to hashes (host): h_i = FNV-1a-64 of the
 * little-endian bytes of (h_{i-1}, the block's block_size tokens, extra_key),
 * h_{-1} = 0.  Returns the number of full blocks, -1 on invalid arguments.  A
 * partial last block has no hash.  The 64-bit hash is trusted: two different
 * prefixes with the same hash would share blocks.
 */
int32_t pa_pool_hash_blocks(const int32_t* tokens, int32_t num_tokens, int32_t block_size, uint64_t extra_key,
                            uint64_t* hashes);

/*
 * The longest run hashes[0..n-1] that is cached: writes a cached block for
 * each to blocks (the oldest physical copy) and returns n (0 .. num_hashes),
 * -1 on invalid arguments.  Changes nothing (pass the blocks to
 * pa_pool_allocate_slots to take them).
 */
int32_t pa_pool_find_longest_cache_hit(const pa_block_pool_t* pool, const uint64_t* hashes, int32_t num_hashes,
                                       int32_t* blocks);

/*
 * Makes request_id hold ceil(num_tokens / block_size) blocks.  On the first
 * call for a request, hit_blocks (cached blocks, e.g. from
 * pa_pool_find_longest_cache_hit) become its leading blocks: each gains a
 * reference and leaves the free list if it was there.  The rest come from the
 * head of the free list (reference count 1; a cached one loses its hash).
 * Later calls (growing a running request) pass no hits.  PA_ERR_NO_SPACE if
 * the free list is too short, with nothing changed.  num_blocks (optional):
 * the request's block count afterwards.
 */
pa_status_t pa_pool_allocate_slots(pa_block_pool_t* pool, int64_t request_id, int32_t num_tokens,
                                   const int32_t* hit_blocks, int32_t num_hit_blocks, int32_t* num_blocks);

/*
 * Commits the hashes of the request's first num_full_blocks blocks once their
 * K/V are written (hashes: as from pa_pool_hash_blocks over the request's
 * tokens).  Blocks already cached and null entries are skipped; a hash that
 * is already cached gains another physical copy.
 */
pa_status_t pa_pool_cache_blocks(pa_block_pool_t* pool, int64_t request_id, const uint64_t* hashes,
                                 int32_t num_full_blocks);

/*
 * Sliding window ([A] §5.1's manager that keeps only the blocks inside the
 * window): releases every block of the request wholly before token position
 * `position` (entries j < position / block_size) and puts the null block in
 * their table entries.  For a window of W and a next step whose first new row
 * is at position p, pass p - W + 1.
 */
pa_status_t pa_pool_release_before(pa_block_pool_t* pool, int64_t request_id, int32_t position);

/* Releases all of the request's blocks (last to first) and forgets it. */
pa_status_t pa_pool_free(pa_block_pool_t* pool, int64_t request_id);

/* Copies up to max_blocks of the request's table (host int32) to out; returns its length, -1 if unknown. */
int32_t pa_pool_block_table(const pa_block_pool_t* pool, int64_t request_id, int32_t* out, int32_t max_blocks);

/* Inspection: a block's reference count, whether it is in the free list, and its hash (if it has one). */
pa_status_t pa_pool_block_state(const pa_block_pool_t* pool, int32_t block, int32_t* ref_count, int32_t* is_free,
                                int32_t* has_hash, uint64_t* hash);
/* Inspection: the free list from head to tail (up to max_blocks ids); returns its length. */
int32_t pa_pool_free_queue(const pa_block_pool_t* pool, int32_t* out, int32_t max_blocks);

/*
 * Kernel timing, for measurement.  Not part of the pages' problem statement:
 * it serves the roofline figures (device time of each kernel of the path).
 * pa_timing_enable(1): from now on every entry point records a pair of HIP
 * events on its stream around each kernel it launches (events are created
 * by the library and reused; no device memory is allocated).  The events
 * serialise nothing but add a small gap between the kernels of one call.
 * pa_timing_read(kernel, &count, &total_ms): waits for the recorded events
 * of that kernel and returns how many launches were timed and their summed
 * duration in milliseconds.  pa_timing_read_launches(kernel, ms, max, &n):
 * the same wait, then the duration of each launch timed since the last reset
 * (the first 2^20 of them), in launch order: n = how many are kept, of which
 * the first min(n, max) are copied to ms (host, may be NULL when max is 0).
 * pa_timing_reset(): zeroes the sums and forgets the durations.
 */
typedef enum pa_kernel {
  PA_K_SLOT_MAPPING = 0,    /* pa_slot_mapping */
  PA_K_RESHAPE_AND_CACHE = 1, /* pa_reshape_and_cache, pa_reshape_and_cache_fp8 */
  PA_K_DECODE = 2,          /* the paged decode kernel (pa_decode(_fp8), decode rows of pa_prefill_varlen), and the prefix-tile + suffix launch of pa_decode_cascade(_fp8) */
  PA_K_DECODE_MERGE = 3,    /* the log-sum-exp merge of split sequences */
  PA_K_PREFILL = 4,         /* the varlen prefill kernel */
  PA_K_PREFILL_MERGE = 5,   /* the log-sum-exp merge of split prefill row tiles */
  PA_K_STAGE_FP8 = 6,       /* no launch is timed under it (fp8 tiles are converted inside the kernels) */
  PA_K_FUSED = 7            /* decode rows and prefill chunks of a mixed batch in one launch (pa_prefill_varlen*) */
} pa_kernel_t;

pa_status_t pa_timing_enable(int on);

/*
 * pa_set_fused(mode) -- how pa_prefill_varlen* run a batch that has both decode rows and
 * chunks: 0 = a decode launch, then a prefill launch; 1 = one launch holding both when the
 * host estimate says it ends sooner (the default); 2 = one launch whenever it can hold the
 * batch's prefill items (at most 440); -1 = follow the environment variable PA_FUSED
 * (0 / 1 / 2, default 1).  The result does not depend on the mode beyond the last bits (the
 * decode rows' split counts differ); the workspace size does, so query
 * pa_prefill_varlen*_workspace_bytes under the same mode.  PA_ERR_SHAPE for other values.
 */
pa_status_t pa_set_fused(int mode);

/*
 * pa_probe_mfma_peak -- measurement only (the denominator of a measured
 * matrix-core peak beside the published one; not part of the pages'
 * problem).  Launches blocks work-groups of 256 threads; each wave runs
 * iters rounds of four independent v_mfma_f32_32x32x16_bf16 (32768 FLOP
 * each) on register operands and writes one float per thread to out
 * (device, blocks * 256 floats).  Time it with events on `stream`:
 * FLOP = blocks * 4 waves * iters * 4 * 32768.
 */
pa_status_t pa_probe_mfma_peak(float* out, int32_t blocks, int32_t iters, void* stream);
pa_status_t pa_timing_reset(void);
pa_status_t pa_timing_read(pa_kernel_t kernel, int64_t* count, double* total_ms);
pa_status_t pa_timing_read_launches(pa_kernel_t kernel, float* ms, int32_t max_launches, int32_t* n);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
