// Internal launch parameters shared by the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Records the thread-local failure message (pa_last_error) and returns st.
pa_status_t set_error(pa_status_t st, const char* fmt, ...);

constexpr int kBlockSize = 16;      // tokens per physical block
constexpr int kDecodeWaves = 4;     // waves per decode work-group
constexpr int kMaxGroup = 16;       // q heads per kv head handled by one MFMA column set (cascade limit)
constexpr int kMaxGqa = 256;        // q heads per kv head: decode takes them 16 at a time, prefill packs
                                    // at least one position of them into a 256-row tile
constexpr int kPrefillRows = 256;   // (position, q head) rows per prefill work-group (8 waves x 32)
constexpr int kPrefillKeys = 64;    // keys per LDS tile in prefill
constexpr int kMaxPrefillItems = 440;  // work items per launch (kernel-argument space: a fused launch
                                       // carries them beside the decode parameters in 4 KB)

enum Dtype { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// One decode launch: grid (n_splits, num_kv_heads) (fp32: (n_splits, num_q_heads)).
// The blocks of all decode sequences, laid end to end, are cut into n_splits
// equal shares; share c leaves one partial result per sequence piece it
// holds, under piece id c + s (unique because shares and sequences are both
// visited in increasing order).
struct DecodeParams {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* qsl;        // optional: rows of a flattened batch; sequences with q_len != 1 are skipped
  float* part_o;             // [n_splits + num_seqs][Hq][D] partial outputs (unnormalised)
  float* part_m;             // [n_splits + num_seqs][Hq] running max (log2 units)
  float* part_l;             // [n_splits + num_seqs][Hq] sum of weights
  int32_t* piece_first;      // [num_seqs] share holding the first piece of each sequence
  int32_t* piece_last;       // [num_seqs] share holding the last piece
  int bt_stride;
  int num_seqs;
  int num_rows;              // rows of query/out (num_seqs, or the flattened token count)
  int num_q_heads;
  int num_kv_heads;
  int group;                 // num_q_heads / num_kv_heads
  int head_groups;           // ceil(group / 16): the matrix-core columns take 16 q heads of a kv head at a time
  int num_blocks;
  int max_seq_len;
  int n_splits;
  int piece_cost;            // blocks' worth of time a piece costs to start (share planning), >= 0
  // cascade (a prefix of blocks shared by every sequence, attended once per group of
  // sequences): the suffix launch skips the shared blocks and leaves every piece partial;
  // the prefix launch writes pre_* partials; the merge folds both in.
  int window;                // sliding window (> 0): the query at position L-1 sees keys L-window .. L-1
  int chunk;                 // chunked local attention (> 0): the query at L-1 sees keys C*((L-1) div C) .. L-1
  int skip_blocks;           // leading table entries the per-sequence pieces skip (0 without cascade)
  int force_partial;         // every piece leaves a partial result, none is finished in place
  int prefix_blocks;         // shared leading blocks (cascade), else 0
  int prefix_shares;         // prefix pieces per sequence (cascade), else 0
  int prefix_waves;          // work-groups per kv head taking prefix pieces (groups x shares), else 0
  float* pre_o;              // [prefix_shares][num_seqs][Hq][D] prefix partial outputs (unnormalised)
  float* pre_m;              // [prefix_shares][num_seqs][Hq]
  float* pre_l;              // [prefix_shares][num_seqs][Hq]
  float scale_log2;          // softmax scale * log2(e) (* k_scale for fp8 pools)
  float v_scale;             // 1, or the fp8 value scale
  int q_f32;                 // query / output are fp32 (else bf16)
  // decode that also writes the step's K/V (the kernels' write_new variant, else unused): row s of
  // new_k / new_v is the K/V of position seq_lens[s] - 1 of sequence s, all kv heads
  const void* new_k;
  const void* new_v;
  int64_t new_k_stride;      // elements between the rows of new_k
  int64_t new_v_stride;
  int new_f32;               // the rows are fp32 (else bf16; bf16 pools take bf16 rows)
  float new_k_scale;         // fp8 pools: the stored codes are those of x / scale
  float new_v_scale;
  int store_chunk_rows;      // the merge launch also stores the new rows of sequences with q_len > 1
};

// One prefill launch: grid (num_kv_heads, n_items).  Item bits: sequence (15),
// whole-row-tile flag (1), row tile (16), first key tile (16), end key tile (16).
// Items that cover only part of their row tile's key tiles come first in the
// plan; their partial results live in slot item_base + blockIdx.y.
struct PrefillParams {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* qsl;
  uint16_t* part_o;          // [slots][num_kv_heads][256 rows][D] (O / l) / sigma, fp16
  float* part_m;             // [slots][num_kv_heads][256 rows] reference maximum (log2 units)
  float* part_l;             // [slots][num_kv_heads][256 rows] sum of weights
  float* part_s;             // [slots][num_kv_heads][256 rows] sigma: a power of two, 2^15 * sigma > max |O / l|
  int bt_stride;
  int num_tokens;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int num_blocks;
  int tile_positions;        // positions per row tile: 256 / group
  int item_base;
  float scale_log2;
  float v_scale;             // 1, or the fp8 value scale (the tiles hold the codes' exact values)
  int window;                // sliding window (> 0): the row at position p sees keys p-window+1 .. p
  int chunk;                 // chunked local attention (> 0): the row at position p sees keys C*(p div C) .. p
  int kv_fp8;                // the pools hold E4M3 codes (k_scale folded into scale_log2)
  // cascade prefix tiles (prefill_body's PREFIX form): the rows of a kv head are the
  // prefix_rows query rows x its G q heads, each sees keys 0 .. prefix_keys-1 of table
  // row 0, and an item's unnormalised partial goes to pre_* at share kt0 / prefix_share_tiles
  int prefix_rows;
  int prefix_keys;
  int prefix_share_tiles;
  float* pre_o;              // [shares][prefix_rows][num_q_heads][D]
  float* pre_m;              // [shares][prefix_rows][num_q_heads] (log2 units)
  float* pre_l;              // [shares][prefix_rows][num_q_heads]
  // fresh rows (the prefill body's FRESH form, a mixed step that also stores its new K/V, bf16
  // pools): keys at or past a chunk's cached length come from row qsl[s] + (key - cached) of
  // new_k / new_v instead of the pool (the decode merge launch after stores them)
  const void* new_k;
  const void* new_v;
  int64_t new_k_stride;      // elements between the rows of new_k
  int64_t new_v_stride;
  int n_items;
  uint64_t items[kMaxPrefillItems];
};

// Merge of split row tiles: grid (n_items x 8 groups of 32 rows, num_kv_heads).  Item bits: sequence
// (16), row tile (16), first slot (20), number of slots (12).
struct PrefillMergeParams {
  void* out;
  const int32_t* qsl;
  const uint16_t* part_o;    // (O / l) / sigma, fp16
  const float* part_m;
  const float* part_l;
  const float* part_s;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int tile_positions;
  float v_scale;
  int n_items;
  uint64_t items[kMaxPrefillItems];
};

// One launch of decode waves and prefill items (a mixed batch): grid (n_decode_wgs +
// pre.n_items * pre.num_kv_heads) x 512 threads.  Work-group w < n_decode_wgs runs decode
// waves g = w * decode_waves_per_wg + wave (< decode_waves), each the decode kernel's wave
// (share g / Y, column g % Y, Y = num_kv_heads * head_groups); the others run prefill items
// (item (w - n_decode_wgs) / num_kv_heads of kv head (w - n_decode_wgs) % num_kv_heads).
struct FusedParams {
  DecodeParams dec;
  PrefillParams pre;
  int n_decode_wgs;
  int decode_waves_per_wg;   // 1 .. 8
  int decode_waves;          // (prefix_waves + n_splits) * Y
};
static_assert(sizeof(FusedParams) <= 4096, "kernel arguments of a fused launch exceed 4 KB");

// Optional kernel timing (pa_timing_enable): a launch site brackets its
// kernel with timing_mark(id, true/false, stream); a no-op unless enabled.
enum KernelId {
  kKSlotMapping = 0,
  kKReshape = 1,
  kKDecode = 2,
  kKDecodeMerge = 3,
  kKPrefill = 4,
  kKPrefillMerge = 5,
  kKStageFp8 = 6,            // no launch is timed under it (the id keeps the others fixed)
  kKFused = 7,
  kNumKernelIds = 8
};
void timing_mark(int kernel, bool begin, hipStream_t stream);

hipError_t launch_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, int bt_stride,
                               const int32_t* seq_lens, const int32_t* qsl, int num_seqs, int num_tokens,
                               int block_size, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, int64_t key_stride, int64_t value_stride,
                                    void* key_cache, void* value_cache, const int32_t* slots, int num_tokens,
                                    int num_kv_heads, int head_dim, int block_size, int num_blocks, int elem_bytes,
                                    hipStream_t stream);

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, int64_t key_stride,
                                        int64_t value_stride, uint8_t* key_cache, uint8_t* value_cache,
                                        const int32_t* slots, int num_tokens, int num_kv_heads, int head_dim,
                                        int block_size, int num_blocks, int src_f32, float k_scale,
                                        float v_scale, hipStream_t stream);

// Slot mapping and KV write in one launch.  kind: kF32 / kBF16 (plain copy, strides in
// elements of that type), kFP8 (E4M3 pools from a bf16 source) or kFP8 + 1 (from fp32);
// slots_out optional; qsl NULL: one new row per sequence, row s of key/value (a decode step).
// Work-groups: num_seqs x ceil(max_q_len / 4).
hipError_t launch_write_kv(const void* key, const void* value, int64_t key_stride, int64_t value_stride,
                           void* key_cache, void* value_cache, int32_t* slots_out, const int32_t* block_tables,
                           int bt_stride, const int32_t* seq_lens, const int32_t* qsl, int num_seqs, int num_tokens,
                           int max_q_len, int num_kv_heads, int head_dim, int block_size, int num_blocks, int kind,
                           float k_scale, float v_scale, hipStream_t stream);

// kv: kF32 (VALU kernel), kBF16 or kFP8 (matrix-core kernel); p.new_k set (kBF16 / kFP8 only):
// the matrix-core kernel also stores the step's new K/V rows and attends them from registers
hipError_t launch_decode(const DecodeParams& p, int kv, int head_dim, hipStream_t stream);
// the log-sum-exp merge of a decode launch's split sequences alone (after a fused launch)
hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, hipStream_t stream);
// decode waves and prefill items in one launch; fp8: both read the E4M3 pools (f.pre.kv_fp8 set)
// (timing_id: the kernel id the launch is timed under -- kKFused for a mixed batch, kKDecode
// for a cascade, whose prefix tiles and suffix shares share the launch)
hipError_t launch_fused(const FusedParams& f, int head_dim, bool fp8, hipStream_t stream, int timing_id = kKFused);

// The decode's static scratch (pa_decode_static): its size, and its device address on the
// current device (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
hipError_t static_scratch(void** ptr);


// the prefill kernel over bf16 pools, or over E4M3 pools when p.kv_fp8 is set
hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream);
// Every query token of a flattened batch attended on its own by one wave per (token, q head),
// on the vector ALU, without scratch: the chunks of pools or queries the prefill kernel does
// not take (fp32 pools and activations; fp32 queries over fp8 pools).  Token t of sequence s
// sits at position c_s + i (c_s = seq_lens[s] - q_len_s, i = t - qsl[s]) and sees the keys a
// decode query of a sequence of length c_s + i + 1 sees (p.window / p.chunk apply).  p: the
// decode parameters of the batch (qsl, seq_lens over num_seqs, q_f32 = 1); out is fp32.
hipError_t launch_rows_f32(const DecodeParams& p, int kv, int head_dim, int num_tokens, hipStream_t stream);
hipError_t launch_prefill_merge(const PrefillMergeParams& p, int head_dim, hipStream_t stream);
// matrix-core peak probe (measurement only): blocks x 256 threads, 4 x iters MFMAs per wave
hipError_t launch_mfma_peak(float* out, int blocks, int iters, hipStream_t stream);

}  // namespace pa
