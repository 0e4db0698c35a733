// C ABI of the paged-KV attention library: argument checks, launch geometry,
// workspace layout and error reporting.  Declarations and the meaning of
// every argument are in include/pa.h.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <functional>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

pa_status_t fail(pa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status_t ok() {
  g_last_error.clear();
  return PA_OK;
}

}  // namespace

// The failure message of the host-only parts of the library (the block pool).
pa_status_t pa::set_error(pa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

namespace {

pa_status_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(PA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// -1: follow PA_VALIDATE; 0 / 1: set by pa_set_validate
std::atomic<int> g_validate_override{-1};

// -1: follow PA_FUSED (default 1); 0 / 1 / 2 set by pa_set_fused
std::atomic<int> g_fused_override{-1};

int fused_mode() {
  const int o = g_fused_override.load(std::memory_order_relaxed);
  if (o >= 0) return o;
  static const int env = [] {
    const char* v = std::getenv("PA_FUSED");
    const int x = v && *v ? std::atoi(v) : 1;
    return x >= 0 && x <= 2 ? x : 1;
  }();
  return env;
}

bool validate_enabled() {
  const int o = g_validate_override.load(std::memory_order_relaxed);
  if (o >= 0) return o != 0;
  static const bool on = [] {
    const char* v = std::getenv("PA_VALIDATE");
    return v && v[0] && std::strcmp(v, "0") != 0;
  }();
  return on;
}

template <typename T>
bool copy_to_host(std::vector<T>& dst, const T* src, size_t n) {
  dst.resize(n);
  if (n == 0) return true;
  // the metadata may have been written by work still queued on any stream of the device (the
  // caller's stream need not be the null stream, which a blocking copy alone would order with)
  if (hipDeviceSynchronize() != hipSuccess) return false;
  return hipMemcpy(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Decode scratch: partial results of sequence pieces (ids share + sequence),
// then the first/last share of every sequence.
struct DecodeLayout {
  size_t o_bytes, m_bytes, idx_bytes, total;
};

DecodeLayout decode_layout(int64_t num_seqs, int64_t heads, int64_t n_splits, int64_t head_dim) {
  const int64_t pieces = n_splits + num_seqs;
  DecodeLayout L;
  L.o_bytes = align_up((size_t)(pieces * heads * head_dim) * sizeof(float));
  L.m_bytes = align_up((size_t)(pieces * heads) * sizeof(float));
  L.idx_bytes = align_up((size_t)num_seqs * sizeof(int32_t));
  L.total = L.o_bytes + 2 * L.m_bytes + 2 * L.idx_bytes;
  return L;
}

int env_int(const char* name, int dflt, int lo, int hi) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  const int x = std::atoi(v);
  return x >= lo && x <= hi ? x : dflt;
}

// The decode scratch of a varlen call is sized for kFusedSplitsFactor waves per SIMD (eight
// decode waves per compute unit of a fused launch); the fused launch never takes more shares.
constexpr int kFusedSplitsFactor = 2;

// decode waves per work-group of a fused launch (PA_FUSED_DECODE_WAVES, 1..8; measurement)
int fused_decode_waves() {
  static const int w = env_int("PA_FUSED_DECODE_WAVES", 8, 1, 8);
  return w;
}

// Compute units of the current device (cached per device; 256 when no device is visible).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Decode waves per SIMD the automatic split aims at: PA_DECODE_WAVES_PER_SIMD when set, else
// one, for every pool type.  With streaming loads, one wave per SIMD with two blocks in flight
// beat two waves on a Llama-3-8B layer (89 against 96 us), and with E4M3 pools as well once the
// block ids came through the scalar cache (48.4-48.9 against 51.3-51.6 us; three, four or six
// register sets at one wave: 51.3, 51.5, 54.2 us).
int decode_waves_per_simd(bool fp8) {
  (void)fp8;
  static const int env = [] {
    const char* v = std::getenv("PA_DECODE_WAVES_PER_SIMD");
    const int x = v ? std::atoi(v) : 0;
    return x >= 1 && x <= 16 ? x : 0;
  }();
  return env ? env : 1;
}

// Blocks' worth of time a decode piece costs to start (PA_DECODE_PIECE_COST overrides): the
// share planner counts it for every sequence, so shares that start several pieces hold fewer
// blocks.  An E4M3 block streams in about half a bf16 block's time, so the same start costs
// more of them: on the Llama-3-8B-shaped batch the fp8 decode launch took 48.5-49.0 us at 3,
// 47.5-47.6 at 5, 48.1 at 6 and 48.2-48.3 at 8; bf16 pools are best at 3.
int decode_piece_cost(bool fp8) {
  static const int env = env_int("PA_DECODE_PIECE_COST", -1, -1, 64);
  return env >= 0 ? env : fp8 ? 5 : 3;
}

// Waves per share of a decode launch: a kv head's q heads go 16 at a time to the matrix-core
// columns, so a kv head with more than 16 of them takes one wave per group of 16.
int decode_columns(int num_q_heads, int num_kv_heads) {
  const int group = num_q_heads / std::max(1, num_kv_heads);
  return num_kv_heads * std::max(1, (group + 15) / 16);
}

// Shares the decode work of each kv head is cut into: num_splits if positive,
// else enough waves to give every SIMD of the device decode_waves_per_simd()
// of them; never more than the blocks there can be.
int resolve_splits(int num_splits, int num_seqs, int num_kv_heads, int max_seq_len, int waves_factor = 1,
                   bool fp8 = false) {
  const int64_t max_blocks = (int64_t)num_seqs * ((max_seq_len + 15) / 16);
  int64_t w = num_splits > 0 ? num_splits
                             : (int64_t)waves_factor * decode_waves_per_simd(fp8) * 4 * device_cu_count() /
                                   std::max(1, num_kv_heads);
  w = std::min<int64_t>(std::max<int64_t>(w, 1), std::max<int64_t>(max_blocks, 1));
  return (int)std::min<int64_t>(w, 1 << 20);
}

// Checks of device metadata under PA_VALIDATE=1 (copies to the host, synchronising).
pa_status_t validate_tables(const int32_t* block_tables, int bt_stride, const int32_t* seq_lens,
                            const int32_t* qsl, int num_seqs, int num_blocks, int max_seq_len, int block_size) {
  std::vector<int32_t> sl, q, bt;
  if (!copy_to_host(sl, seq_lens, num_seqs) || !copy_to_host(bt, block_tables, (size_t)num_seqs * bt_stride))
    return fail(PA_ERR_HIP, "PA_VALIDATE: metadata copy failed");
  if (qsl && !copy_to_host(q, qsl, num_seqs + 1)) return fail(PA_ERR_HIP, "PA_VALIDATE: metadata copy failed");
  if (qsl && q[0] != 0) return fail(PA_ERR_SHAPE, "PA_VALIDATE: query_start_loc[0] = %d, expected 0", q[0]);
  for (int s = 0; s < num_seqs; ++s) {
    const int q_len = qsl ? q[s + 1] - q[s] : 1;
    if (q_len < 1) return fail(PA_ERR_SHAPE, "PA_VALIDATE: sequence %d has q_len %d", s, q_len);
    if (sl[s] < q_len || sl[s] > max_seq_len)
      return fail(PA_ERR_SHAPE, "PA_VALIDATE: seq_lens[%d] = %d outside [%d, %d]", s, sl[s], q_len, max_seq_len);
    const int nb = ceil_div(sl[s], block_size);
    if (nb > bt_stride) return fail(PA_ERR_SHAPE, "PA_VALIDATE: sequence %d needs %d blocks > bt_stride", s, nb);
    for (int j = 0; j < nb; ++j) {
      const int b = bt[(size_t)s * bt_stride + j];
      if (b < 0 || b >= num_blocks)
        return fail(PA_ERR_SHAPE, "PA_VALIDATE: block_tables[%d][%d] = %d out of [0, %d)", s, j, b, num_blocks);
    }
  }
  return PA_OK;
}

pa_status_t validate_slots(const int32_t* slots, int num_tokens, int64_t num_slots) {
  std::vector<int32_t> sm;
  if (!copy_to_host(sm, slots, num_tokens)) return fail(PA_ERR_HIP, "PA_VALIDATE: slot copy failed");
  std::vector<int32_t> seen;
  for (int t = 0; t < num_tokens; ++t) {
    if (sm[t] < 0) continue;
    if (sm[t] >= num_slots) return fail(PA_ERR_SHAPE, "PA_VALIDATE: slot_mapping[%d] = %d >= %lld", t, sm[t],
                                        (long long)num_slots);
    seen.push_back(sm[t]);
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end())
    return fail(PA_ERR_SHAPE, "PA_VALIDATE: duplicate slots in slot_mapping");
  return PA_OK;
}

pa_status_t check_attention_shape(int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                  int bt_stride) {
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", num_q_heads,
                num_kv_heads);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (block_size != pa::kBlockSize) return fail(PA_ERR_UNSUPPORTED, "block_size %d (supported: 16)", block_size);
  if (num_blocks < 1) return fail(PA_ERR_SHAPE, "num_blocks %d < 1", num_blocks);
  if (bt_stride < 1) return fail(PA_ERR_SHAPE, "bt_stride %d < 1", bt_stride);
  return PA_OK;
}

// Shared by pa_decode / pa_decode_fp8 / the decode rows of pa_prefill_varlen.
// Cascade decode: the shared prefix is cut into `shares` pieces per group of 16/G
// sequences (about one wave per SIMD; they run in the suffix launch); the suffix uses the
// split decode's layout (every piece partial), then the prefix partials follow.
int cascade_prefix_shares(int num_seqs, int group, int num_kv_heads, int prefix_blocks) {
  const int per_group = std::max(1, 16 / std::max(1, group));
  const int64_t groups = std::max<int64_t>(1, (num_seqs + per_group - 1) / per_group);
  // about one prefix wave per SIMD (PA_CASCADE_PREFIX_WAVES_PER_CU overrides the 4 per CU):
  // the suffix waves share the launch
  static const int per_cu = env_int("PA_CASCADE_PREFIX_WAVES_PER_CU", 4, 1, 64);
  const int64_t target = (int64_t)per_cu * device_cu_count();
  const int64_t sh = target / std::max<int64_t>(1, groups * num_kv_heads);
  return (int)std::min<int64_t>(std::max<int64_t>(sh, 1), std::max(prefix_blocks, 1));
}

struct CascadeLayout {
  DecodeLayout dec;
  size_t pre_o_bytes, pre_m_bytes, total;
  int n_splits, shares;
};

CascadeLayout cascade_layout(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_seq_len,
                             int prefix_blocks, int num_splits) {
  CascadeLayout L;
  // the suffix waves share the launch with the cache-bound prefix waves: twice the plain
  // decode's count kept the suffix stream busy (prefix-shared fp8 step: 59 against 67 us)
  L.n_splits = resolve_splits(num_splits, num_seqs, num_kv_heads, max_seq_len, 2);
  L.dec = decode_layout(num_seqs, num_q_heads, L.n_splits, head_dim);
  L.shares = cascade_prefix_shares(num_seqs, num_q_heads / std::max(1, num_kv_heads), num_kv_heads, prefix_blocks);
  const size_t rows = (size_t)L.shares * num_seqs * num_q_heads;
  L.pre_o_bytes = align_up(rows * head_dim * sizeof(float));
  L.pre_m_bytes = align_up(rows * sizeof(float));
  L.total = L.dec.total + L.pre_o_bytes + 2 * L.pre_m_bytes;
  return L;
}

// The parameters of one decode launch (its share count and workspace layout).
pa::DecodeParams make_decode_params(void* out, const void* query, const void* key_cache, const void* value_cache,
                                    const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                    const int32_t* qsl, int32_t num_seqs, int32_t num_rows, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len, float scale,
                                    int kv_kind, int q_f32, float k_scale, float v_scale, int32_t num_splits,
                                    void* workspace, int32_t prefix_blocks, int32_t sliding_window,
                                    int32_t local_chunk) {
  // a window (or local chunk) of W keys spans at most W/16 + 2 blocks of each sequence
  const int vis = sliding_window > 0 ? sliding_window : local_chunk;
  const int span = vis > 0 ? std::min<int64_t>(max_seq_len, (int64_t)vis + 16) : max_seq_len;
  const int n_splits =
      resolve_splits(num_splits, num_seqs, decode_columns(num_q_heads, num_kv_heads), span, 1, kv_kind == pa::kFP8);
  pa::DecodeParams p{};
  p.out = out;
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.qsl = qsl;
  p.bt_stride = bt_stride;
  p.num_seqs = num_seqs;
  p.num_rows = num_rows;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.head_groups = (p.group + 15) / 16;  // 1 for a cascade (at most 16 q heads per kv head)
  p.max_seq_len = max_seq_len;
  p.n_splits = n_splits;
  p.piece_cost = decode_piece_cost(kv_kind == pa::kFP8);
  p.window = sliding_window > 0 ? sliding_window : 0;
  p.chunk = local_chunk > 0 ? local_chunk : 0;
  p.scale_log2 = scale * 1.4426950408889634f * (kv_kind == pa::kFP8 ? k_scale : 1.f);
  p.v_scale = kv_kind == pa::kFP8 ? v_scale : 1.f;
  p.q_f32 = q_f32;
  if (prefix_blocks > 0) {  // cascade: prefix launch, then every suffix piece partial, then the merge
    const CascadeLayout cl = cascade_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                            prefix_blocks, num_splits);
    const DecodeLayout& lay = cl.dec;
    p.n_splits = cl.n_splits;
    auto* base = static_cast<unsigned char*>(workspace);
    p.part_o = reinterpret_cast<float*>(base);
    p.part_m = reinterpret_cast<float*>(base + lay.o_bytes);
    p.part_l = reinterpret_cast<float*>(base + lay.o_bytes + lay.m_bytes);
    p.piece_first = reinterpret_cast<int32_t*>(base + lay.o_bytes + 2 * lay.m_bytes);
    p.piece_last = reinterpret_cast<int32_t*>(base + lay.o_bytes + 2 * lay.m_bytes + lay.idx_bytes);
    unsigned char* pre = base + lay.total;
    p.pre_o = reinterpret_cast<float*>(pre);
    p.pre_m = reinterpret_cast<float*>(pre + cl.pre_o_bytes);
    p.pre_l = reinterpret_cast<float*>(pre + cl.pre_o_bytes + cl.pre_m_bytes);
    p.skip_blocks = prefix_blocks;
    p.force_partial = 1;
    p.prefix_blocks = prefix_blocks;
    p.prefix_shares = cl.shares;
    const int per_group = 16 / p.group;
    p.prefix_waves = (num_seqs + per_group - 1) / per_group * cl.shares;
  } else if (n_splits > 1) {
    const DecodeLayout lay = decode_layout(num_seqs, num_q_heads, n_splits, head_dim);
    auto* base = static_cast<unsigned char*>(workspace);
    p.part_o = reinterpret_cast<float*>(base);
    p.part_m = reinterpret_cast<float*>(base + lay.o_bytes);
    p.part_l = reinterpret_cast<float*>(base + lay.o_bytes + lay.m_bytes);
    p.piece_first = reinterpret_cast<int32_t*>(base + lay.o_bytes + 2 * lay.m_bytes);
    p.piece_last = reinterpret_cast<int32_t*>(base + lay.o_bytes + 2 * lay.m_bytes + lay.idx_bytes);
  }
  return p;
}

// The step's new K/V rows for a decode launch that stores them itself (row s: sequence s).
struct NewRows {
  const void* key;
  const void* value;
  int64_t key_stride, value_stride;  // elements
  int src_f32;
  float k_scale, v_scale;            // fp8 pools, else 1
};

pa_status_t run_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens, const int32_t* qsl,
                       int32_t num_seqs, int32_t num_rows, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale, int kv_kind,
                       int q_f32, float k_scale, float v_scale, int32_t num_splits, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, int32_t prefix_blocks = 0,
                       int32_t sliding_window = 0, int32_t local_chunk = 0, const NewRows* rows = nullptr) {
  pa::DecodeParams p = make_decode_params(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, qsl,
                                          num_seqs, num_rows, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                          scale, kv_kind, q_f32, k_scale, v_scale, num_splits, workspace,
                                          prefix_blocks, sliding_window, local_chunk);
  p.num_blocks = num_blocks;
  if (rows) {
    p.new_k = rows->key;
    p.new_v = rows->value;
    p.new_k_stride = rows->key_stride;
    p.new_v_stride = rows->value_stride;
    p.new_f32 = rows->src_f32;
    p.new_k_scale = rows->k_scale;
    p.new_v_scale = rows->v_scale;
  }
  (void)workspace_bytes;
  (void)block_size;
  return hip_status(pa::launch_decode(p, kv_kind, head_dim, stream), "decode launch");
}

pa_status_t check_decode_args(const void* out, const void* query, const void* key_cache, const void* value_cache,
                              const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                              int32_t num_splits, void* workspace, size_t workspace_bytes, size_t need_override = SIZE_MAX) {
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d < 0", num_seqs);
  if (!out || !query || !key_cache || !value_cache || !block_tables || !seq_lens)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  pa_status_t st = check_attention_shape(num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, bt_stride);
  if (st != PA_OK) return st;
  if (max_seq_len < 1) return fail(PA_ERR_SHAPE, "max_seq_len %d < 1", max_seq_len);
  if (ceil_div(max_seq_len, block_size) > bt_stride)
    return fail(PA_ERR_SHAPE, "max_seq_len %d needs %d table columns > bt_stride %d", max_seq_len,
                ceil_div(max_seq_len, block_size), bt_stride);
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "scale is not finite");
  if (num_splits < 0) return fail(PA_ERR_SHAPE, "num_splits %d < 0", num_splits);
  const size_t need = need_override != SIZE_MAX
                          ? need_override
                          : pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                      num_splits);
  if (need && (!workspace || workspace_bytes < need))
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (need && (reinterpret_cast<uintptr_t>(workspace) % kAlign))
    return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(pa_status_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_SHAPE: return "inconsistent shape or metadata";
    case PA_ERR_DTYPE: return "unsupported dtype for this call";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_NO_SPACE: return "not enough free blocks";
    case PA_ERR_STATE: return "unknown request or call out of order";
  }
  return "unknown status";
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

pa_status_t pa_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, int32_t bt_stride,
                            const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                            int32_t num_tokens, int32_t block_size, void* stream) {
  if (num_seqs < 0 || num_tokens < 0) return fail(PA_ERR_SHAPE, "negative num_seqs or num_tokens");
  if (num_seqs == 0) return ok();
  if (!slot_mapping || !block_tables || !seq_lens || !query_start_loc)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  if (block_size < 1) return fail(PA_ERR_SHAPE, "block_size %d < 1", block_size);
  if (bt_stride < 1) return fail(PA_ERR_SHAPE, "bt_stride %d < 1", bt_stride);
  if (validate_enabled()) {
    std::vector<int32_t> q;
    if (!copy_to_host(q, query_start_loc, num_seqs + 1)) return fail(PA_ERR_HIP, "PA_VALIDATE: copy failed");
    if (q[num_seqs] != num_tokens)
      return fail(PA_ERR_SHAPE, "PA_VALIDATE: query_start_loc[num_seqs] = %d != num_tokens %d", q[num_seqs],
                  num_tokens);
    pa_status_t st = validate_tables(block_tables, bt_stride, seq_lens, query_start_loc, num_seqs, INT32_MAX,
                                     bt_stride * block_size, block_size);
    if (st != PA_OK) return st;
  }
  return hip_status(pa::launch_slot_mapping(slot_mapping, block_tables, bt_stride, seq_lens, query_start_loc,
                                            num_seqs, num_tokens, block_size, static_cast<hipStream_t>(stream)),
                    "slot_mapping launch");
}

pa_status_t pa_reshape_and_cache(const void* key, const void* value, int64_t key_tok_stride,
                                 int64_t value_tok_stride, void* key_cache, void* value_cache,
                                 const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype_t dtype,
                                 void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens %d < 0", num_tokens);
  if (num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
    return fail(PA_ERR_SHAPE, "non-positive num_kv_heads/head_dim/block_size/num_blocks");
  if (key_tok_stride < (int64_t)num_kv_heads * head_dim || value_tok_stride < (int64_t)num_kv_heads * head_dim)
    return fail(PA_ERR_SHAPE, "token stride smaller than num_kv_heads * head_dim");
  if (num_tokens == 0) return ok();
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  if ((int64_t)num_blocks * block_size > INT32_MAX) return fail(PA_ERR_SHAPE, "pool has more than 2^31 slots");
  if (validate_enabled()) {
    pa_status_t st = validate_slots(slot_mapping, num_tokens, (int64_t)num_blocks * block_size);
    if (st != PA_OK) return st;
  }
  const int elem = dtype == PA_F32 ? 4 : 2;
  return hip_status(pa::launch_reshape_and_cache(key, value, key_tok_stride, value_tok_stride, key_cache, value_cache,
                                                 slot_mapping, num_tokens, num_kv_heads, head_dim, block_size,
                                                 num_blocks, elem, static_cast<hipStream_t>(stream)),
                    "reshape_and_cache launch");
}

pa_status_t pa_reshape_and_cache_fp8(const void* key, const void* value, int64_t key_tok_stride,
                                     int64_t value_tok_stride, uint8_t* key_cache, uint8_t* value_cache,
                                     const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype_t src_dtype,
                                     float k_scale, float v_scale, void* stream) {
  if (src_dtype != PA_F32 && src_dtype != PA_BF16) return fail(PA_ERR_DTYPE, "src_dtype must be PA_F32 or PA_BF16");
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens %d < 0", num_tokens);
  if (num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
    return fail(PA_ERR_SHAPE, "non-positive num_kv_heads/head_dim/block_size/num_blocks");
  if (key_tok_stride < (int64_t)num_kv_heads * head_dim || value_tok_stride < (int64_t)num_kv_heads * head_dim)
    return fail(PA_ERR_SHAPE, "token stride smaller than num_kv_heads * head_dim");
  if ((num_kv_heads * head_dim) % 8) return fail(PA_ERR_UNSUPPORTED, "num_kv_heads * head_dim must be a multiple of 8");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  if (num_tokens == 0) return ok();
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  if ((int64_t)num_blocks * block_size > INT32_MAX) return fail(PA_ERR_SHAPE, "pool has more than 2^31 slots");
  if (validate_enabled()) {
    pa_status_t st = validate_slots(slot_mapping, num_tokens, (int64_t)num_blocks * block_size);
    if (st != PA_OK) return st;
  }
  return hip_status(pa::launch_reshape_and_cache_fp8(key, value, key_tok_stride, value_tok_stride, key_cache,
                                                     value_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                                                     block_size, num_blocks, src_dtype == PA_F32, k_scale, v_scale,
                                                     static_cast<hipStream_t>(stream)),
                    "reshape_and_cache_fp8 launch");
}

namespace {

pa_status_t check_write_kv(const void* key, const void* value, int64_t key_tok_stride, int64_t value_tok_stride,
                           const void* key_cache, const void* value_cache, const int32_t* block_tables,
                           int32_t bt_stride, const int32_t* seq_lens, const int32_t* query_start_loc,
                           int32_t num_seqs, int32_t num_tokens, int32_t max_q_len, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks) {
  if (num_seqs < 0 || num_tokens < 0 || max_q_len < 0) return fail(PA_ERR_SHAPE, "negative count");
  if (num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1 || bt_stride < 1)
    return fail(PA_ERR_SHAPE, "non-positive num_kv_heads/head_dim/block_size/num_blocks/bt_stride");
  if (key_tok_stride < (int64_t)num_kv_heads * head_dim || value_tok_stride < (int64_t)num_kv_heads * head_dim)
    return fail(PA_ERR_SHAPE, "token stride smaller than num_kv_heads * head_dim");
  if ((int64_t)num_blocks * block_size > INT32_MAX) return fail(PA_ERR_SHAPE, "pool has more than 2^31 slots");
  if (num_seqs == 0 || num_tokens == 0 || max_q_len == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !block_tables || !seq_lens || !query_start_loc)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  if (validate_enabled()) {
    std::vector<int32_t> q;
    if (!copy_to_host(q, query_start_loc, num_seqs + 1)) return fail(PA_ERR_HIP, "PA_VALIDATE: copy failed");
    if (q[num_seqs] != num_tokens)
      return fail(PA_ERR_SHAPE, "PA_VALIDATE: query_start_loc[num_seqs] = %d != num_tokens %d", q[num_seqs],
                  num_tokens);
    pa_status_t st = validate_tables(block_tables, bt_stride, seq_lens, query_start_loc, num_seqs, INT32_MAX,
                                     num_blocks, block_size);
    if (st != PA_OK) return st;
  }
  return PA_OK;
}

}  // namespace

pa_status_t pa_write_kv(const void* key, const void* value, int64_t key_tok_stride, int64_t value_tok_stride,
                        void* key_cache, void* value_cache, int32_t* slot_mapping, const int32_t* block_tables,
                        int32_t bt_stride, const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                        int32_t num_tokens, int32_t max_q_len, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t num_blocks, pa_dtype_t dtype, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  pa_status_t st = check_write_kv(key, value, key_tok_stride, value_tok_stride, key_cache, value_cache, block_tables,
                                  bt_stride, seq_lens, query_start_loc, num_seqs, num_tokens, max_q_len, num_kv_heads,
                                  head_dim, block_size, num_blocks);
  if (st != PA_OK) return st;
  if (num_seqs == 0 || num_tokens == 0 || max_q_len == 0) return ok();
  return hip_status(pa::launch_write_kv(key, value, key_tok_stride, value_tok_stride, key_cache, value_cache,
                                        slot_mapping, block_tables, bt_stride, seq_lens, query_start_loc, num_seqs,
                                        num_tokens, max_q_len, num_kv_heads, head_dim, block_size, num_blocks,
                                        dtype == PA_F32 ? pa::kF32 : pa::kBF16, 1.f, 1.f,
                                        static_cast<hipStream_t>(stream)),
                    "write_kv launch");
}

pa_status_t pa_write_kv_fp8(const void* key, const void* value, int64_t key_tok_stride, int64_t value_tok_stride,
                            uint8_t* key_cache, uint8_t* value_cache, int32_t* slot_mapping,
                            const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                            const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t max_q_len,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            pa_dtype_t src_dtype, float k_scale, float v_scale, void* stream) {
  if (src_dtype != PA_F32 && src_dtype != PA_BF16) return fail(PA_ERR_DTYPE, "src_dtype must be PA_F32 or PA_BF16");
  if ((num_kv_heads * head_dim) % 8) return fail(PA_ERR_UNSUPPORTED, "num_kv_heads * head_dim must be a multiple of 8");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  pa_status_t st = check_write_kv(key, value, key_tok_stride, value_tok_stride, key_cache, value_cache, block_tables,
                                  bt_stride, seq_lens, query_start_loc, num_seqs, num_tokens, max_q_len, num_kv_heads,
                                  head_dim, block_size, num_blocks);
  if (st != PA_OK) return st;
  if (num_seqs == 0 || num_tokens == 0 || max_q_len == 0) return ok();
  return hip_status(pa::launch_write_kv(key, value, key_tok_stride, value_tok_stride, key_cache, value_cache,
                                        slot_mapping, block_tables, bt_stride, seq_lens, query_start_loc, num_seqs,
                                        num_tokens, max_q_len, num_kv_heads, head_dim, block_size, num_blocks,
                                        src_dtype == PA_F32 ? pa::kFP8 + 1 : pa::kFP8, k_scale, v_scale,
                                        static_cast<hipStream_t>(stream)),
                    "write_kv_fp8 launch");
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t num_splits) {
  if (num_seqs < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 || max_seq_len < 1 || num_splits < 0)
    return 0;
  if (num_q_heads % num_kv_heads) return 0;
  // sized for two waves per SIMD: the decode part of a fused decode + prefill launch runs up
  // to eight decode waves per compute unit (an automatic plain decode uses half of it)
  const int n_splits = resolve_splits(num_splits, num_seqs, decode_columns(num_q_heads, num_kv_heads), max_seq_len,
                                      kFusedSplitsFactor);
  if (n_splits <= 1) return 0;
  return decode_layout(num_seqs, num_q_heads, n_splits, head_dim).total;
}

pa_status_t pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, int32_t max_seq_len, float scale, pa_dtype_t dtype, int32_t num_splits,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  pa_status_t st = check_decode_args(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                                     num_splits, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (dtype == PA_BF16 && num_q_heads / num_kv_heads > pa::kMaxGqa)
    return fail(PA_ERR_UNSUPPORTED, "bf16 decode supports up to %d q heads per kv head", pa::kMaxGqa);
  if (num_seqs == 0) return ok();
  if (validate_enabled()) {
    st = validate_tables(block_tables, bt_stride, seq_lens, nullptr, num_seqs, num_blocks, max_seq_len, block_size);
    if (st != PA_OK) return st;
  }
  const int kind = dtype == PA_F32 ? pa::kF32 : pa::kBF16;
  return run_decode(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, nullptr, num_seqs,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale, kind,
                    dtype == PA_F32, 1.f, 1.f, num_splits, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream));
}

pa_status_t pa_decode_static(void* out, const void* query, const void* key_cache, const void* value_cache,
                             const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                             pa_dtype_t dtype, int32_t num_splits, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  pa_status_t st = check_decode_args(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                                     num_splits, nullptr, 0, /*need_override=*/0);
  if (st != PA_OK) return st;
  if (dtype == PA_BF16 && num_q_heads / num_kv_heads > pa::kMaxGqa)
    return fail(PA_ERR_UNSUPPORTED, "bf16 decode supports up to %d q heads per kv head", pa::kMaxGqa);
  const size_t need =
      pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, num_splits);
  if (need > pa::kStaticScratchBytes)
    return fail(PA_ERR_WORKSPACE,
                "pa_decode_static: this batch needs %zu bytes of scratch, more than the library's static %zu "
                "(use pa_decode with a workspace, or fewer sequences, heads or splits)",
                need, pa::kStaticScratchBytes);
  if (num_seqs == 0) return ok();
  if (validate_enabled()) {
    st = validate_tables(block_tables, bt_stride, seq_lens, nullptr, num_seqs, num_blocks, max_seq_len, block_size);
    if (st != PA_OK) return st;
  }
  void* ws = nullptr;
  if (need) {
    st = hip_status(pa::static_scratch(&ws), "pa_decode_static: device address of the static scratch");
    if (st != PA_OK) return st;
  }
  const int kind = dtype == PA_F32 ? pa::kF32 : pa::kBF16;
  return run_decode(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, nullptr, num_seqs,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale, kind,
                    dtype == PA_F32, 1.f, 1.f, num_splits, ws, need ? pa::kStaticScratchBytes : 0,
                    static_cast<hipStream_t>(stream));
}

pa_status_t pa_decode_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                          const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, int32_t max_seq_len, float scale, pa_dtype_t q_dtype, float k_scale,
                          float v_scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (q_dtype != PA_F32 && q_dtype != PA_BF16) return fail(PA_ERR_DTYPE, "q_dtype must be PA_F32 or PA_BF16");
  pa_status_t st = check_decode_args(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                                     num_splits, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  if (num_q_heads / num_kv_heads > pa::kMaxGqa)
    return fail(PA_ERR_UNSUPPORTED, "fp8 decode supports up to %d q heads per kv head", pa::kMaxGqa);
  if (num_seqs == 0) return ok();
  if (validate_enabled()) {
    st = validate_tables(block_tables, bt_stride, seq_lens, nullptr, num_seqs, num_blocks, max_seq_len, block_size);
    if (st != PA_OK) return st;
  }
  return run_decode(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, nullptr, num_seqs,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale, pa::kFP8,
                    q_dtype == PA_F32, k_scale, v_scale, num_splits, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream));
}

namespace {

// pa_decode_write / pa_decode_write_fp8: the decode launch stores the new rows itself when the
// pools are bf16 or fp8 and each kv-head slice of a row is 16-byte aligned; otherwise (fp32
// pools, other alignments) the KV write runs first as its own launch.  Both give the same bytes.
pa_status_t decode_write(void* out, const void* query, const void* key, const void* value, int64_t key_tok_stride,
                         int64_t value_tok_stride, void* key_cache, void* value_cache, const int32_t* block_tables,
                         int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         int32_t max_seq_len, float scale, int kv_kind, pa_dtype_t dtype, float k_scale,
                         float v_scale, int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream,
                         int32_t sliding_window = 0, int32_t local_chunk = 0) {
  pa_status_t st = check_decode_args(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                                     num_splits, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (kv_kind != pa::kF32 && num_q_heads / num_kv_heads > pa::kMaxGqa)
    return fail(PA_ERR_UNSUPPORTED, "decode supports up to %d q heads per kv head", pa::kMaxGqa);
  if (num_seqs > 0 && (!key || !value)) return fail(PA_ERR_NULL, "key or value is NULL");
  if (key_tok_stride < (int64_t)num_kv_heads * head_dim || value_tok_stride < (int64_t)num_kv_heads * head_dim)
    return fail(PA_ERR_SHAPE, "token stride smaller than num_kv_heads * head_dim");
  if ((int64_t)num_blocks * block_size > INT32_MAX) return fail(PA_ERR_SHAPE, "pool has more than 2^31 slots");
  if (num_seqs == 0) return ok();
  if (validate_enabled()) {
    st = validate_tables(block_tables, bt_stride, seq_lens, nullptr, num_seqs, num_blocks, max_seq_len, block_size);
    if (st != PA_OK) return st;
  }
  const int src_f32 = dtype == PA_F32;
  const int64_t elem = src_f32 ? 4 : 2;
  const uintptr_t align = (uintptr_t)key | (uintptr_t)value | (uintptr_t)(key_tok_stride * elem) |
                          (uintptr_t)(value_tok_stride * elem);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (kv_kind != pa::kF32 && (align & 15u) == 0) {
    const NewRows rows{key, value, key_tok_stride, value_tok_stride, src_f32, k_scale, v_scale};
    return run_decode(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, nullptr, num_seqs,
                      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                      kv_kind, src_f32, k_scale, v_scale, num_splits, workspace, workspace_bytes, s, 0,
                      sliding_window, local_chunk, &rows);
  }
  const int write_kind = kv_kind == pa::kFP8 ? (src_f32 ? pa::kFP8 + 1 : pa::kFP8) : kv_kind;
  st = hip_status(pa::launch_write_kv(key, value, key_tok_stride, value_tok_stride, key_cache, value_cache, nullptr,
                                      block_tables, bt_stride, seq_lens, nullptr, num_seqs, num_seqs, 1, num_kv_heads,
                                      head_dim, block_size, num_blocks, write_kind, k_scale, v_scale, s),
                  "write_kv launch");
  if (st != PA_OK) return st;
  return run_decode(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, nullptr, num_seqs, num_seqs,
                    num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale, kv_kind, src_f32,
                    k_scale, v_scale, num_splits, workspace, workspace_bytes, s, 0, sliding_window, local_chunk);
}

}  // namespace

pa_status_t pa_decode_write(void* out, const void* query, const void* key, const void* value, int64_t key_tok_stride,
                            int64_t value_tok_stride, void* key_cache, void* value_cache, const int32_t* block_tables,
                            int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_seq_len, float scale, pa_dtype_t dtype, int32_t num_splits, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  return decode_write(out, query, key, value, key_tok_stride, value_tok_stride, key_cache, value_cache, block_tables,
                      bt_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_seq_len, scale, dtype == PA_F32 ? pa::kF32 : pa::kBF16, dtype, 1.f, 1.f, num_splits,
                      workspace, workspace_bytes, stream);
}

pa_status_t pa_decode_write_fp8(void* out, const void* query, const void* key, const void* value,
                                int64_t key_tok_stride, int64_t value_tok_stride, uint8_t* key_cache,
                                uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                                float scale, pa_dtype_t dtype, float k_scale, float v_scale, int32_t num_splits,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  return decode_write(out, query, key, value, key_tok_stride, value_tok_stride, key_cache, value_cache, block_tables,
                      bt_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_seq_len, scale, pa::kFP8, dtype, k_scale, v_scale, num_splits, workspace, workspace_bytes,
                      stream);
}

// the sliding-window and chunked-local decode steps that also store the new K/V: pa_decode_write's path with
// the mask of pa_decode_window / pa_decode_local (the new row, at L - 1, is always visible)
pa_status_t pa_decode_window_write(void* out, const void* query, const void* key, const void* value,
                                   int64_t key_tok_stride, int64_t value_tok_stride, void* key_cache,
                                   void* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                   const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_seq_len, float scale, pa_dtype_t dtype, int32_t sliding_window,
                                   int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  if (sliding_window < 1) return fail(PA_ERR_SHAPE, "sliding_window %d < 1", sliding_window);
  return decode_write(out, query, key, value, key_tok_stride, value_tok_stride, key_cache, value_cache, block_tables,
                      bt_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_seq_len, scale, dtype == PA_F32 ? pa::kF32 : pa::kBF16, dtype, 1.f, 1.f, num_splits,
                      workspace, workspace_bytes, stream, sliding_window, 0);
}

pa_status_t pa_decode_window_write_fp8(void* out, const void* query, const void* key, const void* value,
                                       int64_t key_tok_stride, int64_t value_tok_stride, uint8_t* key_cache,
                                       uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                       const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_seq_len, float scale, pa_dtype_t dtype, float k_scale,
                                       float v_scale, int32_t sliding_window, int32_t num_splits, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  if (sliding_window < 1) return fail(PA_ERR_SHAPE, "sliding_window %d < 1", sliding_window);
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  return decode_write(out, query, key, value, key_tok_stride, value_tok_stride, key_cache, value_cache, block_tables,
                      bt_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_seq_len, scale, pa::kFP8, dtype, k_scale, v_scale, num_splits, workspace, workspace_bytes,
                      stream, sliding_window, 0);
}

pa_status_t pa_decode_local_write(void* out, const void* query, const void* key, const void* value,
                                  int64_t key_tok_stride, int64_t value_tok_stride, void* key_cache, void* value_cache,
                                  const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                                  pa_dtype_t dtype, int32_t chunk_size, int32_t num_splits, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  if (chunk_size < 1) return fail(PA_ERR_SHAPE, "chunk_size %d < 1", chunk_size);
  return decode_write(out, query, key, value, key_tok_stride, value_tok_stride, key_cache, value_cache, block_tables,
                      bt_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_seq_len, scale, dtype == PA_F32 ? pa::kF32 : pa::kBF16, dtype, 1.f, 1.f, num_splits,
                      workspace, workspace_bytes, stream, 0, chunk_size);
}

pa_status_t pa_decode_local_write_fp8(void* out, const void* query, const void* key, const void* value,
                                      int64_t key_tok_stride, int64_t value_tok_stride, uint8_t* key_cache,
                                      uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                      const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      int32_t max_seq_len, float scale, pa_dtype_t dtype, float k_scale,
                                      float v_scale, int32_t chunk_size, int32_t num_splits, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  if (chunk_size < 1) return fail(PA_ERR_SHAPE, "chunk_size %d < 1", chunk_size);
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  return decode_write(out, query, key, value, key_tok_stride, value_tok_stride, key_cache, value_cache, block_tables,
                      bt_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_seq_len, scale, pa::kFP8, dtype, k_scale, v_scale, num_splits, workspace, workspace_bytes,
                      stream, 0, chunk_size);
}

namespace {

// Arguments of a cascade call on top of the decode checks: a prefix of whole blocks
// inside every sequence, a group of at most 16 q heads, and (PA_VALIDATE=1) tables
// that really share it.
// writes: the step's new rows are stored as well, so each must lie after the shared prefix.
pa_status_t check_cascade(const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t block_size, int32_t max_seq_len,
                          int32_t prefix_blocks, bool writes = false) {
  if (prefix_blocks < 1) return fail(PA_ERR_SHAPE, "prefix_blocks %d < 1", prefix_blocks);
  if ((int64_t)prefix_blocks * block_size > max_seq_len)
    return fail(PA_ERR_SHAPE, "prefix of %d blocks longer than max_seq_len %d", prefix_blocks, max_seq_len);
  if (num_q_heads / num_kv_heads > pa::kMaxGroup)
    return fail(PA_ERR_UNSUPPORTED, "cascade decode supports up to %d q heads per kv head", pa::kMaxGroup);
  if (!validate_enabled() || num_seqs == 0) return PA_OK;
  std::vector<int32_t> sl, bt;
  if (!copy_to_host(sl, seq_lens, num_seqs) || !copy_to_host(bt, block_tables, (size_t)num_seqs * bt_stride))
    return fail(PA_ERR_HIP, "PA_VALIDATE: metadata copy failed");
  for (int s = 0; s < num_seqs; ++s) {
    if (sl[s] < prefix_blocks * block_size)
      return fail(PA_ERR_SHAPE, "PA_VALIDATE: seq_lens[%d] = %d shorter than the shared prefix", s, sl[s]);
    if (writes && sl[s] <= prefix_blocks * block_size)
      return fail(PA_ERR_SHAPE, "PA_VALIDATE: the new row of sequence %d would be stored inside the shared prefix", s);
    for (int j = 0; j < prefix_blocks; ++j)
      if (bt[(size_t)s * bt_stride + j] != bt[j])
        return fail(PA_ERR_SHAPE, "PA_VALIDATE: block_tables[%d][%d] differs from sequence 0's", s, j);
  }
  return PA_OK;
}

}  // namespace

namespace {

// Cascade prefix as dense matrix-core tiles ("vLLM 架构概述" §2: blocks shared by several
// requests are stored once; cascade attention in the backend table of §6).  For each kv
// head the num_seqs query rows x its G q heads are rows of the prefill kernel's 256-row
// tiles (256 / G sequences each), attended against the shared prefix, whose key tiles are
// cut into `shares` key ranges: one work item per (kv head, row tile, share).  The items run
// in one launch with the suffix shares of the split decode (launch_fused: the decode
// work-groups first, eight decode waves each, then the items, one work-group per compute
// unit), each item leaves an unnormalised partial per (share, sequence, head), and the
// decode merge folds them with the suffix pieces.  fp8 pools: the tiles copy the codes and
// convert them to their exact bf16 values in the kernel, on the way to the matrix cores.
//
// The split between the two parts uses the fused launch's host estimate (PA_FUSED_TILE_NS
// per 64-key tile of a 256-row item plus 5 us; PA_FUSED_CU_GBPS per decode compute unit up
// to PA_FUSED_DECODE_GBPS in all).  The host does not see seq_lens here, so the suffix bytes
// are estimated as if suffix lengths were spread evenly up to max_seq_len - prefix.  The
// share count minimises the larger of the item time and the suffix time.
struct CascadeTilePlan {
  bool ok = false;
  int positions = 0;     // sequences per row tile: 256 / G
  int row_tiles = 0;
  int key_tiles = 0;     // 64-key tiles of the prefix
  int tps = 0;           // key tiles per share
  int shares = 0;
  int n_decode_wgs = 0;  // compute units the estimate gives the suffix
  int n_splits = 0;      // suffix shares per kv head
  size_t dec_bytes = 0, pre_o_bytes = 0, pre_m_bytes = 0, total = 0;
};

bool cascade_tiles_enabled() {
  static const int on = env_int("PA_CASCADE_TILES", 1, 0, 1);
  return on != 0;
}

CascadeTilePlan plan_cascade_tiles(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_seq_len,
                                   int prefix_blocks, int num_splits, int kv_elem) {
  CascadeTilePlan cp;
  const int G = num_q_heads / std::max(1, num_kv_heads);
  if (num_seqs < 1 || G < 1 || G > pa::kMaxGroup) return cp;
  cp.positions = pa::kPrefillRows / G;
  cp.row_tiles = ceil_div(num_seqs, cp.positions);
  const int prefix_len = prefix_blocks * pa::kBlockSize;
  cp.key_tiles = ceil_div(prefix_len, pa::kPrefillKeys);
  static const double tile_s = env_int("PA_FUSED_TILE_NS", 2200, 100, 1000000) * 1e-9;
  // the decode shares' rate inside the fused launch: about 30 GB/s per compute unit, and no
  // more than about 5.8 TB/s in all (the items' own traffic shares HBM with it)
  static const double bw = env_int("PA_FUSED_DECODE_GBPS", 5800, 100, 100000) * 1e9;
  static const double bw_cu = env_int("PA_FUSED_CU_GBPS", 30, 1, 100000) * 1e9;
  // an fp8 block is half the bytes for the same work per block: fewer bytes per compute unit
  // (measured on the prefix-shared fp8 step: 18 GB/s per decode compute unit)
  static const double bw_cu8 = env_int("PA_FUSED_CU_GBPS_FP8", 18, 1, 100000) * 1e9;
  const double item_s = 5e-6;
  const int C = device_cu_count();
  const double cu_rate = kv_elem == 1 ? bw_cu8 : bw_cu;
  const double dec_bytes =
      2.0 * num_seqs * 0.5 * std::max(0, max_seq_len - prefix_len) * num_kv_heads * head_dim * kv_elem;
  double best = 1e30;
  static const int forced = env_int("PA_CASCADE_SHARES", 0, 0, 1 << 16);  // measurement: fix the share count
  for (int want = 1; want <= cp.key_tiles; ++want) {
    const int tps = ceil_div(cp.key_tiles, want);  // near-equal key ranges
    const int shares = ceil_div(cp.key_tiles, tps);
    if (shares != want) continue;
    const int items = cp.row_tiles * shares;
    if (items > pa::kMaxPrefillItems) break;
    const int q = C - items * num_kv_heads;
    if (q < 8) break;
    if (forced > 0 && shares != forced) continue;
    const double t = std::max(tps * tile_s + item_s, dec_bytes / std::min(bw, cu_rate * q));
    if (t < best) {
      best = t;
      cp.tps = tps;
      cp.shares = shares;
      cp.n_decode_wgs = q;
    }
  }
  if (cp.tps == 0) return cp;
  // suffix shares: eight decode waves on each compute unit of the estimate (or num_splits),
  // never more than the blocks there can be
  const int64_t max_blocks = (int64_t)num_seqs * ceil_div(max_seq_len, pa::kBlockSize);
  int64_t ns = num_splits > 0 ? num_splits : (int64_t)cp.n_decode_wgs * fused_decode_waves() / num_kv_heads;
  ns = std::min<int64_t>(std::max<int64_t>(ns, 1), std::max<int64_t>(max_blocks, 1));
  cp.n_splits = (int)ns;
  cp.n_decode_wgs = ceil_div((int64_t)cp.n_splits * num_kv_heads, fused_decode_waves());
  cp.dec_bytes = align_up(decode_layout(num_seqs, num_q_heads, cp.n_splits, head_dim).total);
  const size_t rows = (size_t)cp.shares * num_seqs * num_q_heads;
  cp.pre_o_bytes = align_up(rows * head_dim * sizeof(float));
  cp.pre_m_bytes = align_up(rows * sizeof(float));
  cp.total = cp.dec_bytes + cp.pre_o_bytes + 2 * cp.pre_m_bytes;
  cp.ok = true;
  return cp;
}

pa_status_t run_cascade_tiles(const CascadeTilePlan& cp, void* out, const void* query, const void* key_cache,
                              const void* value_cache, const int32_t* block_tables, int32_t bt_stride,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t num_blocks, int32_t max_seq_len, float scale, int kv_kind,
                              float k_scale, float v_scale, void* workspace, hipStream_t stream,
                              int32_t prefix_blocks, const NewRows* rows = nullptr) {
  auto* base = static_cast<unsigned char*>(workspace);
  // the suffix: the split decode's shares over each sequence's own blocks, every piece partial
  pa::FusedParams f{};
  pa::DecodeParams& d = f.dec;
  d = make_decode_params(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, nullptr, num_seqs,
                         num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, scale, kv_kind, 0, k_scale,
                         v_scale, cp.n_splits, workspace, 0, 0, 0);
  d.num_blocks = num_blocks;
  d.n_splits = cp.n_splits;
  const DecodeLayout lay = decode_layout(num_seqs, num_q_heads, cp.n_splits, head_dim);
  d.part_o = reinterpret_cast<float*>(base);
  d.part_m = reinterpret_cast<float*>(base + lay.o_bytes);
  d.part_l = reinterpret_cast<float*>(base + lay.o_bytes + lay.m_bytes);
  d.piece_first = reinterpret_cast<int32_t*>(base + lay.o_bytes + 2 * lay.m_bytes);
  d.piece_last = reinterpret_cast<int32_t*>(base + lay.o_bytes + 2 * lay.m_bytes + lay.idx_bytes);
  unsigned char* pre = base + cp.dec_bytes;
  d.pre_o = reinterpret_cast<float*>(pre);
  d.pre_m = reinterpret_cast<float*>(pre + cp.pre_o_bytes);
  d.pre_l = reinterpret_cast<float*>(pre + cp.pre_o_bytes + cp.pre_m_bytes);
  d.skip_blocks = prefix_blocks;
  d.force_partial = 1;
  d.prefix_blocks = prefix_blocks;
  d.prefix_shares = 0;  // in the launch: no decode wave takes prefix pieces
  d.prefix_waves = 0;
  if (rows) {  // the suffix waves store the new rows (each in its sequence's own blocks)
    d.new_k = rows->key;
    d.new_v = rows->value;
    d.new_k_stride = rows->key_stride;
    d.new_v_stride = rows->value_stride;
    d.new_f32 = rows->src_f32;
    d.new_k_scale = rows->k_scale;
    d.new_v_scale = rows->v_scale;
  }
  // the prefix tiles, over the pools themselves (fp8: converted in the kernel)
  pa::PrefillParams& pp = f.pre;
  pp.out = out;
  pp.query = query;
  pp.key_cache = key_cache;
  pp.value_cache = value_cache;
  pp.block_tables = block_tables;
  pp.seq_lens = seq_lens;
  pp.bt_stride = bt_stride;
  pp.num_tokens = num_seqs;
  pp.num_q_heads = num_q_heads;
  pp.num_kv_heads = num_kv_heads;
  pp.group = num_q_heads / num_kv_heads;
  pp.num_blocks = num_blocks;
  pp.kv_fp8 = kv_kind == pa::kFP8;
  pp.tile_positions = cp.positions;
  pp.scale_log2 = d.scale_log2;
  pp.v_scale = 1.f;
  pp.prefix_rows = num_seqs;
  pp.prefix_keys = prefix_blocks * pa::kBlockSize;
  pp.prefix_share_tiles = cp.tps;
  pp.pre_o = d.pre_o;
  pp.pre_m = d.pre_m;
  pp.pre_l = d.pre_l;
  int n = 0;
  for (int rt = 0; rt < cp.row_tiles; ++rt)
    for (int j = 0; j < cp.shares; ++j) {
      const uint64_t kt0 = (uint64_t)j * cp.tps, kt1 = std::min<uint64_t>(kt0 + cp.tps, cp.key_tiles);
      pp.items[n++] = ((uint64_t)rt << 16) | (kt0 << 32) | (kt1 << 48);
    }
  pp.n_items = n;
  f.decode_waves_per_wg = fused_decode_waves();
  f.decode_waves = d.n_splits * num_kv_heads;
  f.n_decode_wgs = ceil_div(f.decode_waves, fused_decode_waves());
  pa_status_t st = hip_status(pa::launch_fused(f, head_dim, kv_kind == pa::kFP8, stream, pa::kKDecode),
                              "cascade prefix tiles + suffix launch");
  if (st != PA_OK) return st;
  pa::DecodeParams m = d;
  m.prefix_shares = cp.shares;
  return hip_status(pa::launch_decode_merge(m, head_dim, stream), "cascade merge launch");
}

}  // namespace

size_t pa_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_seq_len, int32_t prefix_blocks,
                                         int32_t num_splits) {
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads || max_seq_len < 1 ||
      (head_dim != 64 && head_dim != 128) || num_splits < 0 || prefix_blocks < 1 ||
      (int64_t)prefix_blocks * pa::kBlockSize > max_seq_len || num_q_heads / num_kv_heads > pa::kMaxGroup)
    return 0;
  if (num_seqs == 0) return 0;  // an empty batch needs no scratch (as pa_decode_workspace_bytes)
  size_t need = cascade_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, prefix_blocks, num_splits).total;
  if (cascade_tiles_enabled())
    for (const int elem : {1, 2}) {  // the size query takes no dtype: room for either plan
      const CascadeTilePlan cp = plan_cascade_tiles(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                    prefix_blocks, num_splits, elem);
      if (cp.ok) need = std::max(need, cp.total);
    }
  // fp32 pools run the plain decode
  return std::max(need, pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                  num_splits));
}

namespace {

// The cascade decode (pa_decode_cascade*), and with rows the decode step that also stores the new
// K/V (pa_decode_cascade_write*): the suffix waves of the tiles' launch store them when the pools
// are bf16 or fp8 and every kv-head slice is 16-byte aligned; otherwise the KV write runs first as
// its own launch.  kv_kind: the pools (kF32 pools take the plain fp32 decode over whole sequences).
pa_status_t cascade_call(void* out, const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, int32_t max_seq_len, float scale, int kv_kind, int q_f32, float k_scale,
                         float v_scale, int32_t prefix_blocks, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, const NewRows* rows) {
  const size_t need = pa_decode_cascade_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                        prefix_blocks, num_splits);
  pa_status_t st = check_decode_args(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                                     num_splits, workspace, workspace_bytes, need);
  if (st != PA_OK) return st;
  if (kv_kind == pa::kFP8 &&
      (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale)))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  st = check_cascade(block_tables, bt_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, block_size, max_seq_len,
                     prefix_blocks, rows != nullptr);
  if (st != PA_OK) return st;
  if (rows) {
    if (num_seqs > 0 && (!rows->key || !rows->value)) return fail(PA_ERR_NULL, "key or value is NULL");
    if (rows->key_stride < (int64_t)num_kv_heads * head_dim || rows->value_stride < (int64_t)num_kv_heads * head_dim)
      return fail(PA_ERR_SHAPE, "token stride smaller than num_kv_heads * head_dim");
    if ((int64_t)num_blocks * block_size > INT32_MAX) return fail(PA_ERR_SHAPE, "pool has more than 2^31 slots");
  }
  if (num_seqs == 0) return ok();
  if (validate_enabled()) {
    st = validate_tables(block_tables, bt_stride, seq_lens, nullptr, num_seqs, num_blocks, max_seq_len, block_size);
    if (st != PA_OK) return st;
  }
  // the tiles read bf16 queries; fp32 queries take the decode waves' path
  CascadeTilePlan cp;
  if (kv_kind != pa::kF32 && !q_f32 && cascade_tiles_enabled())
    cp = plan_cascade_tiles(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, prefix_blocks, num_splits,
                            kv_kind == pa::kFP8 ? 1 : 2);
  if (rows) {
    const int64_t elem = rows->src_f32 ? 4 : 2;
    const uintptr_t align = (uintptr_t)rows->key | (uintptr_t)rows->value | (uintptr_t)(rows->key_stride * elem) |
                            (uintptr_t)(rows->value_stride * elem);
    if (cp.ok && (align & 15u) == 0)
      return run_cascade_tiles(cp, out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                               num_q_heads, num_kv_heads, head_dim, num_blocks, max_seq_len, scale, kv_kind, k_scale,
                               v_scale, workspace, stream, prefix_blocks, rows);
    const int write_kind = kv_kind == pa::kFP8 ? (rows->src_f32 ? pa::kFP8 + 1 : pa::kFP8) : kv_kind;
    st = hip_status(pa::launch_write_kv(rows->key, rows->value, rows->key_stride, rows->value_stride,
                                        const_cast<void*>(key_cache), const_cast<void*>(value_cache), nullptr,
                                        block_tables, bt_stride, seq_lens, nullptr, num_seqs, num_seqs, 1,
                                        num_kv_heads, head_dim, block_size, num_blocks, write_kind, k_scale, v_scale,
                                        stream),
                    "write_kv launch");
    if (st != PA_OK) return st;
  }
  // fp32 pools: the plain fp32 decode over each whole sequence (the same attention; only the
  // grouping of keys, and so the order of fp32 sums, would differ)
  if (kv_kind == pa::kF32)
    return run_decode(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, nullptr, num_seqs,
                      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                      pa::kF32, 1, 1.f, 1.f, num_splits, workspace, workspace_bytes, stream);
  if (cp.ok)
    return run_cascade_tiles(cp, out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                             num_q_heads, num_kv_heads, head_dim, num_blocks, max_seq_len, scale, kv_kind, k_scale,
                             v_scale, workspace, stream, prefix_blocks);
  return run_decode(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, nullptr, num_seqs,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale, kv_kind,
                    q_f32, k_scale, v_scale, num_splits, workspace, workspace_bytes, stream, prefix_blocks);
}

}  // namespace

pa_status_t pa_decode_cascade(void* out, const void* query, const void* key_cache, const void* value_cache,
                              const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                              pa_dtype_t dtype, int32_t prefix_blocks, int32_t num_splits, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  return cascade_call(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                      dtype == PA_F32 ? pa::kF32 : pa::kBF16, dtype == PA_F32, 1.f, 1.f, prefix_blocks, num_splits,
                      workspace, workspace_bytes, static_cast<hipStream_t>(stream), nullptr);
}

pa_status_t pa_decode_cascade_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                                  const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                                  pa_dtype_t q_dtype, float k_scale, float v_scale, int32_t prefix_blocks,
                                  int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (q_dtype != PA_F32 && q_dtype != PA_BF16) return fail(PA_ERR_DTYPE, "q_dtype must be PA_F32 or PA_BF16");
  return cascade_call(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale, pa::kFP8,
                      q_dtype == PA_F32, k_scale, v_scale, prefix_blocks, num_splits, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream), nullptr);
}

pa_status_t pa_decode_cascade_write(void* out, const void* query, const void* key, const void* value,
                                    int64_t key_tok_stride, int64_t value_tok_stride, void* key_cache,
                                    void* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    int32_t max_seq_len, float scale, pa_dtype_t dtype, int32_t prefix_blocks,
                                    int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  const NewRows rows{key, value, key_tok_stride, value_tok_stride, dtype == PA_F32, 1.f, 1.f};
  return cascade_call(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                      dtype == PA_F32 ? pa::kF32 : pa::kBF16, dtype == PA_F32, 1.f, 1.f, prefix_blocks, num_splits,
                      workspace, workspace_bytes, static_cast<hipStream_t>(stream), &rows);
}

pa_status_t pa_decode_cascade_write_fp8(void* out, const void* query, const void* key, const void* value,
                                        int64_t key_tok_stride, int64_t value_tok_stride, uint8_t* key_cache,
                                        uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, int32_t max_seq_len, float scale, pa_dtype_t dtype,
                                        float k_scale, float v_scale, int32_t prefix_blocks, int32_t num_splits,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  const NewRows rows{key, value, key_tok_stride, value_tok_stride, dtype == PA_F32, k_scale, v_scale};
  return cascade_call(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale, pa::kFP8, dtype == PA_F32,
                      k_scale, v_scale, prefix_blocks, num_splits, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream), &rows);
}

namespace {

// Host plan of a flattened batch ([P2]'s ahead-of-time scheduling: the control
// plane knows query_start_loc and seq_lens).  Decode rows (q_len == 1) go to the
// decode kernels.  Chunks are cut into row tiles of 256 / G positions x G q
// heads; a row tile needs ceil((c + last position + 1) / 64) key tiles.  The
// key tiles of all row tiles are shared out so that about one work-group per
// compute unit is busy: a row tile longer than the per-item budget is split
// into near-equal key ranges whose partial results a merge kernel combines.
struct VarlenPlan {
  int max_decode_len = 0;        // longest sequence with q_len == 1 (0: none)
  bool any_decode = false;
  int tile_positions = 0;
  std::vector<uint64_t> items;   // split pieces first (grouped by row tile), then whole row tiles
  std::vector<uint64_t> merges;  // one per split row tile
  int n_split_items = 0;         // items that leave partial results (slots 0 .. n_split_items-1)
  int max_item_tiles = 0;        // key tiles of the longest item
  int64_t total_tiles = 0;       // key tiles of all items (one kv head)
};

pa_status_t plan_varlen(const int32_t* qsl, const int32_t* sl, int num_seqs, int num_tokens, int bt_stride,
                        int group, int num_kv_heads, VarlenPlan& plan, int window = 0, int chunk = 0,
                        int items_per_head = 0) {
  if (qsl[0] != 0) return fail(PA_ERR_SHAPE, "query_start_loc_host[0] = %d, expected 0", qsl[0]);
  const int P = pa::kPrefillRows / group;
  plan.tile_positions = P;
  struct RowTile {
    int s, rt, n_kt, kt_lo;  // key tiles kt_lo .. kt_lo + n_kt - 1
  };
  std::vector<RowTile> tiles;
  int64_t total = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int q_len = qsl[s + 1] - qsl[s];
    if (q_len < 1) return fail(PA_ERR_SHAPE, "sequence %d has q_len %d < 1", s, q_len);
    if (sl[s] < q_len) return fail(PA_ERR_SHAPE, "seq_lens[%d] = %d < q_len %d", s, sl[s], q_len);
    if (ceil_div(sl[s], pa::kBlockSize) > bt_stride)
      return fail(PA_ERR_SHAPE, "sequence %d needs more than bt_stride = %d table columns", s, bt_stride);
    if (q_len == 1) {
      plan.any_decode = true;
      plan.max_decode_len = std::max(plan.max_decode_len, (int)sl[s]);
      continue;
    }
    const int c = sl[s] - q_len;
    const int n_rt = ceil_div(q_len, P);
    if (s >= (1 << 15) || n_rt >= (1 << 16) || ceil_div(sl[s], pa::kPrefillKeys) >= (1 << 16))
      return fail(PA_ERR_UNSUPPORTED, "batch too large for the prefill planner");
    for (int rt = 0; rt < n_rt; ++rt) {
      const int pos_end = std::min(q_len, (rt + 1) * P);
      // a sliding window hides the key tiles below the tile's first row's window
      const int first = c + rt * P;
      const int lo = chunk > 0 ? first - first % chunk : window > 0 ? std::max(first - window + 1, 0) : 0;
      const int kt_lo = lo / pa::kPrefillKeys;
      const int n_kt = ceil_div(c + pos_end, pa::kPrefillKeys) - kt_lo;
      tiles.push_back({s, rt, n_kt, kt_lo});
      total += n_kt;
    }
  }
  if (qsl[num_seqs] != num_tokens)
    return fail(PA_ERR_SHAPE, "query_start_loc_host[num_seqs] = %d != num_tokens %d", qsl[num_seqs], num_tokens);
  if (tiles.empty()) return PA_OK;
  // one work-group per compute unit: the smallest per-item budget (>= 4 key tiles) whose
  // pieces, ceil(n_kt / budget) per row tile, number at most target_items.  With at least
  // as many row tiles as that, nothing is split (the longest-first list keeps the compute
  // units busy by itself).  The piece count does not grow with the budget: bisection.
  const int64_t target_items =
      items_per_head > 0 ? items_per_head : std::max<int64_t>(1, device_cu_count() / std::max(1, num_kv_heads));
  int max_kt = 1;
  for (const RowTile& t : tiles) max_kt = std::max(max_kt, t.n_kt);
  auto pieces = [&](int b) {
    int64_t n = 0;
    for (const RowTile& t : tiles) n += ceil_div(t.n_kt, b);
    return n;
  };
  int budget = max_kt;
  if ((int64_t)tiles.size() < target_items) {
    int lo = (int)std::min<int64_t>(max_kt, std::max<int64_t>(4, (total + target_items - 1) / target_items));
    int hi = max_kt;  // pieces(max_kt) = row tiles < target_items
    while (lo < hi) {
      const int mid = lo + (hi - lo) / 2;
      if (pieces(mid) <= target_items) hi = mid; else lo = mid + 1;
    }
    budget = lo;
  }
  // longest row tiles first
  std::stable_sort(tiles.begin(), tiles.end(), [](const RowTile& a, const RowTile& b) { return a.n_kt > b.n_kt; });
  auto code = [](int s, bool whole, int rt, int k0, int k1) {
    return (uint64_t)s | ((uint64_t)whole << 15) | ((uint64_t)rt << 16) | ((uint64_t)k0 << 32) | ((uint64_t)k1 << 48);
  };
  std::vector<uint64_t> whole_items;
  for (const RowTile& t : tiles) {
    const int n = ceil_div(t.n_kt, budget);
    if (n <= 1) {
      whole_items.push_back(code(t.s, true, t.rt, t.kt_lo, t.kt_lo + t.n_kt));
      continue;
    }
    const int first = (int)plan.items.size();
    if (first + n >= (1 << 20) || n >= (1 << 12)) return fail(PA_ERR_UNSUPPORTED, "too many prefill splits");
    for (int i = 0; i < n; ++i)
      plan.items.push_back(code(t.s, false, t.rt, t.kt_lo + (int)((int64_t)t.n_kt * i / n),
                                t.kt_lo + (int)((int64_t)t.n_kt * (i + 1) / n)));
    plan.merges.push_back((uint64_t)t.s | ((uint64_t)t.rt << 16) | ((uint64_t)first << 32) | ((uint64_t)n << 52));
  }
  plan.n_split_items = (int)plan.items.size();
  plan.items.insert(plan.items.end(), whole_items.begin(), whole_items.end());
  plan.total_tiles = total;
  for (const uint64_t it : plan.items)
    plan.max_item_tiles = std::max(plan.max_item_tiles, (int)(it >> 48) - (int)((it >> 32) & 0xFFFFu));
  return PA_OK;
}

// Prefill scratch: partial results of split row-tile pieces, after the decode rows' scratch.
struct PrefillLayout {
  size_t o_bytes, m_bytes, total;
};

PrefillLayout prefill_layout(int n_split_items, int num_kv_heads, int head_dim) {
  const size_t rows = (size_t)n_split_items * num_kv_heads * pa::kPrefillRows;
  PrefillLayout L;
  L.o_bytes = align_up(rows * head_dim * sizeof(uint16_t));  // (O / l) / sigma, fp16
  L.m_bytes = align_up(rows * sizeof(float));                  // m, l and sigma: one fp32 each per row
  L.total = n_split_items ? L.o_bytes + 3 * L.m_bytes : 0;
  return L;
}

size_t varlen_workspace(const VarlenPlan& plan, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim) {
  const size_t dec = plan.max_decode_len
                         ? pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, plan.max_decode_len, 0)
                         : 0;
  return align_up(dec) + prefill_layout(plan.n_split_items, num_kv_heads, head_dim).total;
}

// A batch with decode rows and prefill chunks runs both in one launch (launch_fused) when
// the host estimate says that ends sooner than the two launches one after the other.  The
// estimate (measured on the MI355X with the mixed continuous-batching step): the decode
// work-groups stream K/V at PA_FUSED_CU_GBPS (default 29 GB/s) per compute unit they hold,
// up to PA_FUSED_DECODE_GBPS (default 6000 GB/s) in all; a prefill work item takes
// PA_FUSED_TILE_NS (default 2200 ns) per 64-key tile plus 5 us, and the items of each kv
// head go longest first to the least loaded of the compute units left to them.  The decode
// work-groups get Q compute units and the prefill items the rest, for the Q (multiples of 8
// from a quarter of the device) that minimises the larger of the two times (the largest
// such Q).  PA_FUSED=0 turns fusing off, 2 fuses every batch it can (pa_set_fused switches
// the same at run time); PA_FUSED_DECODE_CUS fixes Q (measurement).
struct StepPlan {
  VarlenPlan plan;
  bool fused = false;
  int n_decode_wgs = 0;   // decode work-groups of the fused launch
  int decode_splits = 0;  // decode shares per column of the fused launch
};


pa_status_t plan_step(const int32_t* qsl, const int32_t* sl, int num_seqs, int num_tokens, int bt_stride,
                      int num_q_heads, int num_kv_heads, int head_dim, int kv_elem, int window, int chunk,
                      StepPlan& sp) {
  const int group = num_q_heads / num_kv_heads;
  pa_status_t st = plan_varlen(qsl, sl, num_seqs, num_tokens, bt_stride, group, num_kv_heads, sp.plan, window, chunk);
  if (st != PA_OK) return st;
  const int mode = fused_mode();
  if (mode == 0 || !sp.plan.any_decode || sp.plan.items.empty() ||
      sp.plan.items.size() > (size_t)pa::kMaxPrefillItems)
    return PA_OK;
  static const double tile_s = env_int("PA_FUSED_TILE_NS", 2200, 100, 1000000) * 1e-9;
  // the decode shares' rate inside the fused launch: about 30 GB/s per compute unit, and no
  // more than about 5.8 TB/s in all (the items' own traffic shares HBM with it)
  static const double bw = env_int("PA_FUSED_DECODE_GBPS", 5800, 100, 100000) * 1e9;
  static const double bw_cu = env_int("PA_FUSED_CU_GBPS", 30, 1, 100000) * 1e9;
  const double item_s = 5e-6;
  const int C = device_cu_count();
  double dec_bytes = 0;
  for (int s = 0; s < num_seqs; ++s) {
    if (qsl[s + 1] - qsl[s] != 1) continue;
    const int vis_lim = window > 0 ? window + 16 : chunk > 0 ? chunk + 16 : INT32_MAX;
    dec_bytes += 2.0 * std::min(sl[s], vis_lim) * num_kv_heads * head_dim * kv_elem;
  }
  auto t_dec = [&](int q) { return dec_bytes / std::min(bw, bw_cu * q); };
  // the kv heads' items run side by side (the grid interleaves them), each head on cus / Hkv
  // compute units: greedy longest-first makespan of one head's items
  auto t_pre = [&](const VarlenPlan& pl, int cus) {
    const int slots = std::max(1, cus / num_kv_heads);
    std::vector<double> load(slots, 0.0);
    std::vector<int> tiles;
    tiles.reserve(pl.items.size());
    for (const uint64_t it : pl.items) tiles.push_back((int)(it >> 48) - (int)((it >> 32) & 0xFFFFu));
    std::sort(tiles.begin(), tiles.end(), std::greater<int>());
    for (const int t : tiles) {
      double& lo = *std::min_element(load.begin(), load.end());
      lo += t * tile_s + item_s;
    }
    return *std::max_element(load.begin(), load.end());
  };
  const double t_seq = dec_bytes / bw + t_pre(sp.plan, C);
  const double limit = mode == 2 ? 1e30 : t_seq * 0.95;  // fuse only for a clear gain (mode 2: always)
  const std::string saved = g_last_error;
  static const int forced_q = env_int("PA_FUSED_DECODE_CUS", 0, 0, 1 << 20);  // measurement: fix Q
  auto plan_for = [&](int q, VarlenPlan& pl) {
    return plan_varlen(qsl, sl, num_seqs, num_tokens, bt_stride, group, num_kv_heads, pl, window, chunk,
                       std::max(1, (C - q) / num_kv_heads)) == PA_OK &&
           pl.items.size() <= (size_t)pa::kMaxPrefillItems;
  };
  // modelled time of every Q; then the smallest Q within 1% of the best: once the decode
  // stream has the compute units it can use, more of them only slow the items down
  std::vector<std::pair<int, double>> cand;
  double best = 1e30;
  for (int q = std::max(8, C / 4); q <= C - num_kv_heads; q += 8) {
    if (forced_q > 0 && q != forced_q) continue;
    VarlenPlan pl;
    if (!plan_for(q, pl)) continue;
    const double t = std::max(t_dec(q), t_pre(pl, C - q));
    cand.emplace_back(q, t);
    best = std::min(best, t);
  }
  int best_q = 0;
  for (const auto& [q, t] : cand)
    if (forced_q > 0 || (t <= limit && t <= best * 1.01)) {
      best_q = q;
      break;
    }
  VarlenPlan best_plan;
  if (best_q > 0 && !plan_for(best_q, best_plan)) best_q = 0;
  g_last_error = saved;
  if (best_q == 0) return PA_OK;
  sp.fused = true;
  sp.plan = std::move(best_plan);
  sp.n_decode_wgs = best_q;
  sp.decode_splits = std::max(1, best_q * fused_decode_waves() / decode_columns(num_q_heads, num_kv_heads));
  return PA_OK;
}

// pa_prefill_varlen(_window)_workspace_bytes without the argument checks.
size_t varlen_workspace_bytes(const int32_t* qsl, const int32_t* sl, int num_seqs, int num_q_heads, int num_kv_heads,
                              int head_dim, int window, int chunk = 0, int kv_elem = 2) {
  StepPlan sp;
  const std::string saved = g_last_error;
  const pa_status_t st = plan_step(qsl, sl, num_seqs, qsl[num_seqs], INT32_MAX, num_q_heads, num_kv_heads, head_dim,
                                   kv_elem, window, chunk, sp);
  g_last_error = saved;
  if (st != PA_OK) return 0;
  return varlen_workspace(sp.plan, num_seqs, num_q_heads, num_kv_heads, head_dim);
}

// The varlen call for bf16 pools (kv_kind kBF16; dtype PA_F32 allowed for decode-only
// batches) and for fp8 pools (kFP8: decode rows and chunks read the codes directly).
pa_status_t run_varlen(void* out, const void* query, const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                       const int32_t* query_start_loc, const int32_t* seq_lens_host,
                       const int32_t* query_start_loc_host, int32_t num_seqs, int32_t num_tokens,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, float scale, pa_dtype_t dtype, int kv_kind, float k_scale, float v_scale,
                       void* workspace, size_t workspace_bytes, void* stream, int32_t sliding_window = 0,
                       int32_t local_chunk = 0, const NewRows* fresh = nullptr) {
  if (num_seqs < 0 || num_tokens < 0) return fail(PA_ERR_SHAPE, "negative num_seqs or num_tokens");
  if (num_seqs == 0) return num_tokens == 0 ? ok() : fail(PA_ERR_SHAPE, "num_tokens > 0 with no sequences");
  if (!out || !query || !key_cache || !value_cache || !block_tables || !seq_lens || !query_start_loc ||
      !seq_lens_host || !query_start_loc_host)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  pa_status_t st = check_attention_shape(num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, bt_stride);
  if (st != PA_OK) return st;
  if (num_q_heads / num_kv_heads > pa::kMaxGqa)
    return fail(PA_ERR_UNSUPPORTED, "up to %d q heads per kv head", pa::kMaxGqa);
  // the prefill kernel masks raw scores and applies the scale inside exp2(s * scale - m),
  // which orders the scores correctly only for a positive scale
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(PA_ERR_SHAPE, "scale must be positive and finite");
  StepPlan sp;
  st = plan_step(query_start_loc_host, seq_lens_host, num_seqs, num_tokens, bt_stride, num_q_heads, num_kv_heads,
                 head_dim, kv_kind == pa::kFP8 ? 1 : 2, sliding_window, local_chunk, sp);
  if (st != PA_OK) return st;
  const VarlenPlan& plan = sp.plan;
  // chunks of fp32 pools, or of fp32 queries over fp8 pools: every token on its own, no scratch
  const bool rows = dtype == PA_F32 && !plan.items.empty();
  const size_t need = rows ? 0 : varlen_workspace(plan, num_seqs, num_q_heads, num_kv_heads, head_dim);
  if (need && (!workspace || workspace_bytes < need))
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (need && (reinterpret_cast<uintptr_t>(workspace) % kAlign))
    return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (validate_enabled()) {
    std::vector<int32_t> q, sl;
    if (!copy_to_host(q, query_start_loc, num_seqs + 1) || !copy_to_host(sl, seq_lens, num_seqs))
      return fail(PA_ERR_HIP, "PA_VALIDATE: metadata copy failed");
    for (int s = 0; s <= num_seqs; ++s)
      if (q[s] != query_start_loc_host[s]) return fail(PA_ERR_SHAPE, "PA_VALIDATE: host/device query_start_loc differ");
    for (int s = 0; s < num_seqs; ++s)
      if (sl[s] != seq_lens_host[s]) return fail(PA_ERR_SHAPE, "PA_VALIDATE: host/device seq_lens differ");
    int max_len = 1;
    for (int s = 0; s < num_seqs; ++s) max_len = std::max(max_len, (int)seq_lens_host[s]);
    st = validate_tables(block_tables, bt_stride, seq_lens, query_start_loc, num_seqs, num_blocks, max_len, block_size);
    if (st != PA_OK) return st;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int dec_kind = kv_kind == pa::kFP8 ? pa::kFP8 : (dtype == PA_F32 ? pa::kF32 : pa::kBF16);
  if (fresh) {
    // the step's new rows: stored by the fused launch itself (bf16 pools and rows, no window,
    // 16-byte aligned kv-head slices), else by the KV write's launch first
    const int64_t elem = fresh->src_f32 ? 4 : 2;
    const uintptr_t align = (uintptr_t)fresh->key | (uintptr_t)fresh->value | (uintptr_t)(fresh->key_stride * elem) |
                            (uintptr_t)(fresh->value_stride * elem);
    const bool in_launch = sp.fused && !rows && kv_kind == pa::kBF16 && dtype == PA_BF16 && sliding_window <= 0 &&
                           local_chunk <= 0 && (align & 15u) == 0;
    if (!in_launch) {
      int max_q = 0;
      for (int s = 0; s < num_seqs; ++s) max_q = std::max(max_q, query_start_loc_host[s + 1] - query_start_loc_host[s]);
      const int write_kind = kv_kind == pa::kFP8 ? (fresh->src_f32 ? pa::kFP8 + 1 : pa::kFP8) : dec_kind;
      st = hip_status(pa::launch_write_kv(fresh->key, fresh->value, fresh->key_stride, fresh->value_stride,
                                          const_cast<void*>(key_cache), const_cast<void*>(value_cache), nullptr,
                                          block_tables, bt_stride, seq_lens, query_start_loc, num_seqs, num_tokens,
                                          max_q, num_kv_heads, head_dim, block_size, num_blocks, write_kind,
                                          k_scale, v_scale, hs),
                      "write_kv launch");
      if (st != PA_OK) return st;
      fresh = nullptr;
    }
  }
  if (rows) {
    int max_len = 1;
    for (int s = 0; s < num_seqs; ++s) max_len = std::max(max_len, (int)seq_lens_host[s]);
    pa::DecodeParams p = make_decode_params(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens,
                                            query_start_loc, num_seqs, num_tokens, num_q_heads, num_kv_heads,
                                            head_dim, max_len, scale, dec_kind, 1, k_scale, v_scale, 1, nullptr, 0,
                                            sliding_window, local_chunk);
    p.num_blocks = num_blocks;
    return hip_status(pa::launch_rows_f32(p, dec_kind, head_dim, num_tokens, hs), "fp32 rows launch");
  }

  if (plan.any_decode && !sp.fused) {
    st = run_decode(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, query_start_loc, num_seqs,
                    num_tokens, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, plan.max_decode_len, scale,
                    dec_kind, dtype == PA_F32, k_scale, v_scale, 0, workspace, workspace_bytes, hs, 0, sliding_window,
                    local_chunk);
    if (st != PA_OK) return st;
  }
  auto* ws = static_cast<unsigned char*>(workspace);
  const size_t dec_bytes = plan.max_decode_len ? align_up(pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                                                    head_dim, plan.max_decode_len, 0))
                                               : 0;
  const PrefillLayout lay = prefill_layout(plan.n_split_items, num_kv_heads, head_dim);
  uint16_t* part_o = plan.n_split_items ? reinterpret_cast<uint16_t*>(ws + dec_bytes) : nullptr;
  float* part_m = plan.n_split_items ? reinterpret_cast<float*>(ws + dec_bytes + lay.o_bytes) : nullptr;
  float* part_l = plan.n_split_items ? reinterpret_cast<float*>(ws + dec_bytes + lay.o_bytes + lay.m_bytes) : nullptr;
  float* part_s =
      plan.n_split_items ? reinterpret_cast<float*>(ws + dec_bytes + lay.o_bytes + 2 * lay.m_bytes) : nullptr;
  auto prefill_params = [&](size_t i0, pa::PrefillParams& p) {
    p.out = out;
    p.query = query;
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.block_tables = block_tables;
    p.seq_lens = seq_lens;
    p.qsl = query_start_loc;
    p.part_o = part_o;
    p.part_m = part_m;
    p.part_l = part_l;
    p.part_s = part_s;
    p.bt_stride = bt_stride;
    p.num_tokens = num_tokens;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_q_heads / num_kv_heads;
    p.num_blocks = num_blocks;
    p.kv_fp8 = kv_kind == pa::kFP8;
    p.tile_positions = plan.tile_positions;
    p.item_base = (int)i0;
    p.scale_log2 = scale * 1.4426950408889634f * (kv_kind == pa::kFP8 ? k_scale : 1.f);
    p.v_scale = kv_kind == pa::kFP8 ? v_scale : 1.f;
    p.window = sliding_window > 0 ? sliding_window : 0;
    p.chunk = local_chunk > 0 ? local_chunk : 0;
    const size_t n = std::min(plan.items.size() - i0, (size_t)pa::kMaxPrefillItems);
    p.n_items = (int)n;
    std::memcpy(p.items, plan.items.data() + i0, n * sizeof(uint64_t));
  };
  if (sp.fused) {  // decode waves and prefill items in one launch (plan_step keeps the items to one launch)
    // never more shares than the decode scratch of the workspace was sized for
    const int ws_splits = resolve_splits(0, num_seqs, decode_columns(num_q_heads, num_kv_heads),
                                         plan.max_decode_len, kFusedSplitsFactor);
    pa::FusedParams f{};
    f.dec = make_decode_params(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens,
                               query_start_loc, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                               plan.max_decode_len, scale, dec_kind, dtype == PA_F32, k_scale, v_scale,
                               std::min(sp.decode_splits, ws_splits), workspace, 0, sliding_window, local_chunk);
    f.dec.num_blocks = num_blocks;
    prefill_params(0, f.pre);
    if (fresh) {  // the decode waves and the prefill items store the new rows themselves
      f.dec.new_k = f.pre.new_k = fresh->key;
      f.dec.new_v = f.pre.new_v = fresh->value;
      f.dec.new_k_stride = f.pre.new_k_stride = fresh->key_stride;
      f.dec.new_v_stride = f.pre.new_v_stride = fresh->value_stride;
      f.dec.new_f32 = 0;
      f.dec.new_k_scale = f.dec.new_v_scale = 1.f;
      f.dec.store_chunk_rows = 1;  // the chunks' rows: stored by the merge launch below
    }
    f.decode_waves_per_wg = fused_decode_waves();
    f.decode_waves = (f.dec.prefix_waves + f.dec.n_splits) * decode_columns(num_q_heads, num_kv_heads);
    f.n_decode_wgs = (f.decode_waves + fused_decode_waves() - 1) / fused_decode_waves();
    st = hip_status(pa::launch_fused(f, head_dim, kv_kind == pa::kFP8, hs), "fused decode + prefill launch");
    if (st != PA_OK) return st;
    st = hip_status(pa::launch_decode_merge(f.dec, head_dim, hs), "decode merge launch");
    if (st != PA_OK) return st;
  } else {
    for (size_t i0 = 0; i0 < plan.items.size(); i0 += pa::kMaxPrefillItems) {
      pa::PrefillParams p{};
      prefill_params(i0, p);
      st = hip_status(pa::launch_prefill(p, head_dim, hs), "prefill launch");
      if (st != PA_OK) return st;
    }
  }
  for (size_t i0 = 0; i0 < plan.merges.size(); i0 += pa::kMaxPrefillItems) {
    pa::PrefillMergeParams p{};
    p.out = out;
    p.qsl = query_start_loc;
    p.part_o = part_o;
    p.part_m = part_m;
    p.part_l = part_l;
    p.part_s = part_s;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_q_heads / num_kv_heads;
    p.tile_positions = plan.tile_positions;
    p.v_scale = kv_kind == pa::kFP8 ? v_scale : 1.f;
    const size_t n = std::min(plan.merges.size() - i0, (size_t)pa::kMaxPrefillItems);
    p.n_items = (int)n;
    std::memcpy(p.items, plan.merges.data() + i0, n * sizeof(uint64_t));
    st = hip_status(pa::launch_prefill_merge(p, head_dim, hs), "prefill merge launch");
    if (st != PA_OK) return st;
  }
  return ok();
}



}  // namespace

size_t pa_prefill_varlen_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim) {
  if (!query_start_loc_host || !seq_lens_host || num_seqs < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
      num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > pa::kMaxGqa)
    return 0;
  return varlen_workspace_bytes(query_start_loc_host, seq_lens_host, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                0);
}

size_t pa_prefill_varlen_window_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t sliding_window) {
  if (!query_start_loc_host || !seq_lens_host || num_seqs < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
      num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > pa::kMaxGqa || sliding_window < 1)
    return 0;
  return varlen_workspace_bytes(query_start_loc_host, seq_lens_host, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                sliding_window);
}

pa_status_t pa_decode_window(void* out, const void* query, const void* key_cache, const void* value_cache,
                             const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_seq_len, float scale, pa_dtype_t dtype,
                             int32_t sliding_window, int32_t num_splits, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  if (sliding_window < 1) return fail(PA_ERR_SHAPE, "sliding_window %d < 1", sliding_window);
  pa_status_t st = check_decode_args(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                                     num_splits, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (dtype == PA_BF16 && num_q_heads / num_kv_heads > pa::kMaxGqa)
    return fail(PA_ERR_UNSUPPORTED, "bf16 decode supports up to %d q heads per kv head", pa::kMaxGqa);
  if (num_seqs == 0) return ok();
  if (validate_enabled()) {
    st = validate_tables(block_tables, bt_stride, seq_lens, nullptr, num_seqs, num_blocks, max_seq_len, block_size);
    if (st != PA_OK) return st;
  }
  return run_decode(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, nullptr, num_seqs,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                    dtype == PA_F32 ? pa::kF32 : pa::kBF16, dtype == PA_F32, 1.f, 1.f, num_splits, workspace,
                    workspace_bytes, static_cast<hipStream_t>(stream), 0, sliding_window);
}

pa_status_t pa_prefill_varlen(void* out, const void* query, const void* key_cache, const void* value_cache,
                              const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                              const int32_t* query_start_loc, const int32_t* seq_lens_host,
                              const int32_t* query_start_loc_host, int32_t num_seqs, int32_t num_tokens,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, float scale, pa_dtype_t dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  return run_varlen(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, query_start_loc,
                    seq_lens_host, query_start_loc_host, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                    block_size, num_blocks, scale, dtype, pa::kBF16, 1.f, 1.f, workspace, workspace_bytes, stream);
}

pa_status_t pa_prefill_varlen_write(void* out, const void* query, const void* key, const void* value,
                                    int64_t key_tok_stride, int64_t value_tok_stride, void* key_cache,
                                    void* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                    const int32_t* seq_lens, const int32_t* query_start_loc,
                                    const int32_t* seq_lens_host, const int32_t* query_start_loc_host,
                                    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                    pa_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  if (num_tokens > 0 && (!key || !value)) return fail(PA_ERR_NULL, "key or value is NULL");
  if (key_tok_stride < (int64_t)num_kv_heads * head_dim || value_tok_stride < (int64_t)num_kv_heads * head_dim)
    return fail(PA_ERR_SHAPE, "token stride smaller than num_kv_heads * head_dim");
  if ((int64_t)num_blocks * block_size > INT32_MAX) return fail(PA_ERR_SHAPE, "pool has more than 2^31 slots");
  const NewRows rows{key, value, key_tok_stride, value_tok_stride, dtype == PA_F32, 1.f, 1.f};
  return run_varlen(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, query_start_loc,
                    seq_lens_host, query_start_loc_host, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                    block_size, num_blocks, scale, dtype, pa::kBF16, 1.f, 1.f, workspace, workspace_bytes, stream, 0,
                    0, &rows);
}

pa_status_t pa_prefill_varlen_window(void* out, const void* query, const void* key_cache, const void* value_cache,
                                     const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                     const int32_t* query_start_loc, const int32_t* seq_lens_host,
                                     const int32_t* query_start_loc_host, int32_t num_seqs, int32_t num_tokens,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, float scale, pa_dtype_t dtype, int32_t sliding_window,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  if (sliding_window < 1) return fail(PA_ERR_SHAPE, "sliding_window %d < 1", sliding_window);
  return run_varlen(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, query_start_loc,
                    seq_lens_host, query_start_loc_host, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                    block_size, num_blocks, scale, dtype, pa::kBF16, 1.f, 1.f, workspace, workspace_bytes, stream,
                    sliding_window);
}

size_t pa_prefill_varlen_local_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t chunk_size) {
  if (!query_start_loc_host || !seq_lens_host || num_seqs < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
      num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > pa::kMaxGqa || chunk_size < 1)
    return 0;
  return varlen_workspace_bytes(query_start_loc_host, seq_lens_host, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                0, chunk_size);
}

pa_status_t pa_decode_local(void* out, const void* query, const void* key_cache, const void* value_cache,
                            const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, int32_t max_seq_len, float scale, pa_dtype_t dtype,
                            int32_t chunk_size, int32_t num_splits, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  if (chunk_size < 1) return fail(PA_ERR_SHAPE, "chunk_size %d < 1", chunk_size);
  pa_status_t st = check_decode_args(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                                     num_splits, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (dtype == PA_BF16 && num_q_heads / num_kv_heads > pa::kMaxGqa)
    return fail(PA_ERR_UNSUPPORTED, "bf16 decode supports up to %d q heads per kv head", pa::kMaxGqa);
  if (num_seqs == 0) return ok();
  if (validate_enabled()) {
    st = validate_tables(block_tables, bt_stride, seq_lens, nullptr, num_seqs, num_blocks, max_seq_len, block_size);
    if (st != PA_OK) return st;
  }
  return run_decode(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, nullptr, num_seqs,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                    dtype == PA_F32 ? pa::kF32 : pa::kBF16, dtype == PA_F32, 1.f, 1.f, num_splits, workspace,
                    workspace_bytes, static_cast<hipStream_t>(stream), 0, 0, chunk_size);
}

pa_status_t pa_prefill_varlen_local(void* out, const void* query, const void* key_cache, const void* value_cache,
                                    const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                    const int32_t* query_start_loc, const int32_t* seq_lens_host,
                                    const int32_t* query_start_loc_host, int32_t num_seqs, int32_t num_tokens,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, float scale, pa_dtype_t dtype, int32_t chunk_size,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_DTYPE, "dtype must be PA_F32 or PA_BF16");
  if (chunk_size < 1) return fail(PA_ERR_SHAPE, "chunk_size %d < 1", chunk_size);
  return run_varlen(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, query_start_loc,
                    seq_lens_host, query_start_loc_host, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                    block_size, num_blocks, scale, dtype, pa::kBF16, 1.f, 1.f, workspace, workspace_bytes, stream, 0,
                    chunk_size);
}

namespace {

// pa_prefill_varlen(_window|_local)_fp8_workspace_bytes without the argument checks: the
// plan's workspace (the kernels read the codes themselves, nothing is staged).
size_t varlen_fp8_workspace_bytes(const int32_t* qsl, const int32_t* sl, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int window, int chunk) {
  return varlen_workspace_bytes(qsl, sl, num_seqs, num_q_heads, num_kv_heads, head_dim, window, chunk,
                                /*kv_elem=*/1);
}

}  // namespace

size_t pa_prefill_varlen_fp8_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t bt_stride) {
  if (!query_start_loc_host || !seq_lens_host || num_seqs < 1 || num_q_heads < 1 || num_kv_heads < 1 ||
      head_dim < 1 || bt_stride < 1 || num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > pa::kMaxGqa)
    return 0;
  return varlen_fp8_workspace_bytes(query_start_loc_host, seq_lens_host, num_seqs, num_q_heads, num_kv_heads,
                                    head_dim, 0, 0);
}

pa_status_t pa_prefill_varlen_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                                  const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                  const int32_t* query_start_loc, const int32_t* seq_lens_host,
                                  const int32_t* query_start_loc_host, int32_t num_seqs, int32_t num_tokens,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float scale, pa_dtype_t q_dtype, float k_scale, float v_scale,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (q_dtype != PA_F32 && q_dtype != PA_BF16) return fail(PA_ERR_DTYPE, "q_dtype must be PA_F32 or PA_BF16");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  return run_varlen(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, query_start_loc,
                    seq_lens_host, query_start_loc_host, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                    block_size, num_blocks, scale, q_dtype, pa::kFP8, k_scale, v_scale, workspace, workspace_bytes,
                    stream);
}


size_t pa_prefill_varlen_window_fp8_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                    int32_t head_dim, int32_t bt_stride, int32_t sliding_window) {
  if (!query_start_loc_host || !seq_lens_host || num_seqs < 1 || num_q_heads < 1 || num_kv_heads < 1 ||
      head_dim < 1 || bt_stride < 1 || num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > pa::kMaxGqa ||
      sliding_window < 1)
    return 0;
  return varlen_fp8_workspace_bytes(query_start_loc_host, seq_lens_host, num_seqs, num_q_heads, num_kv_heads,
                                    head_dim, sliding_window, 0);
}

size_t pa_prefill_varlen_local_fp8_workspace_bytes(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                                                   int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                   int32_t head_dim, int32_t bt_stride, int32_t chunk_size) {
  if (!query_start_loc_host || !seq_lens_host || num_seqs < 1 || num_q_heads < 1 || num_kv_heads < 1 ||
      head_dim < 1 || bt_stride < 1 || num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > pa::kMaxGqa ||
      chunk_size < 1)
    return 0;
  return varlen_fp8_workspace_bytes(query_start_loc_host, seq_lens_host, num_seqs, num_q_heads, num_kv_heads,
                                    head_dim, 0, chunk_size);
}

namespace {

// pa_decode_fp8 with a sliding window or local chunks (exactly one of them > 0).
pa_status_t decode_fp8_masked(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                              const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                              pa_dtype_t q_dtype, float k_scale, float v_scale, int32_t sliding_window,
                              int32_t local_chunk, int32_t num_splits, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (q_dtype != PA_F32 && q_dtype != PA_BF16) return fail(PA_ERR_DTYPE, "q_dtype must be PA_F32 or PA_BF16");
  pa_status_t st = check_decode_args(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                                     num_splits, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  if (num_q_heads / num_kv_heads > pa::kMaxGqa)
    return fail(PA_ERR_UNSUPPORTED, "fp8 decode supports up to %d q heads per kv head", pa::kMaxGqa);
  if (num_seqs == 0) return ok();
  if (validate_enabled()) {
    st = validate_tables(block_tables, bt_stride, seq_lens, nullptr, num_seqs, num_blocks, max_seq_len, block_size);
    if (st != PA_OK) return st;
  }
  return run_decode(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, nullptr, num_seqs,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale, pa::kFP8,
                    q_dtype == PA_F32, k_scale, v_scale, num_splits, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream), 0, sliding_window, local_chunk);
}

}  // namespace

pa_status_t pa_decode_window_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                                 const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                                 pa_dtype_t q_dtype, float k_scale, float v_scale, int32_t sliding_window,
                                 int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (sliding_window < 1) return fail(PA_ERR_SHAPE, "sliding_window %d < 1", sliding_window);
  return decode_fp8_masked(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                           num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale, q_dtype,
                           k_scale, v_scale, sliding_window, 0, num_splits, workspace, workspace_bytes, stream);
}

pa_status_t pa_decode_local_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                                const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                                pa_dtype_t q_dtype, float k_scale, float v_scale, int32_t chunk_size,
                                int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (chunk_size < 1) return fail(PA_ERR_SHAPE, "chunk_size %d < 1", chunk_size);
  return decode_fp8_masked(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, num_seqs,
                           num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale, q_dtype,
                           k_scale, v_scale, 0, chunk_size, num_splits, workspace, workspace_bytes, stream);
}

pa_status_t pa_prefill_varlen_window_fp8(void* out, const void* query, const uint8_t* key_cache,
                                         const uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                         const int32_t* seq_lens, const int32_t* query_start_loc,
                                         const int32_t* seq_lens_host, const int32_t* query_start_loc_host,
                                         int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                         int32_t num_blocks, float scale, pa_dtype_t q_dtype, float k_scale,
                                         float v_scale, int32_t sliding_window, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (q_dtype != PA_F32 && q_dtype != PA_BF16) return fail(PA_ERR_DTYPE, "q_dtype must be PA_F32 or PA_BF16");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  if (sliding_window < 1) return fail(PA_ERR_SHAPE, "sliding_window %d < 1", sliding_window);
  return run_varlen(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, query_start_loc,
                    seq_lens_host, query_start_loc_host, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                    block_size, num_blocks, scale, q_dtype, pa::kFP8, k_scale, v_scale, workspace, workspace_bytes,
                    stream, sliding_window);
}

pa_status_t pa_prefill_varlen_local_fp8(void* out, const void* query, const uint8_t* key_cache,
                                        const uint8_t* value_cache, const int32_t* block_tables, int32_t bt_stride,
                                        const int32_t* seq_lens, const int32_t* query_start_loc,
                                        const int32_t* seq_lens_host, const int32_t* query_start_loc_host,
                                        int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, float scale, pa_dtype_t q_dtype, float k_scale,
                                        float v_scale, int32_t chunk_size, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (q_dtype != PA_F32 && q_dtype != PA_BF16) return fail(PA_ERR_DTYPE, "q_dtype must be PA_F32 or PA_BF16");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  if (chunk_size < 1) return fail(PA_ERR_SHAPE, "chunk_size %d < 1", chunk_size);
  return run_varlen(out, query, key_cache, value_cache, block_tables, bt_stride, seq_lens, query_start_loc,
                    seq_lens_host, query_start_loc_host, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                    block_size, num_blocks, scale, q_dtype, pa::kFP8, k_scale, v_scale, workspace, workspace_bytes,
                    stream, 0, chunk_size);
}

}  // extern "C"

// ---- optional kernel timing ------------------------------------------------
namespace {

struct TimingState {
  std::mutex mu;
  std::atomic<bool> on{false};
  struct Pending {
    hipEvent_t begin, end;
  };
  std::vector<Pending> pending[pa::kNumKernelIds];
  hipEvent_t open[pa::kNumKernelIds] = {};
  int64_t count[pa::kNumKernelIds] = {};
  double total_ms[pa::kNumKernelIds] = {};
  std::vector<float> launch_ms[pa::kNumKernelIds];  // each timed launch, in order (the first kMaxKept)
  std::vector<hipEvent_t> spare;
  static constexpr size_t kMaxKept = 1 << 20;

  hipEvent_t take() {
    if (!spare.empty()) {
      hipEvent_t e = spare.back();
      spare.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    return hipEventCreate(&e) == hipSuccess ? e : nullptr;
  }

  // Folds finished event pairs of one kernel into its totals (waits for them).
  bool drain(int k) {
    bool ok = true;
    for (Pending& pe : pending[k]) {
      float ms = 0.f;
      if (hipEventSynchronize(pe.end) != hipSuccess || hipEventElapsedTime(&ms, pe.begin, pe.end) != hipSuccess) {
        ok = false;
      } else {
        ++count[k];
        total_ms[k] += ms;
        if (launch_ms[k].size() < kMaxKept) launch_ms[k].push_back(ms);
      }
      spare.push_back(pe.begin);
      spare.push_back(pe.end);
    }
    pending[k].clear();
    return ok;
  }
};

TimingState& timing() {
  static TimingState* t = new TimingState();  // lives until the process ends
  return *t;
}

}  // namespace

namespace pa {

void timing_mark(int kernel, bool begin, hipStream_t stream) {
  TimingState& t = timing();
  if (!t.on.load(std::memory_order_relaxed) || kernel < 0 || kernel >= kNumKernelIds) return;
  std::lock_guard<std::mutex> lk(t.mu);
  hipEvent_t e = t.take();
  if (!e) return;
  if (hipEventRecord(e, stream) != hipSuccess) {
    t.spare.push_back(e);
    return;
  }
  if (begin) {
    if (t.open[kernel]) t.spare.push_back(t.open[kernel]);
    t.open[kernel] = e;
  } else if (t.open[kernel]) {
    t.pending[kernel].push_back({t.open[kernel], e});
    t.open[kernel] = nullptr;
  } else {
    t.spare.push_back(e);
  }
}

}  // namespace pa

extern "C" {

pa_status_t pa_set_validate(int on) {
  g_validate_override.store(on < 0 ? -1 : (on != 0 ? 1 : 0), std::memory_order_relaxed);
  return ok();
}

pa_status_t pa_set_fused(int mode) {
  if (mode < -1 || mode > 2) return fail(PA_ERR_SHAPE, "pa_set_fused: mode %d outside -1 .. 2", mode);
  g_fused_override.store(mode, std::memory_order_relaxed);
  return ok();
}

pa_status_t pa_probe_mfma_peak(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (!out) return fail(PA_ERR_NULL, "pa_probe_mfma_peak: out is NULL");
  if (blocks < 1 || iters < 1) return fail(PA_ERR_SHAPE, "pa_probe_mfma_peak: blocks and iters must be >= 1");
  return hip_status(pa::launch_mfma_peak(out, blocks, iters, static_cast<hipStream_t>(stream)), "mfma probe launch");
}

pa_status_t pa_timing_enable(int on) {
  timing().on.store(on != 0, std::memory_order_relaxed);
  return ok();
}

pa_status_t pa_timing_reset(void) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  for (int k = 0; k < pa::kNumKernelIds; ++k) {
    t.drain(k);
    t.count[k] = 0;
    t.total_ms[k] = 0.0;
    t.launch_ms[k].clear();
  }
  return ok();
}

pa_status_t pa_timing_read_launches(pa_kernel_t kernel, float* ms, int32_t max_launches, int32_t* n) {
  if (!n || (max_launches > 0 && !ms)) return fail(PA_ERR_NULL, "n (and ms when max_launches > 0) must not be NULL");
  if ((int)kernel < 0 || (int)kernel >= pa::kNumKernelIds) return fail(PA_ERR_SHAPE, "unknown kernel id %d", (int)kernel);
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  const bool good = t.drain((int)kernel);
  const std::vector<float>& v = t.launch_ms[(int)kernel];
  *n = (int32_t)std::min<size_t>(v.size(), INT32_MAX);
  for (int32_t i = 0; i < std::min(*n, max_launches); ++i) ms[i] = v[i];
  return good ? ok() : fail(PA_ERR_HIP, "a timing event could not be read");
}

pa_status_t pa_timing_read(pa_kernel_t kernel, int64_t* count, double* total_ms) {
  if (!count || !total_ms) return fail(PA_ERR_NULL, "count and total_ms must not be NULL");
  if ((int)kernel < 0 || (int)kernel >= pa::kNumKernelIds) return fail(PA_ERR_SHAPE, "unknown kernel id %d", (int)kernel);
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  const bool good = t.drain((int)kernel);
  *count = t.count[(int)kernel];
  *total_ms = t.total_ms[(int)kernel];
  return good ? ok() : fail(PA_ERR_HIP, "a timing event could not be read");
}

}  // extern "C"
