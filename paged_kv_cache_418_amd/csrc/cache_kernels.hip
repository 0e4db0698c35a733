// Slot mapping and the KV write for gfx950.
//
// Slot mapping (page "vLLM：从 KV Cache 到高吞吐推理服务", tutorial 3; page
// "vLLM 架构概述" §2): new row i of sequence s sits at position
// p = seq_len - q_len + i; its slot is block_tables[s][p / B] * B + p % B.
// KV write (page "vLLM 架构概述" §3, the reshape_and_cache kernel): copy the
// new token's K and V rows of every kv head to cache[slot / B][slot % B].
// fp8 pools (tutorial 6: FP8 E4M3 KV with a scale) store the E4M3 code of
// x / scale.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

__global__ void __launch_bounds__(256) slot_mapping_kernel(int32_t* slots, const int32_t* block_tables,
                                                           int bt_stride, const int32_t* seq_lens,
                                                           const int32_t* qsl, int num_tokens, int block_size) {
  const int s = blockIdx.x;
  const int q0 = qsl[s], q_len = qsl[s + 1] - q0;
  const int cached = seq_lens[s] - q_len;
  const int* bt = block_tables + (size_t)s * bt_stride;
  for (int i = threadIdx.x; i < q_len; i += blockDim.x) {
    if (q0 + i < 0 || q0 + i >= num_tokens) continue;
    const int pos = cached + i;
    const int logical = pos / block_size;
    int slot = -1;
    if (pos >= 0 && logical < bt_stride) slot = bt[logical] * block_size + (pos - logical * block_size);
    slots[q0 + i] = slot;
  }
}

// Slot of new row i of a sequence with `cached` tokens before this step (-1 when its
// position lies past the table).
__device__ __forceinline__ int row_slot(const int32_t* bt, int bt_stride, int cached, int i, int block_size) {
  const int pos = cached + i;
  const int logical = pos / block_size;
  return (pos >= 0 && logical < bt_stride) ? bt[logical] * block_size + (pos - logical * block_size) : -1;
}

// The work-group's threads copy token t's K and V rows (all kv heads) in VecT chunks.
template <typename VecT>
__device__ __forceinline__ void copy_token(const uint8_t* key, const uint8_t* value, int64_t key_stride_b,
                                           int64_t value_stride_b, uint8_t* key_cache, uint8_t* value_cache, int t,
                                           int slot, int row_bytes) {
  const int n = row_bytes / (int)sizeof(VecT);
  const VecT* ks = reinterpret_cast<const VecT*>(key + (int64_t)t * key_stride_b);
  const VecT* vs = reinterpret_cast<const VecT*>(value + (int64_t)t * value_stride_b);
  VecT* kd = reinterpret_cast<VecT*>(key_cache + (int64_t)slot * row_bytes);
  VecT* vd = reinterpret_cast<VecT*>(value_cache + (int64_t)slot * row_bytes);
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

// Elements e .. e+7 of a bf16 or fp32 row (element offset e of the row at src).
template <bool SRC_F32>
__device__ __forceinline__ void load8(const void* src, int64_t e, float (&x)[8]) {
  if constexpr (SRC_F32) {
    const float* s = reinterpret_cast<const float*>(src) + e;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = s[j];
  } else {
    const uint16_t* s = reinterpret_cast<const uint16_t*>(src) + e;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = bf16_to_f32(s[j]);
  }
}

// The E4M3 codes of x / scale, one 8-byte store.
__device__ __forceinline__ void store_e4m3x8(uint8_t* dst, const float (&x)[8], float scale) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j >> 2] |= (uint32_t)f32_to_e4m3(__fdiv_rn(x[j], scale)) << (8 * (j & 3));
  *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
}

// fp8: each thread quantises 8 consecutive elements of token t (one 8-byte store per pool).
template <bool SRC_F32>
__device__ __forceinline__ void quantize_token(const void* key, const void* value, int64_t key_stride,
                                               int64_t value_stride, uint8_t* key_cache, uint8_t* value_cache, int t,
                                               int slot, int row_elems, float k_scale, float v_scale) {
  for (int c = threadIdx.x; c < row_elems / 8; c += blockDim.x) {
    float xk[8], xv[8];
    load8<SRC_F32>(key, (int64_t)t * key_stride + c * 8, xk);
    load8<SRC_F32>(value, (int64_t)t * value_stride + c * 8, xv);
    store_e4m3x8(key_cache + (int64_t)slot * row_elems + c * 8, xk, k_scale);
    store_e4m3x8(value_cache + (int64_t)slot * row_elems + c * 8, xv, v_scale);
  }
}

// One work-group per token; threads copy VEC-byte chunks of all kv heads.
template <typename VecT>
__global__ void __launch_bounds__(256) reshape_kernel(const uint8_t* key, const uint8_t* value, int64_t key_stride_b,
                                                      int64_t value_stride_b, uint8_t* key_cache, uint8_t* value_cache,
                                                      const int32_t* slots, int row_bytes, int num_slots) {
  const int t = blockIdx.x;
  const int slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  copy_token<VecT>(key, value, key_stride_b, value_stride_b, key_cache, value_cache, t, slot, row_bytes);
}

template <bool SRC_F32>
__global__ void __launch_bounds__(256) reshape_fp8_kernel(const void* key, const void* value, int64_t key_stride,
                                                          int64_t value_stride, uint8_t* key_cache,
                                                          uint8_t* value_cache, const int32_t* slots, int row_elems,
                                                          int num_slots, float k_scale, float v_scale) {
  const int t = blockIdx.x;
  const int slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  quantize_token<SRC_F32>(key, value, key_stride, value_stride, key_cache, value_cache, t, slot, row_elems, k_scale,
                          v_scale);
}

// Slot mapping and KV write in one launch: grid (num_seqs, min(ceil(max_q_len / kWriteTokens),
// 65535)); work-group (s, g) takes the groups of kWriteTokens new rows g, g + gridDim.y, ... of
// sequence s, computes each row's slot as slot_mapping_kernel does (stored when slots_out is
// given), and writes the rows as the reshape kernels do (skipped for slots outside the pool).
// A group's table reads are issued together, then every load of its rows before any store, so
// the rows' memory round trips overlap instead of following one another.
constexpr int kWriteTokens = 4;

// Copies rows tok[j] -> slots slot[j] (slot < 0: no row) in VecT chunks.
template <typename VecT>
__device__ __forceinline__ void copy_rows(const uint8_t* key, const uint8_t* value, int64_t key_stride_b,
                                          int64_t value_stride_b, uint8_t* key_cache, uint8_t* value_cache,
                                          const int (&tok)[kWriteTokens], const int (&slot)[kWriteTokens],
                                          int row_bytes) {
  const int n = row_bytes / (int)sizeof(VecT);
  for (int c = threadIdx.x; c < n; c += blockDim.x) {
    VecT kx[kWriteTokens], vx[kWriteTokens];
#pragma unroll
    for (int j = 0; j < kWriteTokens; ++j)
      if (slot[j] >= 0) {
        kx[j] = reinterpret_cast<const VecT*>(key + (int64_t)tok[j] * key_stride_b)[c];
        vx[j] = reinterpret_cast<const VecT*>(value + (int64_t)tok[j] * value_stride_b)[c];
      }
#pragma unroll
    for (int j = 0; j < kWriteTokens; ++j)
      if (slot[j] >= 0) {
        reinterpret_cast<VecT*>(key_cache + (int64_t)slot[j] * row_bytes)[c] = kx[j];
        reinterpret_cast<VecT*>(value_cache + (int64_t)slot[j] * row_bytes)[c] = vx[j];
      }
  }
}

// Quantises rows tok[j] into slots slot[j] (slot < 0: no row), 8 elements per thread and row.
template <bool SRC_F32>
__device__ __forceinline__ void quantize_rows(const void* key, const void* value, int64_t key_stride,
                                              int64_t value_stride, uint8_t* key_cache, uint8_t* value_cache,
                                              const int (&tok)[kWriteTokens], const int (&slot)[kWriteTokens],
                                              int row_elems, float k_scale, float v_scale) {
  for (int c = threadIdx.x; c < row_elems / 8; c += blockDim.x) {
    float xk[kWriteTokens][8], xv[kWriteTokens][8];
#pragma unroll
    for (int j = 0; j < kWriteTokens; ++j)
      if (slot[j] >= 0) {
        load8<SRC_F32>(key, (int64_t)tok[j] * key_stride + c * 8, xk[j]);
        load8<SRC_F32>(value, (int64_t)tok[j] * value_stride + c * 8, xv[j]);
      }
#pragma unroll
    for (int j = 0; j < kWriteTokens; ++j)
      if (slot[j] >= 0) {
        store_e4m3x8(key_cache + (int64_t)slot[j] * row_elems + c * 8, xk[j], k_scale);
        store_e4m3x8(value_cache + (int64_t)slot[j] * row_elems + c * 8, xv[j], v_scale);
      }
  }
}

template <typename VecT, int KIND>  // KIND 0: copy; 1: fp8 from bf16; 2: fp8 from fp32
__global__ void __launch_bounds__(128) write_kv_kernel(const void* key, const void* value, int64_t key_stride,
                                                       int64_t value_stride, uint8_t* key_cache, uint8_t* value_cache,
                                                       int32_t* slots_out, const int32_t* block_tables, int bt_stride,
                                                       const int32_t* seq_lens, const int32_t* qsl, int num_tokens,
                                                       int block_size, int num_slots, int row, float k_scale,
                                                       float v_scale) {
  const int s = blockIdx.x;
  const int q0 = qsl ? qsl[s] : s, q_len = qsl ? qsl[s + 1] - q0 : 1;  // no qsl: one row per sequence
  const int cached = seq_lens[s] - q_len;
  const int* bt = block_tables + (size_t)s * bt_stride;
  // row groups blockIdx.y, blockIdx.y + gridDim.y, ... of kWriteTokens rows (the grid's y extent is capped)
  for (int g0 = blockIdx.y * kWriteTokens; g0 < q_len; g0 += gridDim.y * kWriteTokens) {
    int tok[kWriteTokens], slot[kWriteTokens];
#pragma unroll
    for (int j = 0; j < kWriteTokens; ++j) {
      const int i = g0 + j, t = q0 + i;
      const bool row_ok = i < q_len && t >= 0 && t < num_tokens;
      tok[j] = t;
      slot[j] = row_ok ? row_slot(bt, bt_stride, cached, i, block_size) : -1;
      if (row_ok && slots_out && threadIdx.x == 0) slots_out[t] = slot[j];
      if (slot[j] >= num_slots) slot[j] = -1;  // outside the pool: not written
    }
    if constexpr (KIND == 0)  // key_stride / value_stride in bytes, row in bytes
      copy_rows<VecT>(reinterpret_cast<const uint8_t*>(key), reinterpret_cast<const uint8_t*>(value), key_stride,
                      value_stride, key_cache, value_cache, tok, slot, row);
    else  // strides in elements, row in elements
      quantize_rows<KIND == 2>(key, value, key_stride, value_stride, key_cache, value_cache, tok, slot, row, k_scale,
                               v_scale);
  }
}

}  // namespace

hipError_t launch_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, int bt_stride,
                               const int32_t* seq_lens, const int32_t* qsl, int num_seqs, int num_tokens,
                               int block_size, hipStream_t stream) {
  timing_mark(kKSlotMapping, true, stream);
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(num_seqs), dim3(64), 0, stream, slot_mapping, block_tables, bt_stride,
                     seq_lens, qsl, num_tokens, block_size);
  timing_mark(kKSlotMapping, false, stream);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, int64_t key_stride, int64_t value_stride,
                                    void* key_cache, void* value_cache, const int32_t* slots, int num_tokens,
                                    int num_kv_heads, int head_dim, int block_size, int num_blocks, int elem_bytes,
                                    hipStream_t stream) {
  const int row_bytes = num_kv_heads * head_dim * elem_bytes;  // one token of one pool
  const int64_t ksb = key_stride * elem_bytes, vsb = value_stride * elem_bytes;
  const int num_slots = num_blocks * block_size;
  const uintptr_t align = (uintptr_t)key | (uintptr_t)value | (uintptr_t)key_cache | (uintptr_t)value_cache |
                          (uintptr_t)ksb | (uintptr_t)vsb | (uintptr_t)row_bytes;
  const int threads = 128;
  const auto* k8 = reinterpret_cast<const uint8_t*>(key);
  const auto* v8 = reinterpret_cast<const uint8_t*>(value);
  auto* kc8 = reinterpret_cast<uint8_t*>(key_cache);
  auto* vc8 = reinterpret_cast<uint8_t*>(value_cache);
  timing_mark(kKReshape, true, stream);
  if ((align & 15u) == 0)
    hipLaunchKernelGGL(reshape_kernel<u32x4>, dim3(num_tokens), dim3(threads), 0, stream, k8, v8, ksb, vsb, kc8, vc8,
                       slots, row_bytes, num_slots);
  else if ((align & 3u) == 0)
    hipLaunchKernelGGL(reshape_kernel<uint32_t>, dim3(num_tokens), dim3(threads), 0, stream, k8, v8, ksb, vsb, kc8,
                       vc8, slots, row_bytes, num_slots);
  else
    hipLaunchKernelGGL(reshape_kernel<uint16_t>, dim3(num_tokens), dim3(threads), 0, stream, k8, v8, ksb, vsb, kc8,
                       vc8, slots, row_bytes, num_slots);
  timing_mark(kKReshape, false, stream);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, int64_t key_stride,
                                        int64_t value_stride, uint8_t* key_cache, uint8_t* value_cache,
                                        const int32_t* slots, int num_tokens, int num_kv_heads, int head_dim,
                                        int block_size, int num_blocks, int src_f32, float k_scale,
                                        float v_scale, hipStream_t stream) {
  const int row_elems = num_kv_heads * head_dim;
  const int num_slots = num_blocks * block_size;
  timing_mark(kKReshape, true, stream);
  if (src_f32)
    hipLaunchKernelGGL(reshape_fp8_kernel<true>, dim3(num_tokens), dim3(128), 0, stream, key, value, key_stride,
                       value_stride, key_cache, value_cache, slots, row_elems, num_slots, k_scale, v_scale);
  else
    hipLaunchKernelGGL(reshape_fp8_kernel<false>, dim3(num_tokens), dim3(128), 0, stream, key, value, key_stride,
                       value_stride, key_cache, value_cache, slots, row_elems, num_slots, k_scale, v_scale);
  timing_mark(kKReshape, false, stream);
  return hipGetLastError();
}

hipError_t launch_write_kv(const void* key, const void* value, int64_t key_stride, int64_t value_stride,
                           void* key_cache, void* value_cache, int32_t* slots_out, const int32_t* block_tables,
                           int bt_stride, const int32_t* seq_lens, const int32_t* qsl, int num_seqs, int num_tokens,
                           int max_q_len, int num_kv_heads, int head_dim, int block_size, int num_blocks, int kind,
                           float k_scale, float v_scale, hipStream_t stream) {
  const dim3 grid(num_seqs, std::min((max_q_len + kWriteTokens - 1) / kWriteTokens, 65535));
  const int num_slots = num_blocks * block_size;
  auto* kc8 = reinterpret_cast<uint8_t*>(key_cache);
  auto* vc8 = reinterpret_cast<uint8_t*>(value_cache);
  const int row_elems = num_kv_heads * head_dim;
  timing_mark(kKReshape, true, stream);
  if (kind == kFP8 + 0 || kind == kFP8 + 1) {  // fp8 pools: kind kFP8 (bf16 source) or kFP8 + 1 (fp32 source)
    if (kind == kFP8)
      hipLaunchKernelGGL((write_kv_kernel<uint32_t, 1>), grid, dim3(128), 0, stream, key, value, key_stride,
                         value_stride, kc8, vc8, slots_out, block_tables, bt_stride, seq_lens, qsl, num_tokens,
                         block_size, num_slots, row_elems, k_scale, v_scale);
    else
      hipLaunchKernelGGL((write_kv_kernel<uint32_t, 2>), grid, dim3(128), 0, stream, key, value, key_stride,
                         value_stride, kc8, vc8, slots_out, block_tables, bt_stride, seq_lens, qsl, num_tokens,
                         block_size, num_slots, row_elems, k_scale, v_scale);
  } else {
    const int elem = kind == kF32 ? 4 : 2;
    const int row_bytes = row_elems * elem;
    const int64_t ksb = key_stride * elem, vsb = value_stride * elem;
    const uintptr_t align = (uintptr_t)key | (uintptr_t)value | (uintptr_t)key_cache | (uintptr_t)value_cache |
                            (uintptr_t)ksb | (uintptr_t)vsb | (uintptr_t)row_bytes;
    if ((align & 15u) == 0)
      hipLaunchKernelGGL((write_kv_kernel<u32x4, 0>), grid, dim3(128), 0, stream, key, value, ksb, vsb, kc8, vc8,
                         slots_out, block_tables, bt_stride, seq_lens, qsl, num_tokens, block_size, num_slots,
                         row_bytes, 1.f, 1.f);
    else if ((align & 3u) == 0)
      hipLaunchKernelGGL((write_kv_kernel<uint32_t, 0>), grid, dim3(128), 0, stream, key, value, ksb, vsb, kc8, vc8,
                         slots_out, block_tables, bt_stride, seq_lens, qsl, num_tokens, block_size, num_slots,
                         row_bytes, 1.f, 1.f);
    else
      hipLaunchKernelGGL((write_kv_kernel<uint16_t, 0>), grid, dim3(128), 0, stream, key, value, ksb, vsb, kc8, vc8,
                         slots_out, block_tables, bt_stride, seq_lens, qsl, num_tokens, block_size, num_slots,
                         row_bytes, 1.f, 1.f);
  }
  timing_mark(kKReshape, false, stream);
  return hipGetLastError();
}

}  // namespace pa
