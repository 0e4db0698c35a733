// Paged varlen prefill attention for gfx950 (bf16, matrix cores).
//
// What is computed (reading note on "Inside vLLM", core point 2: the step's
// sequences are concatenated into one super-sequence and each one is masked
// to its own tokens; page "vLLM：从 KV Cache 到高吞吐推理服务", tutorial 5:
// chunked prefill continues a prompt after its cached tokens): for new row i
// of sequence s with c = seq_len - q_len cached tokens,
//   out[row][h] = sum_{j <= c + i} softmax_j(scale * q . K_j) V_j,
// with K_j, V_j read through the block table (page "vLLM 架构概述" §2).
//
// Tiling (tutorial 7 of the same page: tiling plus online softmax; the CDNA4
// mapping is our own).  A work-group of 8 waves owns a row tile of 256
// (position, q head) rows of one kv head: the q heads that share the kv head
// (GQA, tutorial 1) are packed next to each other, so every K/V tile is
// gathered once for all of them.  Wave w owns rows 32w .. 32w+31, one 32-row
// matrix-core block.  K/V tiles of 64 keys (4 paged blocks) are copied through
// the block table straight from HBM into LDS (global_load_lds_dwordx4, no
// registers on the way), row-major with XOR-swizzled 16-byte chunks, in a ring
// of four stages filled three tiles ahead:
//   S^T[key][row] = K Q^T    v_mfma_f32_32x32x16_bf16 (K rows from LDS, Q in registers)
//   O^T[d][row]  += V^T P^T  v_mfma_f32_32x32x16_bf16 (V^T through ds_read_b64_tr_b16,
//                                                      P straight from the S^T registers)
// The scores of tile t+1 are issued to the matrix cores before the softmax
// of tile t.  The running maximum is only moved when a row's
// new maximum exceeds it by more than 2^8 (the probabilities stay <= 256,
// exact enough in bf16), so the accumulators are rarely rescaled.  A work
// item may cover only a range of key tiles (a split of a long row tile); it
// then leaves (O, m, l) for the merge kernel, which combines the splits with
// the log-sum-exp rule.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"
#include "prefill_body.h"

namespace pa {

namespace {

template <int D, bool WINDOW>
__global__ void __launch_bounds__(512) prefill_kernel(PrefillParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  // grid (kv heads, items): the dispatcher walks x fastest, so every kv head's item i
  // starts before any head's item i+1 -- with items listed longest first, the work-groups
  // start in longest-first order across the heads, and the short items fill the tail
  prefill_body<D, WINDOW>(p, smem, blockIdx.y, blockIdx.x);
}

// Log-sum-exp merge of the splits of a row tile: grid (row tiles x 8 groups of 32 rows,
// kv heads), 256 threads.  A wave takes 8 rows; D/8 lanes cover one row, 8 elements (16
// bytes of fp16 partial, 16 bytes of bf16 output) each, so every load and store moves whole
// rows.  Split i of a row holds (O_i / l_i) / sigma_i in fp16 with its scale sigma_i, its
// reference maximum m_i (log2 units) and weight sum l_i; it enters with weight
// l_i * 2^(m_i - M), folded online over the splits.  A split that saw none of the row's keys
// (m_i = -inf), or whose weight underflows to 0 next to the running maximum, is skipped
// rather than multiplied, so no 0 * inf can arise.  The split holding the row's largest
// score has l_i >= 1, so the weight sum is never 0.
template <int D>
__global__ void __launch_bounds__(256) prefill_merge_kernel(PrefillMergeParams p) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerPass = 64 / kLanesPerRow;
  constexpr int kRowsPerWave = 8;
  const uint64_t item = p.items[blockIdx.x >> 3];
  const int s = (int)(item & 0xFFFFu);
  const int rt = (int)((item >> 16) & 0xFFFFu);
  const int first = (int)((item >> 32) & 0xFFFFFu), n = (int)(item >> 52);
  const int kvh = blockIdx.y;
  const int G = p.group, P = p.tile_positions;
  const int q0 = p.qsl[s];
  const int q_len = p.qsl[s + 1] - q0;
  const int pos0 = rt * P;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane / kLanesPerRow, c = lane % kLanesPerRow;
  const size_t slot_step = (size_t)p.num_kv_heads * kPrefillRows;
#pragma unroll
  for (int k = 0; k < kRowsPerWave / kRowsPerPass; ++k) {
    const int R = (blockIdx.x & 7) * 32 + wave * kRowsPerWave + k * kRowsPerPass + sub;
    const int pos = pos0 + R / G;
    if (R >= P * G || pos >= q_len) continue;
    const size_t base = ((size_t)first * p.num_kv_heads + kvh) * kPrefillRows + R;
    float M = -INFINITY, den = 0.f, o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = 0.f;
#pragma unroll 4
    for (int i = 0; i < n; ++i) {
      const size_t pi = base + i * slot_step;
      const float mi = p.part_m[pi], li = p.part_l[pi], si = p.part_s[pi];
      const u32x4 w = *reinterpret_cast<const u32x4*>(p.part_o + pi * D + c * 8);
      if (mi == -INFINITY) continue;  // this split saw none of the row's keys
      const float Mn = fmaxf(M, mi);
      const float b = li * fast_exp2(mi - Mn);
      if (b == 0.f) continue;  // negligible next to the running maximum (then Mn == M)
      const float a = fast_exp2(M - Mn);  // 0 for the first split that counts
      const float bs = b * si;
      den = den * a + b;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = o[2 * j] * a + f16_bits_to_f32(w[j] & 0xFFFFu) * bs;
        o[2 * j + 1] = o[2 * j + 1] * a + f16_bits_to_f32(w[j] >> 16) * bs;
      }
      M = Mn;
    }
    const float inv = p.v_scale / den;
    const int h = kvh * G + (R % G);
    uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + ((size_t)(q0 + pos) * p.num_q_heads + h) * D + c * 8;
    *reinterpret_cast<u32x4*>(op) = u32x4{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                                          pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
  }
}

// fp8 staging: one work-group of 256 threads per (sequence, block) -- blocks past the grid's
// capped y extent (65535) go to work-group y, y + gridDim.y, ....  Sequence s's
// first staging block is the sum of the block counts of the sequences before it that
// have q_len > 1 (a block-wide sum over them; the batch's sequence count is small next
// to the blocks moved).  Each thread turns 16 codes into 16 bf16 values per step.
__global__ void __launch_bounds__(256) stage_fp8_kernel(const uint8_t* key_cache, const uint8_t* value_cache,
                                                         const int32_t* block_tables, int bt_stride,
                                                         const int32_t* seq_lens, const int32_t* qsl, int num_seqs,
                                                         int row_bytes, int num_blocks, uint16_t* stage_k,
                                                         uint16_t* stage_v, int32_t* stage_tables) {
  __shared__ int red[256];
  const int s = blockIdx.x;
  if (qsl[s + 1] - qsl[s] <= 1) return;
  const int nb = (seq_lens[s] + 15) >> 4;
  if ((int)blockIdx.y >= nb) return;
  int acc = 0;
  for (int t = threadIdx.x; t < s; t += 256) acc += qsl[t + 1] - qsl[t] > 1 ? (seq_lens[t] + 15) >> 4 : 0;
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const int base = red[0];
  const int block_bytes = 16 * row_bytes;  // codes per block (one byte each)
  for (int j = blockIdx.y; j < nb; j += gridDim.y) {  // the grid's y extent is capped
    const int phys = min(max(block_tables[(size_t)s * bt_stride + j], 0), num_blocks - 1);
    const int dst = base + j;
    if (threadIdx.x == 0) stage_tables[(size_t)s * bt_stride + j] = dst;
    const uint8_t* ks = key_cache + (size_t)phys * block_bytes;
    const uint8_t* vs = value_cache + (size_t)phys * block_bytes;
    uint16_t* kd = stage_k + (size_t)dst * block_bytes;
    uint16_t* vd = stage_v + (size_t)dst * block_bytes;
    for (int e = threadIdx.x * 16; e < block_bytes; e += 256 * 16) {
      const u32x4 kc = *reinterpret_cast<const u32x4*>(ks + e);
      const u32x4 vc = *reinterpret_cast<const u32x4*>(vs + e);
      u32x4 klo, khi, vlo, vhi;
      const u32x2 k0 = e4m3x4_to_bf16x4(kc.x), k1 = e4m3x4_to_bf16x4(kc.y), k2 = e4m3x4_to_bf16x4(kc.z),
                  k3 = e4m3x4_to_bf16x4(kc.w);
      const u32x2 v0 = e4m3x4_to_bf16x4(vc.x), v1 = e4m3x4_to_bf16x4(vc.y), v2 = e4m3x4_to_bf16x4(vc.z),
                  v3 = e4m3x4_to_bf16x4(vc.w);
      klo = u32x4{k0.x, k0.y, k1.x, k1.y};
      khi = u32x4{k2.x, k2.y, k3.x, k3.y};
      vlo = u32x4{v0.x, v0.y, v1.x, v1.y};
      vhi = u32x4{v2.x, v2.y, v3.x, v3.y};
      *reinterpret_cast<u32x4*>(kd + e) = klo;
      *reinterpret_cast<u32x4*>(kd + e + 8) = khi;
      *reinterpret_cast<u32x4*>(vd + e) = vlo;
      *reinterpret_cast<u32x4*>(vd + e + 8) = vhi;
    }
  }
}

// Cascade prefix over fp8 pools: work-group (j, q) copies quarter q of block j of table row 0
// -- the prefix every sequence's table begins with -- to staging block j as the exact bf16
// values of its codes (16 codes per thread: one load of K and one of V each), and (q = 0)
// writes staging table entry j = j.
__global__ void __launch_bounds__(256) stage_prefix_fp8_kernel(const uint8_t* key_cache, const uint8_t* value_cache,
                                                                const int32_t* block_tables, int row_bytes,
                                                                int num_blocks, uint16_t* stage_k, uint16_t* stage_v,
                                                                int32_t* stage_table) {
  const int j = blockIdx.x;
  const int phys = min(max(block_tables[j], 0), num_blocks - 1);
  if (threadIdx.x == 0 && blockIdx.y == 0) stage_table[j] = j;
  const int block_bytes = 16 * row_bytes;
  const uint8_t* ks = key_cache + (size_t)phys * block_bytes;
  const uint8_t* vs = value_cache + (size_t)phys * block_bytes;
  uint16_t* kd = stage_k + (size_t)j * block_bytes;
  uint16_t* vd = stage_v + (size_t)j * block_bytes;
  for (int e = (blockIdx.y * 256 + threadIdx.x) * 16; e < block_bytes; e += gridDim.y * 256 * 16) {
    const u32x4 kc = *reinterpret_cast<const u32x4*>(ks + e);
    const u32x4 vc = *reinterpret_cast<const u32x4*>(vs + e);
    const u32x2 k0 = e4m3x4_to_bf16x4(kc.x), k1 = e4m3x4_to_bf16x4(kc.y), k2 = e4m3x4_to_bf16x4(kc.z),
                k3 = e4m3x4_to_bf16x4(kc.w);
    const u32x2 v0 = e4m3x4_to_bf16x4(vc.x), v1 = e4m3x4_to_bf16x4(vc.y), v2 = e4m3x4_to_bf16x4(vc.z),
                v3 = e4m3x4_to_bf16x4(vc.w);
    *reinterpret_cast<u32x4*>(kd + e) = u32x4{k0.x, k0.y, k1.x, k1.y};
    *reinterpret_cast<u32x4*>(kd + e + 8) = u32x4{k2.x, k2.y, k3.x, k3.y};
    *reinterpret_cast<u32x4*>(vd + e) = u32x4{v0.x, v0.y, v1.x, v1.y};
    *reinterpret_cast<u32x4*>(vd + e + 8) = u32x4{v2.x, v2.y, v3.x, v3.y};
  }
}

}  // namespace

hipError_t launch_stage_prefix_fp8(const uint8_t* key_cache, const uint8_t* value_cache, const int32_t* block_tables,
                                   int prefix_blocks, int num_kv_heads, int head_dim, int num_blocks,
                                   uint16_t* stage_k, uint16_t* stage_v, int32_t* stage_table, hipStream_t stream) {
  // one 16-code chunk per thread: 256 threads x 16 codes per work-group along y
  const int parts = (16 * num_kv_heads * head_dim + 256 * 16 - 1) / (256 * 16);
  timing_mark(kKStageFp8, true, stream);
  hipLaunchKernelGGL(stage_prefix_fp8_kernel, dim3(prefix_blocks, parts), dim3(256), 0, stream, key_cache, value_cache,
                     block_tables, num_kv_heads * head_dim, num_blocks, stage_k, stage_v, stage_table);
  timing_mark(kKStageFp8, false, stream);
  return hipGetLastError();
}

hipError_t launch_stage_fp8(const uint8_t* key_cache, const uint8_t* value_cache, const int32_t* block_tables,
                            int bt_stride, const int32_t* seq_lens, const int32_t* qsl, int num_seqs, int max_blocks,
                            int num_kv_heads, int head_dim, int num_blocks, uint16_t* stage_k, uint16_t* stage_v,
                            int32_t* stage_tables, hipStream_t stream) {
  const dim3 grid(num_seqs, std::min(max_blocks, 65535));
  timing_mark(kKStageFp8, true, stream);
  hipLaunchKernelGGL(stage_fp8_kernel, grid, dim3(256), 0, stream, key_cache, value_cache, block_tables, bt_stride,
                     seq_lens, qsl, num_seqs, num_kv_heads * head_dim, num_blocks, stage_k, stage_v, stage_tables);
  timing_mark(kKStageFp8, false, stream);
  return hipGetLastError();
}

size_t prefill_lds_bytes(int head_dim) {
  return head_dim == 128 ? PrefillShape<128>::kLdsBytes : PrefillShape<64>::kLdsBytes;
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(p.num_kv_heads, p.n_items);
  const size_t lds = prefill_lds_bytes(head_dim);
  timing_mark(kKPrefill, true, stream);
  auto launch = [&](auto kernel, int threads) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    hipLaunchKernelGGL(kernel, grid, dim3(threads), lds, stream, p);
  };
  if (head_dim == 128) {
    if (p.window > 0 || p.chunk > 0)
      launch(&prefill_kernel<128, true>, PrefillShape<128>::kThreads);
    else
      launch(&prefill_kernel<128, false>, PrefillShape<128>::kThreads);
  } else {
    if (p.window > 0 || p.chunk > 0)
      launch(&prefill_kernel<64, true>, PrefillShape<64>::kThreads);
    else
      launch(&prefill_kernel<64, false>, PrefillShape<64>::kThreads);
  }
  timing_mark(kKPrefill, false, stream);
  return hipGetLastError();
}

// Matrix-core peak probe: every wave runs `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 (the prefill kernel's instruction) on register operands and
// writes one sum per lane, so nothing is optimised away.  256 threads per work-group.
__global__ void __launch_bounds__(256) mfma_peak_kernel(float* out, int iters) {
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  // normal bf16 operands (1.0, 0.5, 0.25, ...): no denormal inputs
  const u32x4 a{0x3f803f80u, 0x3f003f00u, 0x3e803e80u, 0x3f803f00u}, b{0x3f003f80u, 0x3e803f80u, 0x3f803f80u, 0x3f003f00u};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(u4_to_bf16x8(a), u4_to_bf16x8(b), acc[i], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[i][r];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = sum;
}

hipError_t launch_mfma_peak(float* out, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError();
}

hipError_t launch_prefill_merge(const PrefillMergeParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(p.n_items * 8, p.num_kv_heads);
  timing_mark(kKPrefillMerge, true, stream);
  if (head_dim == 128)
    hipLaunchKernelGGL(prefill_merge_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_merge_kernel<64>, grid, dim3(256), 0, stream, p);
  timing_mark(kKPrefillMerge, false, stream);
  return hipGetLastError();
}

}  // namespace pa
