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
// registers on the way), row-major with XOR-swizzled 16-byte chunks, in rings
// (four K stages, five V stages) filled three tiles ahead:
//   S^T[key][row] = K Q^T    v_mfma_f32_32x32x16_bf16 (K rows from LDS, Q in registers)
//   O^T[d][row]  += V^T P^T  v_mfma_f32_32x32x16_bf16 (V^T gathered from the row-major
//                                                      V tile by ds_read_b64_tr_b16,
//                                                      P straight from the S^T registers)
// The scores of tile t+1 are issued to the matrix cores before the softmax
// of tile t.  The running maximum is only moved when a row's
// new maximum exceeds it by more than 2^8 (the probabilities stay <= 256,
// exact enough in bf16), so the accumulators are rarely rescaled.  A work
// item may cover only a range of key tiles (a split of a long row tile); it
// then leaves (O, m, l) for the merge kernel, which combines the splits with
// the log-sum-exp rule.
//
// fp8 pools (tutorial 6 of the same page: E4M3 KV with a scale): the tiles are copied as
// raw codes; K operands are converted to bf16 as they are read, and V is converted into a
// bf16 row-major tile that O += V P reads as it reads bf16 tiles, so the matrix cores see
// the codes' exact bf16 values (the scales go to the score scale and the output).
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"
#include "prefill_body.h"

namespace pa {

namespace {

template <int D, bool WINDOW, bool F8>
__global__ void __launch_bounds__(512) prefill_kernel(PrefillParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  // grid (kv heads, items): the dispatcher walks x fastest, so every kv head's item i
  // starts before any head's item i+1 -- with items listed longest first, the work-groups
  // start in longest-first order across the heads, and the short items fill the tail
  prefill_body<D, WINDOW, false, F8>(p, smem, blockIdx.y, blockIdx.x);
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

}  // namespace

size_t prefill_lds_bytes(int head_dim) {
  return head_dim == 128 ? PrefillShape<128>::kLdsBytes : PrefillShape<64>::kLdsBytes;
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(p.num_kv_heads, p.n_items);
  const size_t lds = prefill_lds_bytes(head_dim);
  const bool win = p.window > 0 || p.chunk > 0;
  timing_mark(kKPrefill, true, stream);
  auto launch = [&](auto kernel) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    hipLaunchKernelGGL(kernel, grid, dim3(512), lds, stream, p);
  };
  auto pick = [&](auto d_c, auto f8_c) {
    constexpr int D = decltype(d_c)::value;
    constexpr bool F8 = decltype(f8_c)::value;
    if (win)
      launch(&prefill_kernel<D, true, F8>);
    else
      launch(&prefill_kernel<D, false, F8>);
  };
  using T = std::true_type;
  using F = std::false_type;
  if (head_dim == 128)
    p.kv_fp8 ? pick(std::integral_constant<int, 128>{}, T{}) : pick(std::integral_constant<int, 128>{}, F{});
  else
    p.kv_fp8 ? pick(std::integral_constant<int, 64>{}, T{}) : pick(std::integral_constant<int, 64>{}, F{});
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
