// Paged decode attention for gfx950: one new token per sequence.
//
// What is computed: for each sequence s and q head h,
//   out[s][h] = sum_j softmax_j(scale * q . K_j) V_j,  j = 0 .. seq_len-1,
// with K_j, V_j gathered through the int32 block table (page "vLLM 架构概述"
// §2: the table is an int32 array looked up inside the kernel plus address
// arithmetic; page "vLLM：从 KV Cache 到高吞吐推理服务", tutorial 3: logical
// block j / B, offset j % B).  Softmax is evaluated online, block by block
// (tutorial 7 of the same page: tiling and online softmax), and long
// contexts are cut into partitions whose partial results are combined with
// the log-sum-exp rule (tutorial 7: the LSE statistic).
//
// Work decomposition (designed for CDNA4, not taken from the pages): the
// blocks of all sequences, laid end to end, are cut into num_splits equal
// shares per kv head, and one wave takes one share.  A share may end inside
// a sequence and may cover several short ones; every piece of a sequence
// that is not the whole sequence leaves a partial result (unnormalised O,
// running max m, sum l) that the merge kernel combines with the log-sum-exp
// rule.  Equal shares keep every wave busy until the end of the launch, which
// fixed-size context partitions of uneven sequences do not.
//
// Inside a wave, the q heads that share the kv head (GQA, tutorial 1) are
// the 16 columns of the matrix-core tiles, so the K/V of a block are read
// once for all of them.  Each 16-lane quarter of the wave loads one whole
// token row of the block (coalesced 16-byte loads for bf16 at head size
// 128); K goes through a small swizzled LDS tile to reach the matrix-core
// operand layout, V is used from registers.  Masked positions (the partly
// filled last block) are removed by selection, never by multiplying with
// zero, so NaN in unused pool slots cannot leak.
#include <mutex>
#include <type_traits>

#include "decode_body.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

// WRITE: the decode that also stores the step's new K/V rows (p.new_k / p.new_v)
template <int D, bool FP8, bool WRITE>
__global__ void __launch_bounds__(64) decode_mfma_kernel(DecodeParams p) {
  __shared__ __align__(16) unsigned char k_lds[DecodeShape<D, FP8>::kLdsBytes];
  // grid y: (kv head, group of 16 of its q heads); a cascade has one group per kv head
  decode_wave<D, FP8, WRITE>(p, k_lds, blockIdx.x, blockIdx.y);
}

// fp32 pools and queries: vector-ALU kernel, one wave per (share, q head).
// Lane = (token t = lane % 16, quarter = lane / 16) holding D/4 elements of a row.
template <int D>
__device__ __forceinline__ void decode_f32_piece(const DecodeParams& p, int split, int h, int s, int b0, int b1,
                                                 int nb) {
  constexpr int QD = D / 4;
  const int row = p.qsl ? p.qsl[s] : s;
  const int L = min(p.seq_lens[s], p.max_seq_len);
  const int skip = decode_skip(p, L);        // blocks wholly before a window / local chunk
  const int key_lo = decode_first_key(p, L);  // keys below it are not visible
  const int tok0 = (skip + b0) * 16;
  const int tok1 = min(L, (skip + b1) * 16);
  const int nblk = b1 - b0;
  const int lane = threadIdx.x;
  const int t = lane & 15, quarter = lane >> 4;
  const int kvh = h / p.group;

  float q[QD];
  const float* qp = reinterpret_cast<const float*>(p.query) + ((size_t)row * p.num_q_heads + h) * D + quarter * QD;
#pragma unroll
  for (int i = 0; i < QD; ++i) q[i] = qp[i];
  float o[QD];
#pragma unroll
  for (int i = 0; i < QD; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int* bt = p.block_tables + (size_t)s * p.bt_stride + skip + b0;
  const float* kc = reinterpret_cast<const float*>(p.key_cache);
  const float* vc = reinterpret_cast<const float*>(p.value_cache);

  for (int b = 0; b < nblk; ++b) {
    int phys = bt[b];
    phys = min(max(phys, 0), p.num_blocks - 1);
    const int pos = tok0 + b * 16 + t;
    const bool live = pos < tok1 && pos >= key_lo;
    const size_t off = (((size_t)phys * 16 + t) * p.num_kv_heads + kvh) * D + quarter * QD;
    float dot = 0.f;
    if (live) {
#pragma unroll
      for (int i = 0; i < QD; ++i) dot += q[i] * kc[off + i];
    }
    dot += shfl_xor(dot, 16);
    dot += shfl_xor(dot, 32);
    const float z = live ? dot * p.scale_log2 : -INFINITY;
    float bmax = z;
#pragma unroll
    for (int msk = 1; msk < 16; msk <<= 1) bmax = fmaxf(bmax, shfl_xor(bmax, msk));
    const float mnew = fmaxf(m, bmax);
    const float alpha = fast_exp2(m - mnew);
    const float pr = fast_exp2(z - mnew);
    l = l * alpha + pr;
    m = mnew;
#pragma unroll
    for (int i = 0; i < QD; ++i) {
      const float v = live ? vc[off + i] : 0.f;
      o[i] = o[i] * alpha + pr * v;
    }
  }
  // sum over the 16 token lanes
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) {
    l += shfl_xor(l, msk);
#pragma unroll
    for (int i = 0; i < QD; ++i) o[i] += shfl_xor(o[i], msk);
  }
  if (t == 0) {
    if (b0 == 0 && b1 == nb) {
      float* op = reinterpret_cast<float*>(p.out) + ((size_t)row * p.num_q_heads + h) * D + quarter * QD;
#pragma unroll
      for (int i = 0; i < QD; ++i) op[i] = o[i] / l;
    } else {
      const size_t pi = (size_t)(split + s) * p.num_q_heads + h;
#pragma unroll
      for (int i = 0; i < QD; ++i) p.part_o[pi * D + quarter * QD + i] = o[i];
      if (quarter == 0) {
        p.part_m[pi] = m;
        p.part_l[pi] = l;
      }
    }
  }
}

template <int D>
__global__ void __launch_bounds__(64) decode_f32_kernel(DecodeParams p) {
  const int split = blockIdx.x, h = blockIdx.y;
  for_each_piece(p, split, [&](int s, int b0, int b1, int nb) {
    if (h == 0 && threadIdx.x == 0) note_piece(p, split, s, b0, b1, nb);
    decode_f32_piece<D>(p, split, h, s, b0, b1, nb);
  });
}

// Log-sum-exp merge of the pieces of a sequence: one wave per (q head,
// sequence), four per work-group, lanes over d.  Pieces of sequence s come
// from shares first..last and have ids share + s; the merge runs online over
// them (running maximum, weight sum and output), so the loads of later pieces
// do not wait for earlier ones.  Sequences held by a single share were
// finished in place.
// Store role of the merge launch (p.store_chunk_rows, a mixed step that also stores its new K/V):
// work-group x (past the merge's num_seqs) stores new rows 8x .. 8x+7 of the flattened batch at
// their slots, as the KV write does, for the rows of sequences with q_len > 1 (the decode waves
// stored the others); kv heads y, y + gridDim.y, ...  Every reader of those rows in the launch
// before took them from the input rows.  Lane (row j = tid / 32, tensor tid / 16 % 2, chunk tid % 16).
template <int D>
__device__ __forceinline__ void store_chunk_rows(const DecodeParams& p, int x) {
  constexpr int kRowChunks = D * 2 / 16;
  const int tid = threadIdx.x;
  const int t = 8 * x + (tid >> 5), chunk = tid & 15;
  const bool is_v = (tid >> 4) & 1;
  if (t >= p.num_rows || chunk >= kRowChunks) return;
  int lo = 0, hi = p.num_seqs - 1;  // the last sequence s with qsl[s] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int s = lo, q0 = p.qsl[s], q_len = p.qsl[s + 1] - q0;
  if (q_len <= 1) return;
  const int pos = p.seq_lens[s] - q_len + (t - q0);
  const int phys = p.block_tables[(size_t)s * p.bt_stride + (pos >> 4)];
  if (phys < 0 || phys >= p.num_blocks) return;
  const uint8_t* src = reinterpret_cast<const uint8_t*>(is_v ? p.new_v : p.new_k) +
                       (size_t)t * (is_v ? p.new_v_stride : p.new_k_stride) * 2 + chunk * 16;
  uint8_t* dst = reinterpret_cast<uint8_t*>(const_cast<void*>(is_v ? p.value_cache : p.key_cache)) +
                 ((size_t)phys * 16 + (pos & 15)) * p.num_kv_heads * D * 2 + chunk * 16;
  for (int kvh = blockIdx.y; kvh < p.num_kv_heads; kvh += gridDim.y)
    *reinterpret_cast<u32x4*>(dst + (size_t)kvh * D * 2) = *reinterpret_cast<const u32x4*>(src + (size_t)kvh * D * 2);
}

template <int D>
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeParams p) {
  constexpr int PER_LANE = D / 64;
  if ((int)blockIdx.x >= p.num_seqs) {
    store_chunk_rows<D>(p, blockIdx.x - p.num_seqs);
    return;
  }
  if (p.n_splits <= 1 && !p.force_partial) return;  // a launch for the stores alone
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + wave, s = blockIdx.x;  // sequences on x: no 65535 limit on the batch
  if (h >= p.num_q_heads) return;
  // the piece range is read beside the length (one memory round trip, not two); it is only
  // meaningful when the sequence has pieces of its own
  const int pf = p.piece_first[s], pl = p.piece_last[s];
  const bool own = decode_blocks(p, s) > 0;  // the sequence has pieces of its own
  if (!own && p.prefix_shares == 0) return;
  const int first = own ? pf : 0, last = own ? pl : -1;
  if (first >= last && !p.force_partial) return;  // finished in place
  const int row = p.qsl ? p.qsl[s] : s;
  const size_t step = (size_t)p.num_q_heads;
  float M = -INFINITY, den = 0.f, o[PER_LANE];
#pragma unroll
  for (int k = 0; k < PER_LANE; ++k) o[k] = 0.f;
  auto fold = [&](const float* po, float mi, float li) {
    float src[PER_LANE];
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) src[k] = po[lane * PER_LANE + k];
    const float Mn = fmaxf(M, mi);
    const float a = fast_exp2(M - Mn), b = fast_exp2(mi - Mn);
    den = den * a + li * b;
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) o[k] = o[k] * a + src[k] * b;
    M = Mn;
  };
  // cascade: the prefix pieces of (s, h) first
  for (int i = 0; i < p.prefix_shares; ++i) {
    const size_t pi = ((size_t)i * p.num_seqs + s) * step + h;
    fold(p.pre_o + pi * D, p.pre_m[pi], p.pre_l[pi]);
  }
  const size_t base = (size_t)(first + s) * step + h;  // piece i: base + i * num_q_heads
#pragma unroll 4
  for (int i = 0; i <= last - first; ++i) {
    const size_t pi = base + i * step;
    fold(p.part_o + pi * D, p.part_m[pi], p.part_l[pi]);
  }
  const float inv = p.v_scale / den;
  const size_t oi = ((size_t)row * p.num_q_heads + h) * D + lane * PER_LANE;
  if (p.q_f32) {
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) reinterpret_cast<float*>(p.out)[oi + k] = o[k] * inv;
  } else if constexpr (PER_LANE == 1) {
    reinterpret_cast<uint16_t*>(p.out)[oi] = f32_to_bf16(o[0] * inv);
  } else {
#pragma unroll
    for (int k = 0; k < PER_LANE; k += 2)
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(p.out) + oi + k) = pack_bf16x2(o[k] * inv, o[k + 1] * inv);
  }
}

template <int D>
hipError_t launch_merge_d(const DecodeParams& p, hipStream_t stream) {
  timing_mark(kKDecodeMerge, true, stream);
  const int store_wgs = p.store_chunk_rows ? (p.num_rows + 7) / 8 : 0;
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(p.num_seqs + store_wgs, (p.num_q_heads + 3) / 4), dim3(256), 0,
                     stream, p);
  timing_mark(kKDecodeMerge, false, stream);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, int kv, hipStream_t stream) {
  timing_mark(kKDecode, true, stream);
  if (kv == kF32) {
    hipLaunchKernelGGL(decode_f32_kernel<D>, dim3(p.n_splits, p.num_q_heads), dim3(64), 0, stream, p);
  } else {
    const dim3 grid(p.prefix_waves + p.n_splits, p.num_kv_heads * p.head_groups);
    if (kv == kFP8 && p.new_k)
      hipLaunchKernelGGL((decode_mfma_kernel<D, true, true>), grid, dim3(64), 0, stream, p);
    else if (kv == kFP8)
      hipLaunchKernelGGL((decode_mfma_kernel<D, true, false>), grid, dim3(64), 0, stream, p);
    else if (p.new_k)
      hipLaunchKernelGGL((decode_mfma_kernel<D, false, true>), grid, dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<D, false, false>), grid, dim3(64), 0, stream, p);
  }
  timing_mark(kKDecode, false, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (p.n_splits <= 1 && !p.force_partial) || p.num_seqs == 0) return e;
  return launch_merge_d<D>(p, stream);
}

}  // namespace

// Scratch of the decode entry point that allocates nothing (pa_decode_static): a
// file-scope device array, one copy per GPU at its own address, held until the process
// ends.  Host code never passes the array's name (a host-side stand-in) to a kernel: it
// looks up the device address once per device, with that device current, and passes that.
// Nothing in it needs to start at zero: the merge reads only what the decode launch before
// it wrote.  Calls that overlap on one GPU share the array and race.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {

// One wave per (token t, q head h) of a flattened batch, fp32 queries and output; fp32 pools or
// E4M3 codes (exact in fp32; k_scale is in scale_log2, v_scale applied at the end).  Lane =
// (key t16 = lane % 16 of a block, quarter = lane / 16 holding D/4 elements of a row), as in
// the fp32 decode.  The token finds its sequence by binary search over query_start_loc.
template <int D, bool FP8>
__global__ void __launch_bounds__(64) rows_f32_kernel(DecodeParams p) {
  constexpr int QD = D / 4;
  const int t = blockIdx.x, h = blockIdx.y;
  int lo = 0, hi = p.num_seqs - 1;  // the last sequence s with qsl[s] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const int q_len = p.qsl[s + 1] - p.qsl[s];
  const int L = p.seq_lens[s] - q_len + (t - p.qsl[s]) + 1;  // keys 0 .. L-1 (causal)
  const int skip = decode_skip(p, L);
  const int key_lo = decode_first_key(p, L);
  const int nblk = (L + 15) / 16 - skip;
  const int lane = threadIdx.x;
  const int t16 = lane & 15, quarter = lane >> 4;
  const int kvh = h / p.group;

  float q[QD];
  const float* qp = reinterpret_cast<const float*>(p.query) + ((size_t)t * p.num_q_heads + h) * D + quarter * QD;
#pragma unroll
  for (int i = 0; i < QD; ++i) q[i] = qp[i];
  float o[QD];
#pragma unroll
  for (int i = 0; i < QD; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int* bt = p.block_tables + (size_t)s * p.bt_stride + skip;
  for (int b = 0; b < nblk; ++b) {
    const int phys = min(max(bt[b], 0), p.num_blocks - 1);
    const int pos = (skip + b) * 16 + t16;
    const bool live = pos < L && pos >= key_lo;
    const size_t off = (((size_t)phys * 16 + t16) * p.num_kv_heads + kvh) * D + quarter * QD;
    float k[QD], v[QD];
    if constexpr (FP8) {
      const uint32_t* kc = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(p.key_cache) + off);
      const uint32_t* vc = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(p.value_cache) + off);
#pragma unroll
      for (int i = 0; i < QD / 4; ++i) {
        const u32x2 kw = e4m3x4_to_bf16x4(live ? kc[i] : 0u), vw = e4m3x4_to_bf16x4(live ? vc[i] : 0u);
        k[4 * i] = __uint_as_float(kw.x << 16);
        k[4 * i + 1] = __uint_as_float(kw.x & 0xFFFF0000u);
        k[4 * i + 2] = __uint_as_float(kw.y << 16);
        k[4 * i + 3] = __uint_as_float(kw.y & 0xFFFF0000u);
        v[4 * i] = __uint_as_float(vw.x << 16);
        v[4 * i + 1] = __uint_as_float(vw.x & 0xFFFF0000u);
        v[4 * i + 2] = __uint_as_float(vw.y << 16);
        v[4 * i + 3] = __uint_as_float(vw.y & 0xFFFF0000u);
      }
    } else {
      const float* kc = reinterpret_cast<const float*>(p.key_cache) + off;
      const float* vc = reinterpret_cast<const float*>(p.value_cache) + off;
#pragma unroll
      for (int i = 0; i < QD; ++i) {
        k[i] = live ? kc[i] : 0.f;
        v[i] = live ? vc[i] : 0.f;
      }
    }
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < QD; ++i) dot += q[i] * k[i];
    dot += shfl_xor(dot, 16);
    dot += shfl_xor(dot, 32);
    const float z = live ? dot * p.scale_log2 : -INFINITY;
    float bmax = z;
#pragma unroll
    for (int msk = 1; msk < 16; msk <<= 1) bmax = fmaxf(bmax, shfl_xor(bmax, msk));
    const float mnew = fmaxf(m, bmax);
    const float alpha = fast_exp2(m - mnew);
    const float pr = fast_exp2(z - mnew);
    l = l * alpha + pr;
    m = mnew;
#pragma unroll
    for (int i = 0; i < QD; ++i) o[i] = o[i] * alpha + pr * v[i];
  }
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) {
    l += shfl_xor(l, msk);
#pragma unroll
    for (int i = 0; i < QD; ++i) o[i] += shfl_xor(o[i], msk);
  }
  if (t16 == 0) {
    const float inv = p.v_scale / l;
    float* op = reinterpret_cast<float*>(p.out) + ((size_t)t * p.num_q_heads + h) * D + quarter * QD;
#pragma unroll
    for (int i = 0; i < QD; ++i) op[i] = o[i] * inv;
  }
}

}  // namespace

hipError_t launch_rows_f32(const DecodeParams& p, int kv, int head_dim, int num_tokens, hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  const dim3 grid(num_tokens, p.num_q_heads);
  timing_mark(kKDecode, true, stream);
  if (head_dim == 128 && kv == kFP8)
    hipLaunchKernelGGL((rows_f32_kernel<128, true>), grid, dim3(64), 0, stream, p);
  else if (head_dim == 128)
    hipLaunchKernelGGL((rows_f32_kernel<128, false>), grid, dim3(64), 0, stream, p);
  else if (kv == kFP8)
    hipLaunchKernelGGL((rows_f32_kernel<64, true>), grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((rows_f32_kernel<64, false>), grid, dim3(64), 0, stream, p);
  timing_mark(kKDecode, false, stream);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int kv, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return launch_decode_d<128>(p, kv, stream);
  return launch_decode_d<64>(p, kv, stream);
}

hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (((p.n_splits <= 1 && !p.force_partial) && !p.store_chunk_rows) || p.num_seqs == 0) return hipSuccess;
  if (head_dim == 128) return launch_merge_d<128>(p, stream);
  return launch_merge_d<64>(p, stream);
}

}  // namespace pa
