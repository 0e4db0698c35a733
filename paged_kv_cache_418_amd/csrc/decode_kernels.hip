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
// Work decomposition (designed for CDNA4, not taken from the pages): one
// work-group of 4 waves per (partition, kv head, sequence).  The q heads that
// share the kv head (GQA, tutorial 1) are the 16 columns of the matrix-core
// tiles, so the K/V of a block are read once for all of them:
//   S^T[token][g] = K[token][:] . Q[g][:]   v_mfma_f32_16x16x32_bf16, K from HBM
//   O^T[d][g]    += V^T[d][token] P^T[token][g]   v_mfma_f32_16x16x16_bf16
// The score layout of the first product is exactly the operand layout the
// second one needs for P, so probabilities never leave registers; V is
// transposed through a per-wave LDS tile.  Each wave streams its share of
// the partition's 16-token blocks with the next block's loads in flight.
// Masked positions (the partly filled last block) are removed by selection,
// never by multiplying with zero, so NaN in unused pool slots cannot leak.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct DecodeShape {
  static constexpr int kKSteps = D / 32;   // 16x16x32 MFMAs per score tile
  static constexpr int kOTiles = D / 16;   // 16-wide d tiles of the output
  static constexpr int kLaneD = D / 4;     // elements of one token row held by one lane
  static constexpr int kVRow = D * 2 + 16;  // bytes per token row of the LDS V tile (padded, 16-aligned)
  static constexpr int kStage = kDecodeWaves * 16 * kVRow;
};

// Raw bytes of one lane's slice of a K or V token row: kLaneD elements.
template <int D, bool FP8>
struct RowSlice {
  static constexpr int kBytes = FP8 ? D / 4 : D / 2;
  static constexpr int kVecs = kBytes / 16;
  u32x4 v[kVecs];
};

template <int D, bool FP8>
__device__ __forceinline__ void load_slice(RowSlice<D, FP8>& r, const uint8_t* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < RowSlice<D, FP8>::kVecs; ++i) r.v[i] = q[i];
}

// Slice -> bf16 words: kLaneD/2 dwords, element order preserved.
template <int D, bool FP8>
__device__ __forceinline__ void slice_to_bf16(const RowSlice<D, FP8>& r, uint32_t (&w)[D / 8]) {
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < RowSlice<D, FP8>::kVecs; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        u32x2 b = e4m3x4_to_bf16x4(r.v[i][k]);
        w[i * 8 + k * 2] = b.x;
        w[i * 8 + k * 2 + 1] = b.y;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < RowSlice<D, FP8>::kVecs; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) w[i * 4 + k] = r.v[i][k];
    }
  }
}

__device__ __forceinline__ bf16x8 words_to_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 t = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, t);
}

template <int D, bool FP8>
__global__ void __launch_bounds__(256) decode_mfma_kernel(DecodeParams p) {
  using Sh = DecodeShape<D>;
  extern __shared__ __align__(16) unsigned char smem[];

  const int s = blockIdx.z, kvh = blockIdx.y, part = blockIdx.x;
  int row = s;
  if (p.qsl) {
    const int a = p.qsl[s], b = p.qsl[s + 1];
    if (b - a != 1) return;
    row = a;
  }
  if (row >= p.num_rows) return;
  const int L = min(p.seq_lens[s], p.max_seq_len);
  const int tok0 = part * p.part_size;
  if (tok0 >= L) return;
  const int n_parts = (L + p.part_size - 1) / p.part_size;
  const int tok1 = min(L, tok0 + p.part_size);
  const int nblk = (tok1 - tok0 + 15) >> 4;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane & 15, grp = lane >> 4;
  const int G = p.group;

  // Q^T operand: lane holds q[head g][grp*D/4 + kk*8 + j]; the same d order is
  // used for K, so the dot products are unchanged.
  bf16x8 qf[Sh::kKSteps];
  {
    uint32_t qw[D / 8];
    if (g < G) {
      const size_t qoff = ((size_t)row * p.num_q_heads + kvh * G + g) * D + grp * Sh::kLaneD;
      if (p.q_f32) {
        const float* qp = reinterpret_cast<const float*>(p.query) + qoff;
#pragma unroll
        for (int i = 0; i < D / 8; ++i) qw[i] = pack_bf16x2(qp[2 * i], qp[2 * i + 1]);
      } else {
        const u32x4* qp = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.query) + qoff);
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
          const u32x4 t = qp[i];
          qw[4 * i] = t.x;
          qw[4 * i + 1] = t.y;
          qw[4 * i + 2] = t.z;
          qw[4 * i + 3] = t.w;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < D / 8; ++i) qw[i] = 0u;
    }
#pragma unroll
    for (int kk = 0; kk < Sh::kKSteps; ++kk)
      qf[kk] = words_to_bf16x8(qw[4 * kk], qw[4 * kk + 1], qw[4 * kk + 2], qw[4 * kk + 3]);
  }

  float m = -INFINITY, l = 0.f;
  f32x4 acc[Sh::kOTiles];
#pragma unroll
  for (int n = 0; n < Sh::kOTiles; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int* bt = p.block_tables + (size_t)s * p.bt_stride + (tok0 >> 4);
  unsigned char* vstage = smem + wave * 16 * Sh::kVRow;
  const int tl = lane & 15;  // token row this lane loads
  constexpr int kElem = FP8 ? 1 : 2;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.key_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.value_cache);
  const size_t lane_off = (size_t)(grp * Sh::kLaneD) * kElem;
  const size_t row_stride = (size_t)p.num_kv_heads * D * kElem;  // bytes between tokens of a block
  const size_t head_off = (size_t)kvh * D * kElem;

  auto slice_addr = [&](const uint8_t* base, int b) {
    int phys = bt[b];
    phys = min(max(phys, 0), p.num_blocks - 1);
    return base + ((size_t)phys * 16 + tl) * row_stride + head_off + lane_off;
  };

  RowSlice<D, FP8> kcur, vcur, knext, vnext;
  int b = wave;
  if (b < nblk) {
    load_slice(kcur, slice_addr(kbase, b));
    load_slice(vcur, slice_addr(vbase, b));
  }
  for (; b < nblk; b += kDecodeWaves) {
    const int bn = b + kDecodeWaves;
    if (bn < nblk) {
      load_slice(knext, slice_addr(kbase, bn));
      load_slice(vnext, slice_addr(vbase, bn));
    }
    const int blk_tok = tok0 + b * 16;

    // V slice -> LDS (zero rows past the sequence end)
    {
      uint32_t vw[D / 8];
      slice_to_bf16(vcur, vw);
      const bool live = blk_tok + tl < L;
      u32x4* dst = reinterpret_cast<u32x4*>(vstage + tl * Sh::kVRow + grp * Sh::kLaneD * 2);
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        u32x4 t = {vw[4 * i], vw[4 * i + 1], vw[4 * i + 2], vw[4 * i + 3]};
        if (!live) t = u32x4{0u, 0u, 0u, 0u};
        dst[i] = t;
      }
    }

    // scores S^T[token 4*grp+i][head g]
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    {
      uint32_t kw[D / 8];
      slice_to_bf16(kcur, kw);
#pragma unroll
      for (int kk = 0; kk < Sh::kKSteps; ++kk) {
        bf16x8 a = words_to_bf16x8(kw[4 * kk], kw[4 * kk + 1], kw[4 * kk + 2], kw[4 * kk + 3]);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], sacc, 0, 0, 0);
      }
    }

    float z[4];
    float bmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool live = blk_tok + grp * 4 + i < L;
      z[i] = live ? sacc[i] * p.scale_log2 : -INFINITY;
      bmax = fmaxf(bmax, z[i]);
    }
    bmax = fmaxf(bmax, shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, shfl_xor(bmax, 32));
    const float mnew = fmaxf(m, bmax);
    const float alpha = fast_exp2(m - mnew);
    float pr[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = fast_exp2(z[i] - mnew);
      psum += pr[i];
    }
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int n = 0; n < Sh::kOTiles; ++n) acc[n] *= alpha;

    i16x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = (short)f32_to_bf16(pr[i]);

    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const uint16_t* vs = reinterpret_cast<const uint16_t*>(vstage);
#pragma unroll
    for (int n = 0; n < Sh::kOTiles; ++n) {
      i16x4 va;
#pragma unroll
      for (int j = 0; j < 4; ++j) va[j] = (short)vs[(grp * 4 + j) * (Sh::kVRow / 2) + n * 16 + g];
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[n], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();

    kcur = knext;
    vcur = vnext;
  }

  // the four lanes of a head hold partial sums over different tokens
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);

  // combine the waves of the work-group
  __syncthreads();
  float* sm_m = reinterpret_cast<float*>(smem);
  float* sm_l = sm_m + kDecodeWaves * 16;
  float* sm_o = sm_l + kDecodeWaves * 16;  // [wave][g < G][D]
  if (grp == 0) {
    sm_m[wave * 16 + g] = m;
    sm_l[wave * 16 + g] = l;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, sm_m[w * 16 + g]);
  const float f = fast_exp2(m - M);
  if (g < G) {
#pragma unroll
    for (int n = 0; n < Sh::kOTiles; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_o[(wave * G + g) * D + n * 16 + grp * 4 + r] = acc[n][r] * f;
  }
  __syncthreads();

  const bool single = n_parts == 1;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int gg = idx / D, d = idx - gg * D;
    float Mg = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) Mg = fmaxf(Mg, sm_m[w * 16 + gg]);
    float Lg = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      Lg += sm_l[w * 16 + gg] * fast_exp2(sm_m[w * 16 + gg] - Mg);
      o += sm_o[(w * G + gg) * D + d];
    }
    const int h = kvh * G + gg;
    if (single) {
      const float val = o * p.v_scale / Lg;
      const size_t oi = ((size_t)row * p.num_q_heads + h) * D + d;
      if (p.q_f32)
        reinterpret_cast<float*>(p.out)[oi] = val;
      else
        reinterpret_cast<uint16_t*>(p.out)[oi] = f32_to_bf16(val);
    } else {
      const size_t pi = ((size_t)s * p.num_q_heads + h) * p.n_parts_max + part;
      p.part_o[pi * D + d] = o;
      if (d == 0) {
        p.part_m[pi] = Mg;
        p.part_l[pi] = Lg;
      }
    }
  }
}

// fp32 pools and queries: vector-ALU kernel, one wave per (partition, q head, sequence).
// Lane = (token t = lane % 16, quarter = lane / 16) holding D/4 elements of a row.
template <int D>
__global__ void __launch_bounds__(64) decode_f32_kernel(DecodeParams p) {
  constexpr int QD = D / 4;
  const int s = blockIdx.z, h = blockIdx.y, part = blockIdx.x;
  int row = s;
  if (p.qsl) {
    const int a = p.qsl[s], b = p.qsl[s + 1];
    if (b - a != 1) return;
    row = a;
  }
  if (row >= p.num_rows) return;
  const int L = min(p.seq_lens[s], p.max_seq_len);
  const int tok0 = part * p.part_size;
  if (tok0 >= L) return;
  const int n_parts = (L + p.part_size - 1) / p.part_size;
  const int tok1 = min(L, tok0 + p.part_size);
  const int nblk = (tok1 - tok0 + 15) >> 4;
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
  const int* bt = p.block_tables + (size_t)s * p.bt_stride + (tok0 >> 4);
  const float* kc = reinterpret_cast<const float*>(p.key_cache);
  const float* vc = reinterpret_cast<const float*>(p.value_cache);

  for (int b = 0; b < nblk; ++b) {
    int phys = bt[b];
    phys = min(max(phys, 0), p.num_blocks - 1);
    const int pos = tok0 + b * 16 + t;
    const bool live = pos < L;
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
    if (n_parts == 1) {
      float* op = reinterpret_cast<float*>(p.out) + ((size_t)row * p.num_q_heads + h) * D + quarter * QD;
#pragma unroll
      for (int i = 0; i < QD; ++i) op[i] = o[i] / l;
    } else {
      const size_t pi = ((size_t)s * p.num_q_heads + h) * p.n_parts_max + part;
#pragma unroll
      for (int i = 0; i < QD; ++i) p.part_o[pi * D + quarter * QD + i] = o[i];
      if (quarter == 0) {
        p.part_m[pi] = m;
        p.part_l[pi] = l;
      }
    }
  }
}

// Log-sum-exp merge of partition partials: one work-group of 256 threads per
// (q head, sequence); the 4 waves take every 4th partition, then combine.
template <int D>
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeParams p) {
  constexpr int PER_LANE = D / 64;
  __shared__ float red_m[4], red_l[4];
  __shared__ float red_o[4][D];
  const int s = blockIdx.y, h = blockIdx.x;
  int row = s;
  if (p.qsl) {
    const int a = p.qsl[s], b = p.qsl[s + 1];
    if (b - a != 1) return;
    row = a;
  }
  if (row >= p.num_rows) return;
  const int L = min(p.seq_lens[s], p.max_seq_len);
  const int n_parts = (L + p.part_size - 1) / p.part_size;
  if (n_parts <= 1) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t base = ((size_t)s * p.num_q_heads + h) * p.n_parts_max;

  float M = -INFINITY;
  for (int i = threadIdx.x; i < n_parts; i += blockDim.x) M = fmaxf(M, p.part_m[base + i]);
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) M = fmaxf(M, shfl_xor(M, msk));
  if (lane == 0) red_m[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

  float o[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) o[i] = 0.f;
  float den = 0.f;
#pragma unroll 4
  for (int pi = wave; pi < n_parts; pi += 4) {
    const float w = fast_exp2(p.part_m[base + pi] - M);
    den += w * p.part_l[base + pi];
    const float* src = p.part_o + (base + pi) * D + lane * PER_LANE;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) o[i] += w * src[i];
  }
  if (lane == 0) red_l[wave] = den;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) red_o[wave][lane * PER_LANE + i] = o[i];
  __syncthreads();
  if (wave == 0) {
    const float dsum = red_l[0] + red_l[1] + red_l[2] + red_l[3];
    const float inv = p.v_scale / dsum;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int d = lane * PER_LANE + i;
      const float val = (red_o[0][d] + red_o[1][d] + red_o[2][d] + red_o[3][d]) * inv;
      const size_t oi = ((size_t)row * p.num_q_heads + h) * D + d;
      if (p.q_f32)
        reinterpret_cast<float*>(p.out)[oi] = val;
      else
        reinterpret_cast<uint16_t*>(p.out)[oi] = f32_to_bf16(val);
    }
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, int kv, hipStream_t stream) {
  const dim3 grid(p.n_parts_max, kv == kF32 ? p.num_q_heads : p.num_kv_heads, p.num_seqs);
  if (kv == kF32) {
    hipLaunchKernelGGL(decode_f32_kernel<D>, grid, dim3(64), 0, stream, p);
  } else {
    using Sh = DecodeShape<D>;
    const size_t merge_bytes = (size_t)(2 * kDecodeWaves * 16 + kDecodeWaves * p.group * D) * sizeof(float);
    const size_t lds = merge_bytes > (size_t)Sh::kStage ? merge_bytes : (size_t)Sh::kStage;
    if (kv == kFP8)
      hipLaunchKernelGGL((decode_mfma_kernel<D, true>), grid, dim3(256), lds, stream, p);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<D, false>), grid, dim3(256), lds, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_parts_max <= 1) return e;
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(p.num_q_heads, p.num_seqs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int kv, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return launch_decode_d<128>(p, kv, stream);
  return launch_decode_d<64>(p, kv, stream);
}

}  // namespace pa
