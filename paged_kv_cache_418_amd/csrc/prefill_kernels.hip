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
// gathered once for all of them.  Wave w owns rows 32w .. 32w+31, one
// 32-row matrix-core block.  K/V tiles of 64 keys (4 paged blocks) are gathered through the
// block table into a double-buffered LDS stage, K row-major (XOR-swizzled
// 16-byte chunks) and V transposed, with one barrier per tile; the next
// tile's global loads are in flight while the current tile is computed:
//   S^T[key][row] = K Q^T    v_mfma_f32_32x32x16_bf16 (K from LDS, Q in registers)
//   O^T[d][row]  += V^T P^T  v_mfma_f32_32x32x16_bf16 (P straight from the S^T registers)
// The running maximum is only moved when a row's new maximum exceeds it by
// more than 2^8 (the probabilities stay <= 256, exact enough in bf16), so the
// accumulators are rarely rescaled.  A work item may cover only a range of
// key tiles (a split of a long row tile); it then leaves (O, m, l) for the
// merge kernel, which combines the splits with the log-sum-exp rule.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

template <int D>
struct PrefillShape {
  static constexpr int kThreads = 512;                 // 8 waves x 32 rows = kPrefillRows rows
  static constexpr int kKeys = kPrefillKeys;           // keys per K/V tile
  static constexpr int kChunks = D / 8;                // 16-byte chunks of one pool row
  static constexpr int kKRowBytes = D * 2;             // one key of the K tile
  static constexpr int kKBytes = kKeys * kKRowBytes;
  // one d of the V^T tile, padded by 8 bytes: 34 dwords per row puts the 8-byte reads of
  // 32 consecutive rows on 32 distinct bank pairs
  static constexpr int kVRowBytes = kKeys * 2 + 8;
  static constexpr int kVBytes = D * kVRowBytes;
  static constexpr int kStageBytes = kKBytes + kVBytes;
  static constexpr int kKSteps = D / 16;               // 32x32x16 MFMAs over d
  static constexpr int kDTiles = D / 32;               // 32-wide d tiles of O^T
  static constexpr int kLoads = kKeys * kChunks / kThreads;  // 16-byte loads per thread per tile and tensor
};

__device__ __forceinline__ bf16x8 u4_to_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float max_halves(float x) {
  const uint32_t u = __float_as_uint(x);
  auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const uint32_t u = __float_as_uint(x);
  auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

template <int D>
__global__ void __launch_bounds__(512) prefill_kernel(PrefillParams p) {
  using Sh = PrefillShape<D>;
  constexpr int NL = Sh::kLoads;
  extern __shared__ __align__(16) unsigned char smem[];

  // ---- work item
  const uint64_t item = p.items[blockIdx.x];
  const int s = (int)(item & 0x7FFFu);
  const bool whole = (item >> 15) & 1u;
  const int rt = (int)((item >> 16) & 0xFFFFu);
  const int kt0 = (int)((item >> 32) & 0xFFFFu), kt1 = (int)(item >> 48);
  const int kvh = blockIdx.y;
  const int G = p.group;
  const int P = p.tile_positions;         // positions per row tile (rows = P * G <= 256)
  const int q0 = p.qsl[s];
  const int q_len = p.qsl[s + 1] - q0;
  const int L = p.seq_lens[s];
  const int c = L - q_len;
  const int pos0 = rt * P;
  const int pos_end = min(q_len, pos0 + P);  // positions of this tile: pos0 .. pos_end-1
  const int kv_end = c + pos_end;            // keys the last row sees (exclusive)

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, rl = lane & 31;

  // ---- the lane's row: R = 32*wave + rl -> (position pos0 + R / G, q head kvh*G + R % G)
  const int R = 32 * wave + rl;
  const bool row_ok = R < P * G && pos0 + R / G < pos_end;
  const int row_pos = c + pos0 + R / G;  // absolute position: keys <= it are visible
  // smallest and largest row position of the wave (masking and skipping whole tiles)
  const int wave_first = c + pos0 + (32 * wave) / G;
  const int wave_last = c + min(pos_end - 1, pos0 + (32 * wave + 31) / G);
  const bool wave_live = 32 * wave < P * G && pos0 + (32 * wave) / G < pos_end;

  // ---- Q^T operand: lane holds q[row rl][16*kk + 8*half .. +7]
  bf16x8 qf[Sh::kKSteps];
  {
    const int h = kvh * G + (R % G);
    const u32x4* qp = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.query) +
                                                     ((size_t)(q0 + (row_ok ? pos0 + R / G : 0)) * p.num_q_heads +
                                                      (row_ok ? h : 0)) * D + 8 * half);
#pragma unroll
    for (int kk = 0; kk < Sh::kKSteps; ++kk) qf[kk] = u4_to_bf16x8(row_ok ? qp[2 * kk] : u32x4{0u, 0u, 0u, 0u});
  }

  f32x16 acc[Sh::kDTiles];
#pragma unroll
  for (int n = 0; n < Sh::kDTiles; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
  float m_ref = -INFINITY, lsum = 0.f;

  // ---- loader role: thread = (chunk lc, key group lq); keys lq*NL .. lq*NL+NL-1
  const int lc = tid % Sh::kChunks, lq = tid / Sh::kChunks;
  const int* bt = p.block_tables + (size_t)s * p.bt_stride;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.key_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.value_cache);
  const size_t tok_stride = (size_t)p.num_kv_heads * D * 2;
  const size_t head_off = (size_t)kvh * D * 2 + (size_t)lc * 16;

  u32x4 kreg[NL], vreg[NL];
  auto gather = [&](int tile) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      // keys past the last visible one read key 0 (always present) and are replaced by zeros:
      // pool data there is never used, and zeros keep 0 * NaN out of the products
      const int key = tile * Sh::kKeys + lq * NL + i;
      const bool live = key < kv_end;
      const int k = live ? key : 0;
      int phys = bt[k >> 4];
      phys = min(max(phys, 0), p.num_blocks - 1);
      const size_t off = ((size_t)phys * 16 + (k & 15)) * tok_stride + head_off;
      const u32x4 kv = *reinterpret_cast<const u32x4*>(kbase + off);
      const u32x4 vv = *reinterpret_cast<const u32x4*>(vbase + off);
      const u32x4 zero = {0u, 0u, 0u, 0u};
      kreg[i] = live ? kv : zero;
      vreg[i] = live ? vv : zero;
    }
  };
  auto stage_write = [&](int stage) {
    unsigned char* kl = smem + stage * Sh::kStageBytes;
    unsigned char* vl = kl + Sh::kKBytes;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int key = lq * NL + i;
      *reinterpret_cast<u32x4*>(kl + key * Sh::kKRowBytes + ((lc ^ (key % Sh::kChunks)) << 4)) = kreg[i];
    }
    // V^T: element j of the chunk is d = 8*lc + j; the NL keys of this thread are adjacent in a V^T row
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      unsigned char* dst = vl + (8 * lc + j) * Sh::kVRowBytes + lq * NL * 2;
      if constexpr (NL == 2) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(vreg[1][j >> 1], vreg[0][j >> 1], sel);
      } else {
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)((j & 1) ? (vreg[0][j >> 1] >> 16) : (vreg[0][j >> 1] & 0xFFFFu));
      }
    }
  };

  gather(kt0);
  stage_write(0);
  __syncthreads();

  for (int tile = kt0; tile < kt1; ++tile) {
    const int st = (tile - kt0) & 1;
    if (tile + 1 < kt1) gather(tile + 1);
    const int key0 = tile * Sh::kKeys;
    const unsigned char* kl = smem + st * Sh::kStageBytes;
    const unsigned char* vl = kl + Sh::kKBytes;

    if (wave_live && key0 <= wave_last) {
      const bool need_mask = key0 + Sh::kKeys - 1 > wave_first;
      // two 32-key halves of the tile, each: S^T, online softmax, O^T += V^T P^T
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
        {
          const int key = kt * 32 + rl;
          const unsigned char* krow = kl + key * Sh::kKRowBytes;
#pragma unroll
          for (int kk = 0; kk < Sh::kKSteps; ++kk) {
            const bf16x8 a =
                u4_to_bf16x8(*reinterpret_cast<const u32x4*>(krow + (((2 * kk + half) ^ (key % Sh::kChunks)) << 4)));
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc, 0, 0, 0);
          }
        }
        // lane's entries: key key0 + kt*32 + 8*(r/4) + 4*half + r%4 of row rl.  Raw scores are
        // masked and maximised; the scale (> 0) is applied inside exp2(fma(s, scale, -m)).
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            sacc[r] = key <= row_pos ? sacc[r] : -INFINITY;
          }
        }
        float bmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, sacc[r]);
        bmax = max_halves(bmax) * p.scale_log2;
        // move the reference maximum only when it is exceeded by more than 8 (log2 units)
        const bool need = bmax > m_ref + 8.f;
        if (__any(need)) {
          const float mnew = need ? bmax : m_ref;
          const float alpha = (m_ref == -INFINITY) ? 0.f : fast_exp2(m_ref - mnew);
          lsum *= alpha;
#pragma unroll
          for (int n = 0; n < Sh::kDTiles; ++n) acc[n] *= alpha;
          m_ref = mnew;
        }
        const float msub = m_ref == -INFINITY ? 0.f : m_ref;
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(__builtin_fmaf(sacc[r], p.scale_log2, -msub));
          sacc[r] = pr;
          ps += pr;
        }
        lsum += ps;
        // O^T += V^T P^T over the two 16-key chunks of this half
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int ch = 2 * kt + cc, r0 = cc * 8;
          u32x4 pw;
#pragma unroll
          for (int j = 0; j < 4; ++j) pw[j] = pack_bf16x2(sacc[r0 + 2 * j], sacc[r0 + 2 * j + 1]);
          const bf16x8 pb = u4_to_bf16x8(pw);
          // logical k = 8*half + j  <->  key ch*16 + 8*(j/4) + 4*half + j%4
#pragma unroll
          for (int n = 0; n < Sh::kDTiles; ++n) {
            const unsigned char* vrow = vl + (n * 32 + rl) * Sh::kVRowBytes + (ch * 16 + 4 * half) * 2;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
            const bf16x8 va = u4_to_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
            acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc[n], 0, 0, 0);
          }
        }
      }
    }
    if (tile + 1 < kt1) stage_write(st ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  const float l = sum_halves(lsum);
  if (!row_ok) return;
  const int pos = pos0 + R / G, h = kvh * G + (R % G);
  // lane's outputs: d = n*32 + 8*(r/4) + 4*half + r%4
  if (whole) {
    const float inv = 1.f / l;
    uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + ((size_t)(q0 + pos) * p.num_q_heads + h) * D;
#pragma unroll
    for (int n = 0; n < Sh::kDTiles; ++n)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = n * 32 + 8 * rq + 4 * half;
        *reinterpret_cast<u32x2*>(op + d) = u32x2{pack_bf16x2(acc[n][4 * rq] * inv, acc[n][4 * rq + 1] * inv),
                                                  pack_bf16x2(acc[n][4 * rq + 2] * inv, acc[n][4 * rq + 3] * inv)};
      }
  } else {
    // partial result of a split row tile: slot (launch base + item) x kv head x row
    const size_t pi = ((size_t)(p.item_base + blockIdx.x) * p.num_kv_heads + kvh) * kPrefillRows + R;
    float* po = p.part_o + pi * D;
#pragma unroll
    for (int n = 0; n < Sh::kDTiles; ++n)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = n * 32 + 8 * rq + 4 * half;
        *reinterpret_cast<f32x4*>(po + d) = f32x4{acc[n][4 * rq], acc[n][4 * rq + 1], acc[n][4 * rq + 2], acc[n][4 * rq + 3]};
      }
    if (half == 0) {
      p.part_m[pi] = m_ref;
      p.part_l[pi] = l;
    }
  }
}

// Log-sum-exp merge of the splits of a row tile: grid (row tiles x 32 groups of
// 8 rows, kv heads), one wave per two rows, lanes over d (coalesced).  Splits
// of one row tile are consecutive items, so their slots are first .. first+n-1.
// The merge runs online over the splits (running maximum, weight sum and
// output), so the loads of later splits do not wait for earlier ones.
template <int D>
__global__ void __launch_bounds__(256) prefill_merge_kernel(PrefillMergeParams p) {
  constexpr int PER_LANE = D / 64;
  const uint64_t item = p.items[blockIdx.x >> 5];
  const int s = (int)(item & 0xFFFFu);
  const int rt = (int)((item >> 16) & 0xFFFFu);
  const int first = (int)((item >> 32) & 0xFFFFFu), n = (int)(item >> 52);
  const int kvh = blockIdx.y;
  const int G = p.group, P = p.tile_positions;
  const int q0 = p.qsl[s];
  const int q_len = p.qsl[s + 1] - q0;
  const int pos0 = rt * P;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t slot_step = (size_t)p.num_kv_heads * kPrefillRows;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int R = (blockIdx.x & 31) * 8 + wave * 2 + k;
    const int pos = pos0 + R / G;
    if (R >= P * G || pos >= q_len) continue;
    const size_t base = ((size_t)first * p.num_kv_heads + kvh) * kPrefillRows + R;
    float M = -INFINITY, den = 0.f, o[PER_LANE];
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) o[j] = 0.f;
#pragma unroll 4
    for (int i = 0; i < n; ++i) {
      const size_t pi = base + i * slot_step;
      const float mi = p.part_m[pi], li = p.part_l[pi];
      float src[PER_LANE];
#pragma unroll
      for (int j = 0; j < PER_LANE; ++j) src[j] = p.part_o[pi * D + lane * PER_LANE + j];
      if (mi == -INFINITY) continue;  // this split saw none of the row's keys
      const float Mn = fmaxf(M, mi);
      const float a = fast_exp2(M - Mn), b = fast_exp2(mi - Mn);
      den = den * a + li * b;
#pragma unroll
      for (int j = 0; j < PER_LANE; ++j) o[j] = o[j] * a + src[j] * b;
      M = Mn;
    }
    const float inv = 1.f / den;
    const int h = kvh * G + (R % G);
    uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + ((size_t)(q0 + pos) * p.num_q_heads + h) * D + lane * PER_LANE;
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) op[j] = f32_to_bf16(o[j] * inv);
  }
}

}  // namespace

size_t prefill_lds_bytes(int head_dim) {
  return head_dim == 128 ? 2 * PrefillShape<128>::kStageBytes : 2 * PrefillShape<64>::kStageBytes;
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(p.n_items, p.num_kv_heads);
  const size_t lds = prefill_lds_bytes(head_dim);
  timing_mark(kKPrefill, true, stream);
  if (head_dim == 128) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<128>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(prefill_kernel<128>, grid, dim3(PrefillShape<128>::kThreads), lds, stream, p);
  } else {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<64>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(PrefillShape<64>::kThreads), lds, stream, p);
  }
  timing_mark(kKPrefill, false, stream);
  return hipGetLastError();
}

hipError_t launch_prefill_merge(const PrefillMergeParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(p.n_items * 32, p.num_kv_heads);
  timing_mark(kKPrefillMerge, true, stream);
  if (head_dim == 128)
    hipLaunchKernelGGL(prefill_merge_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_merge_kernel<64>, grid, dim3(256), 0, stream, p);
  timing_mark(kKPrefillMerge, false, stream);
  return hipGetLastError();
}

}  // namespace pa
