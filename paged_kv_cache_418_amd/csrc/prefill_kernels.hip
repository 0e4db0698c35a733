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
// Tiling (tutorial 7 of the same page: tiling plus online softmax; the
// sliced-Q split is prior art, the CDNA4 mapping is our own): a work-group of
// 4 waves takes 128 query rows of one q head; wave w owns rows 32w..32w+31.
// K/V tiles of 64 keys (4 paged blocks) are gathered through the block table
// into LDS, K row-major and V transposed, and every wave runs
//   S^T[key][row] = K Q^T       v_mfma_f32_32x32x16_bf16 (K from LDS, Q in registers)
//   O^T[d][row]  += V^T P^T     v_mfma_f32_32x32x16_bf16 (P straight from the S^T registers)
// Each lane owns one query row, so the online-softmax statistics are
// lane-local plus one exchange between the two half-waves.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

template <int D>
struct PrefillShape {
  static constexpr int kKRow = D * 2 + 16;     // bytes per key row of the K tile
  static constexpr int kVRow = kPrefillKeys * 2 + 16;  // bytes per d row of the V^T tile
  static constexpr int kKBytes = kPrefillKeys * kKRow;
  static constexpr int kVBytes = D * kVRow;
  static constexpr int kKSteps = D / 16;       // 32x32x16 MFMAs per 32x32 score tile
  static constexpr int kDTiles = D / 32;       // 32-wide d tiles of the output
  static constexpr int kHalfD = D / 2;         // d elements of one half-wave's Q/K slices
};

__device__ __forceinline__ bf16x8 u4_to_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int D>
__global__ void __launch_bounds__(256) prefill_kernel(PrefillParams p) {
  using Sh = PrefillShape<D>;
  __shared__ __align__(16) unsigned char k_lds[Sh::kKBytes];
  __shared__ __align__(16) unsigned char v_lds[Sh::kVBytes];

  const uint32_t item = p.items[blockIdx.x];
  const int s = (int)(item >> 12), qt = (int)(item & 0xFFFu);
  const int h = blockIdx.y;
  const int kvh = h / p.group;
  const int q0 = p.qsl[s];
  const int q_len = p.qsl[s + 1] - q0;
  const int L = p.seq_lens[s];
  if (q_len < 1 || q0 + q_len > p.num_tokens || L < q_len) return;
  const int c = L - q_len;
  const int r_begin = qt * kPrefillRows;
  const int r_end = min(q_len, r_begin + kPrefillRows);
  const int kv_end = c + r_end;  // keys the last row of the tile sees

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = lane >> 5, rl = lane & 31;
  const int my_row = r_begin + wave * 32 + rl;           // row within the sequence
  const int my_pos = c + my_row;                         // its position
  const int wave_rows_end = min(r_end, r_begin + wave * 32 + 32);
  const int wave_kv_end = c + wave_rows_end;             // keys this wave needs (exclusive)
  const bool wave_live = r_begin + wave * 32 < r_end;

  // Q^T operand: lane holds q[row rl][half*D/2 + kk*8 + j]; K uses the same d order.
  bf16x8 qf[Sh::kKSteps];
  {
    const bool valid = my_row < r_end;
    const u32x4* qp = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.query) +
                                                     ((size_t)(q0 + (valid ? my_row : 0)) * p.num_q_heads + h) * D +
                                                     half * Sh::kHalfD);
#pragma unroll
    for (int kk = 0; kk < Sh::kKSteps; ++kk) {
      u32x4 t = valid ? qp[kk] : u32x4{0u, 0u, 0u, 0u};
      qf[kk] = u4_to_bf16x8(t);
    }
  }

  f32x16 acc[Sh::kDTiles];
#pragma unroll
  for (int n = 0; n < Sh::kDTiles; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int* bt = p.block_tables + (size_t)s * p.bt_stride;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.key_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.value_cache);
  const size_t tok_stride = (size_t)p.num_kv_heads * D * 2;
  const size_t head_off = (size_t)kvh * D * 2;

  // loader role: wave w copies d-quarter w of all 64 keys; lane = key
  const int ld_key = lane;
  const int ld_q = wave;
  constexpr int kQuarter = D / 4;  // elements per loader slice
  constexpr int kLdVecs = kQuarter * 2 / 16;

  const int n_tiles = (kv_end + kPrefillKeys - 1) / kPrefillKeys;
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int key0 = tile * kPrefillKeys;
    // ---- gather the tile into LDS
    {
      const int pos = key0 + ld_key;
      u32x4 kv[kLdVecs], vv[kLdVecs];
      if (pos < kv_end) {
        int phys = bt[min(pos >> 4, p.bt_stride - 1)];
        phys = min(max(phys, 0), p.num_blocks - 1);
        const size_t off = ((size_t)phys * 16 + (pos & 15)) * tok_stride + head_off + (size_t)ld_q * kQuarter * 2;
        const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + off);
        const u32x4* vp = reinterpret_cast<const u32x4*>(vbase + off);
#pragma unroll
        for (int i = 0; i < kLdVecs; ++i) {
          kv[i] = kp[i];
          vv[i] = vp[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < kLdVecs; ++i) kv[i] = vv[i] = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();  // previous tile fully consumed
      u32x4* kd = reinterpret_cast<u32x4*>(k_lds + ld_key * Sh::kKRow + ld_q * kQuarter * 2);
#pragma unroll
      for (int i = 0; i < kLdVecs; ++i) kd[i] = kv[i];
      uint16_t* vt = reinterpret_cast<uint16_t*>(v_lds);
#pragma unroll
      for (int i = 0; i < kLdVecs; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w = vv[i][e >> 1];
          const uint16_t x = (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xFFFFu);
          vt[(ld_q * kQuarter + i * 8 + e) * (Sh::kVRow / 2) + ld_key] = x;
        }
      __syncthreads();
    }
    if (!wave_live || key0 >= wave_kv_end) continue;

    // ---- scores for the two 32-key halves of the tile
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
      const unsigned char* krow = k_lds + (kt * 32 + rl) * Sh::kKRow + half * Sh::kHalfD * 2;
#pragma unroll
      for (int kk = 0; kk < Sh::kKSteps; ++kk) {
        const bf16x8 a = u4_to_bf16x8(*reinterpret_cast<const u32x4*>(krow + kk * 16));
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[kt], 0, 0, 0);
      }
    }
    // lane's entries: key = key0 + kt*32 + 8*(r/4) + 4*half + r%4, row = rl
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const float z = key <= my_pos ? sacc[kt][r] * p.scale_log2 : -INFINITY;
        sacc[kt][r] = z;
        bmax = fmaxf(bmax, z);
      }
    bmax = fmaxf(bmax, shfl_xor(bmax, 32));
    const float mnew = fmaxf(m, bmax);
    // rows with nothing visible yet keep m = -inf; guard the -inf - -inf case
    const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m - mnew);
    const float msub = (mnew == -INFINITY) ? 0.f : mnew;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(sacc[kt][r] - msub);
        sacc[kt][r] = pr;
        psum += pr;
      }
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int n = 0; n < Sh::kDTiles; ++n) acc[n] *= alpha;

    // ---- O^T += V^T P^T over four 16-key chunks
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int kt = ch >> 1, r0 = (ch & 1) * 8;
      u32x4 pw;
#pragma unroll
      for (int j = 0; j < 4; ++j) pw[j] = pack_bf16x2(sacc[kt][r0 + 2 * j], sacc[kt][r0 + 2 * j + 1]);
      const bf16x8 pb = u4_to_bf16x8(pw);
      // logical k = 8*half + j  <->  key ch*16 + 8*(j/4) + 4*half + j%4
#pragma unroll
      for (int n = 0; n < Sh::kDTiles; ++n) {
        const unsigned char* vrow = v_lds + (n * 32 + rl) * Sh::kVRow + (ch * 16 + 4 * half) * 2;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
        const u32x4 va = {lo.x, lo.y, hi.x, hi.y};
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(u4_to_bf16x8(va), pb, acc[n], 0, 0, 0);
      }
    }
  }

  if (!wave_live) return;
  l += shfl_xor(l, 32);
  if (my_row >= r_end) return;
  const float inv = 1.f / l;
  uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + ((size_t)(q0 + my_row) * p.num_q_heads + h) * D;
  // lane's outputs: d = n*32 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int n = 0; n < Sh::kDTiles; ++n)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d = n * 32 + 8 * rq + 4 * half;
      u32x2 w = {pack_bf16x2(acc[n][4 * rq] * inv, acc[n][4 * rq + 1] * inv),
                 pack_bf16x2(acc[n][4 * rq + 2] * inv, acc[n][4 * rq + 3] * inv)};
      *reinterpret_cast<u32x2*>(op + d) = w;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(p.n_items, p.num_q_heads);
  timing_mark(kKPrefill, true, stream);
  if (head_dim == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(256), 0, stream, p);
  timing_mark(kKPrefill, false, stream);
  return hipGetLastError();
}

}  // namespace pa
