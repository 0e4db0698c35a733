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
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

template <int D>
struct PrefillShape {
  static constexpr int kThreads = 512;                 // 8 waves x 32 rows = kPrefillRows rows
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kKeys = kPrefillKeys;           // keys per K/V tile
  static constexpr int kRowBytes = D * 2;              // one key row of a tile
  static constexpr int kChunks = kRowBytes / 16;       // 16-byte chunks per row (the swizzle period)
  static constexpr int kTileBytes = kKeys * kRowBytes; // one tensor of one tile
  static constexpr int kStageBytes = 2 * kTileBytes;   // K then V
  static constexpr int kStages = 4;
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;           // rows one wave-wide 1 KB copy fills
  static constexpr int kCopies = kTileBytes / 1024 / kWaves;      // copies per wave per tensor per tile
  static constexpr int kKSteps = D / 16;               // 32x32x16 MFMAs over d
  static constexpr int kDTiles = D / 32;               // 32-wide d tiles of O^T
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

typedef short i16x4_t __attribute__((ext_vector_type(4)));
#define PA_LDS __attribute__((address_space(3)))
#define PA_GLOBAL __attribute__((address_space(1)))

// Waits until at most n vector-memory instructions of this wave are outstanding
// (s_waitcnt with only the vmcnt field active; gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int D>
__global__ void __launch_bounds__(512) prefill_kernel(PrefillParams p) {
  using Sh = PrefillShape<D>;
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

  // ---- copy role: each wave copies kCopies 1 KB slabs of K and of V per tile.  Slab
  // kCopies*wave + i holds rows kRowsPerCopy*(kCopies*wave + i) ...; lane = (row in slab,
  // physical chunk); the chunk it fetches is the logical chunk stored in that slot,
  // physical ^ (row % kChunks).  All rows of a wave's slabs lie in one paged block.
  const int* bt = p.block_tables + (size_t)s * p.bt_stride;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.key_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.value_cache);
  const size_t tok_stride = (size_t)p.num_kv_heads * D * 2;
  const int lanes_per_row = Sh::kChunks;
  const int copy_row0 = Sh::kRowsPerCopy * Sh::kCopies * wave;  // first row of this wave's slabs
  const int bt0 = min(max(bt[0], 0), p.num_blocks - 1);          // block of key 0 (always written)
  auto block_of = [&](int tile) {  // physical block of this wave's rows of a tile
    const int key = tile * Sh::kKeys + copy_row0;
    return key < kv_end ? bt[key >> 4] : bt0;
  };
  // Rows past the last visible key copy the row of key 0 (written and finite): their
  // scores are masked and their probabilities are 0, so pool data there is never used.
  auto copy_tile = [&](int tile, int phys, int stage) {
    phys = min(max(phys, 0), p.num_blocks - 1);
    unsigned char* st = smem + stage * Sh::kStageBytes;
#pragma unroll
    for (int i = 0; i < Sh::kCopies; ++i) {
      const int row = copy_row0 + Sh::kRowsPerCopy * i + lane / lanes_per_row;
      const int slot = lane % lanes_per_row;
      const int chunk = slot ^ (row % Sh::kChunks);
      const int key = tile * Sh::kKeys + row;
      const bool live = key < kv_end;
      const int ph = live ? phys : bt0;
      const size_t off = ((size_t)ph * 16 + (live ? (key & 15) : 0)) * tok_stride + (size_t)kvh * D * 2 + chunk * 16;
      unsigned char* dst = st + (copy_row0 + Sh::kRowsPerCopy * i) * Sh::kRowBytes;
      __builtin_amdgcn_global_load_lds((const void PA_GLOBAL*)(kbase + off), (void PA_LDS*)dst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void PA_GLOBAL*)(vbase + off), (void PA_LDS*)(dst + Sh::kTileBytes), 16,
                                       0, 0);
    }
  };

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

  // S^T for both 32-key halves of a tile from an LDS stage: two independent MFMA chains.
  auto scores = [&](f32x16 (&sacc)[2], int stage) {
    const unsigned char* kl = smem + stage * Sh::kStageBytes;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < Sh::kKSteps; ++kk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = kt * 32 + rl;
        const bf16x8 a = u4_to_bf16x8(
            *reinterpret_cast<const u32x4*>(kl + key * Sh::kRowBytes + (((2 * kk + half) ^ (key % Sh::kChunks)) << 4)));
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[kt], 0, 0, 0);
      }
    }
  };

  // V^T operands of O^T += V^T P^T for the 16-key chunk ch, all d tiles n: lane (d = 32n +
  // l%32, h = l/32) holds keys ch*16 + 4h + 0..3 and ch*16 + 8 + 4h + 0..3.  In each 16-lane
  // group, ds_read_b64_tr_b16 gives output lane i element k = element i%4 of the 8 bytes
  // addressed by lane 4k + i/4; so lane 4k + q addresses key kb + k, d 32n + 16*(group%2) + 4q.
  // The reads are issued from one asm block that also waits for them, so the compiler does
  // not hold them back behind the copies in flight (the barrier protocol already guarantees
  // that the stage read here has landed).
  const int tr_k = (lane & 15) >> 2, tr_q = lane & 3, tr_g = lane >> 4;
  auto v_operands = [&](const unsigned char* vl, int ch, bf16x8 (&ops)[Sh::kDTiles]) {
    uint32_t addr[Sh::kDTiles][2];
#pragma unroll
    for (int n = 0; n < Sh::kDTiles; ++n)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int key = ch * 16 + 8 * w + 4 * (tr_g >> 1) + tr_k;
        const int byte = (32 * n + 16 * (tr_g & 1) + 4 * tr_q) * 2;
        const int phys = (((byte >> 4) ^ (key % Sh::kChunks)) << 4) | (byte & 15);
        addr[n][w] = (uint32_t)(uintptr_t)(vl + key * Sh::kRowBytes + phys);
      }
    u32x2 part[Sh::kDTiles][2];
    if constexpr (Sh::kDTiles == 4) {
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n\t"
          "ds_read_b64_tr_b16 %1, %9\n\t"
          "ds_read_b64_tr_b16 %2, %10\n\t"
          "ds_read_b64_tr_b16 %3, %11\n\t"
          "ds_read_b64_tr_b16 %4, %12\n\t"
          "ds_read_b64_tr_b16 %5, %13\n\t"
          "ds_read_b64_tr_b16 %6, %14\n\t"
          "ds_read_b64_tr_b16 %7, %15\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(part[0][0]), "=&v"(part[0][1]), "=&v"(part[1][0]), "=&v"(part[1][1]), "=&v"(part[2][0]),
            "=&v"(part[2][1]), "=&v"(part[3][0]), "=&v"(part[3][1])
          : "v"(addr[0][0]), "v"(addr[0][1]), "v"(addr[1][0]), "v"(addr[1][1]), "v"(addr[2][0]), "v"(addr[2][1]),
            "v"(addr[3][0]), "v"(addr[3][1])
          : "memory");
    } else {
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4\n\t"
          "ds_read_b64_tr_b16 %1, %5\n\t"
          "ds_read_b64_tr_b16 %2, %6\n\t"
          "ds_read_b64_tr_b16 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(part[0][0]), "=&v"(part[0][1]), "=&v"(part[1][0]), "=&v"(part[1][1])
          : "v"(addr[0][0]), "v"(addr[0][1]), "v"(addr[1][0]), "v"(addr[1][1])
          : "memory");
    }
#pragma unroll
    for (int n = 0; n < Sh::kDTiles; ++n)
      ops[n] = __builtin_bit_cast(bf16x8, u32x4{part[n][0].x, part[n][0].y, part[n][1].x, part[n][1].y});
  };

  // Online softmax of one tile's scores and O^T += V^T P^T with V from an LDS stage.
  auto softmax_pv = [&](f32x16 (&sacc)[2], int key0, int stage) {
    const unsigned char* vl = smem + stage * Sh::kStageBytes + Sh::kTileBytes;
    // lane's entries: key key0 + kt*32 + 8*(r/4) + 4*half + r%4 of row rl.  Raw scores are
    // masked and maximised; the scale (> 0) is applied inside exp2(fma(s, scale, -m)).
    if (key0 + Sh::kKeys - 1 > wave_first) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          sacc[kt][r] = key <= row_pos ? sacc[kt][r] : -INFINITY;
        }
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, sacc[kt][r]);
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
    // per half: P = exp2(s*scale - m) packed to bf16, then O^T += V^T P^T over its two
    // 16-key chunks; the second half's exponentials overlap the first half's MFMAs
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      u32x4 pw[2];
      float ps = 0.f;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(__builtin_fmaf(sacc[kt][8 * cc + 2 * j], p.scale_log2, -msub));
          const float p1 = fast_exp2(__builtin_fmaf(sacc[kt][8 * cc + 2 * j + 1], p.scale_log2, -msub));
          ps += p0 + p1;
          pw[cc][j] = pack_bf16x2(p0, p1);
        }
      lsum += ps;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int ch = 2 * kt + cc;
        const bf16x8 pb = u4_to_bf16x8(pw[cc]);
        // logical k = 8*half + j  <->  key ch*16 + 8*(j/4) + 4*half + j%4
        bf16x8 va[Sh::kDTiles];
        v_operands(vl, ch, va);
#pragma unroll
        for (int n = 0; n < Sh::kDTiles; ++n)
          acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[n], pb, acc[n], 0, 0, 0);
      }
    }
  };

  // Pipeline over the item's key tiles t = kt0 .. kt1-1 (stage of tile t: (t - kt0) % 4).
  // Step t: read the block id of tile t+4, start the copy of tile t+3; the scores of tile
  // t+1 go to the matrix cores while the softmax of tile t runs, then O += V P for tile t;
  // finally wait for the copy of tile t+2 (started one step ago) and meet at a barrier.
  // Vector-memory instructions retire in order and the last ones a step issues are its
  // 2*kCopies copies, so "everything older than this step's copies has landed" is
  // vmcnt <= 2*kCopies.  Each block id is read before the copies of its step, so consuming
  // it never waits for copies still in flight.  Tiles past the item's range are copied too
  // (valid rows, never used) so that every step is alike.
  constexpr int kStepLoads = 2 * Sh::kCopies;
  const int wave_tiles_end = min(kt1, wave_last / Sh::kKeys + 1);  // tiles this wave computes
  {
    const int ph0 = block_of(kt0), ph1 = block_of(kt0 + 1), ph2 = block_of(kt0 + 2);
    int phys_next = block_of(kt0 + 3);
    copy_tile(kt0, ph0, 0);
    copy_tile(kt0 + 1, ph1, 1);
    copy_tile(kt0 + 2, ph2, 2);
    wait_vmcnt<2 * Sh::kCopies>();  // tiles kt0 and kt0+1 have landed
    __builtin_amdgcn_s_barrier();

    f32x16 s_cur[2], s_next[2];
    if (wave_live && kt0 < wave_tiles_end) scores(s_cur, 0);

    auto step = [&](int tile, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
      const int j = tile - kt0;
      const int phys_new = block_of(tile + 4);
      copy_tile(tile + 3, phys_next, (j + 3) & 3);
      phys_next = phys_new;
      if (wave_live && tile + 1 < wave_tiles_end) scores(sn, (j + 1) & 3);
      if (wave_live && tile < wave_tiles_end) softmax_pv(sc, tile * Sh::kKeys, j & 3);
      wait_vmcnt<kStepLoads>();  // tile t+2 has landed (this wave's copies)
      __builtin_amdgcn_s_barrier();
    };
    for (int tile = kt0; tile < kt1; tile += 2) {
      step(tile, s_cur, s_next);
      if (tile + 1 < kt1) step(tile + 1, s_next, s_cur);
    }
    wait_vmcnt<0>();  // no copy may still be writing LDS when the work-group ends
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
  return head_dim == 128 ? PrefillShape<128>::kStages * PrefillShape<128>::kStageBytes
                         : PrefillShape<64>::kStages * PrefillShape<64>::kStageBytes;
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
