// Device code of the varlen prefill (included by the prefill kernels and by the fused
// decode + prefill kernel).  What is computed and the tiling are described at the top of
// prefill_kernels.hip.
#pragma once

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
  static constexpr int kKSlots = 4;                    // K ring: K(t+3) is copied at step t
  static constexpr int kVSlots = 5;                    // V ring: V(t+3) copied at step t, read at t+3 and t+4
  static constexpr int kLdsBytes = (kKSlots + kVSlots) * kTileBytes;
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;           // rows one wave-wide 1 KB copy fills
  static constexpr int kCopies = kTileBytes / 1024 / kWaves;      // copies per wave per tensor per tile
  static constexpr int kKSteps = D / 16;               // 32x32x16 MFMAs over d
  static constexpr int kDTiles = D / 32;               // 32-wide d tiles of O^T
  // fp8 pools: the copies fill raw tiles of E4M3 codes (one byte an element).  K operands
  // are converted as they are read; V is converted into a bf16 tile laid out as the bf16
  // pools' V tiles, which O += V P then reads in the same way.
  static constexpr int kRawRowBytes = D;
  static constexpr int kRawChunks = D / 16;            // 16-byte chunks per raw row (its swizzle period)
  static constexpr int kRawTileBytes = kKeys * kRawRowBytes;
  static constexpr int kRawKSlots = 4;                 // raw K ring: K(t+3) copied at step t
  static constexpr int kRawVSlots = 3;                 // raw V ring: V(t+4) copied at step t, converted at step t+2
  static constexpr int kVRowSlots8 = 4;                // bf16 V tiles: V(t+2) converted at step t, read at t+2 and t+3
  static constexpr int kRawRowsPerWave = kKeys / kWaves;  // rows of a raw tile each wave copies and converts
  static constexpr int kRawLanes = kRawRowsPerWave * kRawChunks;  // lanes that hold one 16-byte raw chunk
  static constexpr int kLdsBytesF8 = (kRawKSlots + kRawVSlots) * kRawTileBytes + kVRowSlots8 * kTileBytes;
  static_assert(kLdsBytesF8 <= kLdsBytes, "the fp8 rings fit the bf16 kernel's LDS");
  static_assert(kRawLanes <= 64, "one raw slab per wave and tensor");
};

__device__ __forceinline__ bf16x8 u4_to_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Placement of the 16-byte chunks of a V tile row: logical chunk c of key row r sits at
// c ^ v_swizzle<D>(r % 4).  O += V P reads, per 16-lane group, 4 consecutive key rows x 2
// chunks (per 32 lanes: 4 rows x 4 chunks); with these four values those chunks land on
// distinct banks whether the LDS serves 16 lanes over 32 banks or 32 lanes over 64.
template <int D>
__device__ __forceinline__ int v_swizzle(int r4) {
  if constexpr (D == 128) return (0xCA60 >> (4 * r4)) & 15;  // 0, 6, 10, 12
  else return 2 * r4;                                        // 0, 2, 4, 6
}

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

// Same, and also waits for all of this wave's LDS (and scalar-memory) operations.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

// WINDOW: a lower edge on the visible keys as well -- a sliding window (p.window > 0: the
// row at p sees p-window+1 .. p) or chunked local attention (p.chunk > 0: C*(p div C) .. p)
// -- a variant of its own so that the plain causal kernel keeps its register budget.
// One work item of a prefill launch: item item_idx (its bits as in PrefillParams) for kv head
// kvh, by a work-group of PrefillShape<D>::kThreads threads with smem =
// PrefillShape<D>::kLdsBytes bytes of LDS.
//
// PREFIX (cascade prefix tiles, without WINDOW): the "positions" of the item are query rows
// 0 .. p.prefix_rows-1 of the batch, each one query of its own sequence, and every row sees
// all of keys 0 .. p.prefix_keys-1 (the blocks that every sequence's table begins with,
// read through table row s = 0); the item leaves its unnormalised partial in pre_*.
//
// F8: the pools hold E4M3 codes (the k_scale is in p.scale_log2, the v_scale is applied to
// the output or by the merge); the tiles are converted to their exact bf16 values in LDS
// and in registers, so the matrix-core work is the bf16 kernel's.
//
// FRESH (a mixed step that also stores its new K/V, bf16 pools): keys at or past the chunk's cached
// length are copied from the input rows p.new_k / p.new_v (row qsl[s] + key - cached, the pool's
// row layout) instead of the pool; the launch after this one stores them there.
template <int D, bool WINDOW, bool PREFIX = false, bool F8 = false, bool FRESH = false>
__device__ __forceinline__ void prefill_body(const PrefillParams& p, unsigned char* smem, int item_idx, int kvh) {
  using Sh = PrefillShape<D>;
  static_assert(!(PREFIX && WINDOW), "prefix tiles see the whole prefix");
  static_assert(!(FRESH && (WINDOW || PREFIX || F8)), "fresh rows: plain causal tiles over bf16 pools");

  // ---- work item
  const uint64_t item = p.items[item_idx];
  const int s = (int)(item & 0x7FFFu);
  const bool whole = (item >> 15) & 1u;
  const int rt = (int)((item >> 16) & 0xFFFFu);
  const int kt0 = (int)((item >> 32) & 0xFFFFu), kt1 = (int)(item >> 48);
  const int G = p.group;
  const int P = p.tile_positions;         // positions per row tile (rows = P * G <= 256)
  const int q0 = PREFIX ? 0 : p.qsl[s];
  const int q_len = PREFIX ? p.prefix_rows : p.qsl[s + 1] - q0;
  const int L = PREFIX ? p.prefix_keys : p.seq_lens[s];
  // every position of a prefix tile sits at L - 1 (all of the prefix visible)
  const int c = PREFIX ? 0 : L - q_len;
  const int pos0 = rt * P;
  const int pos_end = min(q_len, pos0 + P);  // positions of this tile: pos0 .. pos_end-1
  const int kv_end = PREFIX ? L : c + pos_end;  // keys the last row sees (exclusive)

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, rl = lane & 31;

  // ---- the lane's row: R = 32*wave + rl -> (position pos0 + R / G, q head kvh*G + R % G)
  const int R = 32 * wave + rl;
  const bool row_ok = R < P * G && pos0 + R / G < pos_end;
  const int row_pos = PREFIX ? L - 1 : c + pos0 + R / G;  // absolute position: keys <= it are visible
  // smallest and largest row position of the wave (masking and skipping whole tiles)
  const int wave_first = PREFIX ? L - 1 : c + pos0 + (32 * wave) / G;
  const int wave_last = PREFIX ? L - 1 : c + min(pos_end - 1, pos0 + (32 * wave + 31) / G);
  const bool wave_live = 32 * wave < P * G && pos0 + (32 * wave) / G < pos_end;
  // WINDOW: first visible key of the row at position q (non-decreasing in q)
  auto first_visible = [&](int q) { return p.chunk > 0 ? q - q % p.chunk : q - p.window + 1; };
  const uint32_t row_span = WINDOW ? (uint32_t)(row_pos - first_visible(row_pos) + 1) : 0u;  // keys the row sees
  const int wave_lo_max = WINDOW ? first_visible(wave_last) : 0;  // largest first visible key of the wave

  // ---- copy role: each wave copies kCopies 1 KB slabs of K and of V per tile.  Slab
  // kCopies*wave + i holds rows kRowsPerCopy*(kCopies*wave + i) ...; lane = (row in slab,
  // physical chunk); the chunk it fetches is the logical chunk stored in that slot,
  // physical ^ (row % kChunks) for K, physical ^ v_swizzle(row % 4) for V.  All rows of a
  // wave's slabs lie in one paged block.
  const int* bt = p.block_tables + (size_t)s * p.bt_stride;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.key_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.value_cache);
  const size_t tok_stride = (size_t)p.num_kv_heads * D * (F8 ? 1 : 2);
  const int lanes_per_row = Sh::kChunks;
  const int copy_row0 = Sh::kRowsPerCopy * Sh::kCopies * wave;  // first row of this wave's slabs
  // Keys no row of the tile sees are not read from the pool: those past the last visible
  // key and, with a sliding window, those before the first row's first visible key (their
  // blocks may have been given up).  Their rows copy a filler key that is always written
  // and finite -- key 0, or with a window the last visible key -- and their scores are
  // masked, so the probabilities that meet the filler are 0.
  const int fill_key = WINDOW ? kv_end - 1 : 0;
  const int key_first = WINDOW ? first_visible(c + pos0) : 0;
  const int bt_fill = min(max(bt[fill_key >> 4], 0), p.num_blocks - 1);
  // Physical block of this wave's rows of a tile.  The load is unconditional (a key past
  // the last visible one reads the last visible key's entry; any entry read is clamped
  // into the pool), so the compiler can count it among the loads in flight.
  auto block_of = [&](int tile) { return bt[min(tile * Sh::kKeys + copy_row0, kv_end - 1) >> 4]; };
  // Slab i (0 .. kCopies-1) of this wave's part of one tensor of a tile.
  auto copy_slab = [&](bool is_v, int tile, int phys, unsigned char* st, int i) {
    const uint8_t* const base = is_v ? vbase : kbase;
    phys = min(max(phys, 0), p.num_blocks - 1);
    const int row = copy_row0 + Sh::kRowsPerCopy * i + lane / lanes_per_row;
    const int slot = lane % lanes_per_row;
    const int chunk = slot ^ (is_v ? v_swizzle<D>(row & 3) : row % Sh::kChunks);
    const int key = tile * Sh::kKeys + row;
    const bool live = key < kv_end && (!WINDOW || key >= key_first);
    const int ph = live ? phys : bt_fill;
    const size_t off = ((size_t)ph * 16 + ((live ? key : fill_key) & 15)) * tok_stride + (size_t)kvh * D * 2 +
                       chunk * 16;
    const uint8_t* src = base + off;
    if constexpr (FRESH) {  // a new row (the filler too): from the input rows
      const int kk = live ? key : fill_key;
      const uint8_t* nb = reinterpret_cast<const uint8_t*>(is_v ? p.new_v : p.new_k);
      const size_t nrow = (size_t)(is_v ? p.new_v_stride : p.new_k_stride) * 2;
      if (kk >= c) src = nb + (size_t)(q0 + kk - c) * nrow + (size_t)kvh * D * 2 + chunk * 16;
    }
    unsigned char* dst = st + (copy_row0 + Sh::kRowsPerCopy * i) * Sh::kRowBytes;
    __builtin_amdgcn_global_load_lds((const void PA_GLOBAL*)src, (void PA_LDS*)dst, 16, 0, 0);
  };
  auto copy_rows = [&](bool is_v, int tile, int phys, unsigned char* st) {
#pragma unroll
    for (int i = 0; i < Sh::kCopies; ++i) copy_slab(is_v, tile, phys, st, i);
  };
  // fp8: this wave's kRawRowsPerWave rows of a raw tile (kRawChunks lanes a row, 16 codes a
  // lane; physical chunk = logical ^ (row % kRawChunks)), one copy instruction
  auto copy_raw = [&](const uint8_t* base, int tile, int phys, unsigned char* st) {
    phys = min(max(phys, 0), p.num_blocks - 1);
    const int row = Sh::kRawRowsPerWave * wave + lane / Sh::kRawChunks;
    const int chunk = (lane % Sh::kRawChunks) ^ (row % Sh::kRawChunks);
    const int key = tile * Sh::kKeys + row;
    const bool live = key < kv_end && (!WINDOW || key >= key_first);
    const int ph = live ? phys : bt_fill;
    const size_t off = ((size_t)ph * 16 + ((live ? key : fill_key) & 15)) * tok_stride + (size_t)kvh * D + chunk * 16;
    unsigned char* dst = st + Sh::kRawRowsPerWave * wave * Sh::kRawRowBytes;
    if (lane < Sh::kRawLanes)
      __builtin_amdgcn_global_load_lds((const void PA_GLOBAL*)(base + off), (void PA_LDS*)dst, 16, 0, 0);
  };
  // LDS: a ring of four K tiles (tile t in slot (t - kt0) % 4) and a ring of five V tiles
  // (slot (t - kt0) % 5).  fp8: four raw K tiles (slot (t - kt0) % 4), three raw V tiles
  // (slot (t - kt0) % 3) and four bf16 V tiles (slot (t - kt0) % 4).
  constexpr int kRawV0 = Sh::kRawKSlots * Sh::kRawTileBytes;        // fp8 layout offsets
  constexpr int kVRow0 = kRawV0 + Sh::kRawVSlots * Sh::kRawTileBytes;
  auto k_stage = [&](int tile) {
    return smem + ((tile - kt0) & 3) * (F8 ? Sh::kRawTileBytes : Sh::kTileBytes);
  };
  auto v_stage = [&](int tile) {  // the bf16 V tile that O += V P reads
    if constexpr (F8) return smem + kVRow0 + ((tile - kt0) & 3) * Sh::kTileBytes;
    else return smem + (Sh::kKSlots + (tile - kt0) % Sh::kVSlots) * Sh::kTileBytes;
  };
  auto vraw_stage = [&](int tile) { return smem + kRawV0 + ((tile - kt0) % 3) * Sh::kRawTileBytes; };
  auto k_addr = [&](int tile) { return (uint32_t)(uintptr_t)k_stage(tile); };
  auto v_addr = [&](int tile) { return (uint32_t)(uintptr_t)v_stage(tile); };

  // block ids of the first four tiles (fp8: five, V runs a tile further ahead), read before Q
  // so the first copies wait only for them
  const int ph0 = block_of(kt0), ph1 = block_of(kt0 + 1), ph2 = block_of(kt0 + 2);
  int phys_next = block_of(kt0 + 3);
  int phys_v_next = F8 ? block_of(kt0 + 4) : 0;

  // ---- Q^T operand: lane holds q[row rl][16*kk + 8*half .. +7].  A lane without a row
  // (past the tile's last position) reads the sequence's first row instead; its results
  // are never stored.  The loads are unconditional so that the wait below can count them.
  bf16x8 qf[Sh::kKSteps];
  {
    const int h = kvh * G + (R % G);
    const u32x4* qp = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.query) +
                                                     ((size_t)(q0 + (row_ok ? pos0 + R / G : 0)) * p.num_q_heads +
                                                      (row_ok ? h : 0)) * D + 8 * half);
#pragma unroll
    for (int kk = 0; kk < Sh::kKSteps; ++kk) qf[kk] = u4_to_bf16x8(qp[2 * kk]);
  }

  f32x16 acc[Sh::kDTiles];
#pragma unroll
  for (int n = 0; n < Sh::kDTiles; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
  float m_ref = -INFINITY, lsum = 0.f;
  // the score scale, waited for here so that no wait inside the tile loop is attributed to it
  float scale_log2 = p.scale_log2;
  asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(scale_log2));

  // S^T for both 32-key halves of a tile from a K slot: two independent MFMA chains.  The
  // lane's K row (key kt*32 + rl) is read in 16-byte chunks 2*kk + half, stored at chunk
  // (2*kk + half) ^ (rl % kChunks) (32 % kChunks == 0).  Operands are read two k-steps
  // before their MFMAs so the LDS latency hides behind the matrix cores; the reads are
  // issued and waited for from asm, like the V reads below.
  // fp8: the same elements are bytes 16*kk + 8*half .. +7 of raw row rl (raw chunk kk, stored
  // at kk ^ (rl % kRawChunks)), read as 8 bytes and converted to the bf16 operand in registers.
  using KOp = std::conditional_t<F8, u32x2, u32x4>;
  uint32_t koff[Sh::kKSteps];
#pragma unroll
  for (int kk = 0; kk < Sh::kKSteps; ++kk)
    koff[kk] = F8 ? (uint32_t)(rl * Sh::kRawRowBytes + ((kk ^ (rl % Sh::kRawChunks)) << 4) + 8 * half)
                  : (uint32_t)(rl * Sh::kRowBytes + (((2 * kk + half) ^ (rl % Sh::kChunks)) << 4));
  auto k_issue = [&](KOp (&x)[2], uint32_t base, auto kk_c) {
    constexpr int KK = decltype(kk_c)::value;
    const uint32_t a = base + koff[KK];
    if constexpr (F8) {
      asm volatile(
          "ds_read_b64 %0, %2\n\t"
          "ds_read_b64 %1, %2 offset:%3"
          : "=&v"(x[0]), "=&v"(x[1])
          : "v"(a), "i"(32 * Sh::kRawRowBytes)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b128 %0, %2\n\t"
          "ds_read_b128 %1, %2 offset:%3"
          : "=&v"(x[0]), "=&v"(x[1])
          : "v"(a), "i"(32 * Sh::kRowBytes)
          : "memory");
    }
  };
  // the K operand of an MFMA from what k_issue read
  auto k_operand = [&](const KOp& x) {
    if constexpr (F8) {
      const u32x2 lo = e4m3x4_to_bf16x4(x.x), hi = e4m3x4_to_bf16x4(x.y);
      return u4_to_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
    } else {
      return u4_to_bf16x8(x);
    }
  };
  // waits until at most N LDS reads issued after x's are in flight (reads return in order)
  auto op_wait = [&](auto& x, auto n_c) {
    constexpr int N = decltype(n_c)::value;
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N) : "memory");
  };
  auto scores = [&](f32x16 (&sacc)[2], uint32_t kbase_lds) {
    constexpr int kAhead = 2;
    KOp kb[kAhead + 1][2];
    static_for<0, kAhead>([&](auto kk_c) { k_issue(kb[decltype(kk_c)::value], kbase_lds, kk_c); });
    static_for<0, Sh::kKSteps>([&](auto kk_c) {
      constexpr int kk = decltype(kk_c)::value;
      constexpr int nxt = kk + kAhead;
      if constexpr (nxt < Sh::kKSteps) k_issue(kb[nxt % (kAhead + 1)], kbase_lds, std::integral_constant<int, nxt>{});
      // reads issued after this k-step's two: the next steps' (at most kAhead of them)
      constexpr int kLater = 2 * (nxt < Sh::kKSteps ? kAhead : Sh::kKSteps - 1 - kk);
      // each MFMA waits for its own operand only
      static_for<0, 2>([&](auto kt_c) {
        constexpr int kt = decltype(kt_c)::value;
        op_wait(kb[kk % (kAhead + 1)][kt], std::integral_constant<int, kLater + 1 - kt>{});
        const f32x16 c = kk == 0 ? f32x16{} : sacc[kt];
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(kb[kk % (kAhead + 1)][kt]), qf[kk], c, 0, 0, 0);
      });
    });
  };

  // ---- V operands.  O^T += V^T P^T needs, per lane (d = 32n + rl, half), the 8 keys whose
  // probabilities sit in its P register quad -- keys 16*ch + 4*half + 0..3 and 16*ch + 8 +
  // 4*half + 0..3 of the tile for chunk ch -- at one d, while the tile holds rows of d for
  // one key.  ds_read_b64_tr_b16 gathers them straight from the row-major tile: in each
  // 16-lane group g, output lane i element k is element i%4 of the 8 bytes addressed by lane
  // 4k + i/4, so lane 4k + q addresses key kb + k at d d0 + 4q .. +3 (d0 = 32n + 16*(g%2),
  // kb = 16*ch + 4*(g/2), plus 8 for the second four keys) and lane i receives keys
  // kb .. kb+3 of d d0 + i.  Two such reads make one operand.  A lane's address for d tile
  // n sits in v_off[n]; chunk ch and the second read are immediate offsets.
  constexpr int kTileQuad = Sh::kDTiles;  // operands per chunk (one per 32-wide d tile)
  uint32_t v_off[kTileQuad];
  {
    const int g = lane >> 4, i = lane & 15;
    const int row = 4 * (g >> 1) + (i >> 2);  // row % 4 == i >> 2
#pragma unroll
    for (int n = 0; n < kTileQuad; ++n) {
      const int chunk = 4 * n + 2 * (g & 1) + ((i & 3) >> 1);
      v_off[n] = (uint32_t)(row * Sh::kRowBytes + ((chunk ^ v_swizzle<D>(i >> 2)) << 4) + 8 * (i & 1));
    }
  }
  // issues (no wait) the 2*kTileQuad transposing reads of chunk CH of the V tile at vbase:
  // x[2n] and x[2n+1] are the two halves of d tile n's operand
  auto v_issue = [&](u32x2 (&x)[2 * kTileQuad], uint32_t vbase_lds, auto ch_c) {
    constexpr int CH = decltype(ch_c)::value;
    constexpr int o0 = 16 * CH * Sh::kRowBytes, o1 = (16 * CH + 8) * Sh::kRowBytes;
    uint32_t a[kTileQuad];
#pragma unroll
    for (int n = 0; n < kTileQuad; ++n) a[n] = vbase_lds + v_off[n];
    if constexpr (kTileQuad == 4) {
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
          "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
          "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
          "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
          "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
          "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
          "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
          "ds_read_b64_tr_b16 %7, %11 offset:%13"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]),
            "=&v"(x[7])
          : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(o0), "i"(o1)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
          "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
          "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
          "ds_read_b64_tr_b16 %3, %5 offset:%7"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
          : "v"(a[0]), "v"(a[1]), "i"(o0), "i"(o1)
          : "memory");
    }
  };

  // fp8: this wave's rows of a raw V tile -> a bf16 V tile.  Lane (row cv_row, logical raw
  // chunk cv_cr) converts 16 codes (d = 16*cv_cr .. +15) into bf16 chunks 2*cv_cr and
  // 2*cv_cr+1 of the row, each stored at chunk ^ v_swizzle(row % 4), as the copies place them.  With
  // fewer rows' chunks than lanes (D = 64) the upper lanes repeat the lower ones' work.
  const int cv_row = Sh::kRawRowsPerWave * wave + (lane % Sh::kRawLanes) / Sh::kRawChunks;
  const int cv_cr = lane % Sh::kRawChunks;
  const uint32_t cv_src = (uint32_t)(cv_row * Sh::kRawRowBytes + ((cv_cr ^ (cv_row % Sh::kRawChunks)) << 4));
  const uint32_t cv_dst0 = (uint32_t)(cv_row * Sh::kRowBytes + (((2 * cv_cr) ^ v_swizzle<D>(cv_row & 3)) << 4));
  const uint32_t cv_dst1 = (uint32_t)(cv_row * Sh::kRowBytes + (((2 * cv_cr + 1) ^ v_swizzle<D>(cv_row & 3)) << 4));
  auto vraw_issue = [&](u32x4& x, uint32_t raw_base) {
    asm volatile("ds_read_b128 %0, %1" : "=&v"(x) : "v"(raw_base + cv_src) : "memory");
  };
  // x holds landed codes (its read waited for, and x passed through a later asm statement)
  auto vraw_write = [&](const u32x4& x, uint32_t row_base) {
    const u32x2 a = e4m3x4_to_bf16x4(x.x), b = e4m3x4_to_bf16x4(x.y);
    const u32x2 c2 = e4m3x4_to_bf16x4(x.z), d2 = e4m3x4_to_bf16x4(x.w);
    const u32x4 lo = {a.x, a.y, b.x, b.y}, hi = {c2.x, c2.y, d2.x, d2.y};
    asm volatile(
        "ds_write_b128 %0, %2\n\t"
        "ds_write_b128 %1, %3"
        :
        : "v"(row_base + cv_dst0), "v"(row_base + cv_dst1), "v"(lo), "v"(hi)
        : "memory");
  };
  // the whole conversion of this wave's rows of one tile, its read waited for at once
  auto vraw_convert = [&](uint32_t raw_base, uint32_t row_base) {
    u32x4 x;
    vraw_issue(x, raw_base);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x) : : "memory");
    vraw_write(x, row_base);
  };

  // Online softmax of one tile's scores: P = exp2(s*scale - m) packed to bf16 in pw[chunk]
  // (16-key chunk ch = 2*half32 + cc), l and the reference maximum m updated.
  auto softmax = [&](f32x16 (&sacc)[2], int key0, u32x4 (&pw)[4]) {
    // lane's entries: key key0 + kt*32 + 8*(r/4) + 4*half + r%4 of row rl.  Raw scores are
    // masked and maximised; the scale (> 0) is applied inside exp2(fma(s, scale, -m)).
    // a tile needs masking if it reaches past some row's position, or (WINDOW) below some
    // row's first visible key
    if constexpr (WINDOW) {
      if (key0 + Sh::kKeys - 1 > wave_first || key0 < wave_lo_max) {
        // visible: 0 <= row_pos - key < row_span, one unsigned comparison
        const uint32_t rel = (uint32_t)(row_pos - key0 - 4 * half);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t dist = rel - (uint32_t)(kt * 32 + 8 * (r >> 2) + (r & 3));
            sacc[kt][r] = dist < row_span ? sacc[kt][r] : -INFINITY;
          }
      }
    } else if (key0 + Sh::kKeys - 1 > wave_first) {
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
    bmax = max_halves(bmax) * scale_log2;
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
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(__builtin_fmaf(sacc[kt][8 * cc + 2 * j], scale_log2, -msub));
          const float p1 = fast_exp2(__builtin_fmaf(sacc[kt][8 * cc + 2 * j + 1], scale_log2, -msub));
          ps += p0 + p1;
          pw[2 * kt + cc][j] = pack_bf16x2(p0, p1);
        }
    lsum += ps;
  };

  // waits until at most N LDS reads issued after x's and y's are in flight (y issued after
  // x: both have landed) and hands both registers on
  auto op_wait2 = [&](auto& x, auto& y, auto n_c) {
    constexpr int N = decltype(n_c)::value;
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "i"(N) : "memory");
  };
  // O^T += V^T P^T for one tile, from the V tile at byte address vbase_lds.  The reads of
  // chunk ch+1 are in flight while the MFMAs of chunk ch run; between(ch) is called after
  // they are issued (the copies of the step go there, spread over the matrix-core work
  // instead of stalling the wave at once).
  auto pv = [&](const u32x4 (&pw)[4], uint32_t vbase_lds, auto&& between) {
    u32x2 vb[2][2 * kTileQuad];
    v_issue(vb[0], vbase_lds, std::integral_constant<int, 0>{});
    static_for<0, 4>([&](auto ch_c) {
      constexpr int ch = decltype(ch_c)::value;
      if constexpr (ch + 1 < 4) v_issue(vb[(ch + 1) & 1], vbase_lds, std::integral_constant<int, ch + 1>{});
      constexpr int kLater = ch + 1 < 4 ? 2 * kTileQuad : 0;
      const bf16x8 pb = u4_to_bf16x8(pw[ch]);
      static_for<0, kTileQuad>([&](auto n_c) {
        constexpr int n = decltype(n_c)::value;
        u32x2& lo = vb[ch & 1][2 * n];
        u32x2& hi = vb[ch & 1][2 * n + 1];
        op_wait2(lo, hi, std::integral_constant<int, kLater + 2 * (kTileQuad - 1 - n)>{});
        const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(u4_to_bf16x8(a), pb, acc[n], 0, 0, 0);
        if constexpr (n == 0) between(ch);  // the step's copy of this chunk, beside the first MFMA
      });
    });
  };
  // the softmax phase of a step (fp8: with this wave's share of the conversion of raw V(t+2)
  // into its bf16 tile, the read issued before the exponentials and the rows written after)
  auto softmax_cv = [&](bool comp, f32x16 (&sacc)[2], int key0, u32x4 (&pw)[4], uint32_t raw_from,
                        uint32_t row_to) {
    if constexpr (F8) {
      u32x4 vr;
      vraw_issue(vr, raw_from);
      if (comp) softmax(sacc, key0, pw);
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(vr) : : "memory");
      vraw_write(vr, row_to);
    } else {
      if (comp) softmax(sacc, key0, pw);
    }
  };

  // Pipeline over the item's key tiles t = kt0 .. kt1-1, one step per tile between
  // work-group barriers.  Per tile a wave has a matrix-core part (S = K Q^T and
  // O += V P, 32 MFMAs) and a vector part (the softmax), about equally long.  The waves
  // are in two groups, one wave of each on every SIMD, that run the parts in opposite
  // order, so one group's exponentials issue while the other group's MFMAs run:
  //   leading group   (waves 0-3): O += V P(t-1), S(t)  | softmax(t) -> P(t)
  //   following group (waves 4-7): softmax(t) -> P(t)   | O += V P(t), S(t+1)
  // Step t also reads the block id of tile t+4 and starts the copies of K(t+3) and
  // V(t+3) (spread over the matrix-core part).  K slot (t+3)%4 last held K(t-1), read at
  // step t-1; V slot (t+3)%5 last held V(t-2), read at step t-1 (the step reads V(t-1) and
  // V(t)).  Before the barrier a wave waits for its LDS reads and for everything older than
  // this step's copies (vector-memory instructions retire in order and the copies are the
  // last loads of a step: vmcnt <= 2*kCopies), which covers K(t+2) and V(t+2), the newest
  // tiles step t+1 reads.  Block ids are read before the copies of their step, so
  // consuming one never waits on copies in flight.  Tiles past the item's range are copied
  // too (valid rows, never used) so that every step is alike.
  // fp8: step t copies raw K(t+3) and raw V(t+4) (block ids of tiles t+4 and t+5 read), and
  // every wave also converts its rows of raw V(t+2), in its softmax part, into bf16 slot
  // (t+2)%4, which last held V(t-2), read at step t-1.  Raw V slot (t+4)%3 last held V(t+1),
  // converted at step t-1; raw K slot (t+3)%4 last held K(t-1).  The end-of-step wait covers
  // raw K(t+2) and raw V(t+3), the newest raw tiles step t+1 reads.
  constexpr int kStepLoads = F8 ? 2 : 2 * Sh::kCopies;  // copy instructions per wave and step
  const int wave_tiles_end = min(kt1, wave_last / Sh::kKeys + 1);  // tiles this wave computes
  // (a sliding window's lower edge is left to the item's key range and to masking: a wave
  // that also skipped its own leading tiles would need registers the kernel does not have)
  const bool leading = wave < Sh::kWaves / 2;
  auto computes = [&](int tile) { return wave_live && tile < wave_tiles_end; };
  {
    wait_vmcnt<Sh::kKSteps>();  // the block ids have landed; Q may still be in flight
    if constexpr (F8) {
      // raw K and V of tiles kt0 .. kt0+2; V(kt0) and V(kt0+1) converted, and raw V(kt0+3)
      // copied into the slot V(kt0) left, before the first step
      copy_raw(kbase, kt0, ph0, k_stage(kt0));
      copy_raw(vbase, kt0, ph0, vraw_stage(kt0));
      copy_raw(kbase, kt0 + 1, ph1, k_stage(kt0 + 1));
      copy_raw(vbase, kt0 + 1, ph1, vraw_stage(kt0 + 1));
      copy_raw(kbase, kt0 + 2, ph2, k_stage(kt0 + 2));
      copy_raw(vbase, kt0 + 2, ph2, vraw_stage(kt0 + 2));
      wait_vmcnt<2>();  // Q and tiles kt0, kt0+1 have landed
      __builtin_amdgcn_s_barrier();
      vraw_convert((uint32_t)(uintptr_t)vraw_stage(kt0), v_addr(kt0));
      vraw_convert((uint32_t)(uintptr_t)vraw_stage(kt0 + 1), v_addr(kt0 + 1));
      wait_vmcnt_lgkm0<2>();
      __builtin_amdgcn_s_barrier();
      copy_raw(vbase, kt0 + 3, phys_next, vraw_stage(kt0 + 3));
      wait_vmcnt_lgkm0<1>();  // tile kt0+2 has landed; raw V(kt0+3) may be in flight
      __builtin_amdgcn_s_barrier();
    } else {
      copy_rows(false, kt0, ph0, k_stage(kt0));
      copy_rows(true, kt0, ph0, v_stage(kt0));
      copy_rows(false, kt0 + 1, ph1, k_stage(kt0 + 1));
      copy_rows(true, kt0 + 1, ph1, v_stage(kt0 + 1));
      copy_rows(false, kt0 + 2, ph2, k_stage(kt0 + 2));
      copy_rows(true, kt0 + 2, ph2, v_stage(kt0 + 2));
      wait_vmcnt<2 * Sh::kCopies>();  // Q and tiles kt0, kt0+1 have landed
      __builtin_amdgcn_s_barrier();
    }

    f32x16 sc[2];  // scores of the tile the wave softmaxes next
    u32x4 pw[4];   // its probabilities, bf16
    if (!leading && computes(kt0)) scores(sc, k_addr(kt0));
    for (int tile = kt0; tile < kt1; ++tile) {
      const int phys_new = block_of(tile + 4);
      const int phys_v_new = F8 ? block_of(tile + 5) : 0;
      // this step's copies: K(t+3) and V(t+3), kCopies slabs each (fp8: raw K(t+3) and raw
      // V(t+4), one slab each)
      const int phys = phys_next, phys_v = phys_v_next;
      unsigned char* const k_dst = k_stage(tile + 3);
      unsigned char* const v_dst = F8 ? vraw_stage(tile + 4) : v_stage(tile + 3);
      auto copy_part = [&](int part) {
        if constexpr (F8) {
          if (part == 0)
            copy_raw(kbase, tile + 3, phys, k_dst);
          else if (part == 1)
            copy_raw(vbase, tile + 4, phys_v, v_dst);
        } else {
          if (part < Sh::kCopies)
            copy_slab(false, tile + 3, phys, k_dst, part);
          else if (part < 2 * Sh::kCopies)
            copy_slab(true, tile + 3, phys, v_dst, part - Sh::kCopies);
        }
      };
      auto copy_all = [&]() {
#pragma unroll
        for (int part = 0; part < kStepLoads; ++part) copy_part(part);
      };
      phys_next = phys_new;
      phys_v_next = phys_v_new;
      // fp8: raw V(t+2) -> its bf16 tile by every wave; tiles past the range hold valid rows
      // too, so the conversion is unconditional
      const uint32_t raw_from = F8 ? (uint32_t)(uintptr_t)vraw_stage(tile + 2) : 0u;
      const uint32_t row_to = F8 ? v_addr(tile + 2) : 0u;
      if (!leading) softmax_cv(computes(tile), sc, tile * Sh::kKeys, pw, raw_from, row_to);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      if (leading) {
        if (tile > kt0 && computes(tile - 1)) {
          pv(pw, v_addr(tile - 1), copy_part);
        } else {
          copy_all();
        }
        if (computes(tile)) scores(sc, k_addr(tile));
      } else {
        if (computes(tile)) {
          pv(pw, v_addr(tile), copy_part);
        } else {
          copy_all();
        }
        if (computes(tile + 1)) scores(sc, k_addr(tile + 1));
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      if (leading) softmax_cv(computes(tile), sc, tile * Sh::kKeys, pw, raw_from, row_to);
      wait_vmcnt_lgkm0<kStepLoads>();
      __builtin_amdgcn_s_barrier();
    }
    // the last O += V P of the leading group (the copies of the last step went to other slots)
    if (leading && computes(kt1 - 1)) pv(pw, v_addr(kt1 - 1), [](int) {});
    wait_vmcnt<0>();  // no copy may still be writing LDS when the work-group ends
  }


  // ---- epilogue.  The lane's outputs (d = n*32 + 8*(r/4) + 4*half + r%4 of row rl) are
  // scattered pieces of 32 rows; stored as they are, every store instruction would touch 32
  // lines.  Each wave stages its 32 rows in LDS (free now; 16-byte chunks XOR-swizzled by
  // row so that the writes spread over the banks) and stores whole rows from there, 16
  // bytes per lane.  A whole row tile stores bf16 outputs; a split piece stores O / l in
  // fp16 with a per-row scale (below), its reference maximum m and weight sum l, for the
  // merge.
  __syncthreads();  // every wave is done with the rings
  if (!wave_live) return;
  const float l = sum_halves(lsum);
  if constexpr (PREFIX) {
    // unnormalised O, the reference maximum and the weight sum of (sequence pos0 + R / G,
    // q head kvh*G + R % G) for the prefix share of this item's keys; lane (rl, half) holds
    // d = 32n + 8*(r/4) + 4*half + r%4, four consecutive d per (n, r/4)
    if (!row_ok) return;
    const size_t pi = ((size_t)(kt0 / p.prefix_share_tiles) * p.prefix_rows + pos0 + R / G) * p.num_q_heads +
                      kvh * G + R % G;
    float* po = p.pre_o + pi * D + 4 * half;
#pragma unroll
    for (int n = 0; n < Sh::kDTiles; ++n)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *reinterpret_cast<f32x4*>(po + 32 * n + 8 * rq) =
            f32x4{acc[n][4 * rq], acc[n][4 * rq + 1], acc[n][4 * rq + 2], acc[n][4 * rq + 3]};
    if (half == 0) {
      p.pre_m[pi] = m_ref;
      p.pre_l[pi] = l;
    }
    return;
  }
  const float inv = whole ? p.v_scale / l : (l > 0.f ? 1.f / l : 0.f);  // a row that saw no key stores 0
  const size_t slot_row0 = ((size_t)(p.item_base + item_idx) * p.num_kv_heads + kvh) * kPrefillRows + 32 * wave;
  if (whole) {
    unsigned char* const stage = smem + wave * 32 * Sh::kRowBytes;
#pragma unroll
    for (int n = 0; n < Sh::kDTiles; ++n)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int chunk = (n * 4 + rq) ^ (rl % Sh::kChunks);
        const float a0 = acc[n][4 * rq] * inv, a1 = acc[n][4 * rq + 1] * inv;
        const float a2 = acc[n][4 * rq + 2] * inv, a3 = acc[n][4 * rq + 3] * inv;
        *reinterpret_cast<u32x2*>(stage + rl * Sh::kRowBytes + chunk * 16 + half * 8) =
            u32x2{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int kRowsPerStore = 64 / Sh::kChunks;
    const int sc_chunk = lane % Sh::kChunks;
#pragma unroll
    for (int it = 0; it < 32 / kRowsPerStore; ++it) {
      const int row = it * kRowsPerStore + lane / Sh::kChunks;
      const u32x4 v =
          *reinterpret_cast<const u32x4*>(stage + row * Sh::kRowBytes + ((sc_chunk ^ (row % Sh::kChunks)) << 4));
      const int Rw = 32 * wave + row;
      if (Rw >= P * G || pos0 + Rw / G >= pos_end) continue;
      uint16_t* dst = reinterpret_cast<uint16_t*>(p.out) +
                      ((size_t)(q0 + pos0 + Rw / G) * p.num_q_heads + kvh * G + Rw % G) * D;
      *reinterpret_cast<u32x4*>(dst + sc_chunk * 8) = v;
    }
    return;
  }
  // split piece: O / l in fp16 scaled by a per-row power of two sigma = 2^(E-15), where
  // 2^(E-1) <= the row's largest |O / l| < 2^E, so every stored value is below 2^15 (fp16
  // holds up to 65504) and the rounding error is at most 2^-11 of that largest magnitude,
  // whatever the range of V.  sigma goes to the merge beside m and l.
  float amax = 0.f;
#pragma unroll
  for (int n = 0; n < Sh::kDTiles; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(acc[n][r]));
  amax = max_halves(amax) * inv;  // the row's two lanes hold its D values between them
  int e2 = 0;
  (void)frexpf(amax, &e2);  // amax = f * 2^e2, f in [0.5, 1) (e2 = 0 for amax = 0)
  const float sigma = ldexpf(1.f, e2 - 15);
  const float mul = inv * ldexpf(1.f, 15 - e2);
  unsigned char* const stage = smem + wave * 32 * Sh::kRowBytes;
#pragma unroll
  for (int n = 0; n < Sh::kDTiles; ++n)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int chunk = (n * 4 + rq) ^ (rl % Sh::kChunks);
      const float a0 = acc[n][4 * rq] * mul, a1 = acc[n][4 * rq + 1] * mul;
      const float a2 = acc[n][4 * rq + 2] * mul, a3 = acc[n][4 * rq + 3] * mul;
      *reinterpret_cast<u32x2*>(stage + rl * Sh::kRowBytes + chunk * 16 + half * 8) =
          u32x2{pack_f16x2(a0, a1), pack_f16x2(a2, a3)};
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int kRowsPerStore = 64 / Sh::kChunks;
  const int sc_chunk = lane % Sh::kChunks;
#pragma unroll
  for (int it = 0; it < 32 / kRowsPerStore; ++it) {
    const int row = it * kRowsPerStore + lane / Sh::kChunks;
    const u32x4 v =
        *reinterpret_cast<const u32x4*>(stage + row * Sh::kRowBytes + ((sc_chunk ^ (row % Sh::kChunks)) << 4));
    const int Rw = 32 * wave + row;
    if (Rw >= P * G || pos0 + Rw / G >= pos_end) continue;
    *reinterpret_cast<u32x4*>(p.part_o + (slot_row0 + row) * D + sc_chunk * 8) = v;
  }
  if (half == 0 && row_ok) {
    p.part_m[slot_row0 + rl] = m_ref;
    p.part_l[slot_row0 + rl] = l;
    p.part_s[slot_row0 + rl] = sigma;
  }
}

}  // namespace

}  // namespace pa
