// Device code of the paged decode (included by the decode kernels and by the fused
// decode + prefill kernel).  What is computed and how the work is split is described at
// the top of decode_kernels.hip.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

// Per-lane geometry of one 16-token block for head size D.  A wave reads a
// block's rows for one kv head with each 16-lane quarter covering one whole
// token row (coalesced): lane (a = lane / 16, c = lane % 16) holds the VEC
// consecutive elements c*VEC .. c*VEC+VEC-1 of token rows a, a+4, a+8, a+12.
template <int D, bool FP8>
struct DecodeShape {
  static constexpr int kVec = D / 16;                 // elements of one row per lane
  static constexpr int kWords = kVec / 2;             // bf16 dwords of one row slice
  static constexpr int kLoadBytes = kVec * (FP8 ? 1 : 2);
  static constexpr int kKSteps = D / 32;              // 16x16x32 MFMAs per score tile
  static constexpr int kRowBytes = D * 2;             // bf16 bytes of one token row in LDS
  static constexpr int kChunks = kRowBytes / 16;      // 16-byte chunks per LDS row
  static constexpr int kLdsBytes = 16 * kRowBytes;    // one K block per wave
};

template <int N>
struct RawVec;
template <>
struct RawVec<16> {
  u32x4 v;
};
template <>
struct RawVec<8> {
  u32x2 v;
};
template <>
struct RawVec<4> {
  uint32_t v;
};

// The raw bytes of one lane's slices of the four rows it owns, for K and V.
template <int D, bool FP8>
struct BlockRegs {
  using Sh = DecodeShape<D, FP8>;
  RawVec<Sh::kLoadBytes> k[4], v[4];
};

// s_waitcnt operand for vmcnt(0) with the other counters left free (gfx9 encoding)
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);

// pointers into the constant address space: loads through them from wave-uniform addresses
// become scalar loads
#define PA_CONST_AS __attribute__((address_space(4)))

#ifndef PA_DECODE_IN_FLIGHT
#define PA_DECODE_IN_FLIGHT 2
#endif
#ifndef PA_DECODE_IN_FLIGHT_FP8
#define PA_DECODE_IN_FLIGHT_FP8 2
#endif
// blocks whose loads are in flight per wave while one is computed (register sets); an fp8
// block is half the bytes of a bf16 one, but more sets did not help it (Llama-3-8B layer with
// E4M3 pools at one wave per SIMD: 2 sets 60 us, 3 60, 4 64, 6 65): fp8 takes more waves instead
template <bool FP8>
constexpr int kInFlight = FP8 ? PA_DECODE_IN_FLIGHT_FP8 : PA_DECODE_IN_FLIGHT;

template <int N>
__device__ __forceinline__ void load_raw(RawVec<N>& r, const uint8_t* p) {
  if constexpr (N == 16) r.v = *reinterpret_cast<const u32x4*>(p);
  else if constexpr (N == 8) r.v = *reinterpret_cast<const u32x2*>(p);
  else r.v = *reinterpret_cast<const uint32_t*>(p);
}

template <int N>
__device__ __forceinline__ void store_raw(uint8_t* p, const RawVec<N>& r) {
  if constexpr (N == 16) *reinterpret_cast<u32x4*>(p) = r.v;
  else if constexpr (N == 8) *reinterpret_cast<u32x2*>(p) = r.v;
  else *reinterpret_cast<uint32_t*>(p) = r.v;
}

// r = x where take (per lane)
template <int N>
__device__ __forceinline__ void select_raw(RawVec<N>& r, const RawVec<N>& x, bool take) {
  if constexpr (N == 16) {
    r.v.x = take ? x.v.x : r.v.x;
    r.v.y = take ? x.v.y : r.v.y;
    r.v.z = take ? x.v.z : r.v.z;
    r.v.w = take ? x.v.w : r.v.w;
  } else if constexpr (N == 8) {
    r.v.x = take ? x.v.x : r.v.x;
    r.v.y = take ? x.v.y : r.v.y;
  } else {
    r.v = take ? x.v : r.v;
  }
}

// The same as a non-temporal load: KV that one wave streams once is not kept in the
// caches (measured: the decode kernel of a Llama-3-8B layer 103 -> 96 us, the 70B
// long-context one 394 -> 356 us, with less L2/last-level-cache churn).
template <int N>
__device__ __forceinline__ void load_raw_stream(RawVec<N>& r, const uint8_t* p) {
  if constexpr (N == 16) r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else if constexpr (N == 8) r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  else r.v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// Raw slice -> bf16 dwords (element order kept).  E4M3 codes are exact in bf16.
template <int D, bool FP8>
__device__ __forceinline__ void raw_to_words(const RawVec<DecodeShape<D, FP8>::kLoadBytes>& r,
                                             uint32_t (&w)[DecodeShape<D, FP8>::kWords]) {
  constexpr int W = DecodeShape<D, FP8>::kWords;
  if constexpr (FP8) {
    uint32_t b[W / 2];
    if constexpr (W == 4) {
      b[0] = r.v.x;
      b[1] = r.v.y;
    } else {
      b[0] = r.v;
    }
#pragma unroll
    for (int i = 0; i < W / 2; ++i) {
      const u32x2 t = e4m3x4_to_bf16x4(b[i]);
      w[2 * i] = t.x;
      w[2 * i + 1] = t.y;
    }
  } else {
    if constexpr (W == 4) {
      w[0] = r.v.x;
      w[1] = r.v.y;
      w[2] = r.v.z;
      w[3] = r.v.w;
    } else {
      w[0] = r.v.x;
      w[1] = r.v.y;
    }
  }
}

__device__ __forceinline__ bf16x8 words_to_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 t = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, t);
}

// max / sum over the four lanes l, l^16, l^32, l^48 (the four row groups of a wave)
__device__ __forceinline__ float max_across_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  const uint32_t v = __float_as_uint(x);
  auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

__device__ __forceinline__ float sum_across_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  const uint32_t v = __float_as_uint(x);
  auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
}

// A new K/V row's slice of kv head kvh as loaded (row `row` of the input, 16-byte aligned slices,
// checked by the caller).  bf16 pools: lane (a, c) loads elements c*VEC .. c*VEC+VEC-1 of K and
// of V, the pool-format slice it substitutes.  fp8 pools: the quantisation is spread over the
// whole wave -- lane l loads elements (l % 32)*D/32 .. +D/32-1 of K (l < 32) or V (l >= 32), fp32
// or bf16 -- and the codes reach the lanes that substitute them through cross-lane reads.
template <int D>
struct NewRowSrc {
  uint32_t w[D / 32];
};

template <int N>
__device__ __forceinline__ void load_words(uint32_t* w, const void* p) {
  if constexpr (N == 4) {
    const u32x4 t = *reinterpret_cast<const u32x4*>(p);
    w[0] = t.x;
    w[1] = t.y;
    w[2] = t.z;
    w[3] = t.w;
  } else if constexpr (N == 2) {
    const u32x2 t = *reinterpret_cast<const u32x2*>(p);
    w[0] = t.x;
    w[1] = t.y;
  } else {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

template <int D, bool FP8>
__device__ __forceinline__ void load_new_row(const DecodeParams& p, NewRowSrc<D>& k, NewRowSrc<D>& v, int row,
                                             int kvh, int lane) {
  constexpr int VEC = D / 16;
  if constexpr (!FP8) {
    const int64_t e = kvh * D + (lane & 15) * VEC;
    load_words<VEC / 2>(k.w, reinterpret_cast<const uint16_t*>(p.new_k) + (int64_t)row * p.new_k_stride + e);
    load_words<VEC / 2>(v.w, reinterpret_cast<const uint16_t*>(p.new_v) + (int64_t)row * p.new_v_stride + e);
  } else {
    constexpr int N = D / 32;  // elements of this lane
    const bool is_v = lane >= 32;
    const void* src = is_v ? p.new_v : p.new_k;
    const int64_t e = (int64_t)row * (is_v ? p.new_v_stride : p.new_k_stride) + kvh * D + (lane & 31) * N;
    if (p.new_f32) load_words<N>(k.w, reinterpret_cast<const float*>(src) + e);
    else load_words<N / 2>(k.w, reinterpret_cast<const uint16_t*>(src) + e);
  }
}

// The substituting lane's slices in the pool's format: the bf16 values themselves, or for an
// fp8 pool the E4M3 codes of x / scale -- the codes the KV write stores (round to nearest even,
// saturating).  fp8: every lane of the wave takes part (cross-lane reads).
template <int D, bool FP8>
__device__ __forceinline__ void new_row_raw(const DecodeParams& p, const NewRowSrc<D>& k, const NewRowSrc<D>& v,
                                            RawVec<DecodeShape<D, FP8>::kLoadBytes>& nk,
                                            RawVec<DecodeShape<D, FP8>::kLoadBytes>& nv, int lane) {
  constexpr int VEC = D / 16;
  if constexpr (!FP8) {
    if constexpr (VEC == 8) {
      nk.v = u32x4{k.w[0], k.w[1], k.w[2], k.w[3]};
      nv.v = u32x4{v.w[0], v.w[1], v.w[2], v.w[3]};
    } else {
      nk.v = u32x2{k.w[0], k.w[1]};
      nv.v = u32x2{v.w[0], v.w[1]};
    }
  } else {
    constexpr int N = D / 32;
    const float scale = lane >= 32 ? p.new_v_scale : p.new_k_scale;
    uint32_t codes = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float x = p.new_f32 ? __uint_as_float(k.w[j])
                                : __uint_as_float((j & 1) ? (k.w[j >> 1] & 0xFFFF0000u) : (k.w[j >> 1] << 16));
      codes |= (uint32_t)f32_to_e4m3(__fdiv_rn(x, scale)) << (8 * j);
    }
    // lane (a, c) substitutes elements c*VEC .. c*VEC+VEC-1: N codes each from lanes 2c, 2c+1
    // (K) and 32+2c, 33+2c (V)
    const int c = lane & 15;
    const uint32_t k0 = __shfl((int)codes, 2 * c, 64), k1 = __shfl((int)codes, 2 * c + 1, 64);
    const uint32_t v0 = __shfl((int)codes, 32 + 2 * c, 64), v1 = __shfl((int)codes, 33 + 2 * c, 64);
    if constexpr (N == 4) {
      nk.v = u32x2{k0, k1};
      nv.v = u32x2{v0, v1};
    } else {
      nk.v = (k0 & 0xFFFFu) | (k1 << 16);
      nv.v = (v0 & 0xFFFFu) | (v1 << 16);
    }
  }
}

// Blocks of sequence s the decode attends: ceil(seq_len / 16), or 0 when s
// is not a decode row of a flattened batch (q_len != 1).
// First visible key of a sequence of L >= 1 tokens: L - window with a sliding window, the
// start of the last position's chunk with chunked local attention, else 0.
__device__ __forceinline__ int decode_first_key(const DecodeParams& p, int L) {
  if (p.chunk > 0) return (L - 1) - (L - 1) % p.chunk;
  return p.window > 0 ? max(L - p.window, 0) : 0;
}

// Leading blocks of sequence s its own pieces skip: the shared prefix of a cascade, or the
// blocks wholly before the visible keys (sliding window, local chunk).
__device__ __forceinline__ int decode_skip(const DecodeParams& p, int L) {
  return (p.window > 0 || p.chunk > 0) ? decode_first_key(p, L) >> 4 : p.skip_blocks;
}

// Blocks of sequence s that its own pieces cover.
__device__ __forceinline__ int decode_blocks(const DecodeParams& p, int s) {
  if (p.qsl && p.qsl[s + 1] - p.qsl[s] != 1) return 0;
  const int L = min(p.seq_lens[s], p.max_seq_len);
  return L > 0 ? max(((L + 15) >> 4) - decode_skip(p, L), 0) : 0;
}

__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ int wave_incl_scan_i32(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(x, d, 64);
    if (lane >= d) x += t;
  }
  return x;
}

// Calls piece(s, b0, b1, nb) for every piece of share `split` (of n_splits):
// blocks [b0, b1) of sequence s, which has nb blocks in all.  The sequences are laid
// end to end, each as p.piece_cost units (the cost of starting a piece: its Q, its
// table window, the pipeline's first loads, in blocks' worth of time) followed by its
// nb blocks, and cut into n_splits equal shares of units; a share's piece of s is the
// blocks it holds (a share holding only the start units of s has no piece of it).
// Shares are consecutive, so a wave visits its sequences in increasing order and the
// pieces of a sequence come from consecutive shares.  All arguments are wave-uniform.
// (wave-uniform values pass through readfirstlane: the compiler cannot see that a shuffle
// reduction or a ballot loop ends alike in every lane, and would otherwise keep the piece
// bounds, and every loop over blocks after them, in vector registers and divergent branches)
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <typename Fn>
__device__ __forceinline__ void for_each_piece(const DecodeParams& p, int split, Fn&& piece) {
  const int lane = threadIdx.x & 63;
  const int c = p.piece_cost;
  int tot = 0, nb_first = 0;
  for (int base = 0; base < p.num_seqs; base += 64) {
    const int s = base + lane;
    const int nb = s < p.num_seqs ? decode_blocks(p, s) : 0;
    if (base == 0) nb_first = nb;  // kept: the first 64 sequences are not loaded twice
    tot += nb > 0 ? nb + c : 0;
  }
  const long long T = wave_uniform(wave_sum_i32(tot));
  // never more shares than units, so no share is empty
  const long long n = min((long long)p.n_splits, T);
  if (split >= n) return;
  const int lo = (int)(T * split / n), hi = (int)(T * (split + 1) / n);
  int carry = 0;
  for (int base = 0; base < p.num_seqs && carry < hi; base += 64) {
    const int s = base + lane;
    const int nb = base == 0 ? nb_first : (s < p.num_seqs ? decode_blocks(p, s) : 0);
    const int w = nb > 0 ? nb + c : 0;
    const int incl = wave_incl_scan_i32(w, lane);
    const int start = carry + incl - w + c;  // units before block 0 of s
    const unsigned long long hits0 = __ballot(nb > 0 && start < hi && start + nb > lo);
    unsigned long long hits = ((unsigned long long)(unsigned)wave_uniform((int)(hits0 >> 32)) << 32) |
                              (unsigned)wave_uniform((int)hits0);
    while (hits) {
      const int ln = wave_uniform(__ffsll((long long)hits) - 1);
      hits &= hits - 1;
      const int bs = wave_uniform(__builtin_amdgcn_readlane(start, ln));
      const int nbs = wave_uniform(__builtin_amdgcn_readlane(nb, ln));
      piece(base + ln, wave_uniform(max(lo - bs, 0)), wave_uniform(min(hi - bs, nbs)), nbs);
    }
    carry = wave_uniform(carry + __builtin_amdgcn_readlane(incl, 63));
  }
}

// Records which shares hold the first and the last piece of sequence s.
// With a single share every sequence is finished in place and there is no
// scratch (the index arrays are absent).
__device__ __forceinline__ void note_piece(const DecodeParams& p, int split, int s, int b0, int b1, int nb) {
  if (p.n_splits <= 1 && !p.force_partial) return;
  if (b0 == 0) p.piece_first[s] = split;
  if (b1 == nb) p.piece_last[s] = split;
}

// One 16-token block of a piece for the wave's 16 matrix-core columns:
//   S[tok][col] = K[tok][:] . Q[col][:]     v_mfma_f32_16x16x32_bf16, K through a swizzled LDS tile
//   O^T[d][col] += V^T[d][tok] P^T[tok][col] v_mfma_f32_16x16x16_bf16, V straight from registers
// The K tile rows are read in the order sigma(m) = m/4 + 4*(m%4), so score element r of
// lane (a, c) belongs to token a + 4r: exactly the four tokens whose V slices the same lane
// loaded.  P therefore never leaves its lane, and the V^T operand of MFMA j (d = VEC*m + j)
// is two byte permutes of the lane's own V words.  Tokens outside [key_lo, tok1) are
// masked by selection; V rows at or past tok1 are zeroed (never multiplied: NaN-safe).
// SUB: row sub_i of this lane's four (-1: none) takes the slices nk / nv in place of what was
// loaded, each at the point its row is consumed (the loads are waited for row by row as usual).
template <int D, bool FP8, bool SUB = false>
__device__ __forceinline__ void block_step(const DecodeParams& p, const BlockRegs<D, FP8>& r, unsigned char* kl,
                                           int blk_tok, int tok1, int key_lo,
                                           const bf16x8 (&qf)[DecodeShape<D, FP8>::kKSteps], float& m, float& l,
                                           f32x4 (&acc)[DecodeShape<D, FP8>::kVec],
                                           const RawVec<DecodeShape<D, FP8>::kLoadBytes>* nk = nullptr,
                                           const RawVec<DecodeShape<D, FP8>::kLoadBytes>* nv = nullptr,
                                           int sub_i = -1) {
  using Sh = DecodeShape<D, FP8>;
  constexpr int VEC = Sh::kVec, W = Sh::kWords;
  const int lane = threadIdx.x & 63;
  const int a = lane >> 4, c = lane & 15;
  const int m_row = (c >> 2) + 4 * (c & 3);  // sigma(c): the token row this lane feeds into the MFMA
  const bool partial = blk_tok + 16 > tok1;
  // K slices -> LDS (bf16, swizzled: row t, logical 16-byte chunk x lives at chunk x ^ (t % kChunks))
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w[W];
    RawVec<Sh::kLoadBytes> kr = r.k[i];
    if constexpr (SUB) select_raw(kr, *nk, i == sub_i);
    raw_to_words<D, FP8>(kr, w);
    const int t = a + 4 * i;
    const int byte = c * VEC * 2;
    unsigned char* dst = kl + t * Sh::kRowBytes + (((byte >> 4) ^ (t % Sh::kChunks)) << 4) + (byte & 15);
    if constexpr (W == 4)
      *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    else
      *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
  }
  // V slices -> bf16 words, rows past the sequence end zeroed
  uint32_t vw[4][W];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    RawVec<Sh::kLoadBytes> vr = r.v[i];
    if constexpr (SUB) select_raw(vr, *nv, i == sub_i);
    raw_to_words<D, FP8>(vr, vw[i]);
    if (partial && blk_tok + a + 4 * i >= tok1) {
#pragma unroll
      for (int x = 0; x < W; ++x) vw[i][x] = 0u;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < Sh::kKSteps; ++kk) {
    const int x = a + 4 * kk;
    const u32x4 kw = *reinterpret_cast<const u32x4*>(kl + m_row * Sh::kRowBytes + ((x ^ (m_row % Sh::kChunks)) << 4));
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw), qf[kk], sacc, 0, 0, 0);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // online softmax over the block: element r of this lane is token a + 4r of column c
  float z[4];
  float bmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = blk_tok + a + 4 * i;
    const bool live = tok < tok1 && tok >= key_lo;
    z[i] = live ? sacc[i] * p.scale_log2 : -INFINITY;
    bmax = fmaxf(bmax, z[i]);
  }
  bmax = max_across_rows(bmax);
  const float mnew = fmaxf(m, bmax);
  const float alpha = fast_exp2(m - mnew);
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(z[i] - mnew);
  l = l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
  m = mnew;
  i16x4 pb;
  {
    const uint32_t p01 = pack_bf16x2(pr[0], pr[1]), p23 = pack_bf16x2(pr[2], pr[3]);
    pb = __builtin_bit_cast(i16x4, u32x2{p01, p23});
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t lo = __builtin_amdgcn_perm(vw[1][j >> 1], vw[0][j >> 1], sel);
    const uint32_t hi = __builtin_amdgcn_perm(vw[3][j >> 1], vw[2][j >> 1], sel);
    const i16x4 va = __builtin_bit_cast(i16x4, u32x2{lo, hi});
    acc[j] *= alpha;
    acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[j], 0, 0, 0);
  }
}

// Writes a finished piece of q head h (lane (a, column) holds O[column][VEC*(4a + r) + j] in
// acc[j][r]: 4*VEC consecutive d; l already summed over the four row groups).  GROUP: the
// cascade prefix partial of (prefix share split, sequence col_seq); whole: the normalised
// output row; else the partial of piece id split + s (unique: shares and sequences are both
// visited in increasing order).
template <int D, bool GROUP>
__device__ __forceinline__ void piece_output(const DecodeParams& p, const f32x4 (&acc)[D / 16], float m, float l,
                                             int h, int split, int s, int row, int col_seq, bool whole) {
  constexpr int VEC = D / 16;
  const int a = (threadIdx.x & 63) >> 4;
  const int d0 = 4 * VEC * a;
  if constexpr (GROUP) {
    const size_t pi = ((size_t)split * p.num_seqs + col_seq) * p.num_q_heads + h;
    float* po = p.pre_o + pi * D + d0;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < VEC; j += 4)
        *reinterpret_cast<f32x4*>(po + VEC * r + j) = f32x4{acc[j][r], acc[j + 1][r], acc[j + 2][r], acc[j + 3][r]};
    if (a == 0) {
      p.pre_m[pi] = m;
      p.pre_l[pi] = l;
    }
  } else if (whole) {
    const float inv = p.v_scale / l;
    const size_t oi = ((size_t)row * p.num_q_heads + h) * D + d0;
    if (p.q_f32) {
      float* op = reinterpret_cast<float*>(p.out) + oi;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < VEC; j += 4)
          *reinterpret_cast<f32x4*>(op + VEC * r + j) =
              f32x4{acc[j][r] * inv, acc[j + 1][r] * inv, acc[j + 2][r] * inv, acc[j + 3][r] * inv};
    } else {
      uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + oi;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < VEC; j += 4)
          *reinterpret_cast<u32x2*>(op + VEC * r + j) = u32x2{pack_bf16x2(acc[j][r] * inv, acc[j + 1][r] * inv),
                                                              pack_bf16x2(acc[j + 2][r] * inv, acc[j + 3][r] * inv)};
    }
  } else {
    const size_t pi = (size_t)(split + s) * p.num_q_heads + h;
    float* po = p.part_o + pi * D + d0;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < VEC; j += 4)
        *reinterpret_cast<f32x4*>(po + VEC * r + j) = f32x4{acc[j][r], acc[j + 1][r], acc[j + 2][r], acc[j + 3][r]};
    if (a == 0) {
      p.part_m[pi] = m;
      p.part_l[pi] = l;
    }
  }
}

// Q^T operand words of MFMA kk for lane (a, column): q[row][head][8*(a + 4*kk) .. +7] as bf16.
template <int D>
__device__ __forceinline__ u32x4 q_words(const DecodeParams& p, size_t qoff, int a, int kk) {
  const int d0 = 8 * (a + 4 * kk);
  if (p.q_f32) {
    const float* qp = reinterpret_cast<const float*>(p.query) + qoff + d0;
    return u32x4{pack_bf16x2(qp[0], qp[1]), pack_bf16x2(qp[2], qp[3]), pack_bf16x2(qp[4], qp[5]),
                 pack_bf16x2(qp[6], qp[7])};
  }
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.query) + qoff + d0);
}

// One wave, one piece: blocks [b0, b1) of sequence s (nb blocks in all) for q heads
// 16*hg .. 16*hg+15 of kv head kvh (all of them when the kv head has at most 16; more take
// one wave per group of 16, each reading the blocks), kInFlight blocks in flight while one
// is computed.
//
// GROUP (cascade prefix): the 16 columns are 16/G sequences x G heads instead of the G
// heads of one sequence, so each block of the shared prefix feeds 16/G sequences at
// once; s is the group's first sequence, split the prefix share, [b0, b1) blocks of
// the prefix (whole blocks, every key visible).  Otherwise the piece covers blocks
// [b0, b1) of sequence s after its skip_blocks shared blocks.
//
// WRITE (the decode that also writes the step's K/V): position seq_lens[s] - 1 holds the new
// row of s (row s of new_k / new_v).  The piece whose blocks hold it takes the row's slices
// in place of what the loads of that block return (the pool may still hold an older row
// there), and the waves of the first q-head group store them to the pool, at the slot the KV
// write uses.  Nobody else in the launch reads those bytes: the waves of the other q-head
// groups substitute the row as well, and other kv heads read other bytes of the token.
template <int D, bool FP8, bool GROUP = false, bool WRITE = false>
__device__ __forceinline__ void decode_piece(const DecodeParams& p, unsigned char* k_lds, int split, int kvh, int s,
                                             int b0, int b1, int nb, int hg = 0) {
  static_assert(!(GROUP && WRITE), "the cascade prefix holds no new rows");
  using Sh = DecodeShape<D, FP8>;
  constexpr int VEC = Sh::kVec;
  const int row = p.qsl ? p.qsl[s] : s;
  const int L = GROUP ? p.prefix_blocks * 16 : min(p.seq_lens[s], p.max_seq_len);
  const int skip = GROUP ? 0 : decode_skip(p, L);
  const int key_lo = GROUP ? 0 : decode_first_key(p, L);  // keys below it are outside the window
  const int tok0 = (skip + b0) * 16;
  const int tok1 = min(L, (skip + b1) * 16);
  const int nblk = b1 - b0;
  const bool whole = !GROUP && b0 == 0 && b1 == nb && !p.force_partial;

  const int lane = threadIdx.x & 63;
  const int a = lane >> 4, c = lane & 15;  // row group / column within the row group
  const int G = p.group;
  // the lane's column: q head g of query row col_row (col_ok: a real column)
  const int g = GROUP ? c % G : 16 * hg + c;
  const int col_seq = GROUP ? s + c / G : s;
  const bool col_ok = GROUP ? (c < (16 / G) * G && col_seq < p.num_seqs) : g < G;
  const int col_row = GROUP ? col_seq : row;

  bf16x8 qf[Sh::kKSteps];
  {
    const size_t qoff = ((size_t)col_row * p.num_q_heads + kvh * G + g) * D;
#pragma unroll
    for (int kk = 0; kk < Sh::kKSteps; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, col_ok ? q_words<D>(p, qoff, a, kk) : u32x4{0u, 0u, 0u, 0u});
  }

  float m = -INFINITY, l = 0.f;
  f32x4 acc[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int kElem = FP8 ? 1 : 2;
  const size_t row_stride = (size_t)p.num_kv_heads * D * kElem;  // bytes between token rows of a block
  const size_t block_bytes = row_stride * 16;
  // byte offsets of this lane's four rows inside a block (a block of one pool is < 4 GB)
  uint32_t roff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    roff[i] = (uint32_t)((a + 4 * i) * row_stride) + (uint32_t)(kvh * D * kElem) + (uint32_t)(c * Sh::kLoadBytes);
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.key_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.value_cache);
  // Physical block ids of the piece come through the scalar cache (wave-uniform addresses),
  // each read one issue before the loads that use it.  A vector load of the ids (a window of
  // 64 in a VGPR, reloaded when a piece crosses it) made the compiler wait for every vector
  // load in flight before each issue -- the reload might still be pending -- which drained
  // the blocks being prefetched.
  const int PA_CONST_AS* bt =
      (const int PA_CONST_AS*)(uintptr_t)(p.block_tables + (size_t)s * p.bt_stride + skip + b0);
  int phys_next = bt[0];

  // WRITE: block sub_blk of the piece (-1: none) holds the new row, at row sub_t of the block;
  // lanes of row group sub_t % 4 hold its slices
  // WRITE: block sub_blk of the piece (-1: none) holds the new row, at row sub_t of the block;
  // lanes of row group sub_t % 4 hold its slices.  The new row is the sequence's last position,
  // so sub_blk is the piece's last block when the piece holds it.
  int sub_blk = -1, sub_t = 0;
  NewRowSrc<D> ksrc{}, vsrc{};
  RawVec<Sh::kLoadBytes> nk{}, nv{};
  if constexpr (WRITE) {
    const int Lt = p.seq_lens[s];  // a sequence cut to max_seq_len has its new row outside the attended keys
    const int rel = ((Lt - 1) >> 4) - skip - b0;
    if (Lt >= 1 && Lt <= p.max_seq_len && rel == nblk - 1) {
      sub_blk = rel;
      sub_t = (Lt - 1) & 15;
    }
    sub_blk = wave_uniform(sub_blk);
    sub_t = wave_uniform(sub_t);
    // only loaded here: converted after the first blocks' loads are issued, so the wave does not
    // wait for this row before it starts streaming
    if (sub_blk >= 0 && (FP8 || a == (sub_t & 3))) load_new_row<D, FP8>(p, ksrc, vsrc, row, kvh, lane);
  }
  // Loads of block b of the partition.  Indices past the end re-read the last
  // block (cache-resident, no HBM traffic) so that the loop is branch-free and
  // the order of outstanding loads never depends on the data.
  auto issue = [&](BlockRegs<D, FP8>& r, int b) {
    // issues come for b = 0, 1, 2, ... in turn: this one's id was read by the previous one
    int phys = phys_next;
    phys_next = bt[min(b + 1, nblk - 1)];
    phys = min(max(phys, 0), p.num_blocks - 1);
    const uint8_t* kb = kbase + (size_t)phys * block_bytes;  // wave-uniform
    const uint8_t* vb = vbase + (size_t)phys * block_bytes;
    // a sequence's own blocks are streamed once; the shared prefix of a cascade is re-read by
    // every group of sequences and is left to the caches
    if constexpr (GROUP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) load_raw(r.k[i], kb + roff[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) load_raw(r.v[i], vb + roff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) load_raw_stream(r.k[i], kb + roff[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) load_raw_stream(r.v[i], vb + roff[i]);
    }
  };

  // Blocks rotate through kInFlight register sets (loads of the others in flight while one
  // is computed); blocks past the piece's end are fully masked copies of its last block
  // (no effect on m, l or the output).  Measured on the Llama-3-8B layer at one wave per
  // SIMD: 2 sets 89 us, 3 sets 92, 4 sets 94 (1 set 88 with more waves): the memory
  // system, not the wave's latency, is the limit.
  //
  // WRITE: the loop streams the blocks before the new row's block, which it sees fully masked
  // (its loads are the past-the-end re-reads); that block is attended after the loop, from a set
  // holding it, with the new row in place.  The hot loop stays the plain one, and the real
  // blocks are folded in the same order as without the write.
  constexpr int kSets = kInFlight<FP8>;
  const int nloop = sub_blk >= 0 ? sub_blk : nblk;
  const int tok1_loop = sub_blk >= 0 ? tok0 + sub_blk * 16 : tok1;
  BlockRegs<D, FP8> rs[kSets];
  static_for<0, kSets>([&](auto i_c) {
    issue(rs[decltype(i_c)::value], decltype(i_c)::value);
    __builtin_amdgcn_sched_barrier(0);
  });
  if constexpr (WRITE) {
    if (sub_blk >= 0) new_row_raw<D, FP8>(p, ksrc, vsrc, nk, nv, lane);
  }
  for (int b = 0; b < nloop; b += kSets) {
    static_for<0, kSets>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      block_step<D, FP8>(p, rs[i], k_lds, tok0 + (b + i) * 16, tok1_loop, key_lo, qf, m, l, acc);
      // bf16: a refill waits until the other sets have landed, so a wave streams about one
      // block ahead rather than kSets (the Llama-3-8B layer, 1024 waves: 87.7-87.9 us against
      // 88.8-89.7 with both 8 KB sets always in flight -- the memory system is already full);
      // fp8's 4 KB blocks keep every set in flight
      if constexpr (!FP8) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      // this block's registers are consumed: refill them with a later block
      issue(rs[i], b + i + kSets);
    });
  }

  // WRITE: the new row's block (every set holds it: the loop's last issues were past its end), then
  // the waves of the first q-head group store the row, at the slot the KV write uses
  if constexpr (WRITE) {
    if (sub_blk >= 0)
      block_step<D, FP8, true>(p, rs[0], k_lds, tok0 + sub_blk * 16, tok1, key_lo, qf, m, l, acc, &nk, &nv,
                               a == (sub_t & 3) ? sub_t >> 2 : -1);
    if (sub_blk >= 0 && hg == 0) {
      const int phys = bt[sub_blk];
      if (a == (sub_t & 3) && phys >= 0 && phys < p.num_blocks) {
        const size_t off = (size_t)phys * block_bytes + (size_t)sub_t * row_stride + (size_t)kvh * D * kElem +
                           (size_t)c * Sh::kLoadBytes;
        store_raw(const_cast<uint8_t*>(kbase) + off, nk);
        store_raw(const_cast<uint8_t*>(vbase) + off, nv);
      }
    }
  }

  // the four row groups hold partial sums over different tokens of the same head
  l = sum_across_rows(l);
  if (col_ok) piece_output<D, GROUP>(p, acc, m, l, kvh * G + g, split, s, row, col_seq, whole);
}

// With a cascade, the first groups * prefix_shares work-groups of each kv head take the
// shared prefix (cache-bound: every group re-reads the same blocks) and the rest the
// suffixes (HBM-bound), so the two overlap in one launch.
template <int D, bool FP8>
__device__ __forceinline__ bool prefix_piece(const DecodeParams& p, unsigned char* k_lds, int x, int kvh) {
  if (p.prefix_shares == 0) return false;
  const int per_group = 16 / p.group;
  const int groups = (p.num_seqs + per_group - 1) / per_group;
  if (x >= groups * p.prefix_shares) return false;
  const int share = x % p.prefix_shares, group = x / p.prefix_shares;
  const int b0 = (int)((long long)p.prefix_blocks * share / p.prefix_shares);
  const int b1 = (int)((long long)p.prefix_blocks * (share + 1) / p.prefix_shares);
  if (b1 > b0) decode_piece<D, FP8, true>(p, k_lds, share, kvh, group * per_group, b0, b1, p.prefix_blocks);
  return true;
}

// One decode wave: share x (the first prefix_waves ids take the cascade's shared prefix)
// of kv head y / head_groups, q-head group y % head_groups.  k_lds: this wave's 16 rows of
// K (DecodeShape::kLdsBytes).
// WRITE: the waves also store the step's new K/V rows (no cascade).
template <int D, bool FP8, bool WRITE = false>
__device__ __forceinline__ void decode_wave(const DecodeParams& p, unsigned char* k_lds, int x, int y) {
  const int kvh = y / p.head_groups, hg = y % p.head_groups;
  if constexpr (!WRITE) {
    if (prefix_piece<D, FP8>(p, k_lds, x, kvh)) return;
  }
  const int split = x - p.prefix_waves;
  for_each_piece(p, split, [&](int s, int b0, int b1, int nb) {
    if (y == 0 && (threadIdx.x & 63) == 0) note_piece(p, split, s, b0, b1, nb);
    decode_piece<D, FP8, false, WRITE>(p, k_lds, split, kvh, s, b0, b1, nb, hg);
  });
}

}  // namespace

}  // namespace pa
