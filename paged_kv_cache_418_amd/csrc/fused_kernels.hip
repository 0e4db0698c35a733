// Decode rows and prefill chunks of one flattened batch in a single launch.
//
// A continuous-batching step mixes the two regimes the reading note on "Inside vLLM"
// (core point 2) names: decode rows are bound by memory bandwidth, chunked-prefill chunks
// by the matrix cores.  Run one after the other, the chunks' matrix-core work waits for the
// decode stream.  Here one launch holds both: its first n_decode_wgs work-groups run decode
// waves (eight per work-group, the decode kernel's shares), the rest run prefill work items
// (the prefill kernel's items, one per work-group).  Every work-group has the prefill
// kernel's shape (512 threads, the prefill LDS), so each compute unit holds one; the decode
// work-groups are dispatched first and keep their compute units streaming K/V from HBM while
// the prefill items run on the others.  The host plan sizes the two parts so that they end
// together; the decode merge and the prefill merge follow as in the separate launches.
#include <type_traits>

#include "decode_body.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "prefill_body.h"

namespace pa {

namespace {

// WRITE: the launch also stores the step's new K/V rows.  The decode waves store and attend their
// rows as the decode that writes does (f.dec.new_k / new_v); with a cascade those lie in each
// sequence's own blocks, never in the shared prefix the tiles read.  Without one (bf16 pools, no
// window) the prefill items take their chunks' new keys from the input rows (prefill_body's FRESH
// form) and the decode merge launch that follows stores them.
template <int D, bool WINDOW, bool FP8, bool PREFIX, bool WRITE = false>
__global__ void __launch_bounds__(512) fused_kernel(FusedParams f) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int wg = blockIdx.x;
  if (wg < f.n_decode_wgs) {
    const int wave = threadIdx.x >> 6;
    const int g = wg * f.decode_waves_per_wg + wave;  // decode wave: share g / Y of column g % Y
    if (wave >= f.decode_waves_per_wg || g >= f.decode_waves) return;
    const int Y = f.dec.num_kv_heads * f.dec.head_groups;
    decode_wave<D, FP8, WRITE>(f.dec, smem + wave * DecodeShape<D, FP8>::kLdsBytes, g / Y, g % Y);
    return;
  }
  // prefill items in the order of the prefill kernel's grid (kv heads fastest)
  const int w = wg - f.n_decode_wgs;
  prefill_body<D, WINDOW, PREFIX, FP8, WRITE && !PREFIX>(f.pre, smem, w / f.pre.num_kv_heads, w % f.pre.num_kv_heads);
}

}  // namespace

size_t prefill_lds_bytes(int head_dim);

hipError_t launch_fused(const FusedParams& f, int head_dim, bool fp8, hipStream_t stream, int timing_id) {
  const bool win = f.pre.window > 0 || f.pre.chunk > 0;
  const bool prefix = f.pre.prefix_keys > 0;  // cascade prefix tiles (never with a window)
  const dim3 grid(f.n_decode_wgs + f.pre.n_items * f.pre.num_kv_heads);
  const size_t lds = prefill_lds_bytes(head_dim);
  timing_mark(timing_id, true, stream);
  auto launch = [&](auto kernel) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    hipLaunchKernelGGL(kernel, grid, dim3(512), lds, stream, f);
  };
  auto pick = [&](auto d_c, auto fp8_c) {
    constexpr int D = decltype(d_c)::value;
    constexpr bool F = decltype(fp8_c)::value;
    if (prefix && f.dec.new_k)
      launch(&fused_kernel<D, false, F, true, true>);
    else if (prefix)
      launch(&fused_kernel<D, false, F, true>);
    else if (!F && !win && f.dec.new_k)  // the caller checks: fresh rows only over bf16 pools, no window
      launch(&fused_kernel<D, false, false, false, true>);
    else if (win)
      launch(&fused_kernel<D, true, F, false>);
    else
      launch(&fused_kernel<D, false, F, false>);
  };
  using T = std::true_type;
  using F = std::false_type;
  if (head_dim == 128)
    fp8 ? pick(std::integral_constant<int, 128>{}, T{}) : pick(std::integral_constant<int, 128>{}, F{});
  else
    fp8 ? pick(std::integral_constant<int, 64>{}, T{}) : pick(std::integral_constant<int, 64>{}, F{});
  timing_mark(timing_id, false, stream);
  return hipGetLastError();
}

}  // namespace pa
