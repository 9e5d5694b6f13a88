// Both classes' tiles in one launch: the first p.dec_waves / 4 workgroups
// run the decode-class tiles (those the planner gives no work exit at once
// and leave their place to prefill workgroups), the others take
// prefill-class items from the queues until they are empty. The two kinds of
// workgroup have the same size and share one LDS and register budget, so a
// compute unit can hold one of each: the HBM-bound decode streams K/V while
// the MFMA-bound prefill runs beside it. Used wherever the decode and
// prefill workgroups have the same shape (all but the two-group prefill
// kernel's configurations).
#pragma once

#include "rpa_decode.h"
#include "rpa_prefill.h"
#include "rpa_prefill_pp.h"

namespace rpa {

constexpr int tiles_waves_per_simd(int D, bool fp8) {
  return dec_waves_per_simd(D, fp8) < pf_wgs_per_cu(D) ? dec_waves_per_simd(D, fp8) : pf_wgs_per_cu(D);
}

template <int D, int KVT, bool CAP, bool F16, bool Q32 = false>
__global__ __launch_bounds__(kDecWavesPerBlock * 64, tiles_waves_per_simd(D, KVT != kKvBf16)) void tiles_kernel(
    Params p) {
  constexpr bool FP8 = KVT != kKvBf16;
  static_assert(kDecWavesPerBlock == kPfWaves, "one workgroup size for both classes");
  constexpr size_t kDec = (size_t)kDecWavesPerBlock * DecCfg<D, FP8>::WAVE_LDS;
  constexpr size_t kPf = sizeof(PfShared<D, FP8>);
  __shared__ __attribute__((aligned(1024))) char lds[kDec > kPf ? kDec : kPf];
  const int dec_wgs = p.dec_waves / kDecWavesPerBlock;
  if ((int)blockIdx.x < dec_wgs)
    decode_tiles<D, KVT, CAP, F16, Q32>(p, lds, blockIdx.x);
  else
    prefill_tiles<D, KVT, CAP, F16, Q32>(p, *reinterpret_cast<PfShared<D, FP8>*>(lds), blockIdx.x - dec_wgs);
}

// The same for the two-group prefill kernel's configurations (16-bit K/V in
// the q type at head_dim 256): eight-wave workgroups, one per compute unit.
// A decode workgroup runs its decode waves on the first four waves (the
// others exit at once) within the two-group kernel's budget of 256 registers
// per wave, which the head_dim-256 decode fits without spilling. The decode
// workgroups take whole compute units, so the classes share the chip by
// compute unit rather than inside one.
template <int D, bool CAP, bool F16>
__global__ __launch_bounds__(kPpWaves * 64, 1) void tiles_pp_kernel(Params p) {
  static_assert(kPpWaves >= kDecWavesPerBlock, "the decode waves fit a two-group workgroup");
  constexpr size_t kDec = (size_t)kDecWavesPerBlock * DecCfg<D, false>::WAVE_LDS;
  constexpr size_t kPf = sizeof(PpShared<D>);
  __shared__ __attribute__((aligned(1024))) char lds[kDec > kPf ? kDec : kPf];
  const int dec_wgs = p.dec_waves / kDecWavesPerBlock;
  if ((int)blockIdx.x >= dec_wgs) {
    prefill_pp_tiles<D, CAP, F16>(p, *reinterpret_cast<PpShared<D>*>(lds), blockIdx.x - dec_wgs);
  } else if (threadIdx.x < kDecWavesPerBlock * 64) {
    decode_tiles<D, kKvBf16, CAP, F16, false>(p, lds, blockIdx.x);
  }
}

}  // namespace rpa
