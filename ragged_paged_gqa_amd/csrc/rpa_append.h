// rpa_append.h — writing a step's new K and V rows into the paged cache.
//
// The ragged paged attention kernel page (zml platforms/tpu/ragged_paged.zig)
// reads a cache that already holds every query token's own key; this is the
// write that puts it there, by the page's own placement rule (`run` and the
// row ids of `flashAttention`): query token i of sequence s stands at key
// position kv_len - q_len + i, and key j is slot j % page_size of page
// page_indices[s, j / page_size], K of kv head h in combined head 2h and V in
// 2h+1 (`stridedLoadKv`). A stored value inverts the attention's dequant
// factor: RN_f32(x / scale), rounded to nearest even in the cache type
// (e4m3fn saturates at +-448, e5m2 at +-57344; NaN stays NaN; int8 rounds
// to an integer, ties to even, saturating at -128 / 127, NaN to 0). New rows
// come in the q type (bf16, f16 or f32).
//
// HBM-bound: per token 2*Hkv*D elements of the q type are read and 2*Hkv*D
// cache elements written, contiguous on both sides. One wave per token; each lane
// moves 16-byte chunks (8 elements), loads first, then converts and stores.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "rpa_common.h"

namespace rpa {

constexpr int kApWaves = 4;   // waves per workgroup, one token each at a time
constexpr int kApUnroll = 4;  // 16-byte chunks in flight per lane

// Element type of the new rows (template parameter IN): the q type.
constexpr int kInBf16 = 0;
constexpr int kInF16 = 1;
constexpr int kInF32 = 2;

// Eight new elements (one 8-element chunk of a row) as loaded.
template <int IN>
struct ApChunk {
  u32x4 w[IN == kInF32 ? 2 : 1];
};

// Cache element type of an append launch.
enum ApMode : int {
  kApCopy = 0,  // cache in the rows' own 16-bit type, both scales 1: the quotient is x itself
  kApBf16 = 1,  // bf16 cache, general scales
  kApFp8 = 2,   // e4m3fn cache
  kApE5M2 = 3,  // e5m2 cache
  kApF16 = 4,   // f16 cache, general scales
  kApI8 = 5,    // int8 cache
};

struct AppendParams {
  const void* k_new;      // [T, Hkv, D] elements of the q type (bf16, f16 or f32)
  const void* v_new;      // [T, Hkv, D] elements of the q type
  void* kv;               // [P, page_size, 2*Hkv, D] cache elements
  const int32_t* kv_lens;
  const int32_t* page_indices;
  const int32_t* cu_q_lens;
  const int32_t* num_seqs;
  int T, Hkv, P, page_size, max_num_seqs, pps;
  float k_scale, v_scale;
};

// Sequence holding token t: the last s < nseq with cu[s] <= t, given
// cu[0] <= t. The candidate range shrinks 64-fold per round, one probe per
// lane; every probe stays inside cu[0, nseq) whatever cu holds.
__device__ __forceinline__ int ap_seq_of_token(const int32_t* cu, int nseq, int t) {
  const int lane = threadIdx.x & 63;
  int lo = 0, n = nseq;
  while (n > 1) {
    const int step = (n + 63) >> 6;
    const int k = lane * step;
    const bool le = k < n && cu[lo + k] <= t;
    const int c = __popcll(__ballot(le));  // >= 1: lane 0 probes cu[lo] <= t
    lo += (c - 1) * step;
    n = min(step, n - (c - 1) * step);
  }
  return lo;
}

// Element i (0..7) of a chunk as f32, exactly.
template <int IN>
__device__ __forceinline__ float ap_elem(const ApChunk<IN>& x, int i) {
  if constexpr (IN == kInF32) {
    return __uint_as_float(x.w[i >> 2][i & 3]);
  } else {
    const uint32_t w = x.w[0][i >> 1];
    if constexpr (IN == kInF16)
      return (float)__builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFFu)));
    else
      return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
}

// fp8 code pair (e4m3fn, or e5m2) of two f32 quotients into the low (HI
// false) or high 16 bits of `old`: clamp to the finite range (NaN kept),
// then the hardware conversion, round to nearest even.
template <bool HI, bool E5M2>
__device__ __forceinline__ uint32_t ap_fp8_pair(float a, float b, uint32_t old) {
  constexpr float kMax = E5M2 ? 57344.f : 448.f;  // largest finite value
  const float ca = __builtin_amdgcn_fmed3f(a, -kMax, kMax);
  const float cb = __builtin_amdgcn_fmed3f(b, -kMax, kMax);
  if constexpr (E5M2)
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a == a ? ca : a, b == b ? cb : b, (int)old, HI);
  else
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a == a ? ca : a, b == b ? cb : b, (int)old, HI);
}

// Loads chunks c0, c0+64, ... (kApUnroll of them, those below nch) of one
// token's K|V rows: chunk c is 8 elements of combined head c / (D/8).
template <int D, int IN>
__device__ __forceinline__ void load_chunks(ApChunk<IN> (&x)[kApUnroll], const char* kr, const char* vr, int c0,
                                            int nch) {
  constexpr int CPR = D / 8;
  constexpr int ES = IN == kInF32 ? 4 : 2;  // bytes per new element
#pragma unroll
  for (int u = 0; u < kApUnroll; ++u) {
    const int c = c0 + 64 * u;
    if (c < nch) {
      const int ch = c / CPR;  // combined head: 2h = K, 2h+1 = V
      const char* src = ((ch & 1) ? vr : kr) + ((ch >> 1) * D + (c % CPR) * 8) * ES;
#pragma unroll
      for (int k = 0; k < (IN == kInF32 ? 2 : 1); ++k) x[u].w[k] = *reinterpret_cast<const u32x4*>(src + 16 * k);
    }
  }
}

// Converts and stores the chunks load_chunks fetched; e_slot is the slot's
// first cache element.
template <int D, int MODE, int IN>
__device__ __forceinline__ void store_chunks(const ApChunk<IN> (&x)[kApUnroll], const AppendParams& p,
                                             int64_t e_slot, int c0, int nch) {
  static_assert(MODE != kApCopy || IN != kInF32, "a bit copy needs 16-bit rows");
  constexpr int CPR = D / 8;
#pragma unroll
  for (int u = 0; u < kApUnroll; ++u) {
    const int c = c0 + 64 * u;
    if (c >= nch) continue;
    const int64_t e0 = e_slot + (int64_t)c * 8;
    if (MODE == kApCopy) {
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.kv) + e0) = x[u].w[0];
      continue;
    }
    const float sc = ((c / CPR) & 1) ? p.v_scale : p.k_scale;
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = ap_elem<IN>(x[u], i) / sc;
    if (MODE == kApBf16 || MODE == kApF16) {
      u32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = pack2<MODE == kApF16>(f[2 * i], f[2 * i + 1]);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.kv) + e0) = y;
    } else if (MODE == kApI8) {
      // nearest integer, ties to even, saturated to [-128, 127]; NaN -> 0
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float r = __builtin_rintf(__builtin_amdgcn_fmed3f(f[i], -128.f, 127.f));
        b[i] = (uint32_t)(f[i] == f[i] ? (int)r : 0) & 0xFFu;
      }
      const u32x2 y = {b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
      *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(p.kv) + e0) = y;
    } else {
      u32x2 y;
      constexpr bool E5 = MODE == kApE5M2;
      y[0] = ap_fp8_pair<true, E5>(f[2], f[3], ap_fp8_pair<false, E5>(f[0], f[1], 0u));
      y[1] = ap_fp8_pair<true, E5>(f[6], f[7], ap_fp8_pair<false, E5>(f[4], f[5], 0u));
      *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(p.kv) + e0) = y;
    }
  }
}

template <int D, int MODE, int IN>
__global__ __launch_bounds__(kApWaves * 64) void kv_append_kernel(AppendParams p) {
  constexpr int CPR = D / 8;  // 16-byte chunks per head row
  const int lane = threadIdx.x & 63;
  const int nseq = min(max(p.num_seqs[0], 0), p.max_num_seqs);
  if (nseq == 0) return;
  const int t_begin = max(p.cu_q_lens[0], 0);
  const int t_end = min(p.cu_q_lens[nseq], p.T);
  const int nch = 2 * p.Hkv * CPR;
  const int stride = gridDim.x * kApWaves;
  const int64_t pos_cap = (int64_t)p.pps * p.page_size;
  // wave-uniform token loop
  for (int t = t_begin + blockIdx.x * kApWaves + (int)(threadIdx.x >> 6); t < t_end; t += stride) {
    constexpr int ES = IN == kInF32 ? 4 : 2;
    const char* kr = static_cast<const char*>(p.k_new) + (int64_t)t * p.Hkv * D * ES;
    const char* vr = static_cast<const char*>(p.v_new) + (int64_t)t * p.Hkv * D * ES;
    // the token's first rows are in flight while its slot is looked up
    ApChunk<IN> x[kApUnroll];
    load_chunks<D, IN>(x, kr, vr, lane, nch);
    const int s = ap_seq_of_token(p.cu_q_lens, nseq, t);
    const int q0 = p.cu_q_lens[s];
    const int q_len = p.cu_q_lens[s + 1] - q0;
    const int64_t pos = (int64_t)p.kv_lens[s] - q_len + (t - q0);
    if (pos < 0 || pos >= pos_cap) continue;
    const int page = p.page_indices[(int64_t)s * p.pps + pos / p.page_size];
    if (page < 0 || page >= p.P) continue;
    const int64_t slot = (int64_t)page * p.page_size + pos % p.page_size;
    for (int c0 = lane;;) {
      store_chunks<D, MODE, IN>(x, p, slot * 2 * p.Hkv * D, c0, nch);
      c0 += 64 * kApUnroll;
      if (c0 >= nch) break;
      load_chunks<D, IN>(x, kr, vr, c0, nch);
    }
  }
}

}  // namespace rpa
