// Shared device-side definitions of the ragged paged attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rpa_layout.h"

namespace rpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ----------------------------------------------------------------------------
// Everything a kernel needs, passed by value.
struct Params {
  // inputs
  const uint16_t* q;         // [T, Hq, D] q elements: bf16 / f16 bits, or f32 (read as float)
  const uint8_t* kv;         // [P, page, 2Hkv, D] bf16 or fp8 bytes
  const int32_t* kv_lens;
  const int32_t* page_indices;
  const int32_t* cu_q_lens;
  const int32_t* num_seqs;
  // outputs
  uint16_t* out;             // [T, Hq, D] out elements in the q type (f32 written as float)
  float* lse;                // [T, Hq] or null
  // workspace views
  Header* hdr;
  DecSeq* dec_seqs;          // decode sequence table [S_max]
  Unit* pf_units;
  Item* pf_items;
  int32_t* pf_qlist;         // prefill item indices in queue order [kQueues][max_pf_items]
  int32_t* unit_done;        // finished chunks per prefill unit [max_pf_units]
  float* dec_part;           // [2 * dec_waves][kDecRows][D]: partial slots 2w, 2w + 1 of decode wave w
  float* dec_plse;           // [2 * dec_waves][kDecRows]
  float* pf_part;            // [max_pf_items][pf_rows][D]
  float* pf_plse;            // [max_pf_items][pf_rows]
  // shapes
  int32_t T, Hq, Hkv, G, D, page, P, S_max, pps;
  int32_t pf_rows;           // packed rows of a prefill-class unit
  int32_t max_dec_units, max_pf_units, max_pf_items;
  int32_t target_pf_items;
  int32_t dec_waves;         // waves of the decode launch (the stream-K split)
  int32_t dec_blk;           // keys per stream-K block: 16, or 32 for one-byte K/V (kDecBlk)
  int32_t dec_per_cu;        // decode workgroups resident per compute unit
  int32_t fused;             // 1: one launch holds the workgroups of both classes (tiles_kernel)
  const float* sinks;        // [Hq] attention-sink logits, or null
  // numerics
  float sm_scale;      // sm_scale * k_scale
  float soft_cap;      // > 0: on
  float v_scale;
  int32_t is_causal;
  int32_t window;      // > 0: on
};

// ----------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Final statistics of a row from its reference maximum m (base-2 units, -inf
// while no key was seen) and its sum l of 2^(score - m): the factor that
// normalises the row's accumulated O (v_scale folded in) and the row's
// log-sum-exp (natural log). An attention sink (`sink`: a logit in
// natural-log units, compared with the scaled and capped scores; null: none)
// joins the maximum and the denominator and carries no value, as the
// spatial-compiler page's `flat_softmax_rows_at` takes its `sinks`. Without a
// sink this is v_scale / l and (m + log2 l) ln 2 exactly.
__device__ __forceinline__ void row_final(float m, float l, float v_scale, const float* sink, float& inv,
                                          float& lse) {
  const float sb = sink ? *sink * 1.4426950408889634f : -INFINITY;
  const float mf = fmaxf(m, sb);
  if (mf == -INFINITY || !(l > 0.f || sb > -INFINITY)) {
    inv = 0.f;
    lse = -INFINITY;
    return;
  }
  const float a = l > 0.f ? fast_exp2(m - mf) : 0.f;
  const float lt = l * a + (sb > -INFINITY ? fast_exp2(sb - mf) : 0.f);
  inv = v_scale * a / lt;
  lse = (mf + fast_log2(lt)) * 0.6931471805599453f;
}

// Soft-cap in base-2 units: for a raw score s, log2(e) * c * tanh(scale * s /
// c), as c' - 2c' / (1 + e^(2 scale s / c)) with c' = c log2(e): one exp2 and
// one reciprocal (the logistic form of the spatial-compiler page's `capped`
// soft-cap), the scale and the change to base 2 folded into the constants.
// Saturates to +-c' for large |s| (e^.. -> inf gives c', -> 0 gives -c').
struct SoftCapB2 {
  float a;   // scale * 2 log2(e) / c
  float c1;  // c log2(e)
  float c2;  // 2 c log2(e)
  __device__ __forceinline__ SoftCapB2(float scale, float c)
      : a(scale * 2.0f * 1.4426950408889634f / c), c1(c * 1.4426950408889634f), c2(2.0f * c * 1.4426950408889634f) {}
  __device__ __forceinline__ float operator()(float s) const {
    return __builtin_fmaf(-c2, fast_rcp(1.0f + fast_exp2(s * a)), c1);
  }
  // the same plus a uniform offset (folded into the FMA's addend)
  __device__ __forceinline__ float offset(float s, float off) const {
    return __builtin_fmaf(-c2, fast_rcp(1.0f + fast_exp2(s * a)), c1 + off);
  }
};

__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// The 16-bit operand and output type of an attention path is bf16, or f16
// (template parameter F16, the page's `Cfg` q_dtype). 16-bit vectors travel
// as bf16x* bits either way; F16 picks the f16 conversions and MFMAs.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two f32 -> two 16-bit values (round to nearest even), lo in the low half.
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (F16) {
    const f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    return bf16x2_bits(lo, hi);
  }
}

// An f32 q (template parameter Q32 of the attention kernels, computed on the
// bf16 path): each element x is carried as hi = RN_bf16(x) and
// lo = RN_bf16(x - hi), both exact enough that hi + lo is within 2^-17 |x| of
// x (x - hi is an f32 value exactly, and lo rounds it to 8 significant bits).
// The score is K.hi + K.lo, two MFMA chains into one f32 accumulator; K is
// bf16 or a one-byte code widened exactly, so only the lo rounding is lost.
// Out is written in f32. Eight f32 elements -> the hi and lo operands:
__device__ __forceinline__ void split_q8(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack2<false>(x[2 * i], x[2 * i + 1]);
    const float r0 = x[2 * i] - __uint_as_float(h[i] << 16);
    const float r1 = x[2 * i + 1] - __uint_as_float(h[i] & 0xFFFF0000u);
    l[i] = pack2<false>(r0, r1);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// Four results -> out elements [e, e + 4): the 16-bit type, or f32 (Q32).
template <bool F16, bool Q32>
__device__ __forceinline__ void store_out4(uint16_t* out, int64_t e, float a, float b, float c, float d) {
  if constexpr (Q32)
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + e) = f32x4{a, b, c, d};
  else
    *reinterpret_cast<u32x2*>(out + e) = u32x2{pack2<F16>(a, b), pack2<F16>(c, d)};
}

// K/V element types of the attention kernels (template parameter KVT).
constexpr int kKvBf16 = 0;
constexpr int kKvE4M3 = 1;  // OCP fp8 e4m3fn
constexpr int kKvE5M2 = 2;  // OCP fp8 e5m2
constexpr int kKvI8 = 3;    // signed 8-bit integer codes

// Eight fp8 codes (two dwords) -> eight f16, exactly: every e4m3fn and every
// e5m2 value (infinities and NaN included) is an f16 value. (Bits in a bf16x8.)
template <int KVT>
__device__ __forceinline__ bf16x8 fp8x8_to_f16(u32x2 w) {
  static_assert(KVT == kKvE4M3 || KVT == kKvE5M2, "an fp8 kind");
  f16x2 a, b, c, d;
  if constexpr (KVT == kKvE5M2) {
    a = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8((int)w[0], 1.0f, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8((int)w[0], 1.0f, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8((int)w[1], 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8((int)w[1], 1.0f, true);
  } else {
    a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[0], 1.0f, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[0], 1.0f, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[1], 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[1], 1.0f, true);
  }
  const u32x4 r = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                   __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, r);
}

// Eight fp8 codes (two dwords) -> eight bf16, exactly: every e4m3fn and every
// e5m2 value (infinities and NaN included) is a bf16 value.
template <int KVT>
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w) {
  static_assert(KVT == kKvE4M3 || KVT == kKvE5M2, "an fp8 kind");
  bf16x2 a, b, c, d;
  if constexpr (KVT == kKvE5M2) {
    a = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w[0], 1.0f, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w[0], 1.0f, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w[1], 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w[1], 1.0f, true);
  } else {
    a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[0], 1.0f, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[0], 1.0f, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[1], 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[1], 1.0f, true);
  }
  bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Values known to be equal on every lane, moved to scalar registers (so the
// compiler treats them, and what is computed from them, as wave-uniform).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A pointer known to be equal on every lane, moved to scalar registers.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* ptr) {
  const uint64_t v = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

// Scalar (SMEM) loads of metadata the kernel never writes: page-table entries
// and sequence records go to scalar registers through the scalar cache and
// never wait on (or make anything wait on) the K/V stream.
typedef const __attribute__((address_space(4))) int32_t cint32;
__device__ __forceinline__ int sload(const int32_t* ptr) { return *(cint32*)(ptr); }

// A prefill item's record: one 64-byte load (the same address on every
// lane). The planning kernel wrote it before this launch.
__device__ __forceinline__ Item load_item(const Params& p, int item) { return p.pf_items[item]; }

// Index of the XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ int xcc_id() {
  int v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v;
}

// Split-KV partials cross workgroups (and XCDs, whose L2 caches are not
// coherent with each other). They are written and read with device-coherent
// (agent-scope) accesses, which bypass the per-XCD L2 state, so the handoff
// needs no L2 write-back or invalidate: the writer waits for its stores to
// complete, then bumps the unit's counter; the merger reads after the counter.
__device__ __forceinline__ void store_coherent(float* dst, float v) {
  __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent4(float* dst, f32x4 v) {  // dst 16-byte aligned
  unsigned long long* d = reinterpret_cast<unsigned long long*>(dst);
  __hip_atomic_store(d, __builtin_bit_cast(unsigned long long, f32x2{v[0], v[1]}), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 1, __builtin_bit_cast(unsigned long long, f32x2{v[2], v[3]}), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* src) {
  return __hip_atomic_load(const_cast<float*>(src), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The next prefill-class item for a workgroup (called by one thread): this
// XCD's queue first (`home`), then the others in turn; -1 once all are
// drained. `qsel` counts the queues this workgroup has found drained. While
// the home queue lasts an item costs one atomic. After that the heads are
// read together (relaxed, device scope: one round trip), and only queues
// that still look non-empty take an atomic: a head only grows, and all eight
// share one cache line, where an atomic from every workgroup on every
// drained queue would queue up behind each other while items remain.
__device__ inline int take_item(const Params& p, int home, int& qsel) {
  if (qsel == 0) {
    const int k = atomicAdd(&p.hdr->pf_q_next[home], 1);
    if (k < p.hdr->pf_q_count[home]) return p.pf_qlist[p.hdr->pf_q_base[home] + k];
    qsel = 1;
  }
  uint32_t live = 0;  // queues whose head was below their length when read
#pragma unroll
  for (int x = 0; x < kQueues; ++x) {
    const int head = __hip_atomic_load(&p.hdr->pf_q_next[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    live |= (uint32_t)(head < p.hdr->pf_q_count[x]) << x;
  }
  for (; qsel < kQueues; ++qsel) {
    const int x = (home + qsel) % kQueues;
    if (!((live >> x) & 1u)) continue;
    const int k = atomicAdd(&p.hdr->pf_q_next[x], 1);
    if (k < p.hdr->pf_q_count[x]) return p.pf_qlist[p.hdr->pf_q_base[x] + k];
  }
  return -1;
}
__device__ __forceinline__ f32x2 load_coherent2(const float* src) {  // src 8-byte aligned
  unsigned long long* s = reinterpret_cast<unsigned long long*>(const_cast<float*>(src));
  return __builtin_bit_cast(f32x2, __hip_atomic_load(s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// Wait until this wave's stores have completed (and are therefore visible to
// device-coherent reads); also a compiler barrier.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Lane l and lane l ^ 16 (l ^ 32) exchange values with v_permlane16_swap
// (v_permlane32_swap): no LDS round trip. Each swap returns the pair (own,
// partner) in some order, and max / sum do not care which.
__device__ __forceinline__ float max_xor16(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float wave_max_xor16_32(float v) { return max_xor32(max_xor16(v)); }
__device__ __forceinline__ float wave_sum_xor16_32(float v) { return sum_xor32(sum_xor16(v)); }

// Eight int8 codes (two dwords, element k in byte k) -> eight bf16 or f16,
// exactly (|code| <= 128 needs 8 significant bits).
template <bool F16>
__device__ __forceinline__ bf16x8 i8x8_to_16(u32x2 w) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t word = w[i >> 1];
    const int sh = 16 * (i & 1);
    r[i] = pack2<F16>((float)(int8_t)(word >> sh), (float)(int8_t)(word >> (sh + 8)));
  }
  return __builtin_bit_cast(bf16x8, r);
}

// One-byte K/V codes (fp8 kinds, int8) -> the path's 16-bit type.
template <int KVT, bool F16>
__device__ __forceinline__ bf16x8 fp8x8_to_16(u32x2 w) {
  if constexpr (KVT == kKvI8)
    return i8x8_to_16<F16>(w);
  else if constexpr (F16)
    return fp8x8_to_f16<KVT>(w);
  else
    return fp8x8_to_bf16<KVT>(w);
}

template <bool F16>
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS transpose read: within each 16-lane group, lane 4q+r receives element r
// of the 8-byte rows loaded by lanes q, q+4, q+8, q+12 (measured on gfx950).
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// 16 bytes per lane from global memory straight into LDS at lds_addr + 16 *
// lane (global_load_lds_dwordx4; lds_addr is the wave-uniform LDS byte
// address, passed through M0, which is restored afterwards). Written as inline
// assembly so that the compiler does not add its own conservative wait for the
// LDS write before every later LDS read: completion is tracked explicitly with
// wait_vmcnt before the barrier that publishes a stage. An SALU write of M0
// needs one wait state before an instruction that reads M0 (the compiler puts
// the same s_nop between its own M0 write and LDS DMA); one more keeps the
// restore clear of the DMA.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}

// Same, with the global address split into a wave-uniform 64-bit base (SGPR
// pair) and a per-lane 32-bit byte offset: no per-lane 64-bit address math.
__device__ __forceinline__ void dma16_sbase(const uint8_t* sbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_addr)
      : "memory");
}

// N full-width DMA instructions in one M0 window: instruction j reads
// sbase + voff[j] (per lane) into LDS at lds_addr + j * STRIDE + 16 * lane,
// issued only when `go` (wave-uniform) is non-zero. One asm statement, branch
// included, so that nothing the compiler schedules can see the borrowed M0
// and its basic block stays whole; every M0 write is followed by the wait
// state LDS DMA needs.
#define RPA_DMA_LD(j) "global_load_lds_dwordx4 %" #j ", %[sb]\n\t"
#define RPA_DMA_ADV "s_add_u32 m0, m0, %[st]\n\ts_nop 0\n\t"
#define RPA_DMA_HEAD "s_cmp_eq_u32 %[go], 0\n\ts_cbranch_scc1 .Ldma_skip_%=\n\t" \
                     "s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[la]\n\ts_nop 0\n\t"
#define RPA_DMA_TAIL "s_mov_b32 m0, %[sv]\n.Ldma_skip_%=:"
template <int STRIDE>
__device__ __forceinline__ void dma16_rows2(const uint8_t* sbase, const uint32_t (&voff)[2], uint32_t lds_addr,
                                            uint32_t go = 1) {
  uint32_t saved;
  asm volatile(RPA_DMA_HEAD RPA_DMA_LD(1) RPA_DMA_ADV RPA_DMA_LD(2) RPA_DMA_TAIL
               : [sv] "=&s"(saved)
               : "v"(voff[0]), "v"(voff[1]), [sb] "s"(sbase), [la] "s"(lds_addr), [st] "n"(STRIDE), [go] "s"(go)
               : "memory", "scc");
}
template <int STRIDE>
__device__ __forceinline__ void dma16_rows4(const uint8_t* sbase, const uint32_t (&voff)[4], uint32_t lds_addr,
                                            uint32_t go = 1) {
  uint32_t saved;
  asm volatile(RPA_DMA_HEAD RPA_DMA_LD(1) RPA_DMA_ADV RPA_DMA_LD(2) RPA_DMA_ADV RPA_DMA_LD(3) RPA_DMA_ADV
               RPA_DMA_LD(4) RPA_DMA_TAIL
               : [sv] "=&s"(saved)
               : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), [sb] "s"(sbase), [la] "s"(lds_addr),
                 [st] "n"(STRIDE), [go] "s"(go)
               : "memory", "scc");
}
template <int STRIDE>
__device__ __forceinline__ void dma16_rows8(const uint8_t* sbase, const uint32_t (&voff)[8], uint32_t lds_addr,
                                            uint32_t go = 1) {
  uint32_t saved;
  asm volatile(RPA_DMA_HEAD RPA_DMA_LD(1) RPA_DMA_ADV RPA_DMA_LD(2) RPA_DMA_ADV RPA_DMA_LD(3) RPA_DMA_ADV
               RPA_DMA_LD(4) RPA_DMA_ADV RPA_DMA_LD(5) RPA_DMA_ADV RPA_DMA_LD(6) RPA_DMA_ADV RPA_DMA_LD(7)
               RPA_DMA_ADV RPA_DMA_LD(8) RPA_DMA_TAIL
               : [sv] "=&s"(saved)
               : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "v"(voff[4]), "v"(voff[5]), "v"(voff[6]),
                 "v"(voff[7]), [sb] "s"(sbase), [la] "s"(lds_addr), [st] "n"(STRIDE), [go] "s"(go)
               : "memory", "scc");
}
#undef RPA_DMA_LD
#undef RPA_DMA_ADV
#undef RPA_DMA_HEAD
#undef RPA_DMA_TAIL

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(size_t)((const __attribute__((address_space(3))) char*)p);
}

// Physical page of key `key` of sequence s, clamped into [0, P).
__device__ __forceinline__ int32_t page_of(const Params& p, int32_t s, int32_t key) {
  int32_t logical = key / p.page;
  logical = logical < p.pps ? logical : p.pps - 1;
  int32_t phys = p.page_indices[(int64_t)s * p.pps + logical];
  phys = phys < 0 ? 0 : phys;
  phys = phys < p.P ? phys : p.P - 1;
  return phys;
}

// Token range of sequence s, clamped into [0, T].
__device__ __forceinline__ void seq_tokens(const Params& p, int32_t s, int32_t& q0, int32_t& ql) {
  int32_t a = p.cu_q_lens[s], b = p.cu_q_lens[s + 1];
  a = a < 0 ? 0 : (a > p.T ? p.T : a);
  b = b < a ? a : (b > p.T ? p.T : b);
  q0 = a;
  ql = b - a;
}

// floor(a / b) for 0 <= a < 2^48, 0 < b < 2^31, given inv = 1.0 / b: the
// double product is within one of the quotient, which the remainder fixes
// (a multiply instead of a double-precision division).
__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b, double inv) {
  int64_t q = (int64_t)((double)a * inv);
  const int64_t r = a - q * b;
  if (r < 0) --q;
  else if (r >= b) ++q;
  return q;
}

// The stream-K split of the decode work: Tb 16-key blocks (laid end to end in
// the decode sequence table's order) cut into W contiguous ranges, range w =
// [start(w), start(w + 1)) with start(w) = floor(Tb * w / W). The planner
// takes W <= Tb, so that no range is empty.
struct StreamK {
  int64_t Tb;
  int32_t W;
  double inv_Tb, inv_W;
  __device__ static StreamK make(int64_t Tb, int32_t W) {
    return StreamK{Tb, W, Tb > 0 ? 1.0 / (double)Tb : 0.0, W > 0 ? 1.0 / (double)W : 0.0};
  }
  __device__ int32_t start(int32_t w) const { return (int32_t)floor_div(Tb * w, W, inv_W); }
  // the range holding block x (0 <= x < Tb)
  __device__ int32_t wave_of(int32_t x) const {
    const int64_t w = floor_div((int64_t)(x + 1) * W - 1, Tb, inv_Tb);
    return (int32_t)(w < W - 1 ? w : W - 1);
  }
};

}  // namespace rpa
