// Prefill/mixed-class attention kernel: units of up to 128 packed query rows
// (row = token * G + g) of one sequence and one kv head, i.e. the kernel
// page's q block of `num_queries_per_block` tokens times G grouped q heads
// stacked into one MFMA M dimension (`run`, per-kv-head step).
//
// A workgroup of 4 waves owns one item at a time (pulled from a device-wide
// queue); wave w owns rows [32w, 32w + 32) as two 16-wide column blocks.
// Per 32-key step the workgroup
//   1. gathers the step's K and V rows of kv head h (combined heads 2h, 2h+1,
//      adjacent in memory, `stridedLoadKv`) through the page table into
//      registers with 16-byte loads — issued one step ahead so the HBM latency
//      overlaps the MFMA work of the current step — and writes them to a
//      double-buffered LDS tile (V zeroed past kv_len);
//   2. per wave: S^T = K Q^T (v_mfma_f32_16x16x32_bf16, K from LDS, Q^T held in
//      registers), sm_scale (k_scale folded in), soft-cap, masks by selection,
//      base-2 online softmax (`flashAttention`), then O^T += V^T P^T with V^T
//      read by ds_read_b64_tr_b16 and P^T taken straight from the S^T layout.
// One barrier per step protects the double buffer.
#pragma once

#include "rpa_common.h"

namespace rpa {

template <int D>
struct PrefillLds {
  static constexpr int kKStride = D + 8;   // +16 B per K row
  static constexpr int kVStride = D + 16;  // +32 B per V row
  static constexpr int kKElems = kStepKeys * kKStride;
  static constexpr int kVElems = kStepKeys * kVStride;
  static constexpr size_t kBytes = (size_t)2 * (kKElems + kVElems) * 2;
};

template <int D, bool FP8>
__global__ __launch_bounds__(kPfWaves * 64, 1) void prefill_kernel(Params p) {
  constexpr int NI = D / 32;
  constexpr int ND = D / 16;
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int KST = PrefillLds<D>::kKStride;
  constexpr int VST = PrefillLds<D>::kVStride;
  constexpr int NT = kPfWaves * 64;
  // 16-byte global chunks per key (K and V together) and per thread per step
  constexpr int CPK = 2 * D * EB / 16;
  constexpr int CPT = kStepKeys * CPK / NT;
  static_assert(kStepKeys * CPK % NT == 0, "chunks must divide evenly");

  __shared__ __attribute__((aligned(16))) __bf16 ks[2][PrefillLds<D>::kKElems];
  __shared__ __attribute__((aligned(16))) __bf16 vsm[2][PrefillLds<D>::kVElems];
  __shared__ int sh_item[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;

  const int n_items = p.hdr->n_pf_items;
  const int chunk = p.hdr->pf_chunk;
  const int64_t key_stride = (int64_t)2 * p.Hkv * D * EB;
  const bool capped = p.soft_cap > 0.f;
  const float cap_k = capped ? 2.0f * kLog2e / p.soft_cap : 0.f;

  int parity = 0;
  int buf = 0;
  for (;;) {
    if (tid == 0) sh_item[parity] = atomicAdd(&p.hdr->pf_counter, 1);
    __syncthreads();
    const int item = sh_item[parity];
    parity ^= 1;
    if (item >= n_items) break;

    const Item it = p.pf_items[item];
    const Unit u = p.pf_units[it.unit];
    const int s = u.seq;
    const int h = u.kv_head;
    int q0, ql;
    seq_tokens(p, s, q0, ql);
    int kvl = p.kv_lens[s];
    kvl = max(0, min(kvl, p.pps * p.page));
    const int c_lo = u.kv_lo + it.chunk * chunk;
    const int c_hi = min(u.kv_hi, c_lo + chunk);
    const uint8_t* kv_h = p.kv + (int64_t)2 * h * D * EB;

    // this lane's two query rows (one per column block)
    bool rvalid[2];
    int tok[2], qh[2], pos[2];
    bf16x8 qb[2][NI];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int r = 32 * wave + 16 * cb + col;
      rvalid[cb] = r < u.nrows;
      const int prow = u.row0 + r;
      const int t = prow / p.G;
      qh[cb] = h * p.G + (prow - t * p.G);
      tok[cb] = q0 + t;
      pos[cb] = kvl - ql + t;
      if (rvalid[cb]) {
        const uint16_t* qp = p.q + ((int64_t)tok[cb] * p.Hq + qh[cb]) * D;
#pragma unroll
        for (int i = 0; i < NI; ++i) qb[cb][i] = *reinterpret_cast<const bf16x8*>(qp + 32 * i + 8 * g);
      } else {
#pragma unroll
        for (int i = 0; i < NI; ++i) qb[cb][i] = bf16x8{};
      }
    }

    float m[2] = {-INFINITY, -INFINITY};
    float lsum[2] = {0.f, 0.f};
    f32x4 o[2][ND];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int d = 0; d < ND; ++d) o[cb][d] = f32x4{0.f, 0.f, 0.f, 0.f};

    // global -> register staging of one step
    u32x4 stage[CPT];
    auto load_step = [&](int k0) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int idx = tid + NT * c;
        const int key = idx / CPK;
        const int w16 = idx % CPK;
        const int kb = k0 + (key & ~15);
        if (kb < c_hi) {
          const int phys = page_of(p, s, k0 + key);
          const int slot = (k0 + key) % p.page;
          const uint8_t* src = kv_h + ((int64_t)phys * p.page + slot) * key_stride + 16 * w16;
          stage[c] = *reinterpret_cast<const u32x4*>(src);
        } else {
          stage[c] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto store_step = [&](int k0, int b) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int idx = tid + NT * c;
        const int key = idx / CPK;
        const int w16 = idx % CPK;
        const bool valid_v = k0 + key < kvl;
        if constexpr (FP8) {
          // 16 codes -> 16 bf16; K codes occupy the first D bytes of the key
          const int e0 = 16 * w16;
          const bool is_v = e0 >= D;
          const int d0 = is_v ? e0 - D : e0;
          u32x2 lo2 = {stage[c][0], stage[c][1]}, hi2 = {stage[c][2], stage[c][3]};
          bf16x8 a = fp8x8_to_bf16(lo2), bb = fp8x8_to_bf16(hi2);
          if (is_v && !valid_v) {
            a = bf16x8{};
            bb = bf16x8{};
          }
          __bf16* dst = is_v ? &vsm[b][key * VST + d0] : &ks[b][key * KST + d0];
          *reinterpret_cast<bf16x8*>(dst) = a;
          *reinterpret_cast<bf16x8*>(dst + 8) = bb;
        } else {
          const int e0 = 8 * w16;
          const bool is_v = e0 >= D;
          const int d0 = is_v ? e0 - D : e0;
          u32x4 v = stage[c];
          if (is_v && !valid_v) v = u32x4{0u, 0u, 0u, 0u};
          __bf16* dst = is_v ? &vsm[b][key * VST + d0] : &ks[b][key * KST + d0];
          *reinterpret_cast<u32x4*>(dst) = v;
        }
      }
    };

    if (c_lo < c_hi) load_step(c_lo);
    for (int k0 = c_lo; k0 < c_hi; k0 += kStepKeys) {
      store_step(k0, buf);
      __syncthreads();
      if (k0 + kStepKeys < c_hi) load_step(k0 + kStepKeys);

      const __bf16* kt = ks[buf];
      const __bf16* vt = vsm[buf];
      f32x4 sc[2][2];  // [key block][column block]
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        sc[b][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        sc[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + (16 * b + col) * KST + 32 * i + 8 * g);
          sc[b][0] = mfma16x16x32(ka, qb[0][i], sc[b][0]);
          sc[b][1] = mfma16x16x32(ka, qb[1][i], sc[b][1]);
        }
      }

      bf16x8 pb[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = k0 + 16 * b + 4 * g + j;
            float x = sc[b][cb][j] * p.sm_scale;
            if (capped) x = soft_cap_f(x, p.soft_cap, cap_k);
            bool vis = rvalid[cb] && key < kvl && key < c_hi;
            if (p.is_causal) vis = vis && key <= pos[cb];
            if (p.window > 0) vis = vis && key > pos[cb] - p.window;
            const float s2 = vis ? x * kLog2e : -INFINITY;
            sc[b][cb][j] = s2;
            mx = fmaxf(mx, s2);
          }
        }
        mx = wave_max_xor16_32(mx);
        const float m_new = fmaxf(m[cb], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m[cb] - m_use);
        m[cb] = m_new;
        lsum[cb] *= alpha;
#pragma unroll
        for (int d = 0; d < ND; ++d) o[cb][d] *= alpha;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float pv = fast_exp2(sc[b][cb][j] - m_use);
            lsum[cb] += pv;
            pb[cb][4 * b + j] = (__bf16)pv;
          }
      }

      const __bf16* vrow = vt + (4 * g + (col >> 2)) * VST + 4 * (col & 3);
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const bf16x4 lo = lds_read_tr16(vrow + 16 * d);
        const bf16x4 hi = lds_read_tr16(vrow + 16 * VST + 16 * d);
        const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[0][d] = mfma16x16x32(a, pb[0], o[0][d]);
        o[1][d] = mfma16x16x32(a, pb[1], o[1][d]);
      }
      buf ^= 1;
    }

#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float l_row = wave_sum_xor16_32(lsum[cb]);
      const float inv = l_row > 0.f ? p.v_scale / l_row : 0.f;
      const float lse_v = l_row > 0.f ? (m[cb] + fast_log2(l_row)) * kLn2 : -INFINITY;
      const int r = 32 * wave + 16 * cb + col;
      if (!rvalid[cb]) {
        // rows past the unit: nothing to store
      } else if (u.nch == 1) {
        uint16_t* op = p.out + ((int64_t)tok[cb] * p.Hq + qh[cb]) * D;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          u32x2 w = {bf16x2_bits(o[cb][d][0] * inv, o[cb][d][1] * inv),
                     bf16x2_bits(o[cb][d][2] * inv, o[cb][d][3] * inv)};
          *reinterpret_cast<u32x2*>(op + 16 * d + 4 * g) = w;
        }
        if (g == 0 && p.lse) p.lse[(int64_t)tok[cb] * p.Hq + qh[cb]] = lse_v;
      } else {
        float* pp = p.pf_part + ((int64_t)item * kPfRows + r) * D;
#pragma unroll
        for (int d = 0; d < ND; ++d) *reinterpret_cast<f32x4*>(pp + 16 * d + 4 * g) = o[cb][d] * inv;
        if (g == 0) p.pf_plse[(int64_t)item * kPfRows + r] = lse_v;
      }
    }
  }
}

}  // namespace rpa
