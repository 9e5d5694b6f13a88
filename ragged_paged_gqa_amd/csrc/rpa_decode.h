// Decode-class attention kernel: units of at most 16 packed query rows
// (q_len * G <= 16, e.g. one decode token of 4..16 grouped q heads).
//
// One wave owns one item (a key chunk of one sequence and one kv head) at a
// time and pulls items from a device-wide queue. Per 32-key step it
//   1. reads the physical pages of the step through the page table (the kernel
//      page's `createKvAsyncCopyDescriptors`: page_indices[seq, key / page]);
//   2. loads K straight from HBM into MFMA A-operand registers: lane
//      (key = lane % 16, k-group g = lane / 16) reads 16 bytes of its key row,
//      so S^T = K Q^T needs no LDS staging (K of kv head h is combined head
//      2h, V is combined head 2h+1 right after it, `stridedLoadKv`);
//   3. computes S^T [keys x rows] with v_mfma_f32_16x16x32_bf16 against the
//      register-resident Q^T, applies sm_scale (k_scale folded in), the
//      optional soft-cap, then the causal / window / length masks of
//      `flashAttention` by selection (masked scores become -inf, so NaN in
//      unread tail slots cannot leak in);
//   4. runs the online-softmax update of `flashAttention` in base 2 (running
//      max, rescale factor alpha = 2^(m_old - m_new), running sum), keeping
//      the accumulator un-normalised until the end;
//   5. stages V (zeroed past kv_len: 0 * NaN would otherwise poison the sum)
//      through a per-wave LDS tile and reads it back transposed with
//      ds_read_b64_tr_b16 as the A operand of O^T += V^T P^T, whose B operand
//      P^T is exactly the S^T result layout — no shuffle of P.
// fp8 e4m3fn K/V are widened to bf16 exactly with v_cvt_scalef32_pk_bf16_fp8;
// k_scale is folded into the score scale and v_scale into the final
// normalisation.
// An item that is its unit's only chunk writes bf16 out and f32 lse; otherwise
// it writes a normalised f32 partial and its lse, and the wave that finishes
// the unit's last chunk merges them (rpa_merge.h).
#pragma once

#include "rpa_common.h"
#include "rpa_merge.h"

namespace rpa {

constexpr int kDecWavesPerBlock = 4;

template <int D>
struct DecodeLds {
  static constexpr int kVStride = D + 16;  // bf16 elements per staged V row (+32 B)
  static constexpr int kWaveElems = kStepKeys * kVStride;
  static constexpr size_t kBytes = (size_t)kDecWavesPerBlock * kWaveElems * 2;
};

template <int D, bool FP8>
__global__ __launch_bounds__(kDecWavesPerBlock * 64) void decode_kernel(Params p) {
  constexpr int NI = D / 32;  // k-steps of the QK product over head_dim
  constexpr int ND = D / 16;  // 16-row blocks of O^T
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int VST = DecodeLds<D>::kVStride;
  __shared__ __attribute__((aligned(16))) __bf16 lds[kDecWavesPerBlock * DecodeLds<D>::kWaveElems];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  __bf16* vs = lds + wave * DecodeLds<D>::kWaveElems;

  const int n_items = p.hdr->n_dec_items;
  const int chunk = p.hdr->dec_chunk;
  const int64_t key_stride = (int64_t)2 * p.Hkv * D * EB;  // bytes between consecutive slots
  const bool capped = p.soft_cap > 0.f;
  const float cap_k = capped ? 2.0f * kLog2e / p.soft_cap : 0.f;

  // first item of each wave is static; later ones come from the queue
  int item = blockIdx.x * kDecWavesPerBlock + wave;
  const int first_dynamic = gridDim.x * kDecWavesPerBlock;
  while (item < n_items) {
    const Item it = p.dec_items[item];
    const Unit u = p.dec_units[it.unit];
    const int s = u.seq;
    const int h = u.kv_head;
    int q0, ql;
    seq_tokens(p, s, q0, ql);
    int kvl = p.kv_lens[s];
    kvl = max(0, min(kvl, p.pps * p.page));
    const int c_lo = u.kv_lo + it.chunk * chunk;
    const int c_hi = min(u.kv_hi, c_lo + chunk);

    // Column `col` of S^T / O^T is packed row u.row0 + col of the sequence.
    const bool rvalid = col < u.nrows;
    const int prow = u.row0 + col;
    const int t = prow / p.G;
    const int qh = h * p.G + (prow - t * p.G);
    const int tok = q0 + t;
    const int pos = kvl - ql + t;

    bf16x8 qb[NI];
    if (rvalid) {
      const uint16_t* qp = p.q + ((int64_t)tok * p.Hq + qh) * D;
#pragma unroll
      for (int i = 0; i < NI; ++i) qb[i] = *reinterpret_cast<const bf16x8*>(qp + 32 * i + 8 * g);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) qb[i] = bf16x8{};
    }

    float m = -INFINITY;
    float lsum = 0.f;
    f32x4 o[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    // page position of the step start, advanced without division
    const int32_t* ptab = p.page_indices + (int64_t)s * p.pps;
    int lp = c_lo / p.page;
    int sl = c_lo - lp * p.page;
    for (int k0 = c_lo; k0 < c_hi; k0 += kStepKeys) {
      bf16x8 ka[2][NI];
      bf16x8 va[2][NI];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int kb = k0 + 16 * b;
        const int lpb = (b == 0 || sl + 16 < p.page) ? lp : lp + 1;
        const int slb = b == 0 ? sl : (sl + 16 < p.page ? sl + 16 : 0);
        if (kb < c_hi) {
          const int phys = min(max(ptab[min(lpb, p.pps - 1)], 0), p.P - 1);
          const int slot = slb + col;
          const uint8_t* base = p.kv + ((int64_t)phys * p.page + slot) * key_stride + (int64_t)2 * h * D * EB;
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            if constexpr (FP8) {
              ka[b][i] = fp8x8_to_bf16(*reinterpret_cast<const u32x2*>(base + 32 * i + 8 * g));
              va[b][i] = fp8x8_to_bf16(*reinterpret_cast<const u32x2*>(base + D + 32 * i + 8 * g));
            } else {
              ka[b][i] = *reinterpret_cast<const bf16x8*>(base + 2 * (32 * i + 8 * g));
              va[b][i] = *reinterpret_cast<const bf16x8*>(base + 2 * (D + 32 * i + 8 * g));
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            ka[b][i] = bf16x8{};
            va[b][i] = bf16x8{};
          }
        }
      }

      sl += kStepKeys;
      if (sl >= p.page) {
        sl -= p.page;
        ++lp;
      }
      if (sl >= p.page) {
        sl -= p.page;
        ++lp;
      }

      // S^T: lane (col, g) gets keys k0 + 16b + 4g + j of row `col`.
      f32x4 sc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i) sc[b] = mfma16x16x32(ka[b][i], qb[i], sc[b]);
      }

      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = k0 + 16 * b + 4 * g + j;
          float x = sc[b][j] * p.sm_scale;
          if (capped) x = soft_cap_f(x, p.soft_cap, cap_k);
          bool vis = rvalid && key < kvl && key < c_hi;
          if (p.is_causal) vis = vis && key <= pos;
          if (p.window > 0) vis = vis && key > pos - p.window;
          const float s2 = vis ? x * kLog2e : -INFINITY;
          sc[b][j] = s2;
          mx = fmaxf(mx, s2);
        }
      }
      mx = wave_max_xor16_32(mx);
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < ND; ++d) o[d] *= alpha;
      float pv[2][4];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pv[b][j] = fast_exp2(sc[b][j] - m_use);
          lsum += pv[b][j];
        }

      // Stage V rows [k0, k0 + 32) in LDS, zero past kv_len.
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int key = k0 + 16 * b + col;
        const bool vok = (k0 + 16 * b < c_hi) && key < kvl;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          bf16x8 v = vok ? va[b][i] : bf16x8{};
          *reinterpret_cast<bf16x8*>(vs + (16 * b + col) * VST + 32 * i + 8 * g) = v;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      bf16x8 pb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pb[j] = (__bf16)pv[0][j];
        pb[4 + j] = (__bf16)pv[1][j];
      }
      const __bf16* vrow = vs + (4 * g + (col >> 2)) * VST + 4 * (col & 3);
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const bf16x4 lo = lds_read_tr16(vrow + 16 * d);
        const bf16x4 hi = lds_read_tr16(vrow + 16 * VST + 16 * d);
        const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[d] = mfma16x16x32(a, pb, o[d]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    const float l_row = wave_sum_xor16_32(lsum);
    const float inv = l_row > 0.f ? p.v_scale / l_row : 0.f;
    const float lse_v = l_row > 0.f ? (m + fast_log2(l_row)) * kLn2 : -INFINITY;
    if (u.nch == 1) {
      if (rvalid) {
        uint16_t* op = p.out + ((int64_t)tok * p.Hq + qh) * D;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          u32x2 w = {bf16x2_bits(o[d][0] * inv, o[d][1] * inv), bf16x2_bits(o[d][2] * inv, o[d][3] * inv)};
          *reinterpret_cast<u32x2*>(op + 16 * d + 4 * g) = w;
        }
        if (g == 0 && p.lse) p.lse[(int64_t)tok * p.Hq + qh] = lse_v;
      }
    } else {
      if (rvalid) {
        float* pp = p.dec_part + ((int64_t)item * kDecRows + col) * D;
#pragma unroll
        for (int d = 0; d < ND; ++d) store_coherent4(pp + 16 * d + 4 * g, o[d] * inv);
        if (g == 0) store_coherent(p.dec_plse + (int64_t)item * kDecRows + col, lse_v);
      }
      // publish the partial, count the chunk; the last one merges the unit
      wait_stores();
      int done = 0;
      if (lane == 0) done = atomicAdd(&p.unit_done[it.unit], 1);
      done = __builtin_amdgcn_readfirstlane(__shfl(done, 0));
      if (done == u.nch - 1) {
        // the wave's V staging tile is free here; it holds the per-row stats
        auto wave_sync = [] {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };
        merge_unit<D>(p, u, p.dec_part, p.dec_plse, kDecRows, lane, 64, reinterpret_cast<float*>(vs), wave_sync);
        wave_sync();
      }
    }

    int nx = 0;
    if (lane == 0) nx = atomicAdd(&p.hdr->dec_counter, 1);
    item = first_dynamic + __builtin_amdgcn_readfirstlane(__shfl(nx, 0));
  }
}

}  // namespace rpa
