// Split-KV merge: rows whose unit was cut into several key chunks.
//
// Every chunk c of a row left a normalised partial O_c (f32) and its
// log-sum-exp L_c. The row's result is the same merge of softmax blocks the
// kernel page performs block to block inside `flashAttention` (new max, then
// each side rescaled by exp(old max - new max)), applied once over all chunks:
//   L = max_c L_c + log sum_c exp(L_c - max_c L_c),
//   O = sum_c exp(L_c - L) * O_c,
// summed in chunk order (deterministic, no atomics). A row whose chunks all
// saw no key (every L_c = -inf) gets O = 0 and L = -inf.
#pragma once

#include "rpa_common.h"

namespace rpa {

constexpr int kCombineWaves = 4;

template <int D>
__global__ __launch_bounds__(kCombineWaves * 64) void combine_kernel(Params p) {
  constexpr int DPL = D / 64;  // head_dim elements per lane
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_split = p.hdr->n_split_units;
  for (int su = blockIdx.x; su < n_split; su += gridDim.x) {
    const int code = p.split_units[su];
    const int cls = code >> 30;
    const int ui = code & ((1 << 30) - 1);
    const Unit u = cls ? p.pf_units[ui] : p.dec_units[ui];
    const int slot_rows = cls ? kPfRows : kDecRows;
    const float* part = cls ? p.pf_part : p.dec_part;
    const float* plse = cls ? p.pf_plse : p.dec_plse;
    if (u.item0 < 0 || u.item0 + u.nch > (cls ? p.max_pf_items : p.max_dec_items)) continue;
    int q0, ql;
    seq_tokens(p, u.seq, q0, ql);
    for (int r = wave; r < u.nrows; r += kCombineWaves) {
      const int prow = u.row0 + r;
      const int t = prow / p.G;
      const int qh = u.kv_head * p.G + (prow - t * p.G);
      const int64_t orow = (int64_t)(q0 + t) * p.Hq + qh;
      float mx = -INFINITY;
      for (int c = 0; c < u.nch; ++c) mx = fmaxf(mx, plse[(int64_t)(u.item0 + c) * slot_rows + r]);
      float acc[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
      float lse_v = -INFINITY;
      if (mx != -INFINITY) {
        float wsum = 0.f;
        for (int c = 0; c < u.nch; ++c) {
          const int64_t slot = (int64_t)(u.item0 + c) * slot_rows + r;
          const float w = expf(plse[slot] - mx);
          wsum += w;
          const float* src = part + slot * D + lane * DPL;
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] += w * src[e];
        }
        const float inv = 1.0f / wsum;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] *= inv;
        lse_v = mx + logf(wsum);
      }
      uint16_t* op = p.out + orow * D + lane * DPL;
#pragma unroll
      for (int e = 0; e < DPL; e += 2) {
        const uint32_t w = bf16x2_bits(acc[e], DPL > 1 ? acc[e + 1] : 0.f);
        if constexpr (DPL > 1) {
          *reinterpret_cast<uint32_t*>(op + e) = w;
        } else {
          op[0] = (uint16_t)(w & 0xFFFFu);
        }
      }
      if (lane == 0 && p.lse) p.lse[orow] = lse_v;
    }
  }
}

}  // namespace rpa
