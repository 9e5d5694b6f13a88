// Split-KV merge, run by whichever wave/workgroup finishes a split unit's
// last chunk (each chunk bumps the unit's counter after its partial is
// written with device-coherent stores).
//
// Every chunk c of a row left a normalised partial O_c (f32) and its
// log-sum-exp L_c. The row's result is the same merge of softmax blocks the
// kernel page performs block to block inside `flashAttention` (new max, then
// each side rescaled by exp(old max - new max)), applied once over all chunks:
//   L = max_c L_c + log sum_c exp(L_c - max_c L_c),
//   O = sum_c exp(L_c - L) * O_c,
// summed in chunk order, so the result does not depend on which workgroup
// merges or on timing. A row whose chunks all saw no key (every L_c = -inf)
// gets O = 0 and L = -inf. An attention sink (one logit per q head) is one
// more term of the sum that carries no value: it joins max_c L_c and the sum
// here, and never the chunks' partials.
//
// Two phases, both fully parallel over the cooperating threads: (A) per row,
// the max and the normalising sum of the chunk LSEs (kept in LDS, the row's
// LSE written out); (B) per (row, 4-element piece of head_dim), the weighted
// sum over chunks with all loads independent.
#pragma once

#include "rpa_common.h"

namespace rpa {

// Chunk c of the unit left its partial in slot `slot(c)` of `part` / `plse`
// (slot_rows rows each). Threads tid in [0, nt) cooperate; `sync` is called
// between the phases and must synchronise exactly those threads. `stat` is
// LDS scratch of 2 * u.nrows floats. BATCH: issue the loads of several chunks
// before reducing them (the combine kernel, where each wave's merge is one
// long chain of loads); the prefill kernels' last finishers keep the plain
// loops, which need fewer registers beside their main loop's.
template <int D, bool F16, bool Q32, bool BATCH, typename Slot, typename Sync>
__device__ void merge_unit(const Params& p, const Unit& u, const float* part, const float* plse, int slot_rows,
                           Slot slot, int tid, int nt, float* stat, Sync sync) {
  int q0, ql;
  seq_tokens(p, u.seq, q0, ql);
  auto lse_of = [&](int c, int r) { return load_coherent(plse + (int64_t)slot(c) * slot_rows + r); };
  // The partials sit in memory written by other workgroups (coherent loads,
  // long latency): each pass issues a batch of independent loads before it
  // reduces them, always in chunk order, so the sums do not depend on the
  // batching.
  constexpr int BA = BATCH ? 8 : 1, BB = BATCH ? 4 : 1;
  // phase A: per-row max and 1 / sum of exp(L_c - max)
  for (int r = tid; r < u.nrows; r += nt) {
    const int prow = u.row0 + r;
    const int t = prow / p.G;
    const int qh = u.kv_head * p.G + (prow - t * p.G);
    const float sink = p.sinks ? p.sinks[qh] : -INFINITY;
    float held[BA];  // the first BA chunks' L_c, kept for the sum
#pragma unroll
    for (int k = 0; k < BA; ++k) held[k] = k < u.nch ? lse_of(k, r) : -INFINITY;
    float mx = sink;
#pragma unroll
    for (int k = 0; k < BA; ++k) mx = fmaxf(mx, held[k]);
    for (int c0 = BA; c0 < u.nch; c0 += BA) {
      float v[BA];
#pragma unroll
      for (int k = 0; k < BA; ++k) v[k] = c0 + k < u.nch ? lse_of(c0 + k, r) : -INFINITY;
#pragma unroll
      for (int k = 0; k < BA; ++k) mx = fmaxf(mx, v[k]);
    }
    float wsum = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int k = 0; k < BA; ++k)
        if (k < u.nch) wsum += expf(held[k] - mx);
      for (int c0 = BA; c0 < u.nch; c0 += BA) {
        float v[BA];
#pragma unroll
        for (int k = 0; k < BA; ++k) v[k] = c0 + k < u.nch ? lse_of(c0 + k, r) : -INFINITY;
#pragma unroll
        for (int k = 0; k < BA; ++k)
          if (c0 + k < u.nch) wsum += expf(v[k] - mx);
      }
      if (sink != -INFINITY) wsum += expf(sink - mx);
    }
    stat[2 * r] = mx;
    stat[2 * r + 1] = wsum > 0.f ? 1.0f / wsum : 0.f;
    if (p.lse) p.lse[(int64_t)(q0 + t) * p.Hq + qh] = mx != -INFINITY ? mx + logf(wsum) : -INFINITY;
  }
  sync();
  // phase B: out[row, 4 elements] = sum_c exp(L_c - max) / sum * O_c[row, 4 elements]
  constexpr int PIECES = D / 4;
  for (int idx = tid; idx < u.nrows * PIECES; idx += nt) {
    const int r = idx / PIECES;
    const int e0 = 4 * (idx % PIECES);
    const float mx = stat[2 * r];
    const float inv = stat[2 * r + 1];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (mx != -INFINITY) {
      for (int c0 = 0; c0 < u.nch; c0 += BB) {
        float l[BB];
        f32x2 a[BB], b[BB];
#pragma unroll
        for (int k = 0; k < BB; ++k) {
          if (c0 + k < u.nch) {
            const float* src = part + ((int64_t)slot(c0 + k) * slot_rows + r) * D + e0;
            l[k] = lse_of(c0 + k, r);
            a[k] = load_coherent2(src);
            b[k] = load_coherent2(src + 2);
          }
        }
#pragma unroll
        for (int k = 0; k < BB; ++k) {
          if (c0 + k < u.nch) {
            const float w = expf(l[k] - mx);
            acc[0] += w * a[k][0];
            acc[1] += w * a[k][1];
            acc[2] += w * b[k][0];
            acc[3] += w * b[k][1];
          }
        }
      }
    }
    const int prow = u.row0 + r;
    const int t = prow / p.G;
    const int qh = u.kv_head * p.G + (prow - t * p.G);
    store_out4<F16, Q32>(p.out, ((int64_t)(q0 + t) * p.Hq + qh) * D + e0, acc[0] * inv, acc[1] * inv, acc[2] * inv,
                         acc[3] * inv);
  }
}

// The same merge for a unit of at most NMAX chunks, in one pass: every
// thread takes (row, 4-element piece) items and loads all the chunks' LSEs
// and partial pieces at once, so the merge costs one round of coherent loads
// instead of two with a synchronisation between them. The sums run in chunk
// order as above, so both versions give the same bits.
template <int D, bool F16, bool Q32, int NMAX, typename Slot>
__device__ void merge_unit_small(const Params& p, const Unit& u, const float* part, const float* plse, int slot_rows,
                                 Slot slot, int tid, int nt) {
  int q0, ql;
  seq_tokens(p, u.seq, q0, ql);
  constexpr int PIECES = D / 4;
  for (int idx = tid; idx < u.nrows * PIECES; idx += nt) {
    const int r = idx / PIECES;
    const int e0 = 4 * (idx % PIECES);
    const int prow = u.row0 + r;
    const int t = prow / p.G;
    const int qh = u.kv_head * p.G + (prow - t * p.G);
    float l[NMAX];
    f32x2 a[NMAX], b[NMAX];
#pragma unroll
    for (int k = 0; k < NMAX; ++k) {
      if (k < u.nch) {
        const float* src = part + ((int64_t)slot(k) * slot_rows + r) * D + e0;
        l[k] = load_coherent(plse + (int64_t)slot(k) * slot_rows + r);
        a[k] = load_coherent2(src);
        b[k] = load_coherent2(src + 2);
      }
    }
    const float sink = p.sinks ? p.sinks[qh] : -INFINITY;
    float mx = sink;
#pragma unroll
    for (int k = 0; k < NMAX; ++k)
      if (k < u.nch) mx = fmaxf(mx, l[k]);
    float wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (mx != -INFINITY) {
#pragma unroll
      for (int k = 0; k < NMAX; ++k)
        if (k < u.nch) wsum += expf(l[k] - mx);
      if (sink != -INFINITY) wsum += expf(sink - mx);
#pragma unroll
      for (int k = 0; k < NMAX; ++k) {
        if (k < u.nch) {
          const float w = expf(l[k] - mx);
          acc[0] += w * a[k][0];
          acc[1] += w * a[k][1];
          acc[2] += w * b[k][0];
          acc[3] += w * b[k][1];
        }
      }
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    store_out4<F16, Q32>(p.out, ((int64_t)(q0 + t) * p.Hq + qh) * D + e0, acc[0] * inv, acc[1] * inv, acc[2] * inv,
                         acc[3] * inv);
    if (e0 == 0 && p.lse) p.lse[(int64_t)(q0 + t) * p.Hq + qh] = mx != -INFINITY ? mx + logf(wsum) : -INFINITY;
  }
}

}  // namespace rpa
