// Planning kernel: turns the ragged metadata into a list of work items.
//
// The kernel page walks the flattened token axis in fixed q blocks on one
// core, sequence by sequence, streaming every KV block of each sequence
// (`run`: ragged walk over cu_q_lens and kv_lens, KV loop while
// kv_blk * kv_per_blk < kv_len). Here the same walk is made once, up front,
// by one workgroup, and its result is a flat list that thousands of
// workgroups consume concurrently:
//   * every sequence with q_len tokens gives q_len * G packed rows per kv head
//     (row = token * G + g, G = Hq / Hkv: the page's GQA row packing);
//   * sequences with <= kDecRows rows become one decode-class unit per kv
//     head, longer ones become prefill-class units of pf_rows rows;
//   * a unit's key range is only the keys some of its rows can see: up to the
//     last row's causal position and, with a sliding window, from the first
//     row's window start (rounded down to 16), so masked-out blocks are never
//     read;
//   * each unit is cut into chunks of a per-class key count chosen so that
//     the whole batch yields about `target_*_items` items; the unit's
//     finished-chunk counter is cleared for the split merge.
#pragma once

#include "rpa_common.h"

namespace rpa {

constexpr int kPlanThreads = 1024;
constexpr int kDecMinChunk = 256;
constexpr int kPfMinChunk = 512;

struct UnitRange {
  int32_t lo16, hi;
};

// Keys that rows [row0, row0 + nrows) of a sequence (q_len, kv_len) can see.
__device__ __forceinline__ UnitRange unit_range(const Params& p, int32_t ql, int32_t kvl, int32_t row0,
                                                int32_t nrows) {
  const int32_t t_first = row0 / p.G;
  const int32_t t_last = (row0 + nrows - 1) / p.G;
  const int32_t p_first = kvl - ql + t_first;
  const int32_t p_last = kvl - ql + t_last;
  int32_t hi = p.is_causal ? min(kvl, p_last + 1) : kvl;
  hi = max(hi, 0);
  int32_t lo = p.window > 0 ? max(0, p_first - p.window + 1) : 0;
  UnitRange r;
  r.lo16 = lo & ~15;
  r.hi = hi;
  return r;
}

__device__ __forceinline__ int32_t n_chunks(int32_t lo16, int32_t hi, int32_t chunk) {
  int32_t keys = hi > lo16 ? hi - lo16 : 0;
  int32_t n = (keys + chunk - 1) / chunk;
  return n > 0 ? n : 1;
}

__device__ __forceinline__ int32_t pick_chunk(int64_t total_keys, int32_t target, int32_t min_chunk,
                                              int32_t max_chunk) {
  int64_t c = (total_keys + target - 1) / (target > 0 ? target : 1);
  c = (c + 63) & ~(int64_t)63;
  if (c < min_chunk) c = min_chunk;
  if (c > max_chunk) c = max_chunk;
  return (int32_t)c;
}

// Clamped metadata of sequence s.
__device__ __forceinline__ void seq_meta(const Params& p, int32_t s, int32_t& q0, int32_t& ql, int32_t& kvl) {
  seq_tokens(p, s, q0, ql);
  kvl = p.kv_lens[s];
  const int32_t cap = p.pps * p.page;
  kvl = kvl < 0 ? 0 : (kvl > cap ? cap : kvl);
}

// Block-wide exclusive scan of one int per thread; returns the prefix and
// writes the block total to *total. Uses `sh` (kPlanThreads/64 + 1 ints).
__device__ int32_t block_exclusive_scan(int32_t v, int32_t* sh, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t run = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      int32_t t = sh[w];
      sh[w] = run;
      run += t;
    }
    sh[kPlanThreads / 64] = run;
  }
  __syncthreads();
  int32_t r = sh[wave] + x - v;
  *total = sh[kPlanThreads / 64];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(Params p) {
  __shared__ int64_t red[2][kPlanThreads / 64];
  __shared__ int32_t sh[kPlanThreads / 64 + 1];
  const int tid = threadIdx.x;
  int32_t n = *p.num_seqs;
  n = n < 0 ? 0 : (n > p.S_max ? p.S_max : n);

  // pass 1: total visible keys of each class, to size the chunks
  int64_t dec_keys = 0, pf_keys = 0;
  for (int32_t s = tid; s < n; s += kPlanThreads) {
    int32_t q0, ql, kvl;
    seq_meta(p, s, q0, ql, kvl);
    if (ql <= 0) continue;
    const int32_t rows = ql * p.G;
    if (rows <= kDecRows) {
      UnitRange r = unit_range(p, ql, kvl, 0, rows);
      dec_keys += (int64_t)p.Hkv * max(0, r.hi - r.lo16);
    } else {
      for (int32_t r0 = 0; r0 < rows; r0 += p.pf_rows) {
        UnitRange r = unit_range(p, ql, kvl, r0, min(p.pf_rows, rows - r0));
        pf_keys += (int64_t)p.Hkv * max(0, r.hi - r.lo16);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    dec_keys += __shfl_xor(dec_keys, o);
    pf_keys += __shfl_xor(pf_keys, o);
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = dec_keys;
    red[1][tid >> 6] = pf_keys;
  }
  __syncthreads();
  int64_t tot_dec = 0, tot_pf = 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    tot_dec += red[0][w];
    tot_pf += red[1][w];
  }
  const int32_t dec_chunk = pick_chunk(tot_dec, p.target_dec_items, kDecMinChunk, 1 << 28);
  const int32_t pf_chunk = pick_chunk(tot_pf, p.target_pf_items, kPfMinChunk, kPfMaxChunk);

  // pass 1b: prefill items per queue (queue of (seq, kv head) = (seq*Hkv + h) % kQueues)
  __shared__ int32_t q_tot[kQueues];
  if (tid < kQueues) q_tot[tid] = 0;
  __syncthreads();
  for (int32_t s = tid; s < n; s += kPlanThreads) {
    int32_t q0, ql, kvl;
    seq_meta(p, s, q0, ql, kvl);
    const int32_t rows = ql * p.G;
    if (ql <= 0 || rows <= kDecRows) continue;
    int32_t per_head = 0;
    for (int32_t r0 = 0; r0 < rows; r0 += p.pf_rows) {
      UnitRange r = unit_range(p, ql, kvl, r0, min(p.pf_rows, rows - r0));
      per_head += n_chunks(r.lo16, r.hi, pf_chunk);
    }
    for (int32_t h = 0; h < p.Hkv; ++h) atomicAdd(&q_tot[(s * p.Hkv + h) % kQueues], per_head);
  }
  __syncthreads();
  int32_t q_base[kQueues];
  {
    int32_t run = 0;
    for (int x = 0; x < kQueues; ++x) {
      q_base[x] = run;
      run += q_tot[x];
    }
  }

  // pass 2: per-sequence counts -> scans -> records
  int32_t base_du = 0, base_pu = 0, base_di = 0, base_pi = 0, base_sp = 0;
  int32_t q_run[kQueues];
  for (int x = 0; x < kQueues; ++x) q_run[x] = 0;
  for (int32_t s0 = 0; s0 < n; s0 += kPlanThreads) {
    const int32_t s = s0 + tid;
    int32_t q0 = 0, ql = 0, kvl = 0;
    int32_t c_du = 0, c_pu = 0, c_di = 0, c_pi = 0, c_sp = 0;
    bool is_dec = false;
    if (s < n) {
      seq_meta(p, s, q0, ql, kvl);
      if (ql > 0) {
        const int32_t rows = ql * p.G;
        if (rows <= kDecRows) {
          is_dec = true;
          UnitRange r = unit_range(p, ql, kvl, 0, rows);
          const int32_t nch = n_chunks(r.lo16, r.hi, dec_chunk);
          c_du = p.Hkv;
          c_di = p.Hkv * nch;
          c_sp = nch > 1 ? p.Hkv : 0;
        } else {
          int32_t per_head_items = 0, per_head_split = 0, nrb = 0;
          for (int32_t r0 = 0; r0 < rows; r0 += p.pf_rows) {
            UnitRange r = unit_range(p, ql, kvl, r0, min(p.pf_rows, rows - r0));
            const int32_t nch = n_chunks(r.lo16, r.hi, pf_chunk);
            per_head_items += nch;
            per_head_split += nch > 1 ? 1 : 0;
            ++nrb;
          }
          c_pu = p.Hkv * nrb;
          c_pi = p.Hkv * per_head_items;
          c_sp = p.Hkv * per_head_split;
        }
      }
    }
    int32_t t_du, t_pu, t_di, t_pi, t_sp;
    int32_t o_du = base_du + block_exclusive_scan(c_du, sh, &t_du);
    int32_t o_pu = base_pu + block_exclusive_scan(c_pu, sh, &t_pu);
    int32_t o_di = base_di + block_exclusive_scan(c_di, sh, &t_di);
    int32_t o_pi = base_pi + block_exclusive_scan(c_pi, sh, &t_pi);
    (void)block_exclusive_scan(c_sp, sh, &t_sp);
    // this sequence's position in each prefill queue
    int32_t o_q[kQueues];
    for (int x = 0; x < kQueues; ++x) {
      int32_t cnt = 0;
      if (!is_dec && s < n && ql > 0)
        for (int32_t h = 0; h < p.Hkv; ++h) cnt += ((s * p.Hkv + h) % kQueues == x) ? c_pi / p.Hkv : 0;
      int32_t t_q;
      o_q[x] = q_base[x] + q_run[x] + block_exclusive_scan(cnt, sh, &t_q);
      q_run[x] += t_q;
    }

    if (s < n && ql > 0) {
      const int32_t rows = ql * p.G;
      if (is_dec) {
        UnitRange r = unit_range(p, ql, kvl, 0, rows);
        const int32_t nch = n_chunks(r.lo16, r.hi, dec_chunk);
        for (int32_t h = 0; h < p.Hkv; ++h) {
          const int32_t ui = o_du + h;
          if (ui >= p.max_dec_units) break;
          Unit u;
          u.seq = s; u.kv_head = h; u.row0 = 0; u.nrows = rows;
          u.kv_lo = r.lo16; u.kv_hi = r.hi; u.nch = nch; u.item0 = o_di + h * nch;
          p.dec_units[ui] = u;
          p.unit_done[ui] = 0;
          for (int32_t c = 0; c < nch; ++c) {
            const int32_t ii = u.item0 + c;
            if (ii < p.max_dec_items) p.dec_items[ii] = Item{ui, c};
          }
        }
      } else {
        int32_t ui = o_pu, ii = o_pi;
        for (int32_t h = 0; h < p.Hkv; ++h) {
          for (int32_t r0 = 0; r0 < rows; r0 += p.pf_rows) {
            const int32_t nr = min(p.pf_rows, rows - r0);
            UnitRange r = unit_range(p, ql, kvl, r0, nr);
            const int32_t nch = n_chunks(r.lo16, r.hi, pf_chunk);
            if (ui < p.max_pf_units) {
              Unit u;
              u.seq = s; u.kv_head = h; u.row0 = r0; u.nrows = nr;
              u.kv_lo = r.lo16; u.kv_hi = r.hi; u.nch = nch; u.item0 = ii;
              p.pf_units[ui] = u;
              p.unit_done[p.max_dec_units + ui] = 0;
              for (int32_t c = 0; c < nch; ++c)
                if (ii + c < p.max_pf_items) p.pf_items[ii + c] = Item{ui, c};
            }
            ++ui;
            ii += nch;
          }
        }
        // queue entries of each head: chunk-major, then row block
        int32_t ii_h = o_pi;
        for (int32_t h = 0; h < p.Hkv; ++h) {
          const int x = (s * p.Hkv + h) % kQueues;
          int32_t k = o_q[x];
          const int32_t per_head = c_pi / p.Hkv;
          for (int32_t c = 0;; ++c) {
            bool any = false;
            int32_t ii_rb = ii_h;
            for (int32_t r0 = 0; r0 < rows; r0 += p.pf_rows) {
              UnitRange r = unit_range(p, ql, kvl, r0, min(p.pf_rows, rows - r0));
              const int32_t nch = n_chunks(r.lo16, r.hi, pf_chunk);
              if (c < nch) {
                any = true;
                if (k < p.max_pf_items && ii_rb + c < p.max_pf_items) p.pf_qlist[k] = ii_rb + c;
                ++k;
              }
              ii_rb += nch;
            }
            if (!any) break;
          }
          o_q[x] = k;
          ii_h += per_head;
        }
      }
    }
    base_du += t_du; base_pu += t_pu; base_di += t_di; base_pi += t_pi; base_sp += t_sp;
  }
  if (tid == 0) {
    Header h = {};
    h.n_dec_units = min(base_du, p.max_dec_units);
    h.n_pf_units = min(base_pu, p.max_pf_units);
    h.n_dec_items = min(base_di, p.max_dec_items);
    h.n_pf_items = min(base_pi, p.max_pf_items);
    h.dec_chunk = dec_chunk;
    h.pf_chunk = pf_chunk;
    h.n_split_units = base_sp;
    h.dec_counter = 0;
    for (int x = 0; x < kQueues; ++x) {
      h.pf_q_base[x] = min(q_base[x], p.max_pf_items);
      h.pf_q_count[x] = max(0, min(q_tot[x], p.max_pf_items - h.pf_q_base[x]));
      h.pf_q_next[x] = 0;
    }
    *p.hdr = h;
  }
}

}  // namespace rpa
