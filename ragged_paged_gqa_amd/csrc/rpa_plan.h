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
//   * sequences with <= kDecRows rows are decode-class: the planner writes
//     one record per such sequence (its metadata, its units' key range and
//     16-key block count, and the stream-K position of its first block: an
//     exclusive scan of Hkv * blocks over the decode sequences) and nothing
//     per unit or per chunk; the decode waves split the blocks among
//     themselves from these records (see DecSeq);
//   * longer sequences become prefill-class units of pf_rows rows;
//   * a unit's key range is only the keys some of its rows can see: up to the
//     last row's causal position and, with a sliding window, from the first
//     row's window start (rounded down to 16), so masked-out blocks are never
//     read;
//   * each prefill unit is cut into chunks of a key count chosen so that the
//     whole batch yields about `target_pf_items` items; the unit's
//     finished-chunk counter is cleared for the split merge;
//   * prefill items are dealt into one queue per XCD: all items of a
//     (sequence, kv head) go to queue (seq * Hkv + h) % kQueues, chunk-major,
//     so an XCD's concurrently running workgroups stream the same K/V chunk
//     and share it in that XCD's L2. Queue x lives at
//     pf_qlist[x * max_pf_items].
//
// Work split inside the workgroup: sequences are taken in tiles of
// kPlanThreads, one thread per sequence for the per-sequence counts, for the
// one block scan that turns them into record offsets and for the decode
// records; a wave per prefill sequence, a row block per lane.
// Divisions by G and by the chunk size use an exact double-precision
// reciprocal.
#pragma once

#include "rpa_common.h"

namespace rpa {

constexpr int kPlanThreads = 512;  // 1024 would cap a wave at 128 VGPRs and spill
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPfMinChunk = 512;

// a / d for 0 <= a < 2^31, d > 0: the double product is within 1e-6 of the
// quotient, so truncation is off by at most one, which the remainder fixes.
struct FastDiv {
  int32_t d;
  double inv;
};
__device__ __forceinline__ FastDiv make_div(int32_t d) { return FastDiv{d, 1.0 / (double)d}; }
__device__ __forceinline__ int32_t fdiv(int32_t a, const FastDiv& f) {
  int32_t q = (int32_t)((double)a * f.inv);
  const int32_t r = a - q * f.d;
  if (r < 0) --q;
  else if (r >= f.d) ++q;
  return q;
}

struct UnitRange {
  int32_t lo16, hi;
};

// Keys that rows [row0, row0 + nrows) of a sequence (q_len, kv_len) can see.
__device__ __forceinline__ UnitRange unit_range(const Params& p, const FastDiv& G, int32_t ql, int32_t kvl,
                                                int32_t row0, int32_t nrows) {
  const int32_t p_first = kvl - ql + fdiv(row0, G);
  const int32_t p_last = kvl - ql + fdiv(row0 + nrows - 1, G);
  int32_t hi = p.is_causal ? min(kvl, p_last + 1) : kvl;
  hi = max(hi, 0);
  const int32_t lo = p.window > 0 ? max(0, p_first - p.window + 1) : 0;
  return UnitRange{lo & ~15, hi};
}

__device__ __forceinline__ int32_t range_keys(const UnitRange& r) { return r.hi > r.lo16 ? r.hi - r.lo16 : 0; }

__device__ __forceinline__ int32_t n_chunks(const UnitRange& r, const FastDiv& chunk) {
  const int32_t keys = range_keys(r);
  int32_t n = fdiv(keys, chunk);
  n += n * chunk.d < keys;
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
__device__ __forceinline__ void seq_meta(const Params& p, int32_t s, int32_t& ql, int32_t& kvl) {
  int32_t q0;
  seq_tokens(p, s, q0, ql);
  kvl = p.kv_lens[s];
  const int32_t cap = p.pps * p.page;
  kvl = kvl < 0 ? 0 : (kvl > cap ? cap : kvl);
}

// Block-wide exclusive scan of NV ints per thread at once: excl[k] gets the
// sum of v[k] over lower threads, tot[k] the block total. `sh` holds
// kPlanWaves * NV ints.
template <int NV>
__device__ void block_scan(const int32_t (&v)[NV], int32_t (&excl)[NV], int32_t (&tot)[NV], int32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) x[k] = v[k];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int32_t y = __shfl_up(x[k], o);
      if (lane >= o) x[k] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < NV; ++k) sh[wave * NV + k] = x[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    int32_t before = 0, all = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
      const int32_t t = sh[w * NV + k];
      before += w < wave ? t : 0;
      all += t;
    }
    excl[k] = before + x[k] - v[k];
    tot[k] = all;
  }
  __syncthreads();
}

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int32_t wave_max(int32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  return v;
}

// Decode waves given work where one launch holds both classes' workgroups
// (elsewhere: all the launch has, up to one per block). A decode-only batch
// uses half the workgroups wherever two fit on a compute unit: the HBM rate
// holds on half of them. In a batch with prefill work the decode goes to
// 1/RPA_FUSED_DIV_PF of the workgroups when the prefill class's estimated
// time is at least RPA_FUSED_RATIO times the decode class's, else to half of
// them; the workgroups left without work exit at once and free their place on
// the compute unit for a prefill workgroup.
#ifndef RPA_FUSED_DIV_PF
#define RPA_FUSED_DIV_PF 4
#endif
#ifndef RPA_FUSED_RATIO
#define RPA_FUSED_RATIO 0.5
#endif
// rates of the two classes on their own (measured): prefill MFMA flop/s and
// decode K/V bytes/s
constexpr double kPfRate = 0.8e15;
constexpr double kDecRate = 5.5e12;

__device__ inline int32_t fused_dec_waves(const Params& p, int64_t pf_keys, int32_t dec_blocks, int32_t pf_items) {
  const int32_t wgs = max(p.dec_waves, 1) / kDecWavesPerBlock;
  if (!p.fused || dec_blocks <= 0 || wgs <= 1) return max(p.dec_waves, 1);
  int32_t div = 1;
  if (pf_items <= 0) {
    div = p.dec_per_cu >= 2 ? 2 : 1;
  } else {
    // prefill: every packed row of a unit against its key range, 4 * D flops
    // per (row, key); decode: K and V of every block
    const double t_pf = (double)pf_keys * p.pf_rows * 4.0 * p.D / kPfRate;
    const double t_dec = (double)dec_blocks * p.dec_blk * 2.0 * p.D * (p.dec_blk == kDecBlk8 ? 1 : 2) / kDecRate;
    div = t_pf >= RPA_FUSED_RATIO * t_dec ? RPA_FUSED_DIV_PF : 2;
  }
  return max(1, wgs / div) * kDecWavesPerBlock;
}

// Per-sequence counts of the main scan: 0 decode units, 1 prefill units,
// 2 decode blocks, 3 prefill items, 4 split units. The prefill items per queue
// take a second scan, over the tile's prefill sequences heaviest first.
constexpr int kScanN = 5;

// Per prefill sequence of a tile, filled by its wave.
struct PfInfo {
  int32_t s;         // sequence
  int32_t per_head;  // items of one kv head
  int32_t nsplit;    // row blocks with more than one chunk
  int32_t max_nch;   // most chunks of one row block
  int64_t work;      // visible keys of its row blocks (one kv head)
};

// Offsets of a prefill sequence's records, from the block scan.
struct PfOffs {
  int32_t unit, item;
  int32_t queue[kQueues];
};

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(Params p) {
  __shared__ int64_t red[kPlanWaves];
  __shared__ int32_t sh[kPlanWaves * kQueues];
  __shared__ int32_t n_pf_tile;
  __shared__ PfInfo pf_info[kPlanThreads];
  __shared__ int32_t by_rank[kPlanThreads];  // prefill slots of the tile, heaviest sequence first
  __shared__ PfOffs pf_offs[kPlanThreads];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t n = *p.num_seqs;
  n = n < 0 ? 0 : (n > p.S_max ? p.S_max : n);
  const FastDiv G = make_div(p.G);
  const int32_t R = p.pf_rows;

  // Collects this tile's prefill sequences into pf_info[0, n_pf_tile); the
  // thread's sequence gets its slot in `slot` (-1: not prefill).
  auto collect = [&](int32_t s, int32_t ql, int32_t& slot) {
    slot = -1;
    if (s < n && ql * p.G > kDecRows) {
      slot = atomicAdd(&n_pf_tile, 1);
      pf_info[slot].s = s;
    }
  };

  // pass 1: total visible keys of the prefill class, to size its chunks
  int64_t pf_keys = 0;
  for (int32_t s0 = 0; s0 < n; s0 += kPlanThreads) {
    if (tid == 0) n_pf_tile = 0;
    __syncthreads();
    const int32_t s = s0 + tid;
    int32_t ql = 0, kvl = 0, slot;
    if (s < n) seq_meta(p, s, ql, kvl);
    collect(s, ql, slot);
    __syncthreads();
    for (int32_t i = wave; i < n_pf_tile; i += kPlanWaves) {
      const int32_t ps = pf_info[i].s;
      int32_t pql, pkvl;
      seq_meta(p, ps, pql, pkvl);
      const int32_t rows = pql * p.G;
      for (int32_t r0 = lane * R; r0 < rows; r0 += 64 * R)
        pf_keys += (int64_t)p.Hkv * range_keys(unit_range(p, G, pql, pkvl, r0, min(R, rows - r0)));
    }
    __syncthreads();
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) pf_keys += __shfl_xor(pf_keys, o);
  if (lane == 0) red[wave] = pf_keys;
  __syncthreads();
  int64_t tot_pf = 0;
  for (int w = 0; w < kPlanWaves; ++w) tot_pf += red[w];
  const FastDiv pf_chunk = make_div(pick_chunk(tot_pf, p.target_pf_items, kPfMinChunk, kPfMaxChunk));

  // pass 2: per-sequence counts -> one scan per tile -> records
  int32_t base[kScanN], base_q[kQueues];
#pragma unroll
  for (int k = 0; k < kScanN; ++k) base[k] = 0;
#pragma unroll
  for (int x = 0; x < kQueues; ++x) base_q[x] = 0;
  for (int32_t s0 = 0; s0 < n; s0 += kPlanThreads) {
    if (tid == 0) n_pf_tile = 0;
    __syncthreads();
    const int32_t s = s0 + tid;
    int32_t ql = 0, kvl = 0, slot;
    if (s < n) seq_meta(p, s, ql, kvl);
    collect(s, ql, slot);
    __syncthreads();
    // (a) a wave per prefill sequence: chunk counts of its row blocks
    for (int32_t i = wave; i < n_pf_tile; i += kPlanWaves) {
      const int32_t ps = pf_info[i].s;
      int32_t pql, pkvl;
      seq_meta(p, ps, pql, pkvl);
      const int32_t rows = pql * p.G;
      int32_t items = 0, nsplit = 0, max_nch = 0;
      int64_t work = 0;
      for (int32_t r0 = lane * R; r0 < rows; r0 += 64 * R) {
        const UnitRange r = unit_range(p, G, pql, pkvl, r0, min(R, rows - r0));
        const int32_t nch = n_chunks(r, pf_chunk);
        items += nch;
        nsplit += nch > 1;
        max_nch = max(max_nch, nch);
        work += range_keys(r);
      }
      items = wave_sum(items);
      nsplit = wave_sum(nsplit);
      max_nch = wave_max(max_nch);
      work = wave_sum64(work);
      if (lane == 0) {
        pf_info[i].per_head = items;
        pf_info[i].nsplit = nsplit;
        pf_info[i].max_nch = max_nch;
        pf_info[i].work = work;
      }
    }
    __syncthreads();
    // (b) a thread per sequence: counts, scan
    int32_t cnt[kScanN];
#pragma unroll
    for (int k = 0; k < kScanN; ++k) cnt[k] = 0;
    const bool is_dec = s < n && ql > 0 && ql * p.G <= kDecRows;
    UnitRange dr{0, 0};
    int32_t nb = 0;
    if (is_dec) {
      dr = unit_range(p, G, ql, kvl, 0, ql * p.G);
      nb = (range_keys(dr) + p.dec_blk - 1) / p.dec_blk;
      cnt[0] = p.Hkv;
      cnt[2] = p.Hkv * nb;
    } else if (slot >= 0) {
      const PfInfo& f = pf_info[slot];
      const int32_t nrb = (ql * p.G + R - 1) / R;
      cnt[1] = p.Hkv * nrb;
      cnt[3] = p.Hkv * f.per_head;
      cnt[4] = p.Hkv * f.nsplit;
    }
    int32_t off[kScanN], tot[kScanN];
    block_scan<kScanN>(cnt, off, tot, sh);
#pragma unroll
    for (int k = 0; k < kScanN; ++k) off[k] += base[k];
#pragma unroll
    for (int k = 0; k < kScanN; ++k) base[k] += tot[k];

    if (slot >= 0) {
      pf_offs[slot].unit = off[1];
      pf_offs[slot].item = off[3];
    }
    // queue offsets: the tile's prefill sequences take their places in the
    // queues heaviest first (visible keys; ties by sequence index), so that
    // the longest items start first and the queues drain evenly; a sequence's
    // entries in a queue stay contiguous and chunk-major
    if (n_pf_tile > 0) {  // (block-uniform)
      if (slot >= 0) {
        const int64_t wk = pf_info[slot].work;
        int32_t r = 0;
        for (int32_t j = 0; j < n_pf_tile; ++j) {
          const int64_t wj = pf_info[j].work;
          r += wj > wk || (wj == wk && pf_info[j].s < s);
        }
        by_rank[r] = slot;
      }
      __syncthreads();
      int32_t qc[kQueues];
#pragma unroll
      for (int x = 0; x < kQueues; ++x) qc[x] = 0;
      const int32_t rs = tid < n_pf_tile ? by_rank[tid] : -1;
      if (rs >= 0) {
        const PfInfo& f = pf_info[rs];
        for (int32_t h = 0; h < p.Hkv; ++h) {
          const int x = (f.s * p.Hkv + h) % kQueues;
#pragma unroll
          for (int k = 0; k < kQueues; ++k) qc[k] += x == k ? f.per_head : 0;
        }
      }
      int32_t qo[kQueues], qt[kQueues];
      block_scan<kQueues>(qc, qo, qt, sh);
      if (rs >= 0) {
#pragma unroll
        for (int x = 0; x < kQueues; ++x) pf_offs[rs].queue[x] = base_q[x] + qo[x];
      }
#pragma unroll
      for (int x = 0; x < kQueues; ++x) base_q[x] += qt[x];
    }

    // (c) a decode sequence's record, at its rank among the decode sequences
    if (is_dec) {
      int32_t q0, qlx;
      seq_tokens(p, s, q0, qlx);
      const int4 rec[2] = {int4{s, q0, ql, kvl}, int4{dr.lo16, dr.hi, off[2], nb}};
      int4* dst = reinterpret_cast<int4*>(p.dec_seqs + off[0] / p.Hkv);
      dst[0] = rec[0];
      dst[1] = rec[1];
    }
    __syncthreads();

    // (d) a wave per prefill sequence: its units, items and queue entries
    for (int32_t i = wave; i < n_pf_tile; i += kPlanWaves) {
      const PfInfo f = pf_info[i];
      const int32_t ps = f.s;
      int32_t pql, pkvl;
      seq_meta(p, ps, pql, pkvl);
      const int32_t rows = pql * p.G;
      const int32_t nrb = (rows + R - 1) / R;
      const int32_t unit0 = pf_offs[i].unit, item0 = pf_offs[i].item;
      // units and items: unit of (h, rb) is unit0 + h * nrb + rb, its items
      // start at item0 + h * per_head + (chunks of the earlier row blocks)
      int32_t carry = 0;
      for (int32_t rb0 = 0; rb0 < nrb; rb0 += 64) {
        const int32_t rb = rb0 + lane;
        int32_t nch = 0;
        UnitRange r{0, 0};
        int32_t r0 = 0, nr = 0;
        if (rb < nrb) {
          r0 = rb * R;
          nr = min(R, rows - r0);
          r = unit_range(p, G, pql, pkvl, r0, nr);
          nch = n_chunks(r, pf_chunk);
        }
        const int32_t incl = wave_incl_scan(nch);
        const int32_t item_off = carry + incl - nch;
        carry += __shfl(incl, 63);
        if (rb < nrb) {
          for (int32_t h = 0; h < p.Hkv; ++h) {
            const int32_t ui = unit0 + h * nrb + rb;
            const int32_t ii = item0 + h * f.per_head + item_off;
            if (ui >= p.max_pf_units) break;
            Unit u;
            u.seq = ps; u.kv_head = h; u.row0 = r0; u.nrows = nr;
            u.kv_lo = r.lo16; u.kv_hi = r.hi; u.nch = nch; u.item0 = ii;
            p.pf_units[ui] = u;
            p.unit_done[ui] = 0;
            for (int32_t c = 0; c < nch; ++c)
              if (ii + c < p.max_pf_items) p.pf_items[ii + c] = Item{ui, c};
          }
        }
      }
      // queue entries, chunk-major: chunk 0 of every row block, then chunk 1
      // of those that have one, ...; a head's entries are contiguous, after
      // those of this sequence's earlier heads in the same queue
      int32_t pos = 0;  // entries of this sequence's head so far
      for (int32_t c = 0; c < f.max_nch; ++c) {
        int32_t carry_items = 0;
        for (int32_t rb0 = 0; rb0 < nrb; rb0 += 64) {
          const int32_t rb = rb0 + lane;
          int32_t nch = 0;
          if (rb < nrb) {
            const int32_t r0 = rb * R;
            nch = n_chunks(unit_range(p, G, pql, pkvl, r0, min(R, rows - r0)), pf_chunk);
          }
          const int32_t incl = wave_incl_scan(nch);
          const int32_t item_off = carry_items + incl - nch;
          carry_items += __shfl(incl, 63);
          const bool has = c < nch;
          const uint64_t m = __ballot(has);
          const int32_t before = __popcll(m & ((1ull << lane) - 1ull));
          if (has) {
            for (int32_t h = 0; h < p.Hkv; ++h) {
              const int x = (ps * p.Hkv + h) % kQueues;
              const int32_t j = h / kQueues;  // earlier heads of this sequence in queue x
              const int32_t k = pf_offs[i].queue[x] + j * f.per_head + pos + before;
              const int32_t item = item0 + h * f.per_head + item_off + c;
              if (k < p.max_pf_items && item < p.max_pf_items)
                p.pf_qlist[(int64_t)x * p.max_pf_items + k] = item;
            }
          }
          pos += __popcll(m);
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    Header h = {};
    h.n_dec_units = base[0];
    h.n_pf_units = min(base[1], p.max_pf_units);
    h.n_dec_seqs = base[0] / p.Hkv;
    h.n_pf_items = min(base[3], p.max_pf_items);
    h.zero = 0;
    h.pf_chunk = pf_chunk.d;
    h.n_split_units = base[4];
    h.dec_blocks = base[2];
    // decode waves given work: every one of them gets at least one block
    h.pad0[0] = max(1, min(fused_dec_waves(p, tot_pf, base[2], base[3]), base[2]));
    for (int x = 0; x < kQueues; ++x) {
      h.pf_q_base[x] = x * p.max_pf_items;
      h.pf_q_count[x] = max(0, min(base_q[x], p.max_pf_items));
      h.pf_q_next[x] = 0;
    }
    *p.hdr = h;
  }
}

}  // namespace rpa
