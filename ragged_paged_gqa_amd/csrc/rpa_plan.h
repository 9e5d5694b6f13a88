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
//     finished-chunk counter is cleared for the split merge;
//   * prefill items are dealt into one queue per XCD: all items of a
//     (sequence, kv head) go to queue (seq * Hkv + h) % kQueues, chunk-major,
//     so an XCD's concurrently running workgroups stream the same K/V chunk
//     and share it in that XCD's L2. Queue x lives at
//     pf_qlist[x * max_pf_items].
//
// Work split inside the workgroup: sequences are taken in tiles of
// kPlanThreads, one thread per sequence for the per-sequence counts and for
// the one block scan that turns them into record offsets; a thread per
// (decode sequence, kv head) for that unit and its items, staged in LDS and
// stored in contiguous runs; a wave per prefill sequence, a row block per
// lane.
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

// Per-sequence counts (scan slots): 0 decode units, 1 prefill units,
// 2 decode items, 3 prefill items, 4 split units, 5.. prefill items per queue
constexpr int kScanN = 5 + kQueues;

// Per prefill sequence of a tile, filled by its wave.
struct PfInfo {
  int32_t s;         // sequence
  int32_t per_head;  // items of one kv head
  int32_t nsplit;    // row blocks with more than one chunk
  int32_t max_nch;   // most chunks of one row block
};

// A decode sequence of a tile, for the writing of its units and items.
struct DecSeq {
  int32_t s, ql, kvl, q0;
  int32_t blk0, nb;  // its first stream-K block, blocks per kv head
  int32_t lo16, hi;  // key range of its units
};
// Decode items staged in LDS per round of (sequence, kv head) pairs; a round
// with more items writes the rest directly.
constexpr int kPlanItemBuf = 1024;

// Offsets of a prefill sequence's records, from the block scan.
struct PfOffs {
  int32_t unit, item;
  int32_t queue[kQueues];
};

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

// Stream-K split of the decode work: the Tb key blocks of all decode units,
// laid end to end (unit (s, h) at blocks [blk0_s + h * nb_s, + nb_s)), are cut
// into W contiguous ranges, W <= Tb so that none is empty; wave w runs blocks
// [start(w), start(w + 1)). A unit with no key block gets no item (the combine
// kernel writes its rows).
// Range starts of up to this many decode waves are tabulated in LDS.
constexpr int kPlanMaxDecWaves = 4096;

struct StreamK {
  int64_t Tb;
  int32_t W;
  // start(w) for w <= W when W <= kPlanMaxDecWaves, else null (an LDS pointer:
  // a generic one would make every lookup wait for the kernel's global stores)
  const __attribute__((address_space(3))) int32_t* table;
  double inv_Tb, inv_W;
  __device__ int32_t start_exact(int32_t w) const { return (int32_t)floor_div(Tb * w, W, inv_W); }
  __device__ int32_t start(int32_t w) const { return table ? table[w] : start_exact(w); }
  // the wave whose range holds block x (0 <= x < Tb)
  __device__ int32_t wave_of(int32_t x) const {
    const int64_t w = floor_div((int64_t)(x + 1) * W - 1, Tb, inv_Tb);
    return (int32_t)(w < W - 1 ? w : W - 1);
  }
  // items of unit blocks [b0, b0 + nb): one per wave from wa to wb
  __device__ int32_t n_items(int32_t b0, int32_t nb, int32_t& wa) const {
    if (nb <= 0 || Tb <= 0) {
      wa = 0;
      return 0;
    }
    wa = wave_of(b0);
    return wave_of(b0 + nb - 1) - wa + 1;
  }
};

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(Params p) {
  __shared__ int64_t red[2][kPlanWaves];
  __shared__ int32_t sh[kPlanWaves * kScanN];
  __shared__ int32_t n_pf_tile;
  __shared__ PfInfo pf_info[kPlanThreads];
  __shared__ int32_t sk_start[kPlanMaxDecWaves + 1];
  __shared__ PfOffs pf_offs[kPlanThreads];
  __shared__ DecSeq dec_seq[kPlanThreads];
  __shared__ int4 ubuf[kPlanThreads][2];
  __shared__ int4 ibuf[kPlanItemBuf][4];
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

  // pass 1: total visible keys of each class, to size the chunks
  int64_t dec_keys = 0, pf_keys = 0;
  for (int32_t s0 = 0; s0 < n; s0 += kPlanThreads) {
    if (tid == 0) n_pf_tile = 0;
    __syncthreads();
    const int32_t s = s0 + tid;
    int32_t ql = 0, kvl = 0, slot;
    if (s < n) seq_meta(p, s, ql, kvl);
    if (s < n && ql > 0 && ql * p.G <= kDecRows)
      dec_keys += (int64_t)p.Hkv * ((range_keys(unit_range(p, G, ql, kvl, 0, ql * p.G)) + 15) / 16);
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
  for (int o = 32; o > 0; o >>= 1) {
    dec_keys += __shfl_xor(dec_keys, o);
    pf_keys += __shfl_xor(pf_keys, o);
  }
  if (lane == 0) {
    red[0][wave] = dec_keys;
    red[1][wave] = pf_keys;
  }
  __syncthreads();
  int64_t tot_dec = 0, tot_pf = 0;
  for (int w = 0; w < kPlanWaves; ++w) {
    tot_dec += red[0][w];
    tot_pf += red[1][w];
  }
  // tot_dec counts 16-key blocks of decode units; with fewer blocks than
  // waves only the first tot_dec waves get work, so every used wave's range
  // holds at least one block
  const int32_t n_dec_waves = (int32_t)max((int64_t)1, min((int64_t)max(p.dec_waves, 1), tot_dec));
  const bool tabulate = n_dec_waves <= kPlanMaxDecWaves;
  const StreamK sk{tot_dec, n_dec_waves,
                   tabulate ? (const __attribute__((address_space(3))) int32_t*)sk_start : nullptr,
                   tot_dec > 0 ? 1.0 / (double)tot_dec : 0.0, 1.0 / (double)n_dec_waves};
  if (tabulate)
    for (int32_t w = tid; w <= n_dec_waves; w += kPlanThreads) sk_start[w] = sk.start_exact(w);
  for (int32_t w = tid; w < max(p.dec_waves, 1); w += kPlanThreads) p.dec_wave_first[w] = INT32_MAX;
  const FastDiv pf_chunk = make_div(pick_chunk(tot_pf, p.target_pf_items, kPfMinChunk, kPfMaxChunk));

  // pass 2: per-sequence counts -> one scan per tile -> records
  int32_t base[kScanN];
#pragma unroll
  for (int k = 0; k < kScanN; ++k) base[k] = 0;
  int32_t base_blk = 0;  // decode blocks of the earlier tiles
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
      for (int32_t r0 = lane * R; r0 < rows; r0 += 64 * R) {
        const int32_t nch = n_chunks(unit_range(p, G, pql, pkvl, r0, min(R, rows - r0)), pf_chunk);
        items += nch;
        nsplit += nch > 1;
        max_nch = max(max_nch, nch);
      }
      items = wave_sum(items);
      nsplit = wave_sum(nsplit);
      max_nch = wave_max(max_nch);
      if (lane == 0) {
        pf_info[i].per_head = items;
        pf_info[i].nsplit = nsplit;
        pf_info[i].max_nch = max_nch;
      }
    }
    __syncthreads();
    // (b) a thread per sequence: counts, scan
    int32_t cnt[kScanN];
#pragma unroll
    for (int k = 0; k < kScanN; ++k) cnt[k] = 0;
    const bool is_dec = s < n && ql > 0 && ql * p.G <= kDecRows;
    // decode: the sequence's block offset in the stream-K order first
    int32_t nb = 0;
    if (is_dec) nb = (range_keys(unit_range(p, G, ql, kvl, 0, ql * p.G)) + 15) / 16;
    int32_t blk0;
    {
      const int32_t v[1] = {p.Hkv * nb};
      int32_t e[1], t[1];
      block_scan<1>(v, e, t, sh);
      blk0 = base_blk + e[0];
      base_blk += t[0];
    }
    if (is_dec) {
      int32_t items = 0, nsplit = 0;
      for (int32_t h = 0; h < p.Hkv; ++h) {
        int32_t wa;
        const int32_t ni = sk.n_items(blk0 + h * nb, nb, wa);
        items += ni;
        nsplit += ni > 1;
      }
      cnt[0] = p.Hkv;
      cnt[2] = items;
      cnt[4] = nsplit;
    } else if (slot >= 0) {
      const PfInfo& f = pf_info[slot];
      const int32_t nrb = (ql * p.G + R - 1) / R;
      cnt[1] = p.Hkv * nrb;
      cnt[3] = p.Hkv * f.per_head;
      cnt[4] = p.Hkv * f.nsplit;
      for (int32_t h = 0; h < p.Hkv; ++h) {
        const int x = (s * p.Hkv + h) % kQueues;
#pragma unroll
        for (int k = 0; k < kQueues; ++k) cnt[5 + k] += x == k ? f.per_head : 0;
      }
    }
    int32_t off[kScanN], tot[kScanN];
    block_scan<kScanN>(cnt, off, tot, sh);
    const int32_t tile_u0 = base[0], tile_i0 = base[2], n_dec_units_tile = tot[0];
#pragma unroll
    for (int k = 0; k < kScanN; ++k) off[k] += base[k];
#pragma unroll
    for (int k = 0; k < kScanN; ++k) base[k] += tot[k];

    if (slot >= 0) {
      pf_offs[slot].unit = off[1];
      pf_offs[slot].item = off[3];
#pragma unroll
      for (int x = 0; x < kQueues; ++x) pf_offs[slot].queue[x] = off[5 + x];
    }

    // (c) decode units and items. Each decode sequence of the tile leaves its
    // metadata in LDS (at its rank among the tile's decode sequences), then a
    // thread per (sequence, kv head) pair builds that unit and its items (one
    // per decode wave its blocks fall on) in LDS, a block scan placing the
    // items, and the whole block copies them out with contiguous 16-byte
    // stores: the records of consecutive pairs are consecutive in memory, so
    // the stores of one compute unit stay coalesced.
    if (is_dec) {
      const UnitRange r = unit_range(p, G, ql, kvl, 0, ql * p.G);
      int32_t q0, qlx;
      seq_tokens(p, s, q0, qlx);
      dec_seq[(off[0] - tile_u0) / p.Hkv] = DecSeq{s, ql, kvl, q0, blk0, nb, r.lo16, r.hi};
    }
    __syncthreads();
    {
      const int32_t npairs = n_dec_units_tile;  // decode sequences of the tile x Hkv
      int32_t round_i0 = tile_i0;
      for (int32_t P = 0; P < npairs; P += kPlanThreads) {
        const int32_t pair = P + tid;
        const bool valid = pair < npairs;
        DecSeq ds{};
        int32_t h = 0, b0 = 0, nch = 0, wa = 0;
        if (valid) {
          const int32_t i = pair / p.Hkv;
          h = pair - i * p.Hkv;
          ds = dec_seq[i];
          b0 = ds.blk0 + h * ds.nb;
          nch = sk.n_items(b0, ds.nb, wa);
        }
        int32_t excl[1], tot_i[1];
        {
          const int32_t v[1] = {nch};
          block_scan<1>(v, excl, tot_i, sh);
        }
        const int32_t ui = tile_u0 + pair;
        const int32_t ii0 = round_i0 + excl[0];
        const int32_t nrows = ds.ql * p.G;
        if (valid && ui < p.max_dec_units) {
          // Unit {seq, kv_head, row0, nrows | kv_lo, kv_hi, nch, item0}
          ubuf[tid][0] = int4{ds.s, h, 0, nrows};
          ubuf[tid][1] = int4{ds.lo16, ds.hi, nch, ii0};
          p.unit_done[ui] = 0;
          int32_t ws = nch > 0 ? sk.start(wa) : 0;
          for (int32_t c = 0; c < nch; ++c) {
            const int32_t ii = ii0 + c;
            const int32_t w = wa + c;
            if (ii >= p.max_dec_items) break;
            // the unit's blocks inside wave w's range
            const int32_t we = w + 1 < sk.W ? sk.start(w + 1) : (int32_t)sk.Tb;
            const int32_t x0 = max(b0, ws);
            const int32_t x1 = min(b0 + ds.nb, we);
            // DecItem {seq, kv_head, c_lo, c_hi | kvl, q0, ql, row0 |
            //          nrows, nch, unit, chunk | wave, 0, 0, 0}
            const int4 rec[4] = {int4{ds.s, h, ds.lo16 + 16 * (x0 - b0), min(ds.hi, ds.lo16 + 16 * (x1 - b0))},
                                 int4{ds.kvl, ds.q0, ds.ql, 0}, int4{nrows, nch, ui, c}, int4{w, 0, 0, 0}};
            const int32_t loc = ii - round_i0;
            if (loc < kPlanItemBuf) {
#pragma unroll
              for (int k = 0; k < 4; ++k) ibuf[loc][k] = rec[k];
            } else {
#pragma unroll
              for (int k = 0; k < 4; ++k) reinterpret_cast<int4*>(p.dec_items + ii)[k] = rec[k];
            }
            // the item holding a wave's first block starts the wave's items
            if (b0 <= ws) p.dec_wave_first[w] = ii;
            ws = we;
          }
        }
        __syncthreads();
        // copy-out: units [tile_u0 + P, + n_u), items [round_i0, + n_i)
        const int32_t n_u = min(kPlanThreads, npairs - P);
        for (int32_t k = tid; k < 2 * n_u; k += kPlanThreads) {
          const int32_t u = tile_u0 + P + k / 2;
          if (u < p.max_dec_units) reinterpret_cast<int4*>(p.dec_units + u)[k & 1] = ubuf[k / 2][k & 1];
        }
        const int32_t n_i = min(tot_i[0], kPlanItemBuf);
        for (int32_t k = tid; k < 4 * n_i; k += kPlanThreads) {
          const int32_t it = round_i0 + k / 4;
          if (it < p.max_dec_items) reinterpret_cast<int4*>(p.dec_items + it)[k & 3] = ibuf[k / 4][k & 3];
        }
        round_i0 += tot_i[0];
        __syncthreads();
      }
    }

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
            p.unit_done[p.max_dec_units + ui] = 0;
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
    h.n_dec_units = min(base[0], p.max_dec_units);
    h.n_pf_units = min(base[1], p.max_pf_units);
    h.n_dec_items = min(base[2], p.max_dec_items);
    h.n_pf_items = min(base[3], p.max_pf_items);
    h.zero = 0;
    h.pf_chunk = pf_chunk.d;
    h.n_split_units = base[4];
    h.dec_blocks = (int32_t)min(tot_dec, (int64_t)INT32_MAX);
    h.pad0[0] = n_dec_waves;
    for (int x = 0; x < kQueues; ++x) {
      h.pf_q_base[x] = x * p.max_pf_items;
      h.pf_q_count[x] = max(0, min(base[5 + x], p.max_pf_items));
      h.pf_q_next[x] = 0;
    }
    *p.hdr = h;
  }
}

}  // namespace rpa
