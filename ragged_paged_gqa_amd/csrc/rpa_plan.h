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

#include <climits>

#include "rpa_common.h"

namespace rpa {

constexpr int kPlanThreads = 512;  // 1024 would cap a wave at 128 VGPRs and spill
constexpr int kPlanWaves = kPlanThreads / 64;
// Smallest prefill chunk (keys): an item has a fixed cost (its Q tile, block
// table, pipeline fill, partial and share of the merge), so items are kept
// from getting small even when that leaves fewer items than workgroups.
#ifndef RPA_PF_MIN_CHUNK
#define RPA_PF_MIN_CHUNK 8192
#endif
constexpr int kPfMinChunk = RPA_PF_MIN_CHUNK;

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

// Wave-wide scans and reductions with DPP lane moves (VALU operations): a
// shift by 1, 2, 4 and 8 lanes inside each row of 16, then row 0's last lane
// added into row 1 and row 2's into row 3, then lane 31 into rows 2 and 3.
// Lanes whose source falls outside take the identity.
template <typename Op>
__device__ __forceinline__ int32_t dpp_incl_scan(int32_t v, int32_t ident, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
  return dpp_incl_scan(v, 0, [](int32_t a, int32_t b) { return a + b; });
}
__device__ __forceinline__ int32_t wave_sum(int32_t v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}
__device__ __forceinline__ int32_t wave_max(int32_t v) {
  return __builtin_amdgcn_readlane(dpp_incl_scan(v, INT_MIN, [](int32_t a, int32_t b) { return max(a, b); }), 63);
}
// one DPP lane move of a 64-bit value (both halves)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int64_t dpp_move64(int64_t x) {
  const uint64_t u = (uint64_t)x;
  const int32_t lo = __builtin_amdgcn_update_dpp(0, (int32_t)(uint32_t)u, CTRL, ROW_MASK, 0xf, false);
  const int32_t hi = __builtin_amdgcn_update_dpp(0, (int32_t)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xf, false);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
  v += dpp_move64<0x111, 0xf>(v);
  v += dpp_move64<0x112, 0xf>(v);
  v += dpp_move64<0x114, 0xf>(v);
  v += dpp_move64<0x118, 0xf>(v);
  v += dpp_move64<0x142, 0xa>(v);
  v += dpp_move64<0x143, 0xc>(v);
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = __builtin_amdgcn_readlane((int32_t)(uint32_t)u, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int32_t)(uint32_t)(u >> 32), 63);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Block-wide exclusive scan of NV ints per thread at once: excl[k] gets the
// sum of v[k] over lower threads, tot[k] the block total. `sh` holds
// kPlanWaves * NV ints.
template <int NV>
__device__ void block_scan(const int32_t (&v)[NV], int32_t (&excl)[NV], int32_t (&tot)[NV], int32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) x[k] = wave_incl_scan(v[k]);
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < NV; ++k) sh[wave * NV + k] = x[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    int32_t before = 0, all = 0;
#pragma unroll
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
  int32_t nrb;       // row blocks (units of one kv head)
  int32_t lcls;      // size class of its units' last chunks (largest over its row blocks)
  int64_t work;      // visible keys of its row blocks (one kv head)
};

// Offsets of a prefill sequence's records, from the block scan.
struct PfOffs {
  int32_t unit, item;
  int32_t qa[kQueues];  // where its heads' chunks before a unit's last one start in each queue
  int32_t qb[kQueues];  // where its heads' last chunks start in each queue
};

// Size classes of a unit's last chunk (keys * kLastClasses / chunk): the
// queues hold every unit's other chunks first, then the last chunks, larger
// classes first, so that the smallest pieces of work are the last taken.
constexpr int kLastClasses = 16;

// Queue of the g-th (sequence, kv head) in work order: dealt to the queues
// back and forth (0..7, 7..0, ...), so that every queue gets a share of
// the heaviest and of the lightest.
__device__ __forceinline__ int snake_queue(int32_t g) {
  const int32_t round = g / kQueues, k = g % kQueues;
  return (round & 1) ? kQueues - 1 - k : k;
}
// How many of the groups g0 .. g - 1 go to queue x (in every 2 * kQueues
// consecutive groups, queue x takes positions x and 2 * kQueues - 1 - x).
__device__ __forceinline__ int32_t snake_count(int32_t g0, int32_t g, int x) {
  constexpr int32_t P = 2 * kQueues;
  auto upto = [x](int32_t n) { return 2 * (n / P) + (x < n % P) + (P - 1 - x < n % P); };
  return upto(g) - upto(g0);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(Params p) {
  __shared__ int64_t red[kPlanWaves];
  __shared__ int32_t sh[kPlanWaves * kQueues];
  __shared__ int32_t n_pf_tile;
  __shared__ PfInfo pf_info[kPlanThreads];
  __shared__ int32_t by_rank[kPlanThreads];  // prefill slots of the tile, heaviest sequence first
  __shared__ int32_t by_rank_b[kPlanThreads];  // the same by last-chunk class, larger first
  __shared__ int32_t rank_of[kPlanThreads];  // work rank of each prefill slot
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
  pf_keys = wave_sum64(pf_keys);
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
      int32_t items = 0, nsplit = 0, max_nch = 0, lcls = 0;
      int64_t work = 0;
      for (int32_t r0 = lane * R; r0 < rows; r0 += 64 * R) {
        const UnitRange r = unit_range(p, G, pql, pkvl, r0, min(R, rows - r0));
        const int32_t nch = n_chunks(r, pf_chunk);
        items += nch;
        nsplit += nch > 1;
        max_nch = max(max_nch, nch);
        work += range_keys(r);
        const int32_t last = range_keys(r) - (nch - 1) * pf_chunk.d;
        lcls = max(lcls, min(kLastClasses - 1, fdiv(max(last, 0) * kLastClasses, pf_chunk)));
      }
      items = wave_sum(items);
      nsplit = wave_sum(nsplit);
      max_nch = wave_max(max_nch);
      lcls = wave_max(lcls);
      work = wave_sum64(work);
      if (lane == 0) {
        pf_info[i].per_head = items;
        pf_info[i].nsplit = nsplit;
        pf_info[i].max_nch = max_nch;
        pf_info[i].nrb = (rows + R - 1) / R;
        pf_info[i].lcls = lcls;
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
    // queue offsets. The tile's prefill sequences are ranked heaviest first
    // (visible keys; ties by sequence index) and their (sequence, kv head)
    // groups dealt to the queues back and forth in that order. In a queue the
    // tile's groups first place every chunk but their units' last ones, in
    // rank order, then the last chunks, by size class (larger first; ties by
    // rank). A group's entries in each part stay contiguous and chunk-major.
    if (n_pf_tile > 0) {  // (block-uniform)
      if (slot >= 0) {
        const int64_t wk = pf_info[slot].work;
        int32_t r = 0;
#pragma unroll 4
        for (int32_t j = 0; j < n_pf_tile; ++j) {
          const int64_t wj = pf_info[j].work;
          r += wj > wk || (wj == wk && pf_info[j].s < s);
        }
        by_rank[r] = slot;
        rank_of[slot] = r;
      }
      __syncthreads();
      if (slot >= 0) {
        const int32_t ck = pf_info[slot].lcls, rk = rank_of[slot];
        int32_t rb = 0;
#pragma unroll 4
        for (int32_t j = 0; j < n_pf_tile; ++j) {
          const int32_t cj = pf_info[j].lcls;
          rb += cj > ck || (cj == ck && rank_of[j] < rk);
        }
        by_rank_b[rb] = slot;
      }
      __syncthreads();
      // the first part's offsets (thread t: the t-th sequence by work)...
      int32_t ta[kQueues];
      {
        int32_t qa[kQueues], oa[kQueues];
#pragma unroll
        for (int x = 0; x < kQueues; ++x) qa[x] = 0;
        const int32_t ra = tid < n_pf_tile ? by_rank[tid] : -1;
        if (ra >= 0) {
          const int32_t nq = pf_info[ra].per_head - pf_info[ra].nrb;
          for (int32_t h = 0; h < p.Hkv; ++h) {
            const int x = snake_queue(tid * p.Hkv + h);
#pragma unroll
            for (int k = 0; k < kQueues; ++k) qa[k] += x == k ? nq : 0;
          }
        }
        block_scan<kQueues>(qa, oa, ta, sh);
        if (ra >= 0) {
#pragma unroll
          for (int x = 0; x < kQueues; ++x) pf_offs[ra].qa[x] = base_q[x] + oa[x];
        }
      }
      // ...then the second's (thread t: the t-th sequence by last-chunk class)
      {
        int32_t qb[kQueues], ob[kQueues], tb[kQueues];
#pragma unroll
        for (int x = 0; x < kQueues; ++x) qb[x] = 0;
        const int32_t rb = tid < n_pf_tile ? by_rank_b[tid] : -1;
        if (rb >= 0) {
          const int32_t nq = pf_info[rb].nrb, g0 = rank_of[rb] * p.Hkv;
          for (int32_t h = 0; h < p.Hkv; ++h) {
            const int x = snake_queue(g0 + h);
#pragma unroll
            for (int k = 0; k < kQueues; ++k) qb[k] += x == k ? nq : 0;
          }
        }
        block_scan<kQueues>(qb, ob, tb, sh);
        if (rb >= 0) {
#pragma unroll
          for (int x = 0; x < kQueues; ++x) pf_offs[rb].qb[x] = base_q[x] + ta[x] + ob[x];
        }
#pragma unroll
        for (int x = 0; x < kQueues; ++x) base_q[x] += ta[x] + tb[x];
      }
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
      int32_t pql, pkvl, pq0, pql_t;
      seq_meta(p, ps, pql, pkvl);
      seq_tokens(p, ps, pq0, pql_t);
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
        carry += __builtin_amdgcn_readlane(incl, 63);
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
              if (ii + c < p.max_pf_items)
                p.pf_items[ii + c] = Item{ui, c, ps, h, r0, nr, r.lo16, r.hi, nch, ii, pq0, pql, pkvl, {0, 0, 0}};
          }
        }
      }
      // queue entries, chunk-major: chunk 0 of every row block, then chunk 1
      // of those that have one, ...; a unit's last chunk goes to the second
      // part. A head's entries in a part are contiguous, after those of this
      // sequence's earlier heads in the same queue.
      const int32_t rank = rank_of[i];
      int32_t pos_a = 0, pos_b = 0;  // entries of this sequence's head so far, per part
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
          carry_items += __builtin_amdgcn_readlane(incl, 63);
          const bool in_a = c < nch - 1, in_b = c == nch - 1;
          const uint64_t ma = __ballot(in_a), mb = __ballot(in_b);
          const uint64_t below = (1ull << lane) - 1ull;
          if (in_a || in_b) {
            const int32_t before = in_a ? __popcll(ma & below) : __popcll(mb & below);
            for (int32_t h = 0; h < p.Hkv; ++h) {
              const int x = snake_queue(rank * p.Hkv + h);
              const int32_t j = snake_count(rank * p.Hkv, rank * p.Hkv + h, x);  // earlier heads in queue x
              const int32_t k = in_a ? pf_offs[i].qa[x] + j * (f.per_head - f.nrb) + pos_a + before
                                     : pf_offs[i].qb[x] + j * f.nrb + pos_b + before;
              const int32_t item = item0 + h * f.per_head + item_off + c;
              if (k < p.max_pf_items && item < p.max_pf_items)
                p.pf_qlist[(int64_t)x * p.max_pf_items + k] = item;
            }
          }
          pos_a += __popcll(ma);
          pos_b += __popcll(mb);
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
