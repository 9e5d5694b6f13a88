// Launch geometry, work-record layouts and workspace constants of the ragged
// paged attention library: plain C++ shared by the kernels and by the host
// code that sizes and carves the workspace (which is also built without HIP,
// for the host-side sanitizer test).
#pragma once

#include <stdint.h>

namespace rpa {

// Rows of a decode-class unit: one 16-wide MFMA column block.
constexpr int kDecRows = 16;
// A prefill-class tile is worked by 4 waves of 32 packed rows each. For
// head_dim <= 128 two such workgroups share a CU (two waves per SIMD, with
// barriers that couple only their own 4 waves); head_dim 256 needs a whole
// SIMD's registers per wave.
constexpr int kPfWaves = 4;
// 32-row halves per wave of the 4-wave kernel: one (two, with each operand
// read serving two MFMAs, measured slower: one wave per SIMD hides less)
constexpr int kPfHalves = 1;
constexpr int pf_rows_for(int /*head_dim*/) { return 32 * kPfHalves * kPfWaves; }
constexpr int pf_wgs_per_cu(int D) { return D >= 256 ? 1 : 2; }
// Keys per pipeline step in both attention kernels.
constexpr int kStepKeys = 32;
// Largest key chunk of a prefill-class item (bounds the per-item page cache).
constexpr int kPfMaxChunk = 32768;

// ----------------------------------------------------------------------------
// Plan records written by the planning kernel, read by the attention and
// merge kernels. A unit is one sequence, one kv head and a run of packed query
// rows (row = token_in_seq * G + g, the GQA row packing of the kernel page's
// per-kv-head step). An item is one key chunk of a unit.
struct Unit {
  int32_t seq;
  int32_t kv_head;
  int32_t row0;   // first packed row of the unit, relative to the sequence
  int32_t nrows;  // number of packed rows
  int32_t kv_lo;  // start of the unit's chunk grid (16-aligned)
  int32_t kv_hi;  // one past the last key any of the rows can see
  int32_t nch;    // chunks (>= 1)
  int32_t item0;  // index of the unit's first item
};
static_assert(sizeof(Unit) == 32, "unit record is int32[8]");

// A prefill item: chunk `chunk` of unit `unit`, with a copy of the unit's
// record and of its sequence's metadata, so that a workgroup starting the item
// reads one 64-byte record (instead of the item, then the unit, then the
// sequence: three round trips to memory).
struct Item {
  int32_t unit;
  int32_t chunk;
  int32_t seq, kv_head, row0, nrows, kv_lo, kv_hi, nch, item0;  // the unit's record (Unit)
  int32_t q0, ql, kvl;  // the sequence's first query token, query tokens, kv length (clamped to the table)
  int32_t pad[3];
};
static_assert(sizeof(Item) == 64, "item record is int32[16]");

// Decode-class work is scheduled stream-K style: the key blocks (kDecBlk
// keys) of all decode units, laid end to end in (sequence, kv head) order, are cut into
// equal contiguous ranges, one per decode wave; each wave runs the parts of
// the units that fall into its range. The planner writes one record per
// decode sequence and nothing per part: a wave finds the sequence holding its
// first block by a search over `blk0` and derives every part from the records
// and its range. The units of a record are (seq, kv head h) for h < Hkv, each
// with all ql * G packed rows and blocks [blk0 + h * nb, blk0 + (h + 1) * nb).
struct DecSeq {
  int32_t seq;
  int32_t q0;    // first token of the sequence
  int32_t ql;    // its query tokens
  int32_t kvl;   // kv_len, clamped to the page table's reach
  int32_t lo16;  // first key of its units' block grid (16-aligned)
  int32_t hi;    // one past the last key any of its rows can see
  int32_t blk0;  // its first block in the stream-K order
  int32_t nb;    // blocks of each of its units (0: no visible key)
};
static_assert(sizeof(DecSeq) == 32, "decode sequence record is int32[8]");
// Keys per stream-K block: one 16-key pipeline step for 16-bit K/V; two for
// one-byte K/V, whose decode waves compute 32 keys per step (so that every
// part of a unit is a whole number of such steps).
constexpr int kDecBlk16 = 16;
constexpr int kDecBlk8 = 32;

// Prefill-class items are queued per XCD (MI355X: 8 XCDs, each with its own
// L2). All row blocks of one (sequence, kv head) go to the same queue, one
// after the other, so the workgroups of one XCD that run at the same time
// stream the same K/V pages and share them through that XCD's L2.
constexpr int kQueues = 8;

struct Header {
  int32_t n_dec_units;  // decode sequences x Hkv
  int32_t n_pf_units;
  int32_t n_dec_seqs;   // records of the decode sequence table
  int32_t n_pf_items;
  int32_t zero;  // 0 (decode chunks follow the stream-K split)
  int32_t pf_chunk;
  int32_t n_split_units;  // prefill units with more than one chunk
  int32_t dec_blocks;   // 16-key blocks of all decode units (the stream-K total)
  int32_t pad0[8];      // pad0[0]: decode waves given work (min(dec_waves, dec_blocks), >= 1)
  int32_t pf_q_base[kQueues];   // start of each prefill queue in pf_qlist (x * max_pf_items)
  int32_t pf_q_count[kQueues];  // its length
  int32_t pf_q_next[kQueues];   // its head, zeroed by the planning kernel
  int32_t pad1[24];
};
static_assert(sizeof(Header) == 256, "header is int32[64]");

// ----------------------------------------------------------------------------
// Decode-class launch geometry

constexpr int kDecWavesPerBlock = 4;
constexpr int kDecStepKeys = 16;
// LDS budget of one decode wave (4 waves per workgroup; 40 KB: one
// workgroup per CU)
#ifndef RPA_DEC_WAVE_LDS
#define RPA_DEC_WAVE_LDS (20 * 1024)
#endif
constexpr int kDecWaveLds = RPA_DEC_WAVE_LDS;

template <int D, bool FP8>
struct DecCfg {
  static constexpr int EB = FP8 ? 1 : 2;         // bytes per K/V element
  static constexpr int RB = D * EB;              // bytes of one K (or V) row of a head
  static constexpr int REGION = 16 * RB;         // the step's 16 K (or V) rows
  static constexpr int STAGE = 2 * REGION;       // K region, then V region
  static constexpr int NDR = REGION / 1024;      // DMA instructions per region
  static constexpr int NDMA = 2 * NDR;           // DMA instructions per step
  static constexpr int CPR = RB / 16;            // 16-byte chunks per row
  static constexpr int RP = RB >= 256 ? 1 : 256 / RB;  // rows per 256 bytes (one LDS bank sweep)
  static constexpr int NI = D / 32;              // 8-wide k-slots of Q^T per lane (16x16x32 k-steps)
  static constexpr int ND = D / 16;              // 16-row blocks of O^T
  static constexpr int NLD = RB / 64;            // 16-byte K pieces per lane
  // bf16: the next part's 16 Q rows (bf16), DMA'd during the current part.
  // fp8 takes them into registers instead and spends the space on the ring.
  static constexpr int QSLOT = FP8 ? 0 : 16 * D * 2;
  // fp8 head_dim 256 needs more than 256 registers: one wave per SIMD, so
  // each wave takes twice the LDS
  static constexpr int BUDGET = (FP8 && D >= 256) ? 2 * kDecWaveLds : kDecWaveLds;
  static constexpr int NST_FIT = (BUDGET - QSLOT) / STAGE;
  static constexpr int NST = NST_FIT < 2 ? 2 : (NST_FIT > 8 ? 8 : NST_FIT);  // ring slots
  static constexpr int WAVE_LDS = NST * STAGE + QSLOT;
  static_assert(REGION % 1024 == 0, "whole 1 KB DMA instructions per region");
  static_assert(WAVE_LDS * kDecWavesPerBlock <= 160 * 1024, "LDS of a workgroup");
  static_assert((NST - 1) * NDMA < 64, "vmcnt range");
};
template <int D, bool FP8>
constexpr int dec_wgs_per_cu() {
  return (160 * 1024) / (DecCfg<D, FP8>::WAVE_LDS * kDecWavesPerBlock);
}
// resident decode waves per SIMD (sizes the register budget)
constexpr int dec_waves_per_simd(int D, bool fp8) {
  if (fp8) return D == 64 ? dec_wgs_per_cu<64, true>() : D == 128 ? dec_wgs_per_cu<128, true>() : dec_wgs_per_cu<256, true>();
  return D == 64 ? dec_wgs_per_cu<64, false>() : D == 128 ? dec_wgs_per_cu<128, false>() : dec_wgs_per_cu<256, false>();
}

// Waves of a workgroup of the two-group (ping-pong) prefill kernel: two per
// SIMD, 32 packed rows each; a unit of that kernel has kPpRows rows.
constexpr int kPpWaves = 8;
constexpr int kPpRows = 32 * kPpWaves;

}  // namespace rpa
