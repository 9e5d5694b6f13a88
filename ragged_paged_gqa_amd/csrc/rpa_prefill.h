// Prefill/mixed-class attention kernel: units of up to kPfRows packed query
// rows (row = token * G + g) of one sequence and one kv head — the kernel
// page's q block of `num_queries_per_block` tokens times the G q heads of one
// kv head, stacked into one MFMA dimension (`run`, per-kv-head step).
//
// A workgroup of NW waves owns one item (a key chunk of a unit) at a time,
// pulled from a device-wide queue; wave w owns rows [32w, 32w + 32). Split
// units leave partials; the workgroup finishing a unit's last chunk merges
// them (rpa_merge.h).
// Per load step of 32 keys:
//   * loader: the step's K and V rows of kv head h (combined heads 2h and
//     2h+1, adjacent in memory — `stridedLoadKv`) are gathered through the
//     page table into a ring of LDS tiles laid out so that the MFMA operand
//     reads below are bank-conflict free. bf16 rows go straight from HBM to
//     LDS (global_load_lds_dwordx4) two steps ahead of the compute; fp8 rows
//     are staged through registers one step ahead and widened to bf16 on the
//     way. The physical address of every 16-key block of an item is worked
//     out once, into an LDS table, when the item starts. One barrier per step
//     publishes the tile.
// Per 32-key block of the step:
//   * S^T [32 keys x 32 rows] = K Q^T with v_mfma_f32_32x32x16_bf16, Q^T kept
//     in registers; lane (row, half h) holds 16 keys of its row, so a row
//     maximum needs one cross-lane exchange (v_permlane32_swap);
//   * masks (`flashAttention`: causal, sliding window, kv length) are applied
//     only on blocks that can contain a hidden key;
//   * base-2 online softmax with a lazily moved reference maximum: the
//     accumulator is rescaled only when some row's maximum grows by more than
//     kRescaleSlack, and that rescale runs outside the block loop, so inside
//     it the accumulator is only ever an MFMA operand; P = 2^(s*c - m) is one
//     FMA and one exp2 per score;
//   * O^T [D x 32 rows] += V^T P^T with V^T read by ds_read_b64_tr_b16 and P^T
//     taken straight from the S^T accumulator layout.
//
// Element types: the kernel is instantiated per K/V kind KVT (K/V in the q
// type, fp8 e4m3fn, fp8 e5m2, int8) and per 16-bit type F16 (bf16, or f16
// with an f16 q: f16 MFMAs, f16 P and output). In the comments here "bf16"
// stands for that 16-bit type and "fp8" for any one-byte code (widened to it
// exactly: v_cvt_scalef32_pk_*_fp8 / _bf8, or sign extension for int8).
// Q32: an f32 q (bf16 path, K/V bf16 or one-byte): Q is split into bf16 hi
// and lo operands (split_q8), S^T takes both MFMA chains, out is f32.
#pragma once

#include <climits>
#include <type_traits>

#include "rpa_common.h"
#include "rpa_merge.h"

namespace rpa {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// The reference maximum of a row moves only when the row's maximum outgrows
// it by more than this (base-2 units): exponentiated scores stay <= 2^16,
// far inside f32 and bf16 range (one less for f16 P, whose largest finite
// value is 65504), and the accumulator rescale (which leaves the step loop,
// see below) is rare.
constexpr float kRescaleSlack = 16.0f;

template <bool F16>
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

#ifndef RPA_PF_STAGES
#define RPA_PF_STAGES 4
#endif
constexpr int kStagesBf16 = RPA_PF_STAGES;
// Block table entries per item: every 16-key block of the largest chunk, plus
// those of the load steps issued past its end.
constexpr int kPfBlkTable = kPfMaxChunk / 16 + 16;

// LDS layout of a ring slot: the step's K rows (region 0) and V rows (region
// 1), each kStepKeys unpadded rows of 2D bytes whose 16-byte chunks are
// XOR-swizzled by the key (swz_k / swz_v), so that one DMA instruction writes
// 1 KB of whole rows and the MFMA operand reads below are bank-conflict free.
// (No row padding serves both reads: the K reads want 16 consecutive keys in
// distinct 16-byte bank groups, the transposed V reads want 4 consecutive
// keys in distinct 64-byte quarters of the 256-byte bank row.)
template <int D, bool FP8>
struct PrefillLds {
  static constexpr int kRowBytes = 2 * D;      // row stride
  static constexpr int kChunks = 2 * D / 16;   // 16-byte chunks per K or V row
  static constexpr int kStepKeys = rpa::kStepKeys;  // keys per load step (one ring slot, one barrier)
  static constexpr int kRegionBytes = kStepKeys * kRowBytes;  // V region offset
  static constexpr int kBufBytes = 2 * kRegionBytes;
  static constexpr int kStages = FP8 ? 3 : kStagesBf16;
  static constexpr size_t kBytes = (size_t)kStages * kBufBytes;
};

// Chunk swizzles. K is read by MFMA operand loads in which 16 lanes hold 16
// consecutive keys at the same chunk: XOR with the key's low bits spreads
// them over the banks. V is read transposed (ds_read_b64_tr_b16) by 4 keys
// x 4 chunks per 16 lanes: XOR of the chunk's block-of-4 index with key % 4.
template <int D>
__device__ __forceinline__ int swz_k(int key) {
  constexpr int C = 2 * D / 16;
  return key & ((C < 16 ? C : 16) - 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int key) {
  constexpr int C = 2 * D / 16;
  return (4 * (key & 3)) & (C - 1);
}

// LDS of one workgroup of prefill_tiles.
template <int D, bool FP8>
struct PfShared {
  char lds[PrefillLds<D, FP8>::kBytes];  // the K/V ring (and the merge's staging)
  uint32_t blk[kPfBlkTable];             // physical key index of each 16-key block of the item
  int item[2];
  int last;
};

// The prefill-class tiles of one workgroup: it takes items from the queues
// until they are empty. CAP: the soft-cap is on (a template parameter, so the
// uncapped code's block loop has no branch and no cap arithmetic).
template <int D, int KVT, bool CAP, bool F16, bool Q32 = false>
__device__ __forceinline__ void prefill_tiles(const Params& p, PfShared<D, KVT != kKvBf16>& shm, int pf_block) {
  static_assert(!(Q32 && F16), "an f32 q runs on the bf16 path");
  constexpr bool FP8 = KVT != kKvBf16;  // one-byte codes (fp8 kinds, int8), widened in registers
  // f16 P must stay below 65504: exponentiated scores <= 2^15
  constexpr float SLACK = F16 ? kRescaleSlack - 1.0f : kRescaleSlack;
  constexpr int NW = kPfWaves;
  constexpr int NH = kPfHalves;               // 32-row halves per wave
  constexpr int WR = 32 * NH;                 // rows per wave
  constexpr int NS = D / 16;                  // k-steps of the QK product
  constexpr int NDB = D / 32;                 // 32-row blocks of O^T
  constexpr int EB = FP8 ? 1 : 2;             // bytes per K/V element in HBM
  constexpr int NT = NW * 64;
  constexpr int KS = PrefillLds<D, FP8>::kStepKeys;
  constexpr int NB = KS / 32;                 // 32-key score blocks per load step
  constexpr int NB16 = KS / 16;               // 16-key page blocks per load step
  constexpr int RB = PrefillLds<D, FP8>::kRowBytes;
  constexpr int CPR = PrefillLds<D, FP8>::kChunks;
  constexpr int REG = PrefillLds<D, FP8>::kRegionBytes;  // byte offset of a key's V row from its K row
  constexpr int BUF = PrefillLds<D, FP8>::kBufBytes;
  constexpr int NST = PrefillLds<D, FP8>::kStages;
  constexpr int GCH = 2 * D * EB / 16;        // 16-byte global chunks per key (K and V)
  constexpr int CPT = (KS * GCH + NT - 1) / NT;  // fp8 path: chunks per thread per step
  // bf16 path: full-width DMA instructions of 1 KB, RPI rows of one region
  // each, wave w moving region w / 2, keys [16 (w % 2), + 16): a wave's keys
  // lie in one 16-key page block.
  constexpr int RPI = 1024 / RB;              // rows per DMA instruction
  constexpr int NIW = (2 * KS / RPI) / NW;    // DMA instructions per wave per step
  static_assert(NDB >= 2, "head_dim >= 64");
  static_assert(RPI * CPR == 64, "whole rows per full-width DMA instruction");
  static_assert(KS % NW == 0 && (NB == 1 || NB == 2), "step shape");
  static_assert(!FP8 || NST == 3, "fp8 path stages through registers one step ahead");
  static_assert(FP8 || (KS == 32 && NW == 4 && NIW * RPI == 16), "a wave's rows stay in one 16-key block");

  char* const lds = shm.lds;
  uint32_t* const sh_blk = shm.blk;
  int* const sh_item = shm.item;
  int& sh_last = shm.last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r32 = lane & 31;  // S^T column = row within a 32-row half
  const int h = lane >> 5;    // which half of the row's keys this lane holds

  // Every item goes to one workgroup, so workgroups past the item count
  // would only ever find the queues drained: they leave at once.
  if (pf_block >= p.hdr->n_pf_items) return;
  const int chunk = p.hdr->pf_chunk;
  const int64_t key_stride = (int64_t)2 * p.Hkv * D * EB;
  constexpr bool capped = CAP;
  // scores in base-2 units are st * cmul (capped: the cap is applied to st
  // first and cmul = 1); negative scales flip Q's sign instead. A zero scale
  // becomes the smallest normal one, so that hidden keys (-inf) stay -inf
  // through the product while every visible score still rounds to 0.
  const bool neg = p.sm_scale < 0.f;
  const float sm = neg ? -p.sm_scale : p.sm_scale;
  const float cmul = capped ? 1.0f : fmaxf(sm * kLog2e, 1.17549435e-38f);
  const SoftCapB2 cap_b2(sm, capped ? p.soft_cap : 1.0f);
  // Uncapped with head_dim <= 128 (MFMA results in plain VGPRs) the scores
  // stay as the MFMA wrote them and the scale goes into the exponent's FMA
  // (and into the row maximum): one VALU instruction per score less.
  constexpr bool kLate = !CAP && D <= 128;

  // LDS read offsets inside a slot (loop-invariant per lane):
  //   K operand of k-step i: key r32, chunk 2i + h
  //   V^T operand of d-block d: key 4 (g16 / 2) + l16 / 4 (+ 8, + 16 ks),
  //   bytes 32 (g16 % 2) + 8 (l16 % 4) + 64 d of the row
  // The swizzles only permute chunks within 256-byte spans of a row (K: the
  // low 4 bits of the chunk index, V: its bits 2-3), so the offsets of
  // k-steps i and i + 8, and of d-blocks d and d + 4, differ by exactly 256
  // bytes: per-lane tables of KT and VT entries plus immediate offsets.
  constexpr int KT = NS < 8 ? NS : 8;
  constexpr int VT = NDB < 4 ? NDB : 4;
  int k_off[KT];
#pragma unroll
  for (int i = 0; i < KT; ++i) k_off[i] = r32 * RB + 16 * ((2 * i + h) ^ swz_k<D>(r32));
  const int g16 = lane >> 4, l16 = lane & 15;
  const int v_key = 4 * (g16 >> 1) + (l16 >> 2);
  int v_off[VT];
#pragma unroll
  for (int d = 0; d < VT; ++d) {
    const int byte = 32 * (g16 & 1) + 8 * (l16 & 3) + 64 * d;
    v_off[d] = REG + v_key * RB + 16 * ((byte >> 4) ^ swz_v<D>(v_key)) + (byte & 15);
  }
  auto k_at = [&](int i) { return k_off[i % KT] + 256 * (i / KT); };
  auto v_at = [&](int d) { return v_off[d % VT] + 256 * (d / VT); };
  // bf16 loader: this wave's DMA instructions and its lanes' fixed source
  // offsets inside the page block
  const int my_blk = wave & 1;
  const int my_region = wave >> 1;
  uint32_t dma_off[NIW];
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int krow = RPI * j + lane / CPR;  // key within the 16-key block
    const int c_lds = lane % CPR;
    const int c_g = c_lds ^ (my_region ? swz_v<D>(krow) : swz_k<D>(krow));
    dma_off[j] = (uint32_t)(krow * key_stride) + (uint32_t)(my_region * 2 * D) + 16u * c_g;
  }

  // queues: start with this XCD's, then steal from the others in turn
  const int home = xcc_id() % kQueues;
  int qsel = 0;  // used by thread 0 only
  auto next_item = [&]() { return take_item(p, home, qsel); };

  int parity = 0;
  for (;;) {
    if (tid == 0) sh_item[parity] = next_item();
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(sh_item[parity]);  // same on every lane
    parity ^= 1;
    if (item < 0) break;

    // the item's record, which carries
    // its unit's record and its sequence's metadata
    const Item it = load_item(p, item);
    Unit u;
    u.seq = it.seq;
    u.kv_head = it.kv_head;
    u.row0 = it.row0;
    u.nrows = it.nrows;
    u.kv_lo = it.kv_lo;
    u.kv_hi = it.kv_hi;
    u.nch = it.nch;
    u.item0 = it.item0;
    const int s = u.seq;
    const int kvh = u.kv_head;
    const int q0 = it.q0, ql = it.ql, kvl = it.kvl;
    const int c_lo = u.kv_lo + it.chunk * chunk;
    const int c_hi = min(u.kv_hi, c_lo + chunk);
    const int n_sub = c_hi > c_lo ? (c_hi - c_lo + 31) / 32 : 0;  // 32-key score blocks
    const int n_steps = (n_sub + NB - 1) / NB;                     // load steps
    const uint8_t* kv_h = p.kv + (int64_t)2 * kvh * D * EB;
    const int32_t* ptab = p.page_indices + (int64_t)s * p.pps;
    // Block table: physical key index (page * page_size + slot) of 16-key
    // block b of load step m at entry NB16 m + b, for the steps the loader
    // issues ([0, n_steps + NST - 1)). Blocks past the chunk repeat its last
    // block: they are loaded but never computed on.
    const int n_ent = n_steps > 0 ? (n_steps + NST - 1) * NB16 : 0;
    const int last_blk = c_lo + 16 * ((c_hi - c_lo - 1) >> 4);
    for (int i = tid; i < n_ent; i += NT) {
      const int key = min(c_lo + 16 * i, last_blk);
      const int lp = key / p.page;
      const int ph = min(max(ptab[min(lp, p.pps - 1)], 0), p.P - 1);
      sh_blk[i] = (uint32_t)ph * (uint32_t)p.page + (uint32_t)(key - lp * p.page);
    }
    __syncthreads();

    // this lane's query rows, one per half
    const int vis_hi = min(kvl, c_hi);
    int row[NH], tok[NH], qh[NH], vis_end[NH], win_lo[NH];
    bool rvalid[NH];
    bf16x8 qb[NH][NS];
    bf16x8 qlo[Q32 ? NH : 1][Q32 ? NS : 1];  // f32 q: the lo part of the Q operand (split_q8)
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      row[hf] = WR * wave + 32 * hf + r32;
      rvalid[hf] = row[hf] < u.nrows;
      const int prow = u.row0 + row[hf];
      const int t = prow / p.G;
      qh[hf] = kvh * p.G + (prow - t * p.G);
      tok[hf] = q0 + t;
      const int pos = kvl - ql + t;
      // key visibility (`flashAttention` masks, kv length, chunk end)
      win_lo[hf] = p.window > 0 ? pos - p.window : INT_MIN;  // keys <= win_lo are hidden
      vis_end[hf] = p.is_causal ? min(vis_hi, pos + 1) : vis_hi;
      if (rvalid[hf]) {
        const int64_t e = ((int64_t)tok[hf] * p.Hq + qh[hf]) * D;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          if constexpr (Q32) {
            const float* qp = reinterpret_cast<const float*>(p.q) + e + 16 * i + 8 * h;
            f32x4 a = *reinterpret_cast<const f32x4*>(qp), b = *reinterpret_cast<const f32x4*>(qp + 4);
            if (neg) {
              a = -a;
              b = -b;
            }
            split_q8(a, b, qb[hf][i], qlo[hf][i]);
          } else {
            u32x4 v = *reinterpret_cast<const u32x4*>(p.q + e + 16 * i + 8 * h);
            if (neg) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
            qb[hf][i] = __builtin_bit_cast(bf16x8, v);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          qb[hf][i] = bf16x8{};
          if constexpr (Q32) qlo[hf][i] = bf16x8{};
        }
      }
    }
    auto visible = [&](int hf, int key) { return rvalid[hf] && key < vis_end[hf] && key > win_lo[hf]; };
    // the wave's row span, for the masked-block test
    const int wr_last = min(WR * wave + WR - 1, u.nrows - 1);
    const int pos_lo = kvl - ql + (u.row0 + WR * wave) / p.G;
    const int pos_hi = kvl - ql + (u.row0 + max(wr_last, WR * wave)) / p.G;

    float m_ref[NH], lsum[NH];  // reference max (base-2 units) and running sum of this lane's rows
    f32x16 o[NH][NDB];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      m_ref[hf] = -INFINITY;
      lsum[hf] = 0.f;
#pragma unroll
      for (int d = 0; d < NDB; ++d) o[hf][d] = f32x16{};
    }

    // ---- loader ----
    // Ring slots are LDS byte offsets; every item starts its ring at slot 0
    // (the previous item waited for all of its loads). The key block a wave
    // loads comes from the item's block table (sh_blk), so the step loop does
    // no page arithmetic.
    auto adv = [](int off) { return off + BUF < NST * BUF ? off + BUF : 0; };
    auto blk_base = [&](uint32_t ent) { return kv_h + (uint64_t)ent * (uint64_t)key_stride; };

    // bf16: the step's rows straight into the LDS ring, NIW DMA instructions
    // per wave in one M0 window
    constexpr int DSTR = 1024;  // LDS bytes between a wave's DMA instructions
    const int dma_lds = my_region * REG + 16 * my_blk * RB;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr_of(lds));
    auto issue_dma = [&](uint32_t ent, int slot_off) {
      const uint8_t* base = uniform_ptr(blk_base(ent));
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + slot_off + dma_lds);
      static_assert(NIW == 2 || NIW == 4 || NIW == 8, "DMA instructions per wave per step");
      if constexpr (NIW == 2) {
        dma16_rows2<DSTR>(base, dma_off, dst);
      } else if constexpr (NIW == 4) {
        dma16_rows4<DSTR>(base, dma_off, dst);
      } else {
        dma16_rows8<DSTR>(base, dma_off, dst);
      }
    };
    // fp8: registers one step ahead, widened to bf16 on the way into LDS
    u32x4 stage[CPT];
    auto load_regs = [&](int m) {
      const int k0 = c_lo + m * KS;
      const uint8_t* bb[NB16];
#pragma unroll
      for (int b = 0; b < NB16; ++b) bb[b] = blk_base(__builtin_amdgcn_readfirstlane(sh_blk[m * NB16 + b]));
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int idx = tid + NT * c;
        const int key = idx / GCH;
        if (idx < KS * GCH && k0 + 16 * (key >> 4) < c_hi) {
          const int off = (key & 15) * (int)key_stride + 16 * (idx % GCH);
          stage[c] = *reinterpret_cast<const u32x4*>(bb[key >> 4] + off);
        } else {
          stage[c] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto store_regs = [&](int k0, char* dst) {
      if constexpr (FP8) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const int idx = tid + NT * c;
          if (idx >= KS * GCH) continue;
          const int key = idx / GCH;
          const int gc = idx % GCH;              // 16 codes: K chunks first, then V
          const int region = gc / (GCH / 2);
          const int c0 = 2 * (gc % (GCH / 2));   // first of the two bf16 chunks they become
          const int sw = region ? swz_v<D>(key) : swz_k<D>(key);
          char* row_p = dst + region * REG + key * RB;
          u32x2 lo2 = {stage[c][0], stage[c][1]}, hi2 = {stage[c][2], stage[c][3]};
          bf16x8 a = fp8x8_to_16<KVT, F16>(lo2), b = fp8x8_to_16<KVT, F16>(hi2);
          if (k0 + key >= kvl) {  // V past kv_len reads as zero (0 * NaN = NaN); K there is masked
            a = bf16x8{};
            b = bf16x8{};
          }
          *reinterpret_cast<bf16x8*>(row_p + 16 * (c0 ^ sw)) = a;
          *reinterpret_cast<bf16x8*>(row_p + 16 * ((c0 + 1) ^ sw)) = b;
        }
      }
    };

    static_assert(NB == 1, "the pipelined block loop takes 32-key steps");
    static_assert(FP8 || NST >= 3, "bf16 ring: a slot in use, a slot landing, a slot in flight");
    int fill_off = 0;  // bf16: slot that the next DMA step fills
    int ent_v = 0;     // bf16: table entry of that step's block, read one step early
    int issued = 0;    // fp8: load steps staged so far
    // Makes load step n's K/V rows (in slot `cur`) visible to every wave and
    // keeps the ring full. Called one block ahead of the compute (before the
    // QK product of block n), so a slot is refilled only when every wave is
    // past the barrier here, i.e. done with the PV product of the step that
    // used it (bf16: step n - 2; fp8, whose rows go through registers: step
    // n - 3).
    auto sync_step = [&](int n, char* cur) {
      const int k0 = c_lo + n * KS;
      if constexpr (FP8) {
        store_regs(k0, cur);
        __syncthreads();
        if (issued < n_steps) {
          load_regs(issued);
          ++issued;
        }
      } else {
        // every step issues one DMA group (past the chunk: a re-read of its
        // last block, never computed on), so the same count always means
        // "step n has landed, steps n+1 .. n+NST-3 may still be in flight"
        wait_vmcnt<(NST - 3) * NIW>();
        __syncthreads();
        if (k0 + KS > kvl || k0 + KS > c_hi) {
          // zero V of rows past kv_len or in blocks past the chunk
          for (int i = tid; i < KS * CPR; i += NT) {
            const int key = i / CPR;
            if (k0 + key >= kvl || k0 + 16 * (key >> 4) >= c_hi)
              *reinterpret_cast<u32x4*>(cur + REG + key * RB + 16 * (i % CPR)) = u32x4{0u, 0u, 0u, 0u};
          }
          __syncthreads();
        }
        issue_dma(__builtin_amdgcn_readfirstlane(ent_v), fill_off);
        fill_off = adv(fill_off);
        ent_v = sh_blk[(n + NST - 1) * NB16 + my_blk];
      }
    };
    // prologue: the first load steps in flight
    if (n_steps > 0) {
      if constexpr (FP8) {
        load_regs(0);
        issued = 1;
      } else {
#pragma unroll
        for (int k = 0; k < NST - 2; ++k) {
          issue_dma(__builtin_amdgcn_readfirstlane(sh_blk[k * NB16 + my_blk]), fill_off);
          fill_off = adv(fill_off);
        }
        ent_v = sh_blk[(NST - 2) * NB16 + my_blk];
      }
    }

    // S^T [32 keys x 32 rows] = K Q^T of the block in `slot`, for each of
    // the wave's 32-row halves
    auto qk = [&](const char* slot, float (&sv)[NH][16]) {
      bf16x8 ka[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) ka[i] = *reinterpret_cast<const bf16x8*>(slot + k_at(i));
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        f32x16 sc = f32x16{};
#pragma unroll
        for (int i = 0; i < NS; ++i) sc = mfma32x32x16<F16>(ka[i], qb[hf][i], sc);
        if constexpr (Q32) {
#pragma unroll
          for (int i = 0; i < NS; ++i) sc = mfma32x32x16<F16>(ka[i], qlo[hf][i], sc);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) sv[hf][j] = sc[j];
      }
    };
    // Scores of a block to base-2 units (soft-capped first when the cap is
    // on); returns the row maximum. (Written as a product rather than a copy,
    // so that the scores leave the MFMA accumulator registers once.)
    auto to_base2 = [&](float x) {
      if constexpr (CAP) {
        return cap_b2(x);
      } else if constexpr (kLate) {
        return x;
      } else {
        return x * cmul;
      }
    };
    // row maximum (base-2 units) from this lane's maximum of stored scores
    auto row_max = [&](float mx) {
      mx = max_xor32(mx);
      return kLate ? mx * cmul : mx;
    };
    auto finish_scores = [&](float (&sv)[16]) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        sv[j] = to_base2(sv[j]);
        mx = fmaxf(mx, sv[j]);
      }
      return row_max(mx);
    };
    // Hidden keys of the block at kb to -inf (masks of `flashAttention`, kv
    // length, chunk end; by selection, so NaN in unread slots cannot leak);
    // returns the new row maximum in base-2 units.
    auto mask_scores = [&](int hf, float (&sv)[16], int kb) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float x = visible(hf, kb + 8 * (j >> 2) + 4 * h + (j & 3)) ? sv[j] : -INFINITY;
        sv[j] = x;
        mx = fmaxf(mx, x);
      }
      return row_max(mx);
    };
    // Lazily moved reference maximum: the accumulator is rescaled only when a
    // row's maximum outgrows the reference by more than kRescaleSlack. The
    // rescale runs outside the block loop (below), so inside it the
    // accumulator is only ever an MFMA operand and stays in its registers.
    auto needs_rescale = [&](const float (&mb)[NH]) {
      bool any = false;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) any = any || mb[hf] > m_ref[hf] + SLACK;
      return __any(any);
    };
    auto rescale = [&](const float (&mb)[NH]) {
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        const float m_new = fmaxf(m_ref[hf], mb[hf]);
        const float alpha = m_ref[hf] == -INFINITY ? 0.f : fast_exp2(m_ref[hf] - m_new);
        m_ref[hf] = m_new;
        lsum[hf] *= alpha;
#pragma unroll
        for (int d = 0; d < NDB; ++d) o[hf][d] *= alpha;
      }
    };
    // Blocks that can hold a key some row of the wave cannot see: those at
    // or past ub_mask_hi (kv length, chunk end, causal diagonal) and those
    // before ub_mask_lo (sliding window).
    int ub_mask_hi = n_sub, ub_mask_lo = 0;
    {
      int lim = vis_hi - 32;  // blocks with kb <= lim hold no key at or past vis_hi
      if (p.is_causal) lim = min(lim, pos_lo - 31);
      ub_mask_hi = lim < c_lo ? 0 : min(n_sub, (lim - c_lo) / 32 + 1);
      if (p.window > 0) {
        const int w = pos_hi - p.window;  // blocks with kb <= w hold a hidden key
        ub_mask_lo = w < c_lo ? 0 : min(n_sub, (w - c_lo) / 32 + 1);
      }
    }
    auto need_mask = [&](int b) { return b >= ub_mask_hi || b < ub_mask_lo; };

    // Software-pipelined block loop. Entering iteration ub, block ub's scores
    // are final (capped, masked) and the reference maximum covers them. The
    // iteration runs the next block's QK MFMAs beside this block's softmax
    // VALU work, then this block's PV MFMAs beside the next block's score
    // epilogue, so the matrix and vector units work at the same time. With
    // two 32-row halves per wave every K and V^T operand read serves two
    // MFMAs.
    float sc_cur[NH][16];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int j = 0; j < 16; ++j) sc_cur[hf][j] = 0.f;
    float mb_pending[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) mb_pending[hf] = -INFINITY;
    bool pending = false;
    if (n_sub > 0) {
      sync_step(0, lds);
      qk(lds, sc_cur);
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        mb_pending[hf] = finish_scores(sc_cur[hf]);
        if (need_mask(0)) mb_pending[hf] = mask_scores(hf, sc_cur[hf], c_lo);
      }
      pending = needs_rescale(mb_pending);
    }
    int ub = 0;
    int cs = 0;  // ring slot of block ub
    for (;;) {
      if (pending) rescale(mb_pending);
      pending = false;
      for (; ub < n_sub; ++ub) {
        const int ns = adv(cs);
        const bool has_next = ub + 1 < n_sub;
        if (has_next) sync_step(ub + 1, lds + ns);
        // (the last block computes a throw-away QK on its own slot, so that
        // the two units' work stays in one straight-line block)
        const char* nslot = lds + (has_next ? ns : cs);
        const char* cslot = lds + cs;
        float mb_next[NH];
        {
          // The iteration in an explicit order (sched_barrier fences keep the
          // compiler's scheduler from regrouping it): the next block's first K
          // reads; the first P pairs of this block while they land; each QK
          // k-step (NH MFMAs) followed by a K read KA k-steps ahead and a
          // share of the remaining pairs, the last ones by the first V^T
          // reads; each PV step (NH MFMAs) followed by a share of the next
          // block's score epilogue, with V^T reads VA steps ahead.
          constexpr int KA = NS / 2;  // K reads ahead of their MFMA
          bf16x8 ka[NS];
#pragma unroll
          for (int i = 0; i < KA; ++i) ka[i] = *reinterpret_cast<const bf16x8*>(nslot + k_at(i));
          __builtin_amdgcn_sched_barrier(0);
          float negm[NH];
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) negm[hf] = m_ref[hf] == -INFINITY ? 0.f : -m_ref[hf];
          bf16x8 pb[NH][2];
          // P = 2^(score - reference) for scores 2jp, 2jp+1 of half hf
          // (pair index q = 8 hf + jp), packed to bf16; the row sum is taken in
          // f32 over the unrounded values (the LSE needs them: one dominant key
          // rounded to bf16 moves it by up to 2^-8)
          auto p_pair = [&](int q) {
            const int hf = q >> 3, jp = q & 7;
            const float s0 = sc_cur[hf][2 * jp], s1 = sc_cur[hf][2 * jp + 1];
            const float p0 = fast_exp2(kLate ? __builtin_fmaf(s0, cmul, negm[hf]) : s0 + negm[hf]);
            const float p1 = fast_exp2(kLate ? __builtin_fmaf(s1, cmul, negm[hf]) : s1 + negm[hf]);
            lsum[hf] += p0 + p1;
            const bf16x2 pair = __builtin_bit_cast(bf16x2, pack2<F16>(p0, p1));
            pb[hf][jp >> 2][2 * (jp & 3)] = pair[0];
            pb[hf][jp >> 2][2 * (jp & 3) + 1] = pair[1];
          };
          constexpr int NPP = 8 * NH;  // P pairs of the block
          constexpr int PRE = 2;       // pairs before the first QK MFMA
#pragma unroll
          for (int q = 0; q < PRE; ++q) p_pair(q);
          __builtin_amdgcn_sched_barrier(0);
          // O^T += V^T P^T: step m = ks * NDB + d takes key half ks, 32 rows of d
          constexpr int NM = 2 * NDB;
          constexpr int VA = 3;  // V^T reads ahead of their MFMA
          static_assert(NS >= VA && NM > VA, "read-ahead depth");
          bf16x8 va[NM];
          auto read_va = [&](int m) {
            const int ks = m / NDB, d = m % NDB;
            const bf16x4 lo = lds_read_tr16(reinterpret_cast<const __bf16*>(cslot + (16 * ks) * RB + v_at(d)));
            const bf16x4 hi = lds_read_tr16(reinterpret_cast<const __bf16*>(cslot + (16 * ks + 8) * RB + v_at(d)));
            va[m] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          };
          f32x16 sc_next[NH];
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) sc_next[hf] = f32x16{};
#pragma unroll
          for (int i = 0; i < NS; ++i) {
#pragma unroll
            for (int hf = 0; hf < NH; ++hf) {
              sc_next[hf] = mfma32x32x16<F16>(ka[i], qb[hf][i], sc_next[hf]);
              if constexpr (Q32) sc_next[hf] = mfma32x32x16<F16>(ka[i], qlo[hf][i], sc_next[hf]);
            }
            if (i + KA < NS) ka[i + KA] = *reinterpret_cast<const bf16x8*>(nslot + k_at(i + KA));
#pragma unroll
            for (int q = PRE + ((NPP - PRE) * i) / NS; q < PRE + ((NPP - PRE) * (i + 1)) / NS; ++q) p_pair(q);
            if (i >= NS - VA) read_va(i - (NS - VA));
            __builtin_amdgcn_sched_barrier(0);
          }
          float mx[NH];
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) mx[hf] = -INFINITY;
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            if (m + VA < NM) read_va(m + VA);
#pragma unroll
            for (int hf = 0; hf < NH; ++hf)
              o[hf][m % NDB] = mfma32x32x16<F16>(va[m], pb[hf][m / NDB], o[hf][m % NDB]);
#pragma unroll
            for (int e = (16 * NH * m) / NM; e < (16 * NH * (m + 1)) / NM; ++e) {
              const int hf = e >> 4, j = e & 15;
              sc_cur[hf][j] = to_base2(sc_next[hf][j]);
              mx[hf] = fmaxf(mx[hf], sc_cur[hf][j]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) mb_next[hf] = row_max(mx[hf]);
        }
        cs = ns;
        if (has_next) {
          if (need_mask(ub + 1)) {
#pragma unroll
            for (int hf = 0; hf < NH; ++hf) mb_next[hf] = mask_scores(hf, sc_cur[hf], c_lo + 32 * (ub + 1));
          }
          if (needs_rescale(mb_next)) {
            // leave the loop to rescale, then resume at the next block
#pragma unroll
            for (int hf = 0; hf < NH; ++hf) mb_pending[hf] = mb_next[hf];
            pending = true;
            ++ub;
            break;
          }
        }
      }
      if (!pending) break;
    }
    // the re-reads past the chunk have landed: the ring is idle
    if constexpr (!FP8) wait_vmcnt<0>();

    // lane (row, h) holds O^T[32*d + 8*(j/4) + 4*h + (j%4)][row]
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      const float l_row = sum_xor32(lsum[hf]);
      float inv, lse_v;
      // a whole row takes its sink (if any) here; a chunk's partial leaves it
      // to the merge
      row_final(m_ref[hf], l_row, p.v_scale, (u.nch == 1 && p.sinks) ? p.sinks + qh[hf] : nullptr, inv, lse_v);
      if (!rvalid[hf]) continue;
      if (u.nch == 1) {
        const int64_t e = ((int64_t)tok[hf] * p.Hq + qh[hf]) * D + 4 * h;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            store_out4<F16, Q32>(p.out, e + 32 * d + 8 * q4, o[hf][d][4 * q4] * inv, o[hf][d][4 * q4 + 1] * inv,
                                 o[hf][d][4 * q4 + 2] * inv, o[hf][d][4 * q4 + 3] * inv);
        if (h == 0 && p.lse) p.lse[(int64_t)tok[hf] * p.Hq + qh[hf]] = lse_v;
      } else {
        float* pp = p.pf_part + ((int64_t)item * p.pf_rows + row[hf]) * D + 4 * h;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 w = {o[hf][d][4 * q4] * inv, o[hf][d][4 * q4 + 1] * inv, o[hf][d][4 * q4 + 2] * inv,
                       o[hf][d][4 * q4 + 3] * inv};
            store_coherent4(pp + 32 * d + 8 * q4, w);
          }
        if (h == 0) store_coherent(p.pf_plse + (int64_t)item * p.pf_rows + row[hf], lse_v);
      }
    }
    if (u.nch > 1) {
      // publish the partial, count the chunk; the last one merges the unit
      wait_stores();
      __syncthreads();
      if (tid == 0) sh_last = atomicAdd(&p.unit_done[it.unit], 1) == u.nch - 1;
      __syncthreads();
      if (sh_last) {
        // the LDS ring is idle here (every wave is past its last step); it
        // holds the per-row stats of the merge
        auto wg_sync = [] { __syncthreads(); };
        merge_unit<D, F16, Q32, false>(p, u, p.pf_part, p.pf_plse, p.pf_rows, [&](int c) { return u.item0 + c; }, tid, NT,
                                reinterpret_cast<float*>(lds), wg_sync);
      }
    }
    // every wave must be done with the ring before the next item refills it
    __syncthreads();
  }
}

}  // namespace rpa
