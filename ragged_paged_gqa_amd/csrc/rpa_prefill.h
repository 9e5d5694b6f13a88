// Prefill/mixed-class attention kernel: units of up to kPfRows packed query
// rows (row = token * G + g) of one sequence and one kv head — the kernel
// page's q block of `num_queries_per_block` tokens times the G q heads of one
// kv head, stacked into one MFMA dimension (`run`, per-kv-head step).
//
// A workgroup of NW waves owns one item (a key chunk of a unit) at a time,
// pulled from a device-wide queue; wave w owns rows [32w, 32w + 32). Split
// units leave partials; the workgroup finishing a unit's last chunk merges
// them (rpa_merge.h).
// Per load step (64 keys for bf16 with head_dim <= 128, else 32):
//   * loader: the step's K and V rows of kv head h (combined heads 2h and
//     2h+1, adjacent in memory — `stridedLoadKv`) are gathered through the
//     page table into a ring of LDS tiles whose rows are padded so that the
//     MFMA operand reads below are bank-conflict free. bf16 rows go straight
//     from HBM to LDS (global_load_lds_dwordx4, one padded row per
//     instruction) kStagesBf16 - 1 steps ahead of the compute; fp8 rows are
//     staged through registers one step ahead and widened to bf16 on the way.
//     Page position is tracked incrementally (no integer division in the
//     loop). One barrier per step publishes the tile.
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
#pragma once

#include <climits>
#include <type_traits>

#include "rpa_common.h"
#include "rpa_merge.h"

namespace rpa {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// The reference maximum of a row moves only when the row's maximum outgrows
// it by more than this (base-2 units): exponentiated scores stay <= 2^16,
// far inside f32 and bf16 range, and the accumulator rescale (which leaves
// the step loop, see below) is rare.
constexpr float kRescaleSlack = 16.0f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Keys per load step (one LDS ring slot, one barrier). Scores are computed
// 32 keys at a time.
constexpr int pf_step_keys(int D, bool fp8) { return (D > 0 && !fp8) ? 32 : 32; }

#ifndef RPA_PF_STAGES
#define RPA_PF_STAGES 4
#endif
constexpr int kStagesBf16 = RPA_PF_STAGES;
// Cached page-table entries per item: the largest chunk over the smallest page
// (16 keys), plus the partial pages at both ends.
constexpr int kPfPageCache = kPfMaxChunk / 16 + 4;

// Two LDS layouts of a ring slot, both bank-conflict free for the MFMA
// operand reads below:
//   * swizzled (a key's K and V rows together are under 1 KB): the step's K
//     rows (region 0) and V rows (region 1), each kStepKeys unpadded rows of
//     2D bytes whose 16-byte chunks are XOR-swizzled by the key (swz_k /
//     swz_v), so that one DMA instruction writes 1 KB of whole rows;
//   * padded (head_dim 256: K row then V row of a key is exactly 1 KB, one
//     DMA instruction): rows of K|V padded to 16 * (16n + 3) bytes, so 16
//     consecutive keys start in distinct 16-byte bank groups.
template <int D, bool FP8>
struct PrefillLds {
  static constexpr bool kSwizzled = 4 * D < 1024;
  static constexpr int kRowBytes = kSwizzled ? 2 * D : 4 * D + 48;  // row stride
  static constexpr int kChunks = 2 * D / 16;   // 16-byte chunks per K or V row
  static constexpr int kStepKeys = pf_step_keys(D, FP8);
  static constexpr int kRegionBytes = kSwizzled ? kStepKeys * kRowBytes : 2 * D;  // V offset
  static constexpr int kBufBytes = kSwizzled ? 2 * kStepKeys * kRowBytes : kStepKeys * kRowBytes;
  static constexpr int kStages = FP8 ? 2 : kStagesBf16;
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

// Value of lane l ^ 32 (v_permlane32_swap; no LDS round trip).
__device__ __forceinline__ float other_half(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __builtin_bit_cast(float, (uint32_t)(lane_id() < 32 ? r[1] : r[0]));
}

// Scheduling hints: the next `n` LDS reads, then the next `n` MFMAs.
#define RPA_SCHED_DS_READS(n) __builtin_amdgcn_sched_group_barrier(0x100, n, 0)
#define RPA_SCHED_MFMAS(n) __builtin_amdgcn_sched_group_barrier(0x008, n, 0)

template <int D, bool FP8>
__global__ __launch_bounds__(kPfWaves * 64, pf_wgs_per_cu(D)) void prefill_kernel(Params p) {
  constexpr int NW = kPfWaves;
  constexpr int NH = pf_halves_for(D);        // 32-row halves per wave
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
  constexpr bool SWZ = PrefillLds<D, FP8>::kSwizzled;
  constexpr int BUF = PrefillLds<D, FP8>::kBufBytes;
  constexpr int NST = PrefillLds<D, FP8>::kStages;
  constexpr int GCH = 2 * D * EB / 16;        // 16-byte global chunks per key (K and V)
  constexpr int CPT = (KS * GCH + NT - 1) / NT;  // fp8 path: chunks per thread per step
  // bf16 path: full-width DMA instructions of 1 KB. Swizzled: RPI rows of one
  // region each, wave w moving region w / 2, keys [16 (w % 2), + 16).
  // Padded: one key's K|V row each, wave w moving keys [8 w, 8 w + 8). Either
  // way a wave's keys lie in one 16-key page block.
  constexpr int RPI = SWZ ? 1024 / RB : 1;    // rows per DMA instruction
  constexpr int NIW = SWZ ? (2 * KS / RPI) / NW : KS / NW;  // DMA instructions per wave per step
  static_assert(NDB >= 2, "head_dim >= 64");
  static_assert(SWZ ? RPI * CPR == 64 : 2 * CPR == 64, "whole rows per full-width DMA instruction");
  static_assert(KS % NW == 0 && (NB == 1 || NB == 2), "step shape");
  static_assert(!FP8 || NST == 2, "fp8 path stages through registers one step ahead");
  static_assert(FP8 || (KS == 32 && NW == 4 && NIW * RPI == (SWZ ? 16 : 8)), "a wave's rows stay in one 16-key block");

  __shared__ __attribute__((aligned(16))) char lds[PrefillLds<D, FP8>::kBytes];
  __shared__ int sh_pages[kPfPageCache];  // physical pages of the current item
  __shared__ int sh_item[2];
  __shared__ int sh_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r32 = lane & 31;  // S^T column = row within a 32-row half
  const int h = lane >> 5;    // which half of the row's keys this lane holds

  if (p.hdr->n_pf_items == 0) return;  // nothing of this class in the batch
  const int chunk = p.hdr->pf_chunk;
  const int64_t key_stride = (int64_t)2 * p.Hkv * D * EB;
  const bool capped = p.soft_cap > 0.f;
  const float cap_k = capped ? 2.0f * kLog2e / p.soft_cap : 0.f;
  // scores in base-2 units are st * cmul (capped: the cap is applied to st
  // first and cmul = 1); negative scales flip Q's sign instead
  const bool neg = p.sm_scale < 0.f;
  const float sm = neg ? -p.sm_scale : p.sm_scale;
  const float cmul = capped ? 1.0f : sm * kLog2e;

  // LDS read offsets inside a slot (loop-invariant per lane):
  //   K operand of k-step i: key r32, chunk 2i + h
  //   V^T operand of d-block d: key 4 (g16 / 2) + l16 / 4 (+ 8, + 16 ks),
  //   bytes 32 (g16 % 2) + 8 (l16 % 4) + 64 d of the row
  // (swizzled: per-lane tables; padded: one base plus immediate offsets)
  int k_off[SWZ ? NS : 1];
#pragma unroll
  for (int i = 0; i < (SWZ ? NS : 1); ++i) k_off[i] = r32 * RB + 16 * (SWZ ? ((2 * i + h) ^ swz_k<D>(r32)) : h);
  const int g16 = lane >> 4, l16 = lane & 15;
  const int v_key = 4 * (g16 >> 1) + (l16 >> 2);
  int v_off[SWZ ? NDB : 1];
#pragma unroll
  for (int d = 0; d < (SWZ ? NDB : 1); ++d) {
    const int byte = 32 * (g16 & 1) + 8 * (l16 & 3) + 64 * d;
    v_off[d] = REG + v_key * RB + (SWZ ? 16 * ((byte >> 4) ^ swz_v<D>(v_key)) + (byte & 15) : byte);
  }
  auto k_at = [&](int i) { return SWZ ? k_off[SWZ ? i : 0] : k_off[0] + 32 * i; };
  auto v_at = [&](int d) { return SWZ ? v_off[SWZ ? d : 0] : v_off[0] + 64 * d; };
  // bf16 loader: this wave's DMA instructions and its lanes' fixed source
  // offsets inside the page block
  const int my_blk = SWZ ? (wave & 1) : (wave >> 1);
  const int my_region = SWZ ? (wave >> 1) : 0;
  uint32_t dma_off[NIW];
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    if constexpr (SWZ) {
      const int krow = RPI * j + lane / CPR;  // key within the 16-key block
      const int c_lds = lane % CPR;
      const int c_g = c_lds ^ (my_region ? swz_v<D>(krow) : swz_k<D>(krow));
      dma_off[j] = (uint32_t)(krow * key_stride) + (uint32_t)(my_region * 2 * D) + 16u * c_g;
    } else {
      dma_off[j] = (uint32_t)(((wave * NIW + j) & 15) * key_stride) + 16u * lane;
    }
  }

  // queues: start with this XCD's, then steal from the others in turn
  const int home = xcc_id() % kQueues;
  int qsel = 0;  // used by thread 0 only
  auto next_item = [&]() -> int {
    while (qsel < kQueues) {
      const int x = (home + qsel) % kQueues;
      const int k = atomicAdd(&p.hdr->pf_q_next[x], 1);
      if (k < p.hdr->pf_q_count[x]) return p.pf_qlist[p.hdr->pf_q_base[x] + k];
      ++qsel;
    }
    return -1;
  };

  int parity = 0;
  int ring = 0;  // LDS ring slot of the next step to compute
  for (;;) {
    if (tid == 0) sh_item[parity] = next_item();
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(sh_item[parity]);  // same on every lane
    parity ^= 1;
    if (item < 0) break;

    const Item it = p.pf_items[item];
    const Unit u = p.pf_units[it.unit];
    const int s = u.seq;
    const int kvh = u.kv_head;
    int q0, ql;
    seq_tokens(p, s, q0, ql);
    int kvl = p.kv_lens[s];
    kvl = max(0, min(kvl, p.pps * p.page));
    const int c_lo = u.kv_lo + it.chunk * chunk;
    const int c_hi = min(u.kv_hi, c_lo + chunk);
    const int n_sub = c_hi > c_lo ? (c_hi - c_lo + 31) / 32 : 0;  // 32-key score blocks
    const int n_steps = (n_sub + NB - 1) / NB;                     // load steps
    const uint8_t* kv_h = p.kv + (int64_t)2 * kvh * D * EB;
    const int32_t* ptab = p.page_indices + (int64_t)s * p.pps;
    // physical pages of the item's key range, clamped, cached in LDS
    const int lp0 = c_lo / p.page;
    const int n_pg = min(n_steps > 0 ? (c_lo + n_steps * KS - 1) / p.page - lp0 + 1 : 0, kPfPageCache);
    for (int i = tid; i < n_pg; i += NT) sh_pages[i] = min(max(ptab[min(lp0 + i, p.pps - 1)], 0), p.P - 1);
    __syncthreads();

    // this lane's query rows, one per half
    const int vis_hi = min(kvl, c_hi);
    int row[NH], tok[NH], qh[NH], vis_end[NH], win_lo[NH];
    bool rvalid[NH];
    bf16x8 qb[NH][NS];
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
        const uint16_t* qp = p.q + ((int64_t)tok[hf] * p.Hq + qh[hf]) * D;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          u32x4 v = *reinterpret_cast<const u32x4*>(qp + 16 * i + 8 * h);
          if (neg) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
          qb[hf][i] = __builtin_bit_cast(bf16x8, v);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NS; ++i) qb[hf][i] = bf16x8{};
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

    // page position of the next step to load, advanced without division
    int lp = c_lo / p.page;
    int sl = c_lo - lp * p.page;
    auto advance = [&]() {
#pragma unroll
      for (int b = 0; b < NB16; ++b) {
        sl += 16;
        if (sl >= p.page) {
          sl -= p.page;
          ++lp;
        }
      }
    };

    // ---- loader, bf16: rows straight into the LDS ring ----
    auto issue_dma = [&](int k0, char* dst) {
      // page block my_blk of the step at (lp, sl), or block 0 past the chunk
      // (a harmless re-read: its keys are masked and their V rows zeroed)
      int lpb = lp, slb = sl;
      if (k0 + 16 * my_blk < c_hi) {
        for (int b = 0; b < my_blk; ++b) {
          slb += 16;
          if (slb >= p.page) {
            slb = 0;
            ++lpb;
          }
        }
      }
      const int ph = __builtin_amdgcn_readfirstlane(sh_pages[min(lpb - lp0, kPfPageCache - 1)]);
      const uint8_t* base = uniform_ptr(kv_h + ((int64_t)ph * p.page + slb) * key_stride);
      const uint32_t dst0 = __builtin_amdgcn_readfirstlane(
          lds_addr_of(dst + (SWZ ? my_region * REG + 16 * my_blk * RB : wave * NIW * RB)));
#pragma unroll
      for (int j = 0; j < NIW; ++j) dma16_sbase(base, dma_off[j], dst0 + (SWZ ? 1024 : RB) * j);
    };
    // ---- loader, fp8: registers one step ahead, widened to bf16 ----
    // base addresses of the 16-key blocks of the step at (lp, sl)
    auto block_bases = [&](int k0, const uint8_t* (&bb)[NB16]) {
      int lpb = lp, slb = sl;
#pragma unroll
      for (int b = 0; b < NB16; ++b) {
        const int ph = sh_pages[min(lpb - lp0, kPfPageCache - 1)];
        const uint8_t* base = kv_h + ((int64_t)ph * p.page + slb) * key_stride;
        bb[b] = (b == 0 || k0 + 16 * b < c_hi) ? base : bb[0];
        slb += 16;
        if (slb >= p.page) {
          slb = 0;
          ++lpb;
        }
      }
    };
    u32x4 stage[CPT];
    auto load_regs = [&](int k0) {
      const uint8_t* bb[NB16];
      block_bases(k0, bb);
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int idx = tid + NT * c;
        const int key = idx / GCH;
        if (idx < KS * GCH && (key < 16 || k0 + 16 * (key >> 4) < c_hi)) {
          const int off = (key & 15) * (int)key_stride + 16 * (idx % GCH);
          stage[c] = *reinterpret_cast<const u32x4*>(bb[key >> 4] + off);
        } else {
          stage[c] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto store_regs = [&](int k0, char* dst) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int idx = tid + NT * c;
        if (idx >= KS * GCH) continue;
        const int key = idx / GCH;
        const int gc = idx % GCH;              // 16 codes: K chunks first, then V
        const int region = gc / (GCH / 2);
        const int c0 = 2 * (gc % (GCH / 2));   // first of the two bf16 chunks they become
        const int sw = !SWZ ? 0 : (region ? swz_v<D>(key) : swz_k<D>(key));
        char* row_p = dst + region * REG + key * RB;
        u32x2 lo2 = {stage[c][0], stage[c][1]}, hi2 = {stage[c][2], stage[c][3]};
        bf16x8 a = fp8x8_to_bf16(lo2), b = fp8x8_to_bf16(hi2);
        if (k0 + key >= kvl) {  // V past kv_len reads as zero (0 * NaN = NaN); K there is masked
          a = bf16x8{};
          b = bf16x8{};
        }
        *reinterpret_cast<bf16x8*>(row_p + 16 * (c0 ^ sw)) = a;
        *reinterpret_cast<bf16x8*>(row_p + 16 * ((c0 + 1) ^ sw)) = b;
      }
    };
    auto slot_ptr = [&](int k) { return lds + ((ring + k) % NST) * BUF; };

    // prologue: NST - 1 steps in flight
    int issued = 0;
    if constexpr (FP8) {
      if (n_steps > 0) {
        load_regs(c_lo);
        advance();
        issued = 1;
      }
    } else {
#pragma unroll
      for (int k = 0; k < NST - 1; ++k) {
        if (k < n_steps) {
          issue_dma(c_lo + k * KS, slot_ptr(k));
          advance();
          issued = k + 1;
        }
      }
    }

    // Score blocks of 32 keys; block ub belongs to load step ub / NB. The
    // accumulators are touched only by MFMAs inside the loop: when a row's
    // maximum outgrows its reference, the loop is left, the accumulators
    // rescaled, and the same block resumed (its scores kept in st).
    f32x16 st[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) st[hf] = f32x16{};
    float m_blk[NH];
    int ub = 0;
    bool resume = false;
    for (;;) {
      bool pending = false;
      for (; ub < n_sub; ++ub) {
        const int n = ub / NB;
        const int b = ub % NB;
        const int k0 = c_lo + n * KS;
        const int kb = k0 + 32 * b;
        char* cur = slot_ptr(0);
        // does this block hold a key that some row of the wave cannot see?
        const bool need_mask = kb + 32 > vis_hi || (p.is_causal && kb + 31 > pos_lo) ||
                               (p.window > 0 && kb <= pos_hi - p.window);
        if (!resume) {
          if (b == 0) {
            if constexpr (FP8) {
              store_regs(k0, cur);
              __syncthreads();
              if (issued < n_steps) {
                load_regs(c_lo + issued * KS);
                advance();
                ++issued;
              }
            } else {
              // wait for this step's rows: later steps may stay in flight
              const int ahead = issued - n - 1;
              if (ahead >= 2) {
                wait_vmcnt<2 * NIW>();
              } else if (ahead == 1) {
                wait_vmcnt<NIW>();
              } else {
                wait_vmcnt<0>();
              }
              __syncthreads();
              if (k0 + KS > kvl || k0 + KS > c_hi) {
                // zero V of rows past kv_len or in blocks past the chunk
                for (int i = tid; i < KS * CPR; i += NT) {
                  const int key = i / CPR;
                  const bool loaded = key < 16 || k0 + 16 * (key >> 4) < c_hi;
                  if (k0 + key >= kvl || !loaded)
                    *reinterpret_cast<u32x4*>(cur + REG + key * RB + 16 * (i % CPR)) = u32x4{0u, 0u, 0u, 0u};
                }
                __syncthreads();
              }
              // refill the slot freed by the previous step (every wave is past it)
              if (issued < n_steps) {
                issue_dma(c_lo + issued * KS, slot_ptr(NST - 1));
                advance();
                ++issued;
              }
            }
          }

          // S^T = K Q^T for keys [kb, kb + 32): one K operand feeds every half
          {
            const char* kr = cur + 32 * b * RB;
            bf16x8 ka[NS];
#pragma unroll
            for (int i = 0; i < NS; ++i) ka[i] = *reinterpret_cast<const bf16x8*>(kr + k_at(i));
#pragma unroll
            for (int hf = 0; hf < NH; ++hf) st[hf] = f32x16{};
#pragma unroll
            for (int i = 0; i < NS; ++i)
#pragma unroll
              for (int hf = 0; hf < NH; ++hf) st[hf] = mfma32x32x16(ka[i], qb[hf][i], st[hf]);
            RPA_SCHED_DS_READS(NS);
            RPA_SCHED_MFMAS(NS * NH);
          }
          // row maxima over the visible keys, in base-2 units
          bool grow = false;
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) {
            if (capped) {
#pragma unroll
              for (int j = 0; j < 16; ++j) st[hf][j] = soft_cap_f(st[hf][j] * sm, p.soft_cap, cap_k) * kLog2e;
            }
            float mx;
            if (need_mask) {
              mx = -INFINITY;
#pragma unroll
              for (int j = 0; j < 16; ++j)
                mx = fmaxf(mx, visible(hf, kb + 8 * (j >> 2) + 4 * h + (j & 3)) ? st[hf][j] : -INFINITY);
            } else {
              mx = st[hf][0];
#pragma unroll
              for (int j = 1; j < 16; ++j) mx = fmaxf(mx, st[hf][j]);
            }
            mx = fmaxf(mx, other_half(mx));
            m_blk[hf] = mx * cmul;  // -inf stays -inf (cmul > 0 unless the scale is 0)
            grow = grow || m_blk[hf] > m_ref[hf] + kRescaleSlack;
          }
          if (__any(grow)) {
            pending = true;
            break;
          }
        }
        resume = false;

        // P = 2^(score - reference), packed to bf16 for the PV product; the
        // row sum is taken in f32 over the unrounded values (the LSE needs
        // them: one dominant key rounded to bf16 moves it by up to 2^-8)
        bf16x8 pb[NH][2];
        auto make_p = [&](auto hfc, auto masked) {
          constexpr int hf = decltype(hfc)::value;
          const float negm = m_ref[hf] == -INFINITY ? 0.f : -m_ref[hf];
#pragma unroll
          for (int jp = 0; jp < 8; ++jp) {
            float p0 = fast_exp2(__builtin_fmaf(st[hf][2 * jp], cmul, negm));
            float p1 = fast_exp2(__builtin_fmaf(st[hf][2 * jp + 1], cmul, negm));
            if constexpr (decltype(masked)::value) {
              const int key0 = kb + 8 * (jp >> 1) + 4 * h + 2 * (jp & 1);
              p0 = visible(hf, key0) ? p0 : 0.f;
              p1 = visible(hf, key0 + 1) ? p1 : 0.f;
            }
            lsum[hf] += p0 + p1;
            const bf16x2 pair = {(__bf16)p0, (__bf16)p1};
            pb[hf][jp >> 2][2 * (jp & 3)] = pair[0];
            pb[hf][jp >> 2][2 * (jp & 3) + 1] = pair[1];
          }
        };
        auto p_of_half = [&](auto hfc) {
          if (need_mask)
            make_p(hfc, std::true_type{});
          else
            make_p(hfc, std::false_type{});
        };

        // O^T += V^T P^T (two 16-key k-steps); one V^T operand feeds every half
        const char* vr = cur + 32 * b * RB;
        auto read_va = [&](int ks, bf16x8 (&va)[NDB]) {
#pragma unroll
          for (int d = 0; d < NDB; ++d) {
            const bf16x4 lo = lds_read_tr16(reinterpret_cast<const __bf16*>(vr + (16 * ks) * RB + v_at(d)));
            const bf16x4 hi = lds_read_tr16(reinterpret_cast<const __bf16*>(vr + (16 * ks + 8) * RB + v_at(d)));
            va[d] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        };
        if constexpr (NH == 1) {
          p_of_half(std::integral_constant<int, 0>{});
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            bf16x8 va1[NDB];
            read_va(ks, va1);
#pragma unroll
            for (int d = 0; d < NDB; ++d) o[0][d] = mfma32x32x16(va1[d], pb[0][ks], o[0][d]);
            RPA_SCHED_DS_READS(2 * NDB);
            RPA_SCHED_MFMAS(NDB);
          }
        } else {
          bf16x8 va[2][NDB];
          read_va(0, va[0]);
          read_va(1, va[1]);
          p_of_half(std::integral_constant<int, 0>{});
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int d = 0; d < NDB; ++d) o[0][d] = mfma32x32x16(va[ks][d], pb[0][ks], o[0][d]);
          // the second half's softmax runs while the first half's PV MFMAs execute
          p_of_half(std::integral_constant<int, NH - 1>{});
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int d = 0; d < NDB; ++d) o[NH - 1][d] = mfma32x32x16(va[ks][d], pb[NH - 1][ks], o[NH - 1][d]);
        }
        if (b == NB - 1 || ub == n_sub - 1) ring = (ring + 1) % NST;
      }
      if (!pending) break;
      // move the reference max (every row of the wave at once; alpha <= 1)
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        const float m_new = fmaxf(m_ref[hf], m_blk[hf]);
        const float alpha = m_ref[hf] == -INFINITY ? 0.f : fast_exp2(m_ref[hf] - m_new);
        m_ref[hf] = m_new;
        lsum[hf] *= alpha;
#pragma unroll
        for (int d = 0; d < NDB; ++d) o[hf][d] *= alpha;
      }
      resume = true;
    }

    // lane (row, h) holds O^T[32*d + 8*(j/4) + 4*h + (j%4)][row]
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      const float l_row = lsum[hf] + other_half(lsum[hf]);
      const float inv = l_row > 0.f ? p.v_scale / l_row : 0.f;
      const float lse_v = l_row > 0.f ? (m_ref[hf] + fast_log2(l_row)) * kLn2 : -INFINITY;
      if (!rvalid[hf]) continue;
      if (u.nch == 1) {
        uint16_t* op = p.out + ((int64_t)tok[hf] * p.Hq + qh[hf]) * D + 4 * h;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            u32x2 w = {bf16x2_bits(o[hf][d][4 * q4] * inv, o[hf][d][4 * q4 + 1] * inv),
                       bf16x2_bits(o[hf][d][4 * q4 + 2] * inv, o[hf][d][4 * q4 + 3] * inv)};
            *reinterpret_cast<u32x2*>(op + 32 * d + 8 * q4) = w;
          }
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
      if (tid == 0) sh_last = atomicAdd(&p.unit_done[p.max_dec_units + it.unit], 1) == u.nch - 1;
      __syncthreads();
      if (sh_last) {
        // the LDS ring is idle here (every wave is past its last step); it
        // holds the per-row stats of the merge
        auto wg_sync = [] { __syncthreads(); };
        merge_unit<D>(p, u, p.pf_part, p.pf_plse, p.pf_rows, tid, NT, reinterpret_cast<float*>(lds), wg_sync);
      }
    }
    // every wave must be done with the ring before the next item refills it
    __syncthreads();
  }
}

}  // namespace rpa
