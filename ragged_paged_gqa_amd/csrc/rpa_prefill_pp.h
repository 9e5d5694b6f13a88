// Prefill/mixed-class attention kernel for 16-bit q with K/V in the q type
// (bf16, or f16 with F16): the matrix-bound path of the prefill workloads.
//
// A workgroup has 8 waves of 32 packed query rows (row = token * G + g, the
// kernel page's q block times the G q heads of one kv head, stacked into one
// MFMA dimension: `run`, per-kv-head step), 256 rows in all, one workgroup
// per CU. Waves w and w + 4 run on the same SIMD (measured on gfx950), and
// the two groups (waves 0-3: A, waves 4-7: B) take turns on the matrix unit:
// per 32-key step n of an item the waves go through two kinds of phase,
//   M(n): O^T += V^T P^T of step n - 1, then S^T = K Q^T of step n
//         (32 v_mfma_f32_32x32x16 at head_dim 256, operands from LDS),
//   S(n): the softmax of step n (`flashAttention`: scale, soft-cap, masks,
//         online maximum and sum, P = exp(s - m) packed to 16 bits),
// and group B runs one phase behind group A, so while one wave of a SIMD
// issues MFMAs the other does its softmax VALU work. A barrier of all 8
// waves separates the phases.
//
// K/V: each 32-key step's K rows and V rows of kv head h (combined heads 2h
// and 2h + 1, adjacent in memory: `stridedLoadKv`) go straight from HBM into
// one slot of a 4-slot LDS ring (global_load_lds_dwordx4, 1 KB of whole rows
// per instruction, 16-byte chunks XOR-swizzled by key so that the operand
// reads are bank-conflict free), two steps ahead of the first reader. The
// physical address of every 16-key block of an item comes from an LDS table
// built when the item starts (page_indices[seq, key / page_size]).
//
// Items (a key chunk of a 256-row unit) come from the planner's per-XCD
// queues; split units leave normalised f32 partials, and the workgroup that
// finishes a unit's last chunk merges them (rpa_merge.h).
#pragma once

#include <climits>

#include "rpa_common.h"
#include "rpa_merge.h"
#include "rpa_prefill.h"

namespace rpa {

constexpr int kPpStages = 4;  // ring slots: read by M(n-1)/M(n), landed, in flight
constexpr int kPpLead = 2;    // steps between a slot's DMA and its first reader
#ifndef RPA_PP_KA
#define RPA_PP_KA 3
#endif
#ifndef RPA_PP_VA
#define RPA_PP_VA 4  // (3: 0.6 % slower on the long-context workload; 5 and 6 slower still)
#endif

template <int D>
struct PpLds {
  static constexpr int kRowBytes = 2 * D;                // one K (or V) row of 16-bit elements
  static constexpr int kChunks = kRowBytes / 16;         // 16-byte chunks per row
  static constexpr int kRegion = kStepKeys * kRowBytes;  // the step's K rows; its V rows follow
  static constexpr int kSlot = 2 * kRegion;
  static constexpr size_t kBytes = (size_t)kPpStages * kSlot;
};

// LDS of one workgroup of prefill_pp_tiles.
template <int D>
struct PpShared {
  char lds[PpLds<D>::kBytes];  // the K/V ring (and the merge's staging)
  uint32_t blk[kPfBlkTable];   // physical key index of each 16-key block of the item
  int item[2];
  int last;
};

// The prefill-class tiles of one eight-wave workgroup: it takes items from
// the queues until they are empty.
template <int D, bool CAP, bool F16>
__device__ __forceinline__ void prefill_pp_tiles(const Params& p, PpShared<D>& shm, int pf_block) {
  constexpr int NW = kPpWaves;
  constexpr int NT = NW * 64;
  constexpr int NS = D / 16;    // k-steps of the QK product
  constexpr int NDB = D / 32;   // 32-wide d blocks of O^T
  constexpr int NM = 2 * NDB;   // PV MFMAs per step (two 16-key halves per d block)
  constexpr int RB = PpLds<D>::kRowBytes;
  constexpr int CPR = PpLds<D>::kChunks;
  constexpr int REG = PpLds<D>::kRegion;
  constexpr int SLOT = PpLds<D>::kSlot;
  constexpr int RPI = 1024 / RB;  // rows per DMA instruction
  constexpr int NIW = 8 / RPI;    // DMA instructions per wave per step: 8 rows of one region
  // f16 P must stay below 65504: exponentiated scores <= 2^15
  constexpr float SLACK = F16 ? kRescaleSlack - 1.0f : kRescaleSlack;
  static_assert(D == 64 || D == 128 || D == 256, "head_dim");
  static_assert(RPI * CPR == 64 && NIW * RPI == 8, "whole rows per DMA instruction");
  static_assert(kPpStages >= kPpLead + 2, "a slot is refilled once both groups are past its PV");

  char* const lds = shm.lds;
  uint32_t* const sh_blk = shm.blk;
  int* const sh_item = shm.item;
  int& sh_last = shm.last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: group A, 1: group B (one phase behind)
  const int r32 = lane & 31;  // S^T column = this lane's row within the wave's 32
  const int h = lane >> 5;    // which 16 of the row's 32 keys this lane holds

  // Every item goes to one workgroup, so workgroups past the item count
  // would only ever find the queues drained: they leave at once.
  if (pf_block >= p.hdr->n_pf_items) return;
  const int chunk = p.hdr->pf_chunk;
  const int64_t key_stride = (int64_t)2 * p.Hkv * D * 2;
  // Scores in base-2 units are s * cmul (capped: the cap is applied first and
  // folds the scale in); negative scales flip Q's sign instead. A zero scale
  // becomes the smallest normal one, so hidden keys (-inf) stay -inf while
  // every visible score still rounds to 0.
  const bool neg = p.sm_scale < 0.f;
  const float sm = neg ? -p.sm_scale : p.sm_scale;
  const float cmul = CAP ? 1.0f : fmaxf(sm * kLog2e, 1.17549435e-38f);
  const SoftCapB2 cap_b2(sm, CAP ? p.soft_cap : 1.0f);

  // LDS operand offsets inside a slot. The chunk swizzles (rpa_prefill.h)
  // only permute 32-byte (K) or 64-byte (V) steps inside 256-byte spans, and
  // a lane's swizzle bits never overlap its other offset bits, so each
  // operand address is one XOR of a per-lane base with a constant:
  //   K of k-step i: key r32, chunk 2i + h -> k_base ^ 32 (i % KT), + 256 (i / KT);
  //   V^T of d block d: keys 4 (g16 / 2) + l16 / 4 (+ 8), bytes 32 (g16 % 2)
  //   + 8 (l16 % 4) + 64 d of the row -> v_base ^ 64 (d % VT), + 256 (d / VT).
  constexpr int KT = NS < 8 ? NS : 8;
  constexpr int VT = NDB < 4 ? NDB : 4;
  const int sk = swz_k<D>(r32);
  const int k_base = r32 * RB + 16 * (h ^ (sk & 1)) + 32 * (sk >> 1);
  const int g16 = lane >> 4, l16 = lane & 15;
  const int v_key = 4 * (g16 >> 1) + (l16 >> 2);
  const int v_base = REG + v_key * RB + 16 * (2 * (g16 & 1) + ((l16 & 3) >> 1)) + 8 * (l16 & 1) +
                     64 * ((v_key & 3) & (VT - 1));
  // (The bases pass through an empty asm at each use site, so that the
  // compiler forms every address next to its read instead of hoisting all of
  // them out of the step loop into registers.)
  auto opaque = [](int x) {
    asm volatile("" : "+v"(x));
    return x;
  };

  // DMA share of this wave: region w % 2 (K or V), keys [8 (w / 2), + 8) of
  // the step, i.e. 16-key block w / 4 (group A loads a step's first block,
  // group B its second), rows 8 ((w / 2) % 2) of it, in NIW instructions of
  // RPI rows. LDS chunk c of key k holds global chunk c ^ swizzle(k).
  const int dma_region = wave & 1;
  const int dma_blk = wave >> 2;
  const int dma_row0 = 8 * ((wave >> 1) & 1);
  // source offset of this lane's 16 bytes in DMA instruction j (formed at
  // issue time, from an opaque lane index, to keep them out of registers)
  auto dma_off = [&](int ln, int j) {
    const int krow = dma_row0 + RPI * j + ln / CPR;  // key within the 16-key block
    const int key = 16 * dma_blk + krow;             // key within the step
    const int c_g = (ln % CPR) ^ (dma_region ? swz_v<D>(key) : swz_k<D>(key));
    return (uint32_t)(krow * key_stride) + (uint32_t)(dma_region * 2 * D) + 16u * c_g;
  };
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr_of(lds));
  const uint32_t dma_lds = (uint32_t)(dma_region * REG + (16 * dma_blk + dma_row0) * RB);

  // queues: this XCD's first, then the others in turn
  const int home = xcc_id() % kQueues;
  int qsel = 0;  // thread 0 only
  auto next_item = [&]() { return take_item(p, home, qsel); };

  int parity = 0;
  for (;;) {
    if (tid == 0) sh_item[parity] = next_item();
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(sh_item[parity]);
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
    const int N = c_hi > c_lo ? (c_hi - c_lo + kStepKeys - 1) / kStepKeys : 0;  // 32-key steps
    const uint8_t* kv_h = p.kv + (int64_t)2 * kvh * D * 2;
    const int32_t* ptab = p.page_indices + (int64_t)s * p.pps;
    // Block table: physical key index (page * page_size + slot) of 16-key
    // block b of the item at entry b. Blocks past the chunk (the second half
    // of a last step that ends early, and the kPpLead + 1 steps the loader
    // issues past the last one, so that every softmax phase issues the same
    // DMA) repeat its last block: they are loaded and never computed on.
    const int n_ent = N > 0 ? 2 * (N + kPpLead + 1) : 0;
    const int last_blk = c_lo + 16 * ((c_hi - c_lo - 1) >> 4);
    for (int i = tid; i < n_ent; i += NT) {
      const int key = min(c_lo + 16 * i, last_blk);
      const int lp = key / p.page;
      const int ph = min(max(ptab[min(lp, p.pps - 1)], 0), p.P - 1);
      sh_blk[i] = (uint32_t)ph * (uint32_t)p.page + (uint32_t)(key - lp * p.page);
    }
    __syncthreads();

    // this lane's query row
    const int vis_hi = min(kvl, c_hi);
    const int row = 32 * wave + r32;
    const bool rvalid = row < u.nrows;
    const int prow = u.row0 + row;
    const int t = prow / p.G;
    const int qh = kvh * p.G + (prow - t * p.G);
    const int tok = q0 + t;
    const int pos = kvl - ql + t;
    const int win_lo = p.window > 0 ? pos - p.window : INT_MIN;  // keys <= win_lo are hidden
    const int vis_end = p.is_causal ? min(vis_hi, pos + 1) : vis_hi;
    bf16x8 qb[NS];
    if (rvalid) {
      const int64_t e = ((int64_t)tok * p.Hq + qh) * D;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        u32x4 v = *reinterpret_cast<const u32x4*>(p.q + e + 16 * i + 8 * h);
        if (neg) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        qb[i] = __builtin_bit_cast(bf16x8, v);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NS; ++i) qb[i] = bf16x8{};
    }
    // the wave's row span, for the masked-block test
    const int wr_last = min(32 * wave + 31, u.nrows - 1);
    const int pos_lo = kvl - ql + (u.row0 + 32 * wave) / p.G;
    const int pos_hi = kvl - ql + (u.row0 + max(wr_last, 32 * wave)) / p.G;
    // Steps that can hold a key some row of the wave cannot see: those at or
    // past mask_hi (kv length, chunk end, causal diagonal) and those before
    // mask_lo (sliding window).
    int mask_hi, mask_lo = 0;
    {
      int lim = vis_hi - kStepKeys;  // steps starting at or before lim hold no key at or past vis_hi
      if (p.is_causal) lim = min(lim, pos_lo - (kStepKeys - 1));
      mask_hi = lim < c_lo ? 0 : min(N, (lim - c_lo) / kStepKeys + 1);
      if (p.window > 0) {
        const int w = pos_hi - p.window;  // steps starting at or before w hold a hidden key
        mask_lo = w < c_lo ? 0 : min(N, (w - c_lo) / kStepKeys + 1);
      }
    }

    float m_ref = -INFINITY;  // reference maximum of the row, base-2 units
    float lsum = 0.f;         // this lane's part of the row's sum of P
    f32x16 o[NDB];
#pragma unroll
    for (int d = 0; d < NDB; ++d) o[d] = f32x16{};
    f32x16 sacc = f32x16{};  // S^T of the step between its M and S phases
    bf16x8 pb[2];            // P^T of the step between its S phase and the next M phase
    pb[0] = bf16x8{};
    pb[1] = bf16x8{};

    // DMA of step m into its slot: this wave's global base (the block table
    // gives the first key of its 16-key block) and LDS destination, then
    // instruction j of NIW. Each instruction sets M0 for itself, so the NIW
    // of a step can be spread over a phase.
    struct DmaStep {
      const uint8_t* base;
      uint32_t dst;
    };
    auto dma_step_at = [&](int m) {
      const uint32_t ent = __builtin_amdgcn_readfirstlane(sh_blk[2 * m + dma_blk]);
      DmaStep st;
      st.base = uniform_ptr(kv_h + (uint64_t)ent * (uint64_t)key_stride);
      st.dst = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((m % kPpStages) * SLOT) + dma_lds);
      return st;
    };
    auto issue_one = [&](const DmaStep& st, int j) {
      dma16_sbase(st.base, dma_off(opaque(lane), j), st.dst + 1024u * j);
    };
    auto issue = [&](int m) {
      const DmaStep st = dma_step_at(m);
#pragma unroll
      for (int j = 0; j < NIW; ++j) issue_one(st, j);
    };

    // O^T += V^T P^T of step n (the first half of M(n + 1))
    auto pv = [&](int n) {
      const char* cs = lds + (n % kPpStages) * SLOT;
      const int vb = opaque(v_base);
      auto v_at = [&](int d) { return (vb ^ (64 * (d % VT))) + 256 * (d / VT); };
      constexpr int VA = RPA_PP_VA;  // V^T reads ahead of their MFMA
      bf16x8 va[NM];
      auto read_va = [&](int m) {
        const int ks = m / NDB, d = m % NDB;
        const bf16x4 lo = lds_read_tr16(reinterpret_cast<const __bf16*>(cs + (16 * ks) * RB + v_at(d)));
        const bf16x4 hi = lds_read_tr16(reinterpret_cast<const __bf16*>(cs + (16 * ks + 8) * RB + v_at(d)));
        va[m] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
#pragma unroll
      for (int m = 0; m < VA; ++m) read_va(m);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m + VA < NM) read_va(m + VA);
        o[m % NDB] = mfma32x32x16<F16>(va[m], pb[m / NDB], o[m % NDB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // S^T = K Q^T of step n (the second half of M(n))
    auto qk = [&](int n) {
      const char* ns = lds + (n % kPpStages) * SLOT;
      const int kbs = opaque(k_base);
      auto k_at = [&](int i) { return (kbs ^ (32 * (i % KT))) + 256 * (i / KT); };
      constexpr int KA = RPA_PP_KA;  // K reads ahead of their MFMA
      bf16x8 ka[NS];
#pragma unroll
      for (int i = 0; i < KA; ++i) ka[i] = *reinterpret_cast<const bf16x8*>(ns + k_at(i));
      sacc = f32x16{};
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i + KA < NS) ka[i + KA] = *reinterpret_cast<const bf16x8*>(ns + k_at(i + KA));
        sacc = mfma32x32x16<F16>(ka[i], qb[i], sacc);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // S phase of step n: scores -> P (packed), the row's maximum and sum
    auto phase_s = [&](int n, int dma_step) {
      const DmaStep dst = dma_step_at(dma_step);
      const int kb = c_lo + kStepKeys * n;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if constexpr (CAP) sacc[j] = cap_b2(sacc[j]);
        mx = fmaxf(mx, sacc[j]);
      }
      if (n >= mask_hi || n < mask_lo) {
        // hidden keys -> -inf by selection (NaN in unread slots cannot leak)
        mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kb + 8 * (j >> 2) + 4 * h + (j & 3);
          const bool vis = rvalid && key < vis_end && key > win_lo;
          sacc[j] = vis ? sacc[j] : -INFINITY;
          mx = fmaxf(mx, sacc[j]);
        }
      }
      mx = max_xor32(mx);
      if (!CAP) mx *= cmul;
      // lazily moved reference maximum: O and the sum are rescaled only when
      // the row's maximum outgrows the reference by more than SLACK
      if (__any(mx > m_ref + SLACK)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - m_new);
        m_ref = m_new;
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < NDB; ++d) o[d] *= alpha;
      }
      const float negm = m_ref == -INFINITY ? 0.f : -m_ref;
      // P = 2^(score - reference), packed in pairs; the row sum is taken in
      // f32 over the unrounded values
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        // this wave's DMA share of a later step, one instruction at a time
        // between the exponentials
        if (q % (8 / NIW) == 0) issue_one(dst, q / (8 / NIW));
        const float p0 = fast_exp2(CAP ? sacc[2 * q] + negm : __builtin_fmaf(sacc[2 * q], cmul, negm));
        const float p1 = fast_exp2(CAP ? sacc[2 * q + 1] + negm : __builtin_fmaf(sacc[2 * q + 1], cmul, negm));
        asm volatile("" ::"v"(p0), "v"(p1));  // the pair is computed here, between the DMA instructions
        lsum += p0 + p1;
        const bf16x2 pair = __builtin_bit_cast(bf16x2, pack2<F16>(p0, p1));
        pb[q >> 2][2 * (q & 3)] = pair[0];
        pb[q >> 2][2 * (q & 3) + 1] = pair[1];
        __builtin_amdgcn_sched_barrier(0);  // keep the DMA spread over the pairs
      }
    };

    // V rows of step n past kv_len, or in a 16-key block past the chunk,
    // read as zero (0 * NaN would poison the PV sum); group A clears them in
    // the phase between the step's publication and its first PV
    auto clear_tail = [&](int n) {
      const int k0 = c_lo + kStepKeys * n;
      if (k0 + kStepKeys <= vis_hi && k0 + kStepKeys <= c_hi) return;
      char* cur = lds + (n % kPpStages) * SLOT;
      for (int i = tid; i < kStepKeys * CPR; i += NT / 2) {
        const int key = i / CPR;
        if (k0 + key >= kvl || k0 + 16 * (key >> 4) >= c_hi)
          *reinterpret_cast<u32x4*>(cur + REG + key * RB + 16 * (i % CPR)) = u32x4{0u, 0u, 0u, 0u};
      }
    };

    if (N > 0) {
      issue(0);
      if (N > 1) {
        issue(1);
        wait_vmcnt<NIW>();
      } else {
        wait_vmcnt<0>();
      }
    }
    // Every wave runs M(0), S(0), M(1), S(1), ..., S(N - 1), M(N) (M(0) is
    // only a QK, M(N) only a PV), one phase per barrier; group B passes one
    // extra barrier first (and group A one last), so barrier k starts phase k
    // of group A and phase k - 1 of group B. `k` counts the barriers passed.
    // Each group issues its half of step k / 2 + kPpLead during its own S
    // phases (group A at odd k, group B at even k), so the matrix phases
    // never wait on DMA issue; every S phase issues (steps past the last one
    // re-read its block), so step (k + 1) / 2 has landed once at most the
    // wave's latest NIW instructions are outstanding at the end of an odd
    // phase.
    int k = 0;
    int dma_step = 0;  // the step whose DMA this wave issues in the current phase
    auto begin_phase = [&]() {
      __syncthreads();
      dma_step = (k >> 1) + kPpLead;
    };
    auto end_phase = [&]() {
      if (k & 1) wait_vmcnt<NIW>();
      ++k;
    };
    // group B's leading idle phase issues its half of step kPpLead; group
    // A's trailing one issues nothing
    auto idle_phase = [&](bool dma) {
      begin_phase();
      if (dma && N > 0) issue(dma_step);
      end_phase();
    };
    // S phase of step n with this phase's DMA share spread over it
    auto softmax_phase = [&](int n) {
      phase_s(n, dma_step);
      if (grp == 0) clear_tail(n);
    };
    if (grp == 1) idle_phase(true);
    if (N > 0) {
      begin_phase();
      qk(0);
      end_phase();
      begin_phase();
      softmax_phase(0);
      end_phase();
      for (int n = 1; n < N; ++n) {
        begin_phase();
        pv(n - 1);
        qk(n);
        end_phase();
        begin_phase();
        softmax_phase(n);
        end_phase();
      }
      begin_phase();
      pv(N - 1);
      end_phase();
    }
    if (grp == 0) idle_phase(false);
    // the re-reads past the chunk have landed: the ring is idle
    wait_vmcnt<0>();

    // lane (row, h) holds O^T[32 d + 8 (j / 4) + 4 h + (j % 4)][row]
    const float l_row = sum_xor32(lsum);
    float inv, lse_v;
    // a whole row takes its sink (if any) here; a chunk's partial leaves it
    // to the merge
    row_final(m_ref, l_row, p.v_scale, (u.nch == 1 && p.sinks) ? p.sinks + qh : nullptr, inv, lse_v);
    if (rvalid) {
      if (u.nch == 1) {
        const int64_t e = ((int64_t)tok * p.Hq + qh) * D + 4 * h;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            store_out4<F16, false>(p.out, e + 32 * d + 8 * q4, o[d][4 * q4] * inv, o[d][4 * q4 + 1] * inv,
                                   o[d][4 * q4 + 2] * inv, o[d][4 * q4 + 3] * inv);
        if (h == 0 && p.lse) p.lse[(int64_t)tok * p.Hq + qh] = lse_v;
      } else {
        float* pp = p.pf_part + ((int64_t)item * p.pf_rows + row) * D + 4 * h;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 w = {o[d][4 * q4] * inv, o[d][4 * q4 + 1] * inv, o[d][4 * q4 + 2] * inv,
                             o[d][4 * q4 + 3] * inv};
            store_coherent4(pp + 32 * d + 8 * q4, w);
          }
        if (h == 0) store_coherent(p.pf_plse + (int64_t)item * p.pf_rows + row, lse_v);
      }
    }
    if (u.nch > 1) {
      // publish the partial, count the chunk; the last one merges the unit
      wait_stores();
      __syncthreads();
      if (tid == 0) sh_last = atomicAdd(&p.unit_done[it.unit], 1) == u.nch - 1;
      __syncthreads();
      if (sh_last) {
        // the ring is idle (every wave is past its last phase); it holds the
        // merge's per-row statistics
        auto wg_sync = [] { __syncthreads(); };
        merge_unit<D, F16, false, false>(p, u, p.pf_part, p.pf_plse, p.pf_rows, [&](int c) { return u.item0 + c; }, tid, NT,
                                  reinterpret_cast<float*>(lds), wg_sync);
      }
    }
    // every wave must be done with the ring and the block table before the
    // next item refills them
    __syncthreads();
  }
}

}  // namespace rpa
