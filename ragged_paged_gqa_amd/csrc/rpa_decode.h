// Decode-class attention kernel: units of at most 16 packed query rows
// (q_len * G <= 16, e.g. one decode token of 4..16 grouped q heads).
//
// The kernel streams K/V from HBM and is bound by it. A wave works through a
// sequence of items (key chunks of one sequence and one kv head), the first
// one fixed by its position in the grid and the rest claimed from a
// device-wide queue, as one continuous pipeline of 32-key steps:
//   * loads: K and V rows go straight from HBM into registers, one step ahead
//     of the compute. Lane (key = lane % 16, k-group g = lane / 16) reads
//     16-byte pieces of its key row; K of kv head h is combined head 2h and V
//     is combined head 2h+1 right after it (`stridedLoadKv` on the kernel
//     page). The load side moves on to the next item as soon as the current
//     one has no step left, so the pipeline never drains between items;
//   * pages: each 16-key block takes its physical page (the kernel page's
//     `createKvAsyncCopyDescriptors`: page_indices[seq, key / page]) from a
//     128-entry window of the page table that the wave holds in registers, one
//     entry per lane (v_readlane); a chunk never spans more than 128 pages;
//   * next item: its queue slot is claimed when the current item starts, and
//     its descriptor, page window and Q rows are loaded one dependent step at
//     a time behind the current item's loads, so no load on the critical
//     path ever waits for another.
// Per 32-key block:
//   1. S^T [keys x rows] = K Q^T with v_mfma_f32_16x16x32_bf16 against the
//      register-resident Q^T, times sm_scale (k_scale folded in), the optional
//      soft-cap, then the causal / window / length masks of `flashAttention`
//      by selection (masked scores become -inf, so NaN in unread tail slots
//      cannot leak in); blocks that every row sees whole skip the mask;
//   2. the online-softmax update of `flashAttention` in base 2 (running max,
//      rescale factor alpha = 2^(m_old - m_new), running sum), with the
//      accumulator kept un-normalised until the end;
//   3. V (zeroed past kv_len: 0 * NaN would otherwise poison the sum) is
//      staged through a per-wave LDS tile and read back transposed with
//      ds_read_b64_tr_b16 as the A operand of O^T += V^T P^T, whose B operand
//      P^T is exactly the S^T result layout — no shuffle of P.
// fp8 e4m3fn K/V are widened to bf16 exactly with v_cvt_scalef32_pk_bf16_fp8
// at compute time (the in-flight registers hold raw bytes); k_scale is folded
// into the score scale and v_scale into the final normalisation.
// The contraction over head_dim may visit d in any order as long as K and Q
// use the same one: for fp8 a lane's 16-byte piece covers 16 consecutive d,
// which become two 8-wide k-slots of the MFMA, and Q is loaded to match.
// An item that is its unit's only chunk writes bf16 out and f32 lse; otherwise
// it writes a normalised f32 partial and its lse, which the combine kernel
// merges once every item is done (combine_kernel below).
#pragma once

#include "rpa_common.h"
#include "rpa_merge.h"

namespace rpa {

constexpr int kDecWavesPerBlock = 4;

template <int D>
struct DecodeLds {
  static constexpr int kVStride = D + 16;  // bf16 elements per staged V row (+32 B)
  static constexpr int kWaveElems = kStepKeys * kVStride;
  static constexpr size_t kBytes = (size_t)kDecWavesPerBlock * kWaveElems * 2;
};

template <int D, bool FP8>
struct DecShape {
  static constexpr int NI = D / 32;        // 8-wide k-slots per lane over head_dim (MFMA k-steps)
  static constexpr int ND = D / 16;        // 16-row blocks of O^T
  static constexpr int EB = FP8 ? 1 : 2;   // bytes per K/V element
  static constexpr int NLD = D * EB / 64;  // 16-byte loads per lane per 16-key block, K or V
};
// waves per SIMD the register budget is sized for
constexpr int dec_waves_per_simd(int D) { return D >= 256 ? 1 : 2; }

// First d of k-slot i for lane group g (K rows, Q rows and staged V rows use
// the same map). bf16: the 16-byte piece i of lane g is d = 32 i + 8 g; fp8:
// piece j = i / 2 of lane g covers d = 64 j + 16 g .. + 15, split in two
// 8-wide slots.
template <bool FP8>
__device__ __forceinline__ int slot_d(int i, int g) {
  return FP8 ? 64 * (i >> 1) + 16 * g + 8 * (i & 1) : 32 * i + 8 * g;
}

// CAP: the soft-cap is on (a template parameter, so the uncapped kernel
// carries no cap arithmetic at all).
template <int D, bool FP8, bool CAP>
__global__ __launch_bounds__(kDecWavesPerBlock * 64, dec_waves_per_simd(D)) void decode_kernel(Params p) {
  using S = DecShape<D, FP8>;
  constexpr int NI = S::NI, ND = S::ND, EB = S::EB, NLD = S::NLD;
  constexpr int VST = DecodeLds<D>::kVStride;
  __shared__ __attribute__((aligned(16))) __bf16 lds[kDecWavesPerBlock * DecodeLds<D>::kWaveElems];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  __bf16* vs = lds + wave * DecodeLds<D>::kWaveElems;

  const int n_items = uni(p.hdr->n_dec_items);
  const int64_t key_stride = (int64_t)2 * p.Hkv * D * EB;  // bytes between consecutive slots
  const float cap_k = CAP ? 2.0f * kLog2e / p.soft_cap : 0.f;
  const float sc_mul = CAP ? p.sm_scale : p.sm_scale * kLog2e;  // uncapped: straight to base 2
  // this lane's byte offset inside a 16-key block (piece 0 of K)
  const uint32_t lane_off = (uint32_t)(col * key_stride) + 16u * g;

  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // ---- item descriptors: one load of 16 words, one word per lane ----
  struct Info {
    int idx, s, h, c_lo, c_hi, kvl, q0, ql, row0, nrows, nch;
  };
  auto load_desc = [&](int idx) -> int {
    return lane < 16 ? reinterpret_cast<const int32_t*>(p.dec_items + idx)[lane] : 0;
  };
  auto unpack = [&](int idx, int dv) {
    Info I;
    I.idx = idx;
    I.s = __builtin_amdgcn_readlane(dv, 0);
    I.h = __builtin_amdgcn_readlane(dv, 1);
    I.c_lo = __builtin_amdgcn_readlane(dv, 2);
    I.c_hi = max(__builtin_amdgcn_readlane(dv, 3), I.c_lo);
    I.kvl = __builtin_amdgcn_readlane(dv, 4);
    I.q0 = __builtin_amdgcn_readlane(dv, 5);
    I.ql = __builtin_amdgcn_readlane(dv, 6);
    I.row0 = __builtin_amdgcn_readlane(dv, 7);
    I.nrows = __builtin_amdgcn_readlane(dv, 8);
    I.nch = __builtin_amdgcn_readlane(dv, 9);
    return I;
  };
  // the item's physical pages: lane l of window w holds logical page
  // c_lo / page + 64 w + l, clamped to the item's last page (entries past it
  // are never read)
  auto load_window = [&](const Info& I, int (&win)[2]) {
    const int lp0 = I.c_lo / p.page;
    const int lp_last = max(I.c_hi - 1, I.c_lo) / p.page;
    const int32_t* ptab = p.page_indices + (int64_t)I.s * p.pps;
#pragma unroll
    for (int w = 0; w < 2; ++w) win[w] = ptab[min(min(lp0 + 64 * w + lane, lp_last), p.pps - 1)];
  };
  auto load_q = [&](const Info& I, bf16x8 (&qb)[NI]) {
    const int prow = I.row0 + col;
    const int t = prow / p.G;
    const int qh = I.h * p.G + (prow - t * p.G);
    if (col < I.nrows) {
      const uint16_t* qp = p.q + ((int64_t)(I.q0 + t) * p.Hq + qh) * D;
#pragma unroll
      for (int i = 0; i < NI; ++i) qb[i] = *reinterpret_cast<const bf16x8*>(qp + slot_d<FP8>(i, g));
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) qb[i] = bf16x8{};
    }
  };

  // 32-key steps of an item; an empty key range (only outside the data
  // preconditions) still takes one fully masked step, so that the load and
  // compute sides always agree on the step count
  auto item_steps = [](const Info& I) { return max(1, (I.c_hi - I.c_lo + kStepKeys - 1) / kStepKeys); };

  // ---- loader: the item whose steps are being loaded ----
  struct Loader {
    int h, c_hi, lp0, lp, sl, key, left;  // left: steps not yet loaded
  };
  auto loader_for = [&](const Info& I) {
    Loader L;
    L.h = I.h;
    L.c_hi = I.c_hi;
    L.lp0 = I.c_lo / p.page;
    L.lp = L.lp0;
    L.sl = I.c_lo - L.lp0 * p.page;
    L.key = I.c_lo;
    L.left = item_steps(I);
    return L;
  };
  struct Stage {
    u32x4 k[2][NLD];
    u32x4 v[2][NLD];
  };
  // Loads the next step of L (or, with nothing left, re-reads its last block:
  // harmless, never computed).
  auto load_step = [&](Loader& L, const int (&win)[2], Stage& st) {
    const bool real = L.left > 0;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int rel = min(L.lp - L.lp0, kDecPageWindow - 1);
      int phys = rel < 64 ? __builtin_amdgcn_readlane(win[0], rel) : __builtin_amdgcn_readlane(win[1], rel - 64);
      phys = min(max(phys, 0), p.P - 1);
      const uint8_t* base = p.kv + uni64(((int64_t)phys * p.page + L.sl) * key_stride + (int64_t)2 * L.h * D * EB);
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        st.k[b][j] = *reinterpret_cast<const u32x4*>(base + lane_off + 64 * j);
        st.v[b][j] = *reinterpret_cast<const u32x4*>(base + lane_off + D * EB + 64 * j);
      }
      // advance to the next 16-key block if it is still inside the item
      if (real && L.key + 16 < L.c_hi) {
        L.key += 16;
        L.sl += 16;
        if (L.sl >= p.page) {
          L.sl = 0;
          ++L.lp;
        }
      }
    }
    if (real) --L.left;
  };
  // ---- compute state of the current item ----
  Info C;
  bf16x8 qb[NI];
  float m, lsum;
  f32x4 o[ND];
  int steps_done, n_steps;
  bool rvalid;
  int tok, qh, pos, pos_lo, pos_hi, vis_hi;
  auto begin_item = [&]() {
    m = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    steps_done = 0;
    n_steps = item_steps(C);
    // column `col` of S^T / O^T is packed row C.row0 + col of the sequence
    rvalid = col < C.nrows;
    const int prow = C.row0 + col;
    const int t = prow / p.G;
    qh = C.h * p.G + (prow - t * p.G);
    tok = C.q0 + t;
    pos = C.kvl - C.ql + t;
    pos_lo = C.kvl - C.ql + C.row0 / p.G;
    pos_hi = C.kvl - C.ql + (C.row0 + max(C.nrows, 1) - 1) / p.G;
    vis_hi = min(C.c_hi, C.kvl);
  };

  // One 32-key block: keys [kb, kb + 32).
  auto compute_block = [&](const Stage& st, int kb) {
    bf16x8 ka[2][NI];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        if constexpr (FP8) {
          ka[b][2 * j] = fp8x8_to_bf16(u32x2{st.k[b][j][0], st.k[b][j][1]});
          ka[b][2 * j + 1] = fp8x8_to_bf16(u32x2{st.k[b][j][2], st.k[b][j][3]});
        } else {
          ka[b][j] = __builtin_bit_cast(bf16x8, st.k[b][j]);
        }
      }
    }
    // S^T: lane (col, g) gets keys kb + 16b + 4g + j of row `col`.
    f32x4 sc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NI; ++i) sc[b] = mfma16x16x32(ka[b][i], qb[i], sc[b]);
    }
    // does the block hold a key that some row of the unit cannot see?
    const bool need_mask = kb + 32 > vis_hi || (p.is_causal && kb + 31 > pos_lo) ||
                           (p.window > 0 && kb <= pos_hi - p.window);
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = sc[b][j] * sc_mul;
        if constexpr (CAP) x = soft_cap_f(x, p.soft_cap, cap_k) * kLog2e;
        if (need_mask) {
          const int key = kb + 16 * b + 4 * g + j;
          bool vis = key < vis_hi;
          if (p.is_causal) vis = vis && key <= pos;
          if (p.window > 0) vis = vis && key > pos - p.window;
          x = vis ? x : -INFINITY;
        }
        sc[b][j] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = wave_max_xor16_32(mx);
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] *= alpha;
    float pv[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pv[b][j] = fast_exp2(sc[b][j] - m_use);
        lsum += pv[b][j];
      }

    // Stage V rows [kb, kb + 32) in LDS as bf16, zero past kv_len / the chunk.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const bool vok = kb + 16 * b + col < vis_hi;
      __bf16* vrow_w = vs + (16 * b + col) * VST;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        if constexpr (FP8) {
          bf16x8 lo = fp8x8_to_bf16(u32x2{st.v[b][j][0], st.v[b][j][1]});
          bf16x8 hi = fp8x8_to_bf16(u32x2{st.v[b][j][2], st.v[b][j][3]});
          if (!vok) {
            lo = bf16x8{};
            hi = bf16x8{};
          }
          *reinterpret_cast<bf16x8*>(vrow_w + slot_d<FP8>(2 * j, g)) = lo;
          *reinterpret_cast<bf16x8*>(vrow_w + slot_d<FP8>(2 * j + 1, g)) = hi;
        } else {
          const u32x4 v = vok ? st.v[b][j] : u32x4{0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(vrow_w + slot_d<FP8>(j, g)) = v;
        }
      }
    }
    wave_sync();

    bf16x8 pb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pb[j] = (__bf16)pv[0][j];
      pb[4 + j] = (__bf16)pv[1][j];
    }
    const __bf16* vrow = vs + (4 * g + (col >> 2)) * VST + 4 * (col & 3);
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const bf16x4 lo = lds_read_tr16(vrow + 16 * d);
      const bf16x4 hi = lds_read_tr16(vrow + 16 * VST + 16 * d);
      const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[d] = mfma16x16x32(a, pb, o[d]);
    }
    wave_sync();
  };

  // Result of the current item: bf16 out + lse, or an f32 partial + lse.
  auto finish_item = [&]() {
    const float l_row = wave_sum_xor16_32(lsum);
    const float inv = l_row > 0.f ? p.v_scale / l_row : 0.f;
    const float lse_v = l_row > 0.f ? (m + fast_log2(l_row)) * kLn2 : -INFINITY;
    if (!rvalid) return;
    if (C.nch == 1) {
      uint16_t* op = p.out + ((int64_t)tok * p.Hq + qh) * D;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        u32x2 w = {bf16x2_bits(o[d][0] * inv, o[d][1] * inv), bf16x2_bits(o[d][2] * inv, o[d][3] * inv)};
        *reinterpret_cast<u32x2*>(op + 16 * d + 4 * g) = w;
      }
      if (g == 0 && p.lse) p.lse[(int64_t)tok * p.Hq + qh] = lse_v;
    } else {
      float* pp = p.dec_part + ((int64_t)C.idx * kDecRows + col) * D;
#pragma unroll
      for (int d = 0; d < ND; ++d) *reinterpret_cast<f32x4*>(pp + 16 * d + 4 * g) = o[d] * inv;
      if (g == 0) p.dec_plse[(int64_t)C.idx * kDecRows + col] = lse_v;
    }
  };

  // ---- the next item, prepared one dependent load per step ----
  // nstate: 0 slot claimed (claim_v in flight), 1 descriptor in flight,
  // 2 window and Q in flight / ready, 3 the queue is empty
  const int first_dynamic = gridDim.x * kDecWavesPerBlock;
  int nstate = 3, claim_v = 0, ndv = 0;
  Info N;
  N.idx = -1;
  int nwin[2] = {0, 0};
  bf16x8 nq[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) nq[i] = bf16x8{};
  auto claim = [&]() {
    claim_v = 0;
    if (lane == 0) claim_v = atomicAdd(&p.hdr->dec_counter, 1);
    nstate = 0;
  };
  auto hop = [&]() {
    if (nstate == 0) {
      const int idx = first_dynamic + __builtin_amdgcn_readfirstlane(__shfl(claim_v, 0));
      if (idx < n_items) {
        N.idx = idx;
        ndv = load_desc(idx);
        nstate = 1;
      } else {
        nstate = 3;
      }
    } else if (nstate == 1) {
      N = unpack(N.idx, ndv);
      load_window(N, nwin);
      load_q(N, nq);
      nstate = 2;
    }
  };

  // ---- first item (fixed by grid position) ----
  {
    const int first = blockIdx.x * kDecWavesPerBlock + wave;
    if (first >= n_items) return;
    C = unpack(first, load_desc(first));
  }
  int lwin[2];
  load_window(C, lwin);
  load_q(C, qb);
  Loader L = loader_for(C);
  bool loader_on_next = false;
  claim();
  begin_item();

  Stage st[2];
  load_step(L, lwin, st[0]);
  for (;;) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      // load side: the step after the one computed below
      if (L.left == 0 && !loader_on_next) {
        while (nstate < 2) hop();  // only for items shorter than the chain
        if (nstate == 2) {
          L = loader_for(N);
          lwin[0] = nwin[0];
          lwin[1] = nwin[1];
          loader_on_next = true;
        }
      }
      load_step(L, lwin, st[k ^ 1]);
      // compute side
      compute_block(st[k], C.c_lo + steps_done * kStepKeys);
      ++steps_done;
      hop();
      if (steps_done == n_steps) {
        finish_item();
        if (!loader_on_next) return;  // the queue is empty
        C = N;
#pragma unroll
        for (int i = 0; i < NI; ++i) qb[i] = nq[i];
        loader_on_next = false;
        claim();
        begin_item();
      }
    }
  }
}

// Merges the split decode-class units once every decode item is done: one
// wave per unit, the chunks' partials combined by merge_unit.
template <int D>
__global__ __launch_bounds__(kDecWavesPerBlock * 64) void combine_kernel(Params p) {
  __shared__ float stat[kDecWavesPerBlock][2 * kDecRows];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_units = uni(p.hdr->n_dec_units);
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  for (int u = blockIdx.x * kDecWavesPerBlock + wave; u < n_units; u += gridDim.x * kDecWavesPerBlock) {
    Unit U;
    U.seq = uni(p.dec_units[u].seq);
    U.kv_head = uni(p.dec_units[u].kv_head);
    U.row0 = uni(p.dec_units[u].row0);
    U.nrows = uni(p.dec_units[u].nrows);
    U.kv_lo = uni(p.dec_units[u].kv_lo);
    U.kv_hi = uni(p.dec_units[u].kv_hi);
    U.nch = uni(p.dec_units[u].nch);
    U.item0 = uni(p.dec_units[u].item0);
    if (U.nch <= 1) continue;
    merge_unit<D>(p, U, p.dec_part, p.dec_plse, kDecRows, lane, 64, stat[wave], wave_sync);
    wave_sync();
  }
}

}  // namespace rpa
