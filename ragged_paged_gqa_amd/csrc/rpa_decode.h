// Decode-class attention kernel: units of at most 16 packed query rows
// (q_len * G <= 16, e.g. one decode token of 4..16 grouped q heads).
//
// The kernel streams K/V from HBM and is bound by it. Work is split
// stream-K style: the key blocks (16 keys; 32 for one-byte K/V) of all decode
// units, laid end to end, are cut into one equal contiguous range per wave,
// so every wave moves the same number of bytes and no queue is needed. The planner writes only one record
// per decode sequence (DecSeq); a wave finds the sequence holding its first
// block by a 64-way search over the records' first blocks and walks the units
// from there. It runs its parts (the pieces of units inside its range) as one
// continuous pipeline of 16-key DMA steps (computed one at a time for 16-bit
// K/V, two at a time for one-byte K/V):
//   * loads: each step's K rows and V rows of kv head h (combined heads 2h and
//     2h+1, adjacent in memory: `stridedLoadKv` on the kernel page) go
//     straight from HBM into a per-wave ring of LDS slots with
//     global_load_lds_dwordx4, 1 KB of whole rows per instruction, kept
//     NST - 1 steps ahead of the compute across part boundaries. The 16-byte
//     chunks of a row are XOR-swizzled by the key, so that the MFMA operand
//     reads below hit distinct LDS banks. Completion is tracked by counting
//     vector-memory instructions (s_waitcnt vmcnt), so nothing else waits on
//     the stream;
//   * pages and metadata: the physical page of each 16-key block (the kernel
//     page's `createKvAsyncCopyDescriptors`: page_indices[seq, key / page])
//     and the sequence records are read with scalar loads one step ahead, and
//     the next part's Q rows are fetched into an LDS slot by the same DMA
//     while the current part runs.
// Per 16-key step:
//   1. S^T [16 keys x 16 rows] = K Q^T with v_mfma_f32_16x16x32_bf16 against
//      the register-resident Q^T, times sm_scale (k_scale folded in), the
//      optional soft-cap, then the causal / window / length masks of
//      `flashAttention` by selection (masked scores become -inf, so NaN in
//      unread tail slots cannot leak in); steps that every row sees whole skip
//      the mask;
//   2. the online-softmax update of `flashAttention` in base 2, with a lazily
//      moved reference maximum (the accumulator is rescaled only when a row's
//      maximum outgrows it by more than kDecSlack);
//   3. O^T [D x 16 rows] += V^T P^T with v_mfma_f32_16x16x16_bf16: V^T read
//      with ds_read_b64_tr_b16, P^T exactly the S^T result layout. V rows past
//      kv_len are zeroed first (0 * NaN would otherwise poison the sum).
// One-byte K/V codes are widened exactly after the LDS read
// (v_cvt_scalef32_pk_bf16_fp8 / _bf8, or sign extension for int8). Their
// compute step covers 32 keys (two DMA slots): S^T of each 16-key half, one
// softmax update, then O^T += V^T P^T with v_mfma_f32_16x16x32, V^T read
// straight out of the two slots with ds_read_b64_tr_b8 and widened in
// registers; the slots are refilled once those reads are done. k_scale is
// folded into the score scale and v_scale into the final normalisation. The
// contraction over head_dim may visit d in any order as long as K and Q use
// the same one: a lane's 16-byte K piece covers 16 consecutive d for fp8,
// which become two 8-wide k-slots of the MFMA, and Q is read to match.
// A part that is its unit's only one writes bf16 out and f32 lse; otherwise
// it writes a normalised f32 partial and its lse into a slot of its wave
// (2w for a part that continues a unit from the previous range, 2w + 1 for
// the first part of a unit that runs on), which the combine kernel merges
// once every wave is done (combine_kernel below).
//
// Element types: the kernel is instantiated per K/V kind KVT (K/V in the q
// type, fp8 e4m3fn, fp8 e5m2, int8) and per 16-bit type F16 (bf16, or f16
// with an f16 q: f16 MFMAs, f16 P and output). In the comments below "bf16"
// stands for that 16-bit type and "fp8" for any one-byte code.
// Q32: an f32 q (bf16 path, K/V bf16 or one-byte): Q is split into bf16 hi
// and lo operands (split_q8), S^T takes both MFMA chains, out is f32.
#pragma once

#include "rpa_common.h"
#include "rpa_merge.h"

namespace rpa {

// The reference maximum of a row moves only when the row's maximum outgrows it
// by more than this (base-2 units): exponentiated scores stay <= 2^12.
constexpr float kDecSlack = 12.0f;

// Chunk swizzles of a region's rows (key = row 0..15): K pieces are read by
// 16 lanes holding 16 keys at the same chunk; V is read transposed by 4 keys
// x 2 chunks per 16 lanes. Both spread a read over all 64 banks.
template <int D, bool FP8>
__device__ __forceinline__ int dswz_k(int key) {
  using C = DecCfg<D, FP8>;
  return (key / C::RP) & ((C::CPR < 16 ? C::CPR : 16) - 1);
}
template <int D, bool FP8>
__device__ __forceinline__ int dswz_v(int key) {
  using C = DecCfg<D, FP8>;
  return 2 * ((key / C::RP) & ((C::CPR < 16 ? C::CPR : 16) / 2 - 1));
}

// fp8: chunk swizzle of a key's K|V segment (2 * D bytes) in a ring slot:
// the 16 keys' reads of one chunk, and the DMA's writes, cover all banks.
template <int D>
__device__ __forceinline__ int dswz_kv(int key) {
  constexpr int SEG = 2 * D;
  constexpr int RPS = SEG >= 256 ? 1 : 256 / SEG;
  constexpr int CPS = SEG / 16 < 16 ? SEG / 16 : 16;
  return (key / RPS) & (CPS - 1);
}

// First d of k-slot i for lane group g (K pieces and Q use the same map).
// bf16: the 16-byte piece i of lane g is d = 32 i + 8 g; fp8: piece j = i / 2
// of lane g covers d = 64 j + 16 g .. + 15, split in two 8-wide slots.
template <bool FP8>
__device__ __forceinline__ int slot_d(int i, int g) {
  return FP8 ? 64 * (i >> 1) + 16 * g + 8 * (i & 1) : 32 * i + 8 * g;
}


typedef short s16x4 __attribute__((ext_vector_type(4)));
template <bool F16>
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0,
                                                 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                     0, 0);
}

// The decode-class tiles of one workgroup (`block`: its index among the
// decode workgroups), in the workgroup's LDS `lds` (kDecWavesPerBlock *
// WAVE_LDS bytes, 1 KB aligned). CAP: the soft-cap is on (a template
// parameter, so the uncapped code carries no cap arithmetic at all).
template <int D, int KVT, bool CAP, bool F16, bool Q32 = false>
__device__ __forceinline__ void decode_tiles(const Params& p, char* lds, int block) {
  constexpr bool FP8 = KVT != kKvBf16;  // one-byte codes (fp8 kinds, int8)
  constexpr bool QREG = FP8 || Q32;     // Q operand loaded into registers (no LDS Q slot)
  static_assert(!(Q32 && F16), "an f32 q runs on the bf16 path");
  using Cf = DecCfg<D, FP8>;
  constexpr int EB = Cf::EB, RB = Cf::RB, REGION = Cf::REGION, STAGE = Cf::STAGE, NDR = Cf::NDR,
                NDMA = Cf::NDMA, NI = Cf::NI, ND = Cf::ND, NLD = Cf::NLD, NST = Cf::NST;

  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);  // wave-uniform: the loader and part logic stay scalar
  const int col = lane & 15;
  const int g = lane >> 4;
  char* wl = lds + wave * Cf::WAVE_LDS;       // this wave's LDS: ring slots, then the Q slot
  char* ring = wl;
  __bf16* qs = reinterpret_cast<__bf16*>(wl + NST * STAGE);
  const uint32_t ring_lds = lds_addr_of(ring);
  const uint32_t qs_lds = lds_addr_of(qs);

  // keys per stream-K block, 16-key DMA steps per compute step
  constexpr int BK = FP8 ? kDecBlk8 : kDecBlk16, CS = BK / kDecStepKeys;
  static_assert(NST >= 2 * CS, "a compute step's slots and the next ones fit the ring");
  const int key_stride = 2 * p.Hkv * D * EB;  // bytes between consecutive slots (< 2^26)
  const float sc_mul = p.sm_scale * kLog2e;  // uncapped: straight to base 2
  const SoftCapB2 cap_b2(p.sm_scale, CAP ? p.soft_cap : 1.0f);

  // per-lane DMA source offsets inside a 16-key block (loop-invariant): LDS
  // chunk c of row `key` holds global chunk c ^ swizzle(key)
  // bf16: the K region (16 rows), then the V region. fp8: every key's K row
  // and V row are adjacent in memory (combined heads 2h, 2h+1) and move
  // together, as one 2*RB-byte segment per key, so each DMA instruction reads
  // whole K|V segments; chunks are swizzled over the segment (dswz_kv).
  uint32_t voff[2][NDR];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int j = 0; j < NDR; ++j) {
      if constexpr (FP8) {
        const int o = 1024 * (r * NDR + j) + 16 * lane;
        const int key = o / (2 * RB);
        const int cl = (o % (2 * RB)) / 16;
        voff[r][j] = (uint32_t)(key * key_stride + 16 * (cl ^ dswz_kv<D>(key)));
      } else {
        const int o = 1024 * j + 16 * lane;
        const int key = o / RB;
        const int cl = (o % RB) / 16;
        const int sw = r == 1 ? dswz_v<D, FP8>(key) : dswz_k<D, FP8>(key);
        voff[r][j] = (uint32_t)(key * key_stride + r * RB + 16 * (cl ^ sw));
      }
    }

  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // ---- the wave's range of the stream-K split, and its parts ----
  const int w = block * kDecWavesPerBlock + wave;  // stream-K rank
  const int n_dseq = uni(p.hdr->n_dec_seqs);
  const int W = uni(p.hdr->pad0[0]);
  const StreamK sk = StreamK::make(uni(p.hdr->dec_blocks), W);
  // A part: the blocks of unit (decode sequence i, kv head h) that fall into
  // this wave's range [ws, we), keys [c_lo, c_hi).
  // (Kept small: three of these are live at once, in scalar registers; the
  // sequence's own metadata is loaded where a part starts, see Seq.)
  struct Info {
    bool valid;
    int i;          // decode sequence record
    int h, b0, nb;  // the unit: kv head h, blocks [b0, b0 + nb)
    int lo16, hi;   // the units' key range
    int c_lo, c_hi;
  };
  int ws = 0, we = 0;
  auto load_seq = [&](Info& I, int i) {
    const int32_t* d = reinterpret_cast<const int32_t*>(p.dec_seqs + i);
    I.i = i;
    I.lo16 = sload(d + 4);
    I.hi = sload(d + 5);
    I.b0 = sload(d + 6);  // the unit of kv head 0
    I.nb = sload(d + 7);
    I.h = 0;
  };
  auto set_part = [&](Info& I) {
    const int x0 = max(I.b0, ws), x1 = min(I.b0 + I.nb, we);
    I.c_lo = I.lo16 + BK * (x0 - I.b0);
    I.c_hi = max(min(I.hi, I.lo16 + BK * (x1 - I.b0)), I.c_lo);
    I.valid = true;
  };
  // the unit has parts in other ranges too
  auto is_split = [&](const Info& I) { return I.b0 < ws || I.b0 + I.nb > we; };
  // partial slot of a split part: 2w for a part that continues a unit from
  // the previous range, 2w + 1 for the first part of a unit that runs on
  auto slot_of = [&](const Info& I) { return 2 * w + (I.b0 < ws ? 0 : 1); };
  struct Seq {
    int s, q0, ql, kvl, nrows;
  };
  auto seq_of = [&](const Info& I) {
    const int32_t* d = reinterpret_cast<const int32_t*>(p.dec_seqs + I.i);
    Seq m;
    m.s = sload(d + 0);
    m.q0 = sload(d + 1);
    m.ql = sload(d + 2);
    m.kvl = sload(d + 3);
    m.nrows = m.ql * p.G;
    return m;
  };
  // The first part: the unit holding block ws, of the last decode sequence
  // whose first block is <= ws (it has blocks: a later sequence starts after
  // ws). The table is searched 64 probes at a time.
  auto first_info = [&]() {
    const int32_t* blk0 = reinterpret_cast<const int32_t*>(p.dec_seqs) + 6;  // record stride: 8 ints
    int lo = 0, hi = n_dseq;  // blk0[lo] <= ws (blk0[0] = 0); the sequence is in [lo, hi)
    while (hi - lo > 64) {
      const int step = (hi - lo + 63) / 64;
      const int j = lo + lane * step;
      const int k = __popcll(__ballot(j < hi && blk0[(int64_t)j * 8] <= ws));  // lane 0 probes lo
      hi = min(hi, lo + k * step);
      lo += (k - 1) * step;
    }
    const int j = lo + lane;
    const int i = uni(lo + __popcll(__ballot(j < hi && blk0[(int64_t)j * 8] <= ws)) - 1);
    Info I;
    load_seq(I, i);
    if (I.nb <= 0) {  // only if the table were inconsistent
      I.valid = false;
      return I;
    }
    I.h = (ws - I.b0) / I.nb;
    I.b0 += I.h * I.nb;
    set_part(I);
    return I;
  };
  // The part after I in the range (invalid once I reaches its end).
  auto next_info = [&](const Info& I) {
    Info N = I;
    N.valid = false;
    if (!I.valid || I.b0 + I.nb >= we) return N;
    if (I.h + 1 < p.Hkv) {
      N.h = I.h + 1;
      N.b0 = I.b0 + I.nb;
    } else {
      // the next decode sequence with blocks (blocks remain in the range)
      int i = I.i + 1;
      if (i >= n_dseq) return N;
      load_seq(N, i);
      while (N.nb <= 0 && i + 1 < n_dseq) load_seq(N, ++i);
    }
    set_part(N);
    return N;
  };
  // 16-key DMA steps of a part: whole compute steps of BK keys (the last may
  // run past c_hi and is masked); an empty key range (only outside the data
  // preconditions) still takes one fully masked compute step, so that the
  // load and compute sides always agree on the step count
  auto item_steps = [](const Info& I) { return CS * max(1, (I.c_hi - I.c_lo + BK - 1) / BK); };

  // Q rows of a part, 16 x D bf16, straight into the wave's Q slot (row r =
  // packed row r of the sequence; rows past nrows re-read row 0 and are
  // ignored).
  auto dma_q = [&](const Info& I) {
    constexpr int QROW = 2 * D, QRPI = 1024 / QROW, QNI = 16 / QRPI;
    const Seq m = seq_of(I);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier reads of the slot are done
#pragma unroll
    for (int j = 0; j < QNI; ++j) {
      const int r = QRPI * j + (lane * 16) / QROW;
      const int prow = r < m.nrows ? r : 0;
      const int t = prow / p.G;
      const int qh = I.h * p.G + (prow - t * p.G);
      const uint8_t* src =
          reinterpret_cast<const uint8_t*>(p.q + ((int64_t)(m.q0 + t) * p.Hq + qh) * D) + (lane * 16) % QROW;
      dma16(src, qs_lds + 1024u * j);
    }
  };
  // Q^T operand from the Q slot: lane (row col, group g) takes k-slot i
  auto read_q = [&](int nrows, bf16x8 (&qb)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qs + col * D + slot_d<FP8>(i, g));
      qb[i] = col < nrows ? v : bf16x8{};
    }
  };
  // fp8 and f32 q: the same operand straight from global memory (row col of
  // the part; rows past nrows re-read row 0 and are zeroed); an f32 q also
  // gives its lo part (split_q8)
  auto load_q = [&](const Info& I, bf16x8 (&qr)[NI], bf16x8 (&qlr)[Q32 ? NI : 1]) {
    const Seq m = seq_of(I);
    const int prow = col < m.nrows ? col : 0;
    const int t = prow / p.G;
    const int qh = I.h * p.G + (prow - t * p.G);
    const int64_t e = ((int64_t)(m.q0 + t) * p.Hq + qh) * D;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (Q32) {
        const float* qp = reinterpret_cast<const float*>(p.q) + e + slot_d<FP8>(i, g);
        bf16x8 hi, lo;
        split_q8(*reinterpret_cast<const f32x4*>(qp), *reinterpret_cast<const f32x4*>(qp + 4), hi, lo);
        qr[i] = col < m.nrows ? hi : bf16x8{};
        qlr[i] = col < m.nrows ? lo : bf16x8{};
      } else {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(p.q + e + slot_d<FP8>(i, g));
        qr[i] = col < m.nrows ? v : bf16x8{};
      }
    }
  };

  // ---- loader: the part whose steps are being loaded ----
  struct Loader {
    int s;      // sequence (its page-table row)
    int hoff;   // byte offset of combined head 2h in a slot
    int lp, sl, key;  // next block: logical page, slot in the page, first key
    int left;   // steps not yet loaded
    int pg;     // physical page of the next block (scalar-loaded ahead)
  };
  auto page_id = [&](int s, int lp) { return sload(p.page_indices + (int64_t)s * p.pps + min(lp, p.pps - 1)); };
  auto loader_for = [&](const Info& I) {
    Loader L;
    L.s = seq_of(I).s;
    L.hoff = 2 * I.h * D * EB;
    L.lp = I.c_lo / p.page;
    L.sl = I.c_lo - L.lp * p.page;
    L.key = I.c_lo;
    L.left = item_steps(I);
    L.pg = page_id(L.s, L.lp);
    return L;
  };
  // Issues the DMA of L's next step into ring slot `slot`, then moves L on.
  auto issue_step = [&](Loader& L, int slot) {
    const int phys = min(max(L.pg, 0), p.P - 1);
    const uint8_t* base = uniform_ptr(p.kv + ((int64_t)phys * p.page + L.sl) * key_stride + L.hoff);
    const uint32_t dst = (uint32_t)uni((int)(ring_lds + (uint32_t)(slot * STAGE)));
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int j = 0; j < NDR; ++j) dma16_sbase(base, voff[r][j], dst + r * REGION + 1024 * j);
    --L.left;
    if (L.left > 0) {
      L.key += kDecStepKeys;
      L.sl += kDecStepKeys;
      if (L.sl >= p.page) {
        L.sl = 0;
        ++L.lp;
        L.pg = page_id(L.s, L.lp);
      }
    }
  };

  // ---- compute state of the current part ----
  Info C;
  Seq cs;  // its sequence
  bf16x8 qb[NI];
  bf16x8 ql[Q32 ? NI : 1];  // f32 q: the lo part of the Q operand
  float m_ref, lsum;
  f32x4 o[ND];
  int steps_done, n_steps;
  bool rvalid;
  int tok, qh, pos, pos_lo, pos_hi, vis_hi;
  auto begin_item = [&]() {
    m_ref = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    steps_done = 0;
    n_steps = item_steps(C);
    // column `col` of S^T / O^T is packed row col of the sequence
    rvalid = col < cs.nrows;
    const int t = col / p.G;
    qh = C.h * p.G + (col - t * p.G);
    tok = cs.q0 + t;
    pos = cs.kvl - cs.ql + t;
    pos_lo = cs.kvl - cs.ql;
    pos_hi = cs.kvl - cs.ql + (max(cs.nrows, 1) - 1) / p.G;
    vis_hi = min(C.c_hi, cs.kvl);
  };

  // Operands of one compute step, read out of its ring slots so that they
  // can be refilled while the step is computed (bf16: V^T here too; one-byte
  // K/V: V^T is read from the slots during the step).
  struct Ops {
    u32x4 k[CS][NLD];             // K pieces (raw bf16 or one-byte codes) of each 16-key slot
    bf16x4 vt[FP8 ? 1 : ND];      // bf16: V^T operand of each 16-row block of O^T
  };
  // V^T operand layout (ds_read_b64_tr_b16): lane x of group g reads
  // V[4g + x/4][16 d + 4 (x%4) .. + 3] and receives V^T[16 d + x][4g .. 4g + 3]
  const int vkey = 4 * g + (col >> 2);
  const int q4 = col & 3;
  // one-byte V^T (ds_read_b64_tr_b8, measured on gfx950: within a 16-lane
  // group, lane 8q + b receives byte b of the 8-byte pieces loaded by lanes
  // q, q + 2, ..., q + 14): lane x of group g loads 8 bytes (d = 16 d0 + 8 (x%2)
  // .. + 7) of key row j = x/2 of the group's eight keys, so that lane x
  // receives V^T[16 d0 + x][those eight keys]. The eight keys of group g are
  // the four whose scores it holds in each 16-key half: keys 4g .. 4g + 3 of
  // the first slot, then of the second.
  const int tr_key = 4 * g + ((col >> 1) & 3);  // key row within its slot
  const int tr_half = col >> 3;                 // 0: first slot, 1: second
  const int tr_byte = 8 * (col & 1);
  auto read_ops = [&](int n, Ops& op) {
#pragma unroll
    for (int c = 0; c < CS; ++c) {
      const char* kr = ring + ((n + c) % NST) * STAGE;
      if constexpr (FP8) {
        // key col's segment: K chunks 0 .. RB/16 - 1, then V
        const char* seg = kr + col * (2 * RB);
#pragma unroll
        for (int j = 0; j < NLD; ++j)
          op.k[c][j] = *reinterpret_cast<const u32x4*>(seg + 16 * ((4 * j + g) ^ dswz_kv<D>(col)));
      } else {
        const char* vr = kr + REGION;
#pragma unroll
        for (int j = 0; j < NLD; ++j)
          op.k[c][j] = *reinterpret_cast<const u32x4*>(kr + col * RB + 16 * ((4 * j + g) ^ dswz_k<D, FP8>(col)));
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const int chunk = 2 * d + (q4 >> 1);
          op.vt[d] = lds_read_tr16(
              reinterpret_cast<const __bf16*>(vr + vkey * RB + 16 * (chunk ^ dswz_v<D, FP8>(vkey)) + 8 * (q4 & 1)));
        }
      }
    }
    if constexpr (!FP8) {
      // every read of the slot has completed: it may be refilled
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  };

  // One compute step: keys [kb, kb + 16 CS), its rows in the ring slots of
  // DMA steps n .. n + CS - 1. Lane (col, g) holds the scores of keys
  // kb + 16 c + 4g + j (c < CS, j < 4) of packed row col.
  auto compute_step = [&](const Ops& op, int kb_in, int n) {
    const int kb = __builtin_amdgcn_readfirstlane(kb_in);  // wave-uniform: scalar mask tests
    constexpr int NS = 4 * CS;  // scores per lane
    float sc[NS];
#pragma unroll
    for (int c = 0; c < CS; ++c) {
      bf16x8 ka[NI];
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        if constexpr (FP8) {
          ka[2 * j] = fp8x8_to_16<KVT, F16>(u32x2{op.k[c][j][0], op.k[c][j][1]});
          ka[2 * j + 1] = fp8x8_to_16<KVT, F16>(u32x2{op.k[c][j][2], op.k[c][j][3]});
        } else {
          ka[j] = __builtin_bit_cast(bf16x8, op.k[c][j]);
        }
      }
      // S^T of the slot: lane (col, g) gets keys kb + 16c + 4g + j of row `col`
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NI; ++i) s4 = mfma16x16x32<F16>(ka[i], qb[i], s4);
      if constexpr (Q32) {
#pragma unroll
        for (int i = 0; i < NI; ++i) s4 = mfma16x16x32<F16>(ka[i], ql[i], s4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[4 * c + j] = s4[j];
    }
    auto key_of = [&](int e) { return kb + 16 * (e >> 2) + 4 * g + (e & 3); };
    // does the step hold a key that some row of the unit cannot see?
    const bool need_mask = kb + 16 * CS > vis_hi || (p.is_causal && kb + 16 * CS - 1 > pos_lo) ||
                           (p.window > 0 && kb <= pos_hi - p.window);
    // the scores' chains first (independent, so their latencies overlap),
    // then the masks in one uniform branch
#pragma unroll
    for (int e = 0; e < NS; ++e) {
      if constexpr (CAP) {
        sc[e] = cap_b2(sc[e]);
      } else {
        sc[e] = sc[e] * sc_mul;
      }
    }
    if (need_mask) {
#pragma unroll
      for (int e = 0; e < NS; ++e) {
        const int key = key_of(e);
        bool vis = key < vis_hi;
        if (p.is_causal) vis = vis && key <= pos;
        if (p.window > 0) vis = vis && key > pos - p.window;
        sc[e] = vis ? sc[e] : -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int e = 1; e < NS; ++e) mx = fmaxf(mx, sc[e]);
    mx = wave_max_xor16_32(mx);
    // lazily moved reference maximum
    if (__any(mx > m_ref + kDecSlack)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < ND; ++d) o[d] *= alpha;
    }
    const float negm = m_ref == -INFINITY ? 0.f : -m_ref;
    float pj[NS];
#pragma unroll
    for (int e = 0; e < NS; ++e) {
      pj[e] = fast_exp2(sc[e] + negm);
      lsum += pj[e];
    }

    if constexpr (FP8) {
      // O^T += V^T P^T over the 32 keys with v_mfma_f32_16x16x32: P^T's k-slots
      // of lane group g are exactly its eight scores; V^T comes transposed out
      // of the two slots and is widened in registers (keys at or past vis_hi
      // read as 0: 0 * NaN would poison the sum)
      const bf16x8 pb = __builtin_bit_cast(
          bf16x8, u32x4{pack2<F16>(pj[0], pj[1]), pack2<F16>(pj[2], pj[3]), pack2<F16>(pj[4], pj[5]),
                        pack2<F16>(pj[6], pj[7])});
      const char* tr_row = ring + ((n + tr_half) % NST) * STAGE + tr_key * (2 * RB) + tr_byte;
      const bool partial = kb + 32 > vis_hi;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        typedef int i32x2 __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
        const u32x2 raw = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                       (lds_i32x2*)(tr_row + 16 * ((RB / 16 + d) ^ dswz_kv<D>(tr_key)))));
        bf16x8 a = fp8x8_to_16<KVT, F16>(raw);
        if (partial) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (key_of(e) >= vis_hi) a[e] = (__bf16)0.f;
        }
        o[d] = mfma16x16x32<F16>(a, pb, o[d]);
      }
    } else {
      const bf16x4 pb = __builtin_bit_cast(bf16x4, u32x2{pack2<F16>(pj[0], pj[1]), pack2<F16>(pj[2], pj[3])});
      // V of keys at or past vis_hi reads as 0 (0 * NaN would poison the sum)
      const bool partial = kb + 16 > vis_hi;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        bf16x4 a = op.vt[d];
        if (partial) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            if (kb + 4 * g + kk >= vis_hi) a[kk] = (__bf16)0.f;
        }
        o[d] = mfma16x16x16<F16>(a, pb, o[d]);
      }
    }
  };

  // Result of the current part: bf16 out + lse, or an f32 partial + lse.
  auto finish_item = [&]() {
    const float l_row = wave_sum_xor16_32(lsum);
    float inv, lse_v;
    if (!is_split(C)) {
      // the whole row: the sink (if any) joins it here
      row_final(m_ref, l_row, p.v_scale, p.sinks ? p.sinks + qh : nullptr, inv, lse_v);
    } else {
      // a chunk's partial; the combine kernel adds the sink
      row_final(m_ref, l_row, p.v_scale, nullptr, inv, lse_v);
    }
    if (!rvalid) return;
    if (!is_split(C)) {
      const int64_t e = ((int64_t)tok * p.Hq + qh) * D + 4 * g;
#pragma unroll
      for (int d = 0; d < ND; ++d)
        store_out4<F16, Q32>(p.out, e + 16 * d, o[d][0] * inv, o[d][1] * inv, o[d][2] * inv, o[d][3] * inv);
      if (g == 0 && p.lse) p.lse[(int64_t)tok * p.Hq + qh] = lse_v;
    } else {
      const int slot = slot_of(C);
      float* pp = p.dec_part + ((int64_t)slot * kDecRows + col) * D;
#pragma unroll
      for (int d = 0; d < ND; ++d) *reinterpret_cast<f32x4*>(pp + 16 * d + 4 * g) = o[d] * inv;
      if (g == 0) p.dec_plse[(int64_t)slot * kDecRows + col] = lse_v;
    }
  };

  // ---- the wave's parts, one continuous pipeline ----
  if (w >= W || w >= p.dec_waves || n_dseq <= 0 || sk.Tb <= 0) return;
  ws = uni(sk.start(w));
  we = uni(sk.start(w + 1));
  C = first_info();
  if (!C.valid) return;
  cs = seq_of(C);
  Info Cn = next_info(C);  // the compute side's next part
  bf16x8 qn[QREG ? NI : 1];        // fp8, f32 q: the next part's Q operand, loaded ahead
  bf16x8 qnl[Q32 ? NI : 1];        // f32 q: its lo part
  if constexpr (QREG) {
    load_q(C, qb, ql);
    if (Cn.valid) load_q(Cn, qn, qnl);
  } else {
    dma_q(C);
    wait_vmcnt<0>();
    wave_sync();
    read_q(cs.nrows, qb);
    if (Cn.valid) dma_q(Cn);
  }
  int q_age = 0;  // steps computed since the Q slot's DMA was issued
  begin_item();

  Loader L = loader_for(C);
  Info Ln = Cn;          // the load side's next part
  bool loading = true;   // the load side still has steps to issue
  // Moves the load side to its next step: the same part, or the next of the wave.
  auto loader_next = [&]() {
    if (L.left > 0) return;
    if (Ln.valid) {
      L = loader_for(Ln);
      Ln = next_info(Ln);
    } else {
      loading = false;
    }
  };

  // prologue: NST steps in flight
  int ahead = 0;  // steps issued beyond the one being computed
#pragma unroll
  for (int k = 0; k < NST; ++k) {
    if (loading) {
      issue_step(L, k);
      ++ahead;
      loader_next();
    }
  }
  --ahead;  // the first issued step is the one computed first
  Ops op;
  for (int n = 0;; n += CS) {
    // this compute step's DMA steps n .. n + CS - 1 have landed once at most
    // `ahead - (CS - 1)` later steps are in flight
    if (ahead == NST - 1) {
      wait_vmcnt<(NST - CS) * NDMA>();
    } else {
      wait_vmcnt<0>();
    }
    read_ops(n, op);
    // refill the slot just read (one-byte K/V: once the step's transposed V
    // reads are done as well)
    if (!FP8 && loading) {
      issue_step(L, n % NST);
      ++ahead;
      loader_next();
    }
    compute_step(op, C.c_lo + steps_done * kDecStepKeys, n);
    if (FP8 && loading) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int c = 0; c < CS; ++c) {
        if (loading) {
          issue_step(L, (n + c) % NST);
          ++ahead;
          loader_next();
        }
      }
    }
    steps_done += CS;
    q_age += CS;
    ahead -= CS;
    if (steps_done == n_steps) {
      finish_item();
      if (!Cn.valid) return;  // the wave's range is done
      C = Cn;
      cs = seq_of(C);
      Cn = next_info(C);
      if constexpr (QREG) {
#pragma unroll
        for (int i = 0; i < NI; ++i) qb[i] = qn[i];
        if constexpr (Q32) {
#pragma unroll
          for (int i = 0; i < NI; ++i) ql[i] = qnl[i];
        }
        if (Cn.valid) load_q(Cn, qn, qnl);
      } else {
        // the Q slot's DMA is complete once a wait above covered a step
        // issued after it (NST + 1 steps later); for short parts wait here
        if (q_age <= NST) wait_vmcnt<0>();
        wave_sync();
        read_q(cs.nrows, qb);
        if (Cn.valid) {
          dma_q(Cn);
          q_age = 0;
        }
      }
      begin_item();
    }
  }
}

// Merges the split decode-class units once every decode wave is done: one
// wave per unit (decode sequence u / Hkv, kv head u % Hkv), the parts'
// partials combined by merge_unit in block order; a unit with no key to see
// (and so no block) gets out = 0 and lse = -inf.
template <int D, bool F16, bool Q32 = false>
__global__ __launch_bounds__(kDecWavesPerBlock * 64) void combine_kernel(Params p) {
  __shared__ float stat[kDecWavesPerBlock][2 * kDecRows];
  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);  // wave-uniform: the unit's record comes by scalar loads
  const int n_units = uni(p.hdr->n_dec_units);
  const StreamK sk = StreamK::make(uni(p.hdr->dec_blocks), uni(p.hdr->pad0[0]));
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  for (int u = blockIdx.x * kDecWavesPerBlock + wave; u < n_units; u += gridDim.x * kDecWavesPerBlock) {
    const int i = u / p.Hkv;
    const int32_t* d = reinterpret_cast<const int32_t*>(p.dec_seqs + i);
    Unit U;
    U.seq = uni(d[0]);
    U.kv_head = u - i * p.Hkv;
    U.row0 = 0;
    U.nrows = uni(d[2]) * p.G;
    U.kv_lo = uni(d[4]);
    U.kv_hi = uni(d[5]);
    const int nb = uni(d[7]);
    if (nb <= 0) {
      // no visible key (only outside the data preconditions): out 0, lse -inf
      // (with a sink: lse = the sink, its own term)
      int q0, ql;
      seq_tokens(p, U.seq, q0, ql);
      for (int e = lane; e < U.nrows * (D / 4); e += 64) {
        const int prow = e / (D / 4);
        const int t = prow / p.G;
        const int qh = U.kv_head * p.G + (prow - t * p.G);
        store_out4<F16, Q32>(p.out, ((int64_t)(q0 + t) * p.Hq + qh) * D + 4 * (e % (D / 4)), 0.f, 0.f, 0.f, 0.f);
        if (p.lse && e % (D / 4) == 0) p.lse[(int64_t)(q0 + t) * p.Hq + qh] = p.sinks ? p.sinks[qh] : -INFINITY;
      }
      continue;
    }
    const int b0 = uni(d[6]) + U.kv_head * nb;
    const int f = sk.wave_of(b0), l = sk.wave_of(b0 + nb - 1);
    if (f == l) continue;  // one part: its wave wrote the rows
    U.nch = l - f + 1;
    U.item0 = 0;
    // part c ran on wave f + c: the first in slot 2f + 1, the others in 2(f + c)
    auto slot = [&](int c) { return c == 0 ? 2 * f + 1 : 2 * (f + c); };
    if (U.nch <= 4) {
      merge_unit_small<D, F16, Q32, 4>(p, U, p.dec_part, p.dec_plse, kDecRows, slot, lane, 64);
    } else {
      merge_unit<D, F16, Q32, true>(p, U, p.dec_part, p.dec_plse, kDecRows, slot, lane, 64, stat[wave], wave_sync);
      wave_sync();
    }
  }
}

}  // namespace rpa
