/*
 * rpa.h — C ABI of the MI355X (gfx950) ragged paged GQA attention library.
 *
 * The operation is the one defined by the ragged paged attention kernel page
 * (zml platforms/tpu/ragged_paged.zig): for every sequence s < num_seqs, its
 * q_len = cu_q_lens[s+1] - cu_q_lens[s] query tokens attend, head by head,
 * to the kv_lens[s] keys and values that the page table gathers from a
 * paged cache. In detail (`Cfg`, `run` and `flashAttention` on that page):
 *
 *   - key j of sequence s is slot j % page_size of physical page
 *     page_indices[s, j / page_size]; combined head 2h of that slot holds
 *     K of kv head h and combined head 2h+1 holds V (`stridedLoadKv`);
 *   - q head n reads kv head n / (num_q_heads / num_kv_heads);
 *   - query token i of sequence s sits at key position kv_len - q_len + i;
 *   - score = (q . K * k_scale) * sm_scale; if soft_cap > 0 the score becomes
 *     soft_cap * tanh(score / soft_cap);
 *   - with is_causal a key at position j is hidden when j > the query's
 *     position p; with sliding_window w > 0 it is also hidden when
 *     p - w >= j;
 *   - out = softmax over the visible keys of the scores, times V * v_scale;
 *   - lse (not on the page; an output of this library) = natural log of the
 *     sum over visible keys of exp(score).
 *
 * All data pointers are DEVICE pointers, owned by the caller, and must stay
 * valid until the work enqueued on `stream` has finished. Nothing in this
 * library allocates device memory on the call path, synchronises, or keeps
 * state between calls beyond cached device properties (and the contents of
 * rpa_forward_noalloc's scratch array). `stream` is a
 * hipStream_t passed as void* (NULL = the null stream).
 */
#ifndef RPA_H
#define RPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types (the page's `Cfg` q_dtype / kv_dtype). */
typedef enum {
  RPA_DTYPE_BF16 = 0,       /* bfloat16 */
  RPA_DTYPE_FP8_E4M3FN = 1, /* OCP FP8 E4M3 (finite, NaN = S.1111.111) */
  RPA_DTYPE_FP8_E5M2 = 2,   /* OCP FP8 E5M2 (bias 15, infinities and NaN at exponent 31) */
  RPA_DTYPE_F16 = 3,        /* IEEE binary16 */
  RPA_DTYPE_INT8 = 4,       /* signed 8-bit integer codes (K/V only; value = code * scale) */
  RPA_DTYPE_F32 = 5,        /* IEEE binary32 (q and out only; the page's packing-1 q type) */
} rpa_dtype;

typedef enum {
  RPA_OK = 0,
  RPA_ERR_INVALID_ARGUMENT = 1,   /* bad shape, scale, window or null pointer */
  RPA_ERR_UNSUPPORTED = 2,        /* valid but not built: head_dim, page_size, dtype */
  RPA_ERR_WORKSPACE_TOO_SMALL = 3,
  RPA_ERR_HIP = 4,                /* a HIP runtime call or kernel launch failed */
  RPA_ERR_METADATA = 5,           /* rpa_check_metadata found a broken precondition */
} rpa_status;

/*
 * Shapes and numeric knobs: the page's `Cfg` (shape fields, dtypes, sm_scale,
 * soft_cap, k_scale, v_scale, is_causal, sliding_window). Block-size tuning
 * knobs of the page are not part of this ABI; tiling is internal.
 */
typedef struct rpa_config {
  int32_t num_q_tokens;    /* rows of q, out and lse (>= cu_q_lens[num_seqs]) */
  int32_t num_q_heads;     /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;    /* Hkv; kv_pages holds 2*Hkv combined heads */
  int32_t head_dim;        /* D: 64, 128 or 256 */
  int32_t total_num_pages; /* P: first dimension of kv_pages */
  int32_t page_size;       /* keys per page: a multiple of 16, at most 1024 */
  int32_t max_num_seqs;    /* rows of page_indices and kv_lens */
  int32_t pages_per_seq;   /* columns of page_indices */
  int32_t q_dtype;         /* rpa_dtype of q and out: RPA_DTYPE_BF16, RPA_DTYPE_F16 or RPA_DTYPE_F32 */
  int32_t kv_dtype;        /* rpa_dtype: q_dtype (RPA_DTYPE_BF16 with an f32 q), RPA_DTYPE_FP8_E4M3FN,
                              RPA_DTYPE_FP8_E5M2 or RPA_DTYPE_INT8 */
  float sm_scale;          /* score scale, finite */
  float soft_cap;          /* > 0: cap on; 0: off */
  float k_scale;           /* dequant factor of K; 1.0f for none */
  float v_scale;           /* dequant factor of V; 1.0f for none */
  int32_t is_causal;       /* 0 or 1 */
  int32_t sliding_window;  /* > 0: window in keys; 0: off */
} rpa_config;

/*
 * Bytes of device workspace rpa_forward needs for `cfg` on the current HIP
 * device (the tile plan, work counters and split-KV partial results). The
 * size depends only on cfg and the device's compute-unit count.
 * Errors: RPA_ERR_INVALID_ARGUMENT / RPA_ERR_UNSUPPORTED as rpa_forward.
 */
rpa_status rpa_workspace_bytes(const rpa_config* cfg, size_t* bytes);

/*
 * Ragged paged attention forward pass (the page's `run` operands):
 *   q            [num_q_tokens, num_q_heads, head_dim]                 q_dtype
 *   kv_pages     [total_num_pages, page_size, 2*num_kv_heads, head_dim] kv_dtype
 *   kv_lens      [max_num_seqs] int32
 *   page_indices [max_num_seqs, pages_per_seq] int32
 *   cu_q_lens    [max_num_seqs + 1] int32, non-decreasing
 *   num_seqs     [1] int32, device-resident
 *   out          [num_q_tokens, num_q_heads, head_dim]                 q_dtype
 *   lse          [num_q_tokens, num_q_heads] float32, or NULL
 *   workspace    >= rpa_workspace_bytes(cfg) bytes, 256-byte aligned
 * All arrays are dense, row-major, in device memory; out and lse must not
 * alias any input. Rows of tokens >= cu_q_lens[num_seqs] are left untouched.
 * An f32 q (16-byte aligned) is computed on the bf16 path with each element
 * carried as a bf16 pair hi + lo (within 2^-17 of it, relative); scores take
 * both, and out is written in f32. P (the exponentiated scores) is rounded to
 * bf16 for the P.V product as with a bf16 q.
 *
 * Data preconditions (not checked here; rpa_check_metadata checks host copies):
 * 0 <= q_len <= kv_len <= pages_per_seq * page_size, page ids in
 * [0, total_num_pages), num_seqs <= max_num_seqs, cu_q_lens[num_seqs] <=
 * num_q_tokens. Broken preconditions give unspecified values in the affected
 * rows but no out-of-bounds access: page ids are clamped, the page count is
 * clamped to pages_per_seq and token ranges to num_q_tokens. A row with no
 * visible key gets out = 0 and lse = -inf.
 *
 * The call validates cfg and pointers on the host, then enqueues on `stream`
 * and returns: the plan; the tiles of both classes in one launch, whose
 * workgroups run decode-class or prefill-class tiles side by side; and the
 * merge of split decode units (a split prefill unit is merged by whichever
 * workgroup finishes its last key chunk).
 * Errors: RPA_ERR_INVALID_ARGUMENT, RPA_ERR_UNSUPPORTED,
 * RPA_ERR_WORKSPACE_TOO_SMALL (nothing enqueued), RPA_ERR_HIP (launch failed).
 */
rpa_status rpa_forward(const rpa_config* cfg, const void* q, const void* kv_pages, const int32_t* kv_lens,
                       const int32_t* page_indices, const int32_t* cu_q_lens, const int32_t* num_seqs, void* out,
                       float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * rpa_forward with attention sinks: one logit per q head that joins each of
 * that head's rows' softmax and carries no value (gpt-oss's attention sinks;
 * the spatial-compiler page's `flat_softmax_rows_at` with `sinks`): the row's
 * maximum starts from it and exp(sink - max) joins the denominator, so
 *   out = sum_j e^(s_j) v_j / (sum_j e^(s_j) + e^sink),
 *   lse = log(sum_j e^(s_j) + e^sink),
 * with s_j the scores after scale, soft-cap and masks (a row with no visible
 * key: out = 0, lse = sink).
 *   sinks   [num_q_heads] float32 in device memory, finite or -inf; NULL: none
 *           (exactly rpa_forward).
 * Every other argument, precondition and error is rpa_forward's.
 */
rpa_status rpa_forward_sinks(const rpa_config* cfg, const void* q, const void* kv_pages, const int32_t* kv_lens,
                             const int32_t* page_indices, const int32_t* cu_q_lens, const int32_t* num_seqs,
                             const float* sinks, void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * rpa_forward_sinks without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The workspace is the library's own
 * scratch array: a static device array of 256 MiB, one copy per GPU, created with the library's code on that GPU
 * and held until the process ends; its address is looked up once per device
 * (hipGetSymbolAddress) on the first call. The call allocates nothing and
 * never synchronises. `sinks` may be NULL (then exactly rpa_forward).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or host threads, without ordering between them)
 * race on it and give undefined results; calls ordered on one stream are
 * safe (each call's planning kernel rewrites everything the others read).
 * Errors: those of rpa_forward_sinks, and RPA_ERR_WORKSPACE_TOO_SMALL when
 * rpa_workspace_bytes(cfg) exceeds the array (nothing is enqueued).
 */
rpa_status rpa_forward_noalloc(const rpa_config* cfg, const void* q, const void* kv_pages, const int32_t* kv_lens,
                               const int32_t* page_indices, const int32_t* cu_q_lens, const int32_t* num_seqs,
                               const float* sinks, void* out, float* lse, void* stream);

/*
 * KV-cache append: writes every query token's new K and V rows into the
 * paged cache, in place, before attention reads them. The pages read a cache
 * that already holds each query token's own key; this is the write that puts
 * it there, by the placement the ragged paged attention kernel page reads
 * with (`run` and the row ids of `flashAttention`): query token i of sequence
 * s (cu_q_lens[s] + i) stands at key position kv_len - q_len + i, which is
 * slot pos % page_size of page page_indices[s, pos / page_size]; K of kv head
 * h goes to combined head 2h, V to 2h+1 (`stridedLoadKv`).
 *   k_new, v_new [num_q_tokens, num_kv_heads, head_dim] q_dtype (bf16, f16 or f32)
 *   kv_pages     [total_num_pages, page_size, 2*num_kv_heads, head_dim]
 *                kv_dtype, updated in place
 *   kv_lens, page_indices, cu_q_lens, num_seqs: as rpa_forward (kv_lens
 *                already counts the new tokens)
 * Stored value: RN_f32(x / scale) with scale = k_scale for K and v_scale for
 * V (IEEE binary32 division), rounded to nearest even in kv_dtype; e4m3fn
 * saturates at +-448 and e5m2 at +-57344, bf16 and f16 overflow to +-inf; a
 * NaN input stores a NaN; int8 stores the nearest integer (ties to even)
 * saturated to [-128, 127], and 0 for NaN. With rows and cache of one 16-bit
 * type and both scales 1 this is a bit copy. Device pointers, owned by the
 * caller; k_new, v_new and kv_pages 16-byte aligned; k_new/v_new must not
 * overlap kv_pages. Tokens past cu_q_lens[num_seqs] and tokens whose position
 * or page id falls outside the table (a broken precondition) write nothing;
 * two tokens that map to one slot race. Enqueues one kernel on `stream`; no
 * workspace. Errors: RPA_ERR_INVALID_ARGUMENT (null or misaligned pointer,
 * bad cfg, a scale that is not > 0), RPA_ERR_UNSUPPORTED, RPA_ERR_HIP.
 */
rpa_status rpa_kv_append(const rpa_config* cfg, const void* k_new, const void* v_new, void* kv_pages,
                         const int32_t* kv_lens, const int32_t* page_indices, const int32_t* cu_q_lens,
                         const int32_t* num_seqs, void* stream);

/* Static description of a status code; never NULL. */
const char* rpa_status_string(rpa_status status);

/*
 * Host-side check of the data preconditions listed for rpa_forward, on HOST
 * copies of the metadata (kv_lens [max_num_seqs], page_indices
 * [max_num_seqs, pages_per_seq], cu_q_lens [max_num_seqs + 1]).
 * Returns RPA_OK or RPA_ERR_METADATA (or RPA_ERR_INVALID_ARGUMENT for a bad
 * cfg / null pointer). Touches no device.
 */
rpa_status rpa_check_metadata(const rpa_config* cfg, const int32_t* kv_lens, const int32_t* page_indices,
                              const int32_t* cu_q_lens, int32_t num_seqs);

/*
 * Plan inspection, for tests: runs only the planning kernel on `stream` into
 * `workspace`, then describes where the plan lives in it. The plan is a list
 * of prefill units (one sequence, one kv head, a run of packed query rows
 * row = token_in_seq * (Hq/Hkv) + g, and the key range those rows can see)
 * with their items (a unit and one key chunk of it), and a table of the
 * decode sequences; see rpa_plan_layout. Same errors as rpa_forward.
 */
rpa_status rpa_plan(const rpa_config* cfg, const int32_t* kv_lens, const int32_t* cu_q_lens,
                    const int32_t* num_seqs, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Byte offsets inside the workspace (host-only, no device access):
 *   offsets[0] header: int32[64] = {n_dec_units, n_pf_units, n_dec_seqs,
 *              n_pf_items, 0, pf_chunk, n_split_units, dec_blocks,
 *              dec_waves_used, pad[7], queue_base[8], queue_count[8],
 *              queue_next[8], pad[24]}
 *              (n_split_units counts prefill units with more than one item;
 *              n_dec_units = n_dec_seqs * Hkv; dec_blocks is the number of
 *              16-key blocks (32 for one-byte K/V) of all decode units, split
 *              over the first dec_waves_used decode waves, at least 1 and at
 *              most min(dec_waves, dec_blocks): min(V, dec_blocks) with V
 *              whole 4-wave workgroups, half of dec_waves for a batch with no
 *              prefill work where two decode workgroups fit on a compute
 *              unit (else all of them), and for a batch with prefill work a
 *              quarter when its estimated prefill time is at least half its
 *              decode time, else half; the prefill items are dealt into 8
 *              queues, one per XCD, by (sequence, kv head), the heaviest
 *              first and back and forth over the queues; a queue lists the
 *              units' other chunks before their last ones, those by size;
 *              queue x is queue_count[x] entries of the queue list from
 *              queue_base[x] = x * max_pf_items on)
 *   offsets[1] decode sequences int32[max_num_seqs][8]
 *   offsets[2] prefill units    int32[max_pf_units][8]
 *   offsets[3] 0 (reserved)
 *   offsets[4] prefill items    int32[max_pf_items][16]
 *   offsets[5] queue list       int32[8][max_pf_items] (prefill item indices)
 *   offsets[6], offsets[7] 0 (reserved)
 * A prefill unit is {seq, kv_head, row0, nrows, kv_lo, kv_hi, nch, item0}. A
 * prefill item is {unit, chunk, the unit's 8 ints, q0, ql, kv_len, 3 pad}
 * (the sequence's first query token, query tokens and kv length, clamped),
 * covering keys [kv_lo + chunk*C, min(kv_hi, kv_lo + (chunk+1)*C)) with
 * C = pf_chunk. A decode sequence
 * record is {seq, q0, q_len, kv_len, kv_lo, kv_hi, blk0, nb}, one per
 * sequence with 1 <= q_len * Hq/Hkv <= 16, in sequence order: its units are
 * (seq, h) for every kv head h, all q_len * Hq/Hkv rows, keys [kv_lo, kv_hi)
 * in nb 16-key blocks, at blocks [blk0 + h*nb, blk0 + (h+1)*nb) of the
 * decode blocks laid end to end. Decode wave w runs blocks
 * [floor(dec_blocks*w/W), floor(dec_blocks*(w+1)/W)) with W = dec_waves_used.
 * limits = {max_dec_units, max_pf_units, decode partial slots (2 * dec_waves),
 * max_pf_items, dec_rows_max, pf_rows_max, dec_waves, 0}.
 */
rpa_status rpa_plan_layout(const rpa_config* cfg, size_t offsets[8], int32_t limits[8]);

/*
 * Debug helper for tests: decode n fp8 e4m3fn codes (device array) to
 * float32 (device array) with the same conversion the attention kernels use.
 */
rpa_status rpa_debug_decode_fp8(const uint8_t* codes, float* values, int32_t n, void* stream);

/*
 * Event timing for benchmarks. rpa_profile_begin(max_calls) makes the next
 * max_calls forward calls (process-wide) record HIP events on their stream
 * around their launches. rpa_profile_end waits for the last recorded event
 * and returns in kernel_ms[0..3] the elapsed milliseconds, summed over the
 * recorded calls, of: the plan; the tile launch (both classes); the merge of
 * split decode units; the whole call. It also returns how many calls were
 * recorded, then releases the events. Events are created in
 * rpa_profile_begin, never on the forward path.
 * Not meant for concurrent forward calls from several threads.
 * Errors: RPA_ERR_INVALID_ARGUMENT (bad count, nested begin, end without
 * begin), RPA_ERR_HIP.
 */
rpa_status rpa_profile_begin(int32_t max_calls);
rpa_status rpa_profile_end(float kernel_ms[4], int32_t* n_calls);

/*
 * Debugging switches, read from the environment once per process (a value
 * other than empty or "0" turns a switch on):
 *   RPA_TRACE  every forward call and every launch in it (and each
 *              rpa_kv_append) is a roctx range on the calling thread, for
 *              rocprofv3 --marker-trace: the launcher's counterpart of the
 *              kernel page's trace region around QK^T. The roctx library is
 *              opened when the first range is needed; without it the ranges
 *              are off. Results are unchanged.
 *   RPA_LOG    each forward call prints its plan to stderr (decode sequences,
 *              units, blocks and waves given work; prefill units, items,
 *              chunk size, split units and queue lengths). To read the plan
 *              it copies it back and waits for `stream`, so the call then
 *              synchronises; under stream capture it prints nothing.
 */

#ifdef __cplusplus
}
#endif

#endif /* RPA_H */
