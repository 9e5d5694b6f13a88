// Host-side logic of the C ABI that touches no device (see rpa_host.h) and
// the C entry points built on it alone: rpa_status_string and
// rpa_check_metadata.
#include "rpa_host.h"

#include <cmath>
#include <cstdint>

namespace rpa {
namespace host {

rpa_status validate(const rpa_config* c) {
  if (!c) return RPA_ERR_INVALID_ARGUMENT;
  if (c->num_q_tokens < 0 || c->num_q_heads < 1 || c->num_kv_heads < 1) return RPA_ERR_INVALID_ARGUMENT;
  if (c->num_q_heads % c->num_kv_heads != 0) return RPA_ERR_INVALID_ARGUMENT;
  if (c->total_num_pages < 1 || c->max_num_seqs < 1 || c->pages_per_seq < 1) return RPA_ERR_INVALID_ARGUMENT;
  if (c->page_size < 1 || c->head_dim < 1) return RPA_ERR_INVALID_ARGUMENT;
  if (c->is_causal != 0 && c->is_causal != 1) return RPA_ERR_INVALID_ARGUMENT;
  if (c->sliding_window < 0) return RPA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(c->sm_scale) || !std::isfinite(c->k_scale) || !std::isfinite(c->v_scale))
    return RPA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(c->soft_cap) || c->soft_cap < 0.f) return RPA_ERR_INVALID_ARGUMENT;
  if (c->max_num_seqs >= (1 << 28)) return RPA_ERR_INVALID_ARGUMENT;
  if ((int64_t)c->pages_per_seq * c->page_size > INT32_MAX) return RPA_ERR_INVALID_ARGUMENT;
  if ((int64_t)c->max_num_seqs * c->pages_per_seq > INT32_MAX) return RPA_ERR_INVALID_ARGUMENT;
  // 16 key slots of K|V rows must be addressable with 32-bit offsets
  if ((int64_t)c->num_kv_heads * c->head_dim > (1 << 24)) return RPA_ERR_INVALID_ARGUMENT;
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return RPA_ERR_UNSUPPORTED;
  if (c->page_size % 16 != 0 || c->page_size > 1024) return RPA_ERR_UNSUPPORTED;
  // q (and out) bf16, f16 or f32; K/V in the q type (bf16 with an f32 q), or
  // a one-byte kind
  if (c->q_dtype != RPA_DTYPE_BF16 && c->q_dtype != RPA_DTYPE_F16 && c->q_dtype != RPA_DTYPE_F32)
    return RPA_ERR_UNSUPPORTED;
  const int32_t kv16 = c->q_dtype == RPA_DTYPE_F32 ? RPA_DTYPE_BF16 : c->q_dtype;
  if (c->kv_dtype != kv16 && c->kv_dtype != RPA_DTYPE_FP8_E4M3FN && c->kv_dtype != RPA_DTYPE_FP8_E5M2 &&
      c->kv_dtype != RPA_DTYPE_INT8)
    return RPA_ERR_UNSUPPORTED;
  return RPA_OK;
}

namespace {

// Workgroups of the decode launch: one resident set (the stream-K split is
// made over exactly these waves).
template <int D, bool FP8>
int dec_grid(int cus) {
  const int per_cu = dec_wgs_per_cu<D, FP8>();
  return cus * (per_cu > 0 ? per_cu : 1);
}
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int dec_grid_for(const rpa_config* c, int cus) {
  const bool fp8 = c->kv_dtype == RPA_DTYPE_FP8_E4M3FN || c->kv_dtype == RPA_DTYPE_FP8_E5M2 ||
                   c->kv_dtype == RPA_DTYPE_INT8;
  switch (c->head_dim) {
    case 64: return fp8 ? dec_grid<64, true>(cus) : dec_grid<64, false>(cus);
    case 128: return fp8 ? dec_grid<128, true>(cus) : dec_grid<128, false>(cus);
    default: return fp8 ? dec_grid<256, true>(cus) : dec_grid<256, false>(cus);
  }
}

// The prefill class of `c` runs on the two-group tiles (prefill_pp_tiles in
// tiles_pp_kernel): 16-bit q with K/V in the q type.
bool uses_pp(const rpa_config* c) {
  return (c->q_dtype == RPA_DTYPE_BF16 || c->q_dtype == RPA_DTYPE_F16) && c->kv_dtype == c->q_dtype &&
         c->head_dim >= RPA_PP_MIN_D && c->head_dim <= RPA_PP_MAX_D;
}

// Sizes follow from cfg alone (see the item bound in the planning kernel:
// items <= units + target because every chunk size is >= total / target).
bool make_layout(const rpa_config* c, int cus, Layout* L) {
  const int64_t G = c->num_q_heads / c->num_kv_heads;
  const int64_t Hkv = c->num_kv_heads;
  const int64_t D = c->head_dim;
  const int64_t pf_rows = uses_pp(c) ? kPpRows : pf_rows_for(c->head_dim);
  const int64_t max_du = Hkv * c->max_num_seqs;
  const int64_t max_pu = Hkv * (((int64_t)c->num_q_tokens * G + pf_rows - 1) / pf_rows + c->max_num_seqs);
  const int64_t tgt_p = (int64_t)cus * RPA_PF_ITEMS_PER_CU;
  // stream-K: a decode wave writes at most two partials (slots 2w, 2w + 1),
  // and the decode blocks of all units must be countable in int32
  const int64_t dec_waves = (int64_t)dec_grid_for(c, cus) * kDecWavesPerBlock;
  const int64_t dec_slots = 2 * dec_waves;
  const int64_t max_dec_blocks = max_du * (((int64_t)c->pages_per_seq * c->page_size + kDecBlk16 - 1) / kDecBlk16);
  // prefill chunks are also capped at kPfMaxChunk keys
  const int64_t per_unit_cap = ((int64_t)c->pages_per_seq * c->page_size + kPfMaxChunk - 1) / kPfMaxChunk;
  const int64_t max_pi = max_pu + (tgt_p > max_pu * per_unit_cap ? tgt_p : max_pu * per_unit_cap);
  if (max_du >= (1 << 30) || max_pu >= (1 << 30) || dec_slots >= INT32_MAX || max_dec_blocks >= INT32_MAX ||
      max_pi >= INT32_MAX / kQueues)
    return false;
  size_t off = 0;
  L->hdr = off;   off = align256(off + sizeof(Header));
  L->dseq = off;  off = align256(off + sizeof(DecSeq) * (size_t)c->max_num_seqs);
  L->pu = off;    off = align256(off + sizeof(Unit) * (size_t)max_pu);
  L->pi = off;    off = align256(off + sizeof(Item) * (size_t)max_pi);
  L->qlist = off; off = align256(off + sizeof(int32_t) * kQueues * (size_t)max_pi);
  L->done = off;  off = align256(off + sizeof(int32_t) * (size_t)max_pu);
  L->dpart = off; off = align256(off + sizeof(float) * (size_t)dec_slots * kDecRows * D);
  L->dplse = off; off = align256(off + sizeof(float) * (size_t)dec_slots * kDecRows);
  L->ppart = off; off = align256(off + sizeof(float) * (size_t)max_pi * pf_rows * D);
  L->pplse = off; off = align256(off + sizeof(float) * (size_t)max_pi * pf_rows);
  L->total = off;
  L->max_du = (int32_t)max_du;
  L->max_pu = (int32_t)max_pu;
  L->dec_slots = (int32_t)dec_slots;
  L->max_pi = (int32_t)max_pi;
  L->tgt_p = (int32_t)tgt_p;
  L->pf_rows = (int32_t)pf_rows;
  L->dec_waves = (int32_t)dec_waves;
  return true;
}

}  // namespace host
}  // namespace rpa

using namespace rpa;
using namespace rpa::host;

extern "C" {

const char* rpa_status_string(rpa_status s) {
  switch (s) {
    case RPA_OK: return "ok";
    case RPA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case RPA_ERR_UNSUPPORTED: return "unsupported configuration";
    case RPA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RPA_ERR_HIP: return "HIP runtime error";
    case RPA_ERR_METADATA: return "metadata violates a precondition";
  }
  return "unknown status";
}

rpa_status rpa_check_metadata(const rpa_config* cfg, const int32_t* kv_lens, const int32_t* page_indices,
                              const int32_t* cu_q_lens, int32_t num_seqs) {
  rpa_status st = validate(cfg);
  if (st != RPA_OK) return st;
  if (!kv_lens || !page_indices || !cu_q_lens) return RPA_ERR_INVALID_ARGUMENT;
  if (num_seqs < 0 || num_seqs > cfg->max_num_seqs) return RPA_ERR_METADATA;
  if (cu_q_lens[0] < 0) return RPA_ERR_METADATA;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t ql = (int64_t)cu_q_lens[s + 1] - cu_q_lens[s];
    const int64_t kvl = kv_lens[s];
    if (ql < 0 || kvl < ql) return RPA_ERR_METADATA;
    if (kvl > (int64_t)cfg->pages_per_seq * cfg->page_size) return RPA_ERR_METADATA;
    const int64_t pages = (kvl + cfg->page_size - 1) / cfg->page_size;
    for (int64_t j = 0; j < pages; ++j) {
      const int32_t ph = page_indices[(int64_t)s * cfg->pages_per_seq + j];
      if (ph < 0 || ph >= cfg->total_num_pages) return RPA_ERR_METADATA;
    }
  }
  if (cu_q_lens[num_seqs] > cfg->num_q_tokens) return RPA_ERR_METADATA;
  return RPA_OK;
}

}  // extern "C"
