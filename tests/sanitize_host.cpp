// Host-side C-ABI logic under the address and undefined-behaviour sanitizers
// (built with g++ by tests/test_sanitize.py, no HIP): configuration checks
// over a grid of shapes and types, the workspace layout for every valid one
// on several compute-unit counts, the metadata check on random and broken
// tables, and the status strings. Exits non-zero on the first failed check;
// a sanitizer report aborts the run.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "rpa_host.h"

using namespace rpa;
using namespace rpa::host;

static int failures = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static rpa_config base_cfg() {
  rpa_config c;
  std::memset(&c, 0, sizeof c);
  c.num_q_tokens = 64;
  c.num_q_heads = 8;
  c.num_kv_heads = 2;
  c.head_dim = 128;
  c.total_num_pages = 64;
  c.page_size = 16;
  c.max_num_seqs = 8;
  c.pages_per_seq = 16;
  c.q_dtype = RPA_DTYPE_BF16;
  c.kv_dtype = RPA_DTYPE_BF16;
  c.sm_scale = 0.1f;
  c.k_scale = c.v_scale = 1.f;
  c.is_causal = 1;
  return c;
}

// every region of a layout 256-byte aligned, in order, inside the total
static void check_layout(const Layout& L, const rpa_config& c) {
  const size_t offs[] = {L.hdr, L.dseq, L.pu, L.pi, L.qlist, L.done, L.dpart, L.dplse, L.ppart, L.pplse};
  for (size_t i = 0; i < sizeof offs / sizeof offs[0]; ++i) {
    CHECK(offs[i] % 256 == 0);
    if (i) CHECK(offs[i] >= offs[i - 1]);
    CHECK(offs[i] <= L.total);
  }
  CHECK(L.max_du == c.num_kv_heads * c.max_num_seqs);
  CHECK(L.pf_rows == (uses_pp(&c) ? kPpRows : pf_rows_for(c.head_dim)));
  CHECK(L.ppart + sizeof(float) * (size_t)L.max_pi * L.pf_rows * c.head_dim <= L.pplse);
  CHECK(L.dseq + sizeof(DecSeq) * (size_t)c.max_num_seqs <= L.pu);
  CHECK(L.dec_slots == 2 * L.dec_waves);
  CHECK(L.dpart + sizeof(float) * (size_t)L.dec_slots * kDecRows * c.head_dim <= L.dplse);
}

int main() {
  // 1. validate over a grid; the layout of every accepted configuration
  const int dtypes[] = {RPA_DTYPE_BF16, RPA_DTYPE_FP8_E4M3FN, RPA_DTYPE_FP8_E5M2, RPA_DTYPE_F16, RPA_DTYPE_INT8,
                        RPA_DTYPE_F32, 6, -1};
  const int dims[] = {64, 96, 128, 256, 0};
  const int pages[] = {16, 24, 64, 1024, 2048, 0};
  const int cus_list[] = {1, 80, 256, 304};
  int accepted = 0;
  for (int qd : dtypes)
    for (int kd : dtypes)
      for (int D : dims)
        for (int pg : pages)
          for (int G : {1, 3, 16}) {
            rpa_config c = base_cfg();
            c.q_dtype = qd;
            c.kv_dtype = kd;
            c.head_dim = D;
            c.page_size = pg;
            c.num_q_heads = c.num_kv_heads * G;
            const rpa_status st = validate(&c);
            CHECK(st == RPA_OK || st == RPA_ERR_INVALID_ARGUMENT || st == RPA_ERR_UNSUPPORTED);
            if (st != RPA_OK) continue;
            ++accepted;
            for (int cus : cus_list) {
              Layout L;
              CHECK(make_layout(&c, cus, &L));
              check_layout(L, c);
            }
          }
  CHECK(accepted > 0);
  // invalid shapes and numbers are refused, never computed on
  {
    rpa_config c = base_cfg();
    c.num_q_heads = 7;  // not a multiple of num_kv_heads
    CHECK(validate(&c) == RPA_ERR_INVALID_ARGUMENT);
    c = base_cfg();
    c.sm_scale = std::strtof("nan", nullptr);
    CHECK(validate(&c) == RPA_ERR_INVALID_ARGUMENT);
    c = base_cfg();
    c.soft_cap = -1.f;
    CHECK(validate(&c) == RPA_ERR_INVALID_ARGUMENT);
    CHECK(validate(nullptr) == RPA_ERR_INVALID_ARGUMENT);
  }
  // extreme but accepted sizes: the layout either fits or says it overflows
  {
    rpa_config c = base_cfg();
    c.num_q_tokens = 1 << 30;
    c.max_num_seqs = (1 << 28) - 1;
    c.pages_per_seq = 8;
    c.total_num_pages = 1 << 30;
    if (validate(&c) == RPA_OK) {
      Layout L;
      if (make_layout(&c, 304, &L)) check_layout(L, c);
    }
    c = base_cfg();
    c.pages_per_seq = (int)((1u << 31) / 1024) - 1;
    c.page_size = 1024;
    c.max_num_seqs = 1;
    c.num_q_tokens = 1 << 20;
    if (validate(&c) == RPA_OK) {
      Layout L;
      if (make_layout(&c, 256, &L)) check_layout(L, c);
    }
  }

  // 2. the metadata check on random tables, then on broken ones
  std::mt19937 rng(1234);
  for (int trial = 0; trial < 2000; ++trial) {
    rpa_config c = base_cfg();
    c.max_num_seqs = 1 + (int)(rng() % 9);
    c.pages_per_seq = 1 + (int)(rng() % 6);
    c.total_num_pages = 1 + (int)(rng() % 40);
    c.num_q_tokens = (int)(rng() % 70);
    const int S = c.max_num_seqs;
    std::vector<int32_t> kvl(S), pi((size_t)S * c.pages_per_seq), cu(S + 1);
    const int n = (int)(rng() % (S + 2));  // may exceed max_num_seqs
    cu[0] = (int)(rng() % 3) - 1;          // may be negative
    for (int s = 0; s < S; ++s) {
      cu[s + 1] = cu[s] + (int)(rng() % 12) - 1;  // may decrease
      kvl[s] = (int)(rng() % (c.pages_per_seq * c.page_size + 8)) - 2;
    }
    for (auto& x : pi) x = (int)(rng() % (c.total_num_pages + 4)) - 2;
    const rpa_status st = rpa_check_metadata(&c, kvl.data(), pi.data(), cu.data(), n);
    CHECK(st == RPA_OK || st == RPA_ERR_METADATA);
    // an independent reading of the preconditions agrees
    bool ok = n >= 0 && n <= S && cu[0] >= 0;
    for (int s = 0; ok && s < n; ++s) {
      const long ql = (long)cu[s + 1] - cu[s];
      ok = ql >= 0 && kvl[s] >= ql && kvl[s] <= (long)c.pages_per_seq * c.page_size;
      for (long j = 0; ok && j < (kvl[s] + c.page_size - 1) / c.page_size; ++j) {
        const int32_t ph = pi[(size_t)s * c.pages_per_seq + j];
        ok = ph >= 0 && ph < c.total_num_pages;
      }
    }
    if (ok) ok = cu[n] <= c.num_q_tokens;
    CHECK((st == RPA_OK) == ok);
  }
  {
    rpa_config c = base_cfg();
    int32_t x = 0;
    CHECK(rpa_check_metadata(&c, nullptr, &x, &x, 0) == RPA_ERR_INVALID_ARGUMENT);
    CHECK(rpa_check_metadata(nullptr, &x, &x, &x, 0) == RPA_ERR_INVALID_ARGUMENT);
  }

  // 3. status strings: static text for every code (and for the unused values of the enum range)
  for (int s = 0; s < 8; ++s) CHECK(rpa_status_string((rpa_status)s) != nullptr);

  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host checks passed (%d accepted configurations)\n", accepted);
  return 0;
}
