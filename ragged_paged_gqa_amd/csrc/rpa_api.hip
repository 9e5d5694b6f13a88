// C ABI of the ragged paged GQA attention library: host-side validation,
// workspace carving and the launch sequence, all on the caller's stream: the
// plan, the tiles of both classes (one launch; two in turn, prefill then
// decode, where the prefill runs on the two-group kernel), and the merge of
// split decode units. (A split prefill unit is merged inside the prefill
// tiles.)
#include <hip/hip_runtime.h>

#include <dlfcn.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "rpa.h"
#include "rpa_append.h"
#include "rpa_common.h"
#include "rpa_host.h"
#include "rpa_decode.h"
#include "rpa_plan.h"
#include "rpa_prefill.h"
#include "rpa_prefill_pp.h"
#include "rpa_tiles.h"

namespace {

using namespace rpa;
using namespace rpa::host;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device (cached per device ordinal).
bool device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (dev >= 0 && dev < kMaxDevices) {
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return true;
    }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) return false;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return true;
}

Params make_params(const rpa_config* c, const Layout& L, void* ws) {
  Params p;
  std::memset(&p, 0, sizeof p);
  char* w = static_cast<char*>(ws);
  p.hdr = reinterpret_cast<Header*>(w + L.hdr);
  p.dec_seqs = reinterpret_cast<DecSeq*>(w + L.dseq);
  p.pf_units = reinterpret_cast<Unit*>(w + L.pu);
  p.pf_items = reinterpret_cast<Item*>(w + L.pi);
  p.pf_qlist = reinterpret_cast<int32_t*>(w + L.qlist);
  p.unit_done = reinterpret_cast<int32_t*>(w + L.done);
  p.dec_waves = L.dec_waves;
  p.dec_per_cu = dec_grid_for(c, 1);
  p.fused = 1;
  p.dec_blk = (c->kv_dtype == RPA_DTYPE_FP8_E4M3FN || c->kv_dtype == RPA_DTYPE_FP8_E5M2 ||
               c->kv_dtype == RPA_DTYPE_INT8)
                  ? kDecBlk8
                  : kDecBlk16;
  p.dec_part = reinterpret_cast<float*>(w + L.dpart);
  p.dec_plse = reinterpret_cast<float*>(w + L.dplse);
  p.pf_part = reinterpret_cast<float*>(w + L.ppart);
  p.pf_plse = reinterpret_cast<float*>(w + L.pplse);
  p.T = c->num_q_tokens;
  p.Hq = c->num_q_heads;
  p.Hkv = c->num_kv_heads;
  p.G = c->num_q_heads / c->num_kv_heads;
  p.D = c->head_dim;
  p.page = c->page_size;
  p.P = c->total_num_pages;
  p.S_max = c->max_num_seqs;
  p.pps = c->pages_per_seq;
  p.pf_rows = L.pf_rows;
  p.max_dec_units = L.max_du;
  p.max_pf_units = L.max_pu;
  p.max_pf_items = L.max_pi;
  p.target_pf_items = L.tgt_p;
  p.sm_scale = c->sm_scale * c->k_scale;
  p.soft_cap = c->soft_cap;
  p.v_scale = c->v_scale;
  p.is_causal = c->is_causal;
  p.window = c->sliding_window;
  return p;
}

rpa_status check_launch() { return hipGetLastError() == hipSuccess ? RPA_OK : RPA_ERR_HIP; }

// Optional event timing of the launches of each call (for benchmarks):
// events before the plan, after it, after the tile launch and after the
// merge.
struct Profiler {
  std::mutex mu;
  std::atomic<bool> on{false};  // read without the lock on every forward call
  int max_calls = 0;
  int n_calls = 0;
  std::vector<hipEvent_t> ev;  // kProfEvents per recorded call
};
constexpr int kProfEvents = 4;
Profiler g_prof;

void prof_record(hipEvent_t* ev, int k, hipStream_t st) {
  if (ev) (void)hipEventRecord(ev[k], st);
}

// A non-empty environment variable other than "0".
bool env_on(const char* name) {
  const char* e = std::getenv(name);
  return e && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

// Optional host-side trace ranges, the launcher's counterpart of the kernel
// page's trace region around QK^T: with RPA_TRACE set when the library first
// needs them, every forward call and every launch in it is a roctx range
// (shown by rocprofv3 --marker-trace beside the kernels it enqueued). The
// roctx library is opened then (dlopen), so it is no load-time dependency;
// without it the ranges are off.
struct Tracer {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};
const Tracer& tracer() {
  static const Tracer t = [] {
    Tracer r;
    if (!env_on("RPA_TRACE")) return r;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (!h) h = dlopen("librocprofiler-sdk-roctx.so", RTLD_NOW | RTLD_LOCAL);
    if (!h) return r;
    r.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    r.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    if (!r.push || !r.pop) r = Tracer{};
    return r;
  }();
  return t;
}
struct TraceRange {
  bool on;
  explicit TraceRange(const char* name) : on(tracer().push != nullptr) {
    if (on) tracer().push(name);
  }
  ~TraceRange() {
    if (on) tracer().pop();
  }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

// With RPA_LOG set, each forward call prints its plan to stderr: it copies
// the plan header back and waits for `st` (a debugging aid; the call then
// synchronises, and it prints nothing while `st` is being captured).
void log_plan(const Params& p, hipStream_t st) {
  static const bool on = env_on("RPA_LOG");
  if (!on) return;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return;
  }
  Header h;
  if (hipMemcpyAsync(&h, p.hdr, sizeof h, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  std::fprintf(stderr,
               "rpa plan: decode %d seqs, %d units, %d blocks of %d keys over %d of %d waves; prefill %d units, "
               "%d items of <= %d keys, %d split units; queues",
               h.n_dec_seqs, h.n_dec_units, h.dec_blocks, p.dec_blk, h.pad0[0], p.dec_waves, h.n_pf_units,
               h.n_pf_items, h.pf_chunk, h.n_split_units);
  for (int x = 0; x < kQueues; ++x) std::fprintf(stderr, " %d", h.pf_q_count[x]);
  std::fprintf(stderr, "\n");
}

// Prefill-class workgroups of a launch: the two-group kernel runs one per
// compute unit, the 4-wave kernel as many as its LDS and registers allow;
// never more than there are items.
template <int D, bool FP8, bool PP>
int prefill_grid(const Params& p, int cus) {
  int per_cu = 1;
  if constexpr (!PP) {
    constexpr int by_lds = (int)((160 * 1024) / sizeof(PfShared<D, FP8>));
    per_cu = pf_wgs_per_cu(D) < by_lds ? pf_wgs_per_cu(D) : by_lds;
    if (per_cu < 1) per_cu = 1;
  }
  int grid = cus * per_cu;
  if (grid > p.max_pf_items) grid = p.max_pf_items;
  return grid < 1 ? 1 : grid;
}

template <int D, bool F16, bool Q32>
rpa_status launch_combine(const Params& p, int cus, hipStream_t st) {
  TraceRange r("rpa combine");
  // merge of the split decode units (a wave per unit, grid-stride)
  int cgrid = (p.max_dec_units + kDecWavesPerBlock - 1) / kDecWavesPerBlock;
  if (cgrid > cus * 4) cgrid = cus * 4;
  if (cgrid < 1) cgrid = 1;
  hipLaunchKernelGGL((combine_kernel<D, F16, Q32>), dim3(cgrid), dim3(kDecWavesPerBlock * 64), 0, st, p);
  return check_launch();
}

// The launches after the plan: one launch holds the workgroups of both
// classes (tiles_pp_kernel where the prefill class runs on the two-group
// kernel, tiles_kernel elsewhere), then the merge.
template <int D, int KVT, bool F16, bool Q32>
rpa_status launch_attention(const Params& p, int cus, hipStream_t st, hipEvent_t* ev) {
  constexpr bool FP8 = KVT != kKvBf16;
  // the decode workgroups: the waves of the stream-K split (those the planner
  // gives no work exit at once)
  const int dec_wgs = p.dec_waves / kDecWavesPerBlock;
  if (dec_wgs < 1) return RPA_ERR_HIP;
  {
    TraceRange r("rpa tiles");
    if constexpr (!FP8 && !Q32 && D >= RPA_PP_MIN_D && D <= RPA_PP_MAX_D) {
      const int grid = dec_wgs + prefill_grid<D, FP8, true>(p, cus);
      if (p.soft_cap > 0.f)
        hipLaunchKernelGGL((tiles_pp_kernel<D, true, F16>), dim3(grid), dim3(kPpWaves * 64), 0, st, p);
      else
        hipLaunchKernelGGL((tiles_pp_kernel<D, false, F16>), dim3(grid), dim3(kPpWaves * 64), 0, st, p);
    } else {
      const int grid = dec_wgs + prefill_grid<D, FP8, false>(p, cus);
      if (p.soft_cap > 0.f)
        hipLaunchKernelGGL((tiles_kernel<D, KVT, true, F16, Q32>), dim3(grid), dim3(kDecWavesPerBlock * 64), 0, st,
                           p);
      else
        hipLaunchKernelGGL((tiles_kernel<D, KVT, false, F16, Q32>), dim3(grid), dim3(kDecWavesPerBlock * 64), 0, st,
                           p);
    }
    if (check_launch() != RPA_OK) return RPA_ERR_HIP;
  }
  prof_record(ev, 2, st);
  if (launch_combine<D, F16, Q32>(p, cus, st) != RPA_OK) return RPA_ERR_HIP;
  prof_record(ev, 3, st);
  return RPA_OK;
}

// (q dtype, K/V dtype) -> kernels: K/V in the q type, or fp8 widened to it.
template <int D>
rpa_status launch_for_kv(int32_t q_dtype, int32_t kv_dtype, const Params& p, int cus, hipStream_t st,
                         hipEvent_t* ev) {
  if (q_dtype == RPA_DTYPE_F16) {
    switch (kv_dtype) {
      case RPA_DTYPE_F16: return launch_attention<D, kKvBf16, true, false>(p, cus, st, ev);
      case RPA_DTYPE_FP8_E4M3FN: return launch_attention<D, kKvE4M3, true, false>(p, cus, st, ev);
      case RPA_DTYPE_FP8_E5M2: return launch_attention<D, kKvE5M2, true, false>(p, cus, st, ev);
      case RPA_DTYPE_INT8: return launch_attention<D, kKvI8, true, false>(p, cus, st, ev);
      default: return RPA_ERR_UNSUPPORTED;
    }
  }
  if (q_dtype == RPA_DTYPE_F32) {
    switch (kv_dtype) {
      case RPA_DTYPE_BF16: return launch_attention<D, kKvBf16, false, true>(p, cus, st, ev);
      case RPA_DTYPE_FP8_E4M3FN: return launch_attention<D, kKvE4M3, false, true>(p, cus, st, ev);
      case RPA_DTYPE_FP8_E5M2: return launch_attention<D, kKvE5M2, false, true>(p, cus, st, ev);
      case RPA_DTYPE_INT8: return launch_attention<D, kKvI8, false, true>(p, cus, st, ev);
      default: return RPA_ERR_UNSUPPORTED;
    }
  }
  switch (kv_dtype) {
    case RPA_DTYPE_BF16: return launch_attention<D, kKvBf16, false, false>(p, cus, st, ev);
    case RPA_DTYPE_FP8_E4M3FN: return launch_attention<D, kKvE4M3, false, false>(p, cus, st, ev);
    case RPA_DTYPE_FP8_E5M2: return launch_attention<D, kKvE5M2, false, false>(p, cus, st, ev);
    case RPA_DTYPE_INT8: return launch_attention<D, kKvI8, false, false>(p, cus, st, ev);
    default: return RPA_ERR_UNSUPPORTED;
  }
}

rpa_status launch_plan(const Params& p, hipStream_t st) {
  TraceRange r("rpa plan");
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, p);
  return check_launch();
}

template <int D, int IN>
void launch_append_in(int mode, int grid, hipStream_t st, const AppendParams& p) {
  const dim3 blk(kApWaves * 64);
  // a bit copy needs the rows in the cache type
  if (IN == kInF32 && mode == kApCopy) mode = kApBf16;
  switch (mode) {
    case kApFp8: hipLaunchKernelGGL((kv_append_kernel<D, kApFp8, IN>), dim3(grid), blk, 0, st, p); break;
    case kApE5M2: hipLaunchKernelGGL((kv_append_kernel<D, kApE5M2, IN>), dim3(grid), blk, 0, st, p); break;
    case kApI8: hipLaunchKernelGGL((kv_append_kernel<D, kApI8, IN>), dim3(grid), blk, 0, st, p); break;
    case kApCopy: hipLaunchKernelGGL((kv_append_kernel<D, (IN == kInF32 ? kApBf16 : kApCopy), IN>), dim3(grid), blk, 0, st, p); break;
    case kApF16: hipLaunchKernelGGL((kv_append_kernel<D, (IN == kInF32 ? kApBf16 : kApF16), IN>), dim3(grid), blk, 0, st, p); break;
    default: hipLaunchKernelGGL((kv_append_kernel<D, kApBf16, IN>), dim3(grid), blk, 0, st, p); break;
  }
}
template <int D>
void launch_append(int mode, int in, int grid, hipStream_t st, const AppendParams& p) {
  if (in == kInF16)
    launch_append_in<D, kInF16>(mode, grid, st, p);
  else if (in == kInF32)
    launch_append_in<D, kInF32>(mode, grid, st, p);
  else
    launch_append_in<D, kInBf16>(mode, grid, st, p);
}

__global__ void decode_fp8_kernel(const uint8_t* codes, float* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * i >= n) return;
  uint32_t w = 0;
  for (int k = 0; k < 4; ++k)
    if (4 * i + k < n) w |= (uint32_t)codes[4 * i + k] << (8 * k);
  u32x2 ww = {w, 0u};
  bf16x8 b = fp8x8_to_bf16<kKvE4M3>(ww);
  for (int k = 0; k < 4; ++k)
    if (4 * i + k < n) out[4 * i + k] = (float)b[k];
}

// Workspace of rpa_forward_noalloc, for callers that cannot allocate: a
// file-scope device array, one copy per GPU, held until the process ends.
// Host code never uses its name as an address (that is a host-side stand-in):
// scratch_ptr() resolves each device's copy once, with hipGetSymbolAddress,
// and every launch takes that address.
constexpr size_t kScratchBytes = (size_t)256 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];

// This device's copy of `scratch` (resolved on the first call per device, with
// that device current), or null if it cannot be resolved.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

rpa_status prepare(const rpa_config* cfg, void* workspace, size_t workspace_bytes, Params* p, int* cus_out) {
  rpa_status st = validate(cfg);
  if (st != RPA_OK) return st;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return RPA_ERR_INVALID_ARGUMENT;
  int cus = 0;
  if (!device_cus(&cus)) return RPA_ERR_HIP;
  Layout L;
  if (!make_layout(cfg, cus, &L)) return RPA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < L.total) return RPA_ERR_WORKSPACE_TOO_SMALL;
  *p = make_params(cfg, L, workspace);
  // every workspace view the kernels dereference must be assigned
  const void* views[] = {p->hdr,       p->dec_seqs, p->pf_units, p->pf_items, p->pf_qlist,
                         p->unit_done, p->dec_part, p->dec_plse, p->pf_part,  p->pf_plse};
  for (const void* v : views)
    if (!v) return RPA_ERR_INVALID_ARGUMENT;
  *cus_out = cus;
  return RPA_OK;
}

// The forward call: checks, then the plan and the attention launches on
// `stream`.
rpa_status forward(const rpa_config* cfg, const void* q, const void* kv_pages, const int32_t* kv_lens,
                   const int32_t* page_indices, const int32_t* cu_q_lens, const int32_t* num_seqs,
                   const float* sinks, void* out, float* lse, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (!q || !kv_pages || !kv_lens || !page_indices || !cu_q_lens || !num_seqs || !out)
    return RPA_ERR_INVALID_ARGUMENT;
  // the kernels move q, K/V and out in 16-byte pieces and lse / sinks as f32
  for (const void* a : {q, kv_pages, (const void*)out})
    if ((reinterpret_cast<uintptr_t>(a) & 15u) != 0) return RPA_ERR_INVALID_ARGUMENT;
  for (const void* a : {(const void*)lse, (const void*)sinks})
    if ((reinterpret_cast<uintptr_t>(a) & 3u) != 0) return RPA_ERR_INVALID_ARGUMENT;
  Params p;
  int cus = 0;
  rpa_status st = prepare(cfg, workspace, workspace_bytes, &p, &cus);
  if (st != RPA_OK) return st;
  p.q = static_cast<const uint16_t*>(q);
  p.kv = static_cast<const uint8_t*>(kv_pages);
  p.kv_lens = kv_lens;
  p.page_indices = page_indices;
  p.cu_q_lens = cu_q_lens;
  p.num_seqs = num_seqs;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.sinks = sinks;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = nullptr;
  if (g_prof.on.load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lock(g_prof.mu);
    if (g_prof.on.load(std::memory_order_relaxed) && g_prof.n_calls < g_prof.max_calls)
      ev = &g_prof.ev[kProfEvents * g_prof.n_calls++];
  }
  TraceRange r("rpa_forward");
  prof_record(ev, 0, s);
  st = launch_plan(p, s);
  if (st != RPA_OK) return st;
  prof_record(ev, 1, s);
  log_plan(p, s);
  switch (cfg->head_dim) {
    case 64: return launch_for_kv<64>(cfg->q_dtype, cfg->kv_dtype, p, cus, s, ev);
    case 128: return launch_for_kv<128>(cfg->q_dtype, cfg->kv_dtype, p, cus, s, ev);
    case 256: return launch_for_kv<256>(cfg->q_dtype, cfg->kv_dtype, p, cus, s, ev);
    default: return RPA_ERR_UNSUPPORTED;
  }
}

}  // namespace

extern "C" {

rpa_status rpa_workspace_bytes(const rpa_config* cfg, size_t* bytes) {
  if (!bytes) return RPA_ERR_INVALID_ARGUMENT;
  rpa_status st = validate(cfg);
  if (st != RPA_OK) return st;
  int cus = 0;
  if (!device_cus(&cus)) return RPA_ERR_HIP;
  Layout L;
  if (!make_layout(cfg, cus, &L)) return RPA_ERR_INVALID_ARGUMENT;
  *bytes = L.total;
  return RPA_OK;
}

rpa_status rpa_forward(const rpa_config* cfg, const void* q, const void* kv_pages, const int32_t* kv_lens,
                       const int32_t* page_indices, const int32_t* cu_q_lens, const int32_t* num_seqs, void* out,
                       float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return rpa_forward_sinks(cfg, q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, nullptr, out, lse, workspace,
                           workspace_bytes, stream);
}

rpa_status rpa_forward_sinks(const rpa_config* cfg, const void* q, const void* kv_pages, const int32_t* kv_lens,
                             const int32_t* page_indices, const int32_t* cu_q_lens, const int32_t* num_seqs,
                             const float* sinks, void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return forward(cfg, q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, sinks, out, lse, workspace,
                 workspace_bytes, stream);
}

rpa_status rpa_forward_noalloc(const rpa_config* cfg, const void* q, const void* kv_pages, const int32_t* kv_lens,
                               const int32_t* page_indices, const int32_t* cu_q_lens, const int32_t* num_seqs,
                               const float* sinks, void* out, float* lse, void* stream) {
  if (!q || !kv_pages || !kv_lens || !page_indices || !cu_q_lens || !num_seqs || !out)
    return RPA_ERR_INVALID_ARGUMENT;
  size_t need = 0;
  rpa_status st = rpa_workspace_bytes(cfg, &need);
  if (st != RPA_OK) return st;
  if (need > kScratchBytes) return RPA_ERR_WORKSPACE_TOO_SMALL;
  void* ws = scratch_ptr();
  if (!ws) return RPA_ERR_HIP;
  // the planning kernel rewrites every record, counter and queue head the
  // attention kernels read, so nothing is cleared here
  return forward(cfg, q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, sinks, out, lse, ws, kScratchBytes,
                 stream);
}

rpa_status rpa_profile_begin(int32_t max_calls) {
  if (max_calls < 1 || max_calls > (1 << 20)) return RPA_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (g_prof.on) return RPA_ERR_INVALID_ARGUMENT;
  g_prof.ev.assign((size_t)kProfEvents * max_calls, nullptr);
  for (auto& e : g_prof.ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      for (auto& f : g_prof.ev)
        if (f) (void)hipEventDestroy(f);
      g_prof.ev.clear();
      return RPA_ERR_HIP;
    }
  }
  g_prof.max_calls = max_calls;
  g_prof.n_calls = 0;
  g_prof.on.store(true, std::memory_order_release);
  return RPA_OK;
}

rpa_status rpa_profile_end(float kernel_ms[4], int32_t* n_calls) {
  if (!kernel_ms || !n_calls) return RPA_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (!g_prof.on) return RPA_ERR_INVALID_ARGUMENT;
  rpa_status st = RPA_OK;
  for (int k = 0; k < 4; ++k) kernel_ms[k] = 0.f;
  if (g_prof.n_calls > 0 && hipEventSynchronize(g_prof.ev[kProfEvents * g_prof.n_calls - 1]) != hipSuccess)
    st = RPA_ERR_HIP;
  // plan 0 -> 1, tiles 1 -> 2, merge 2 -> 3, the whole call 0 -> 3
  for (int c = 0; c < g_prof.n_calls && st == RPA_OK; ++c) {
    const hipEvent_t* e = &g_prof.ev[kProfEvents * c];
    const int from[4] = {0, 1, 2, 0}, to[4] = {1, 2, 3, 3};
    for (int k = 0; k < 4; ++k) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, e[from[k]], e[to[k]]) != hipSuccess) {
        st = RPA_ERR_HIP;
        break;
      }
      kernel_ms[k] += ms;
    }
  }
  *n_calls = g_prof.n_calls;
  for (auto& e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.on.store(false, std::memory_order_release);
  g_prof.n_calls = 0;
  return st;
}

rpa_status rpa_plan(const rpa_config* cfg, const int32_t* kv_lens, const int32_t* cu_q_lens, const int32_t* num_seqs,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!kv_lens || !cu_q_lens || !num_seqs) return RPA_ERR_INVALID_ARGUMENT;
  Params p;
  int cus = 0;
  rpa_status st = prepare(cfg, workspace, workspace_bytes, &p, &cus);
  if (st != RPA_OK) return st;
  p.kv_lens = kv_lens;
  p.cu_q_lens = cu_q_lens;
  p.num_seqs = num_seqs;
  return launch_plan(p, static_cast<hipStream_t>(stream));
}

rpa_status rpa_plan_layout(const rpa_config* cfg, size_t offsets[8], int32_t limits[8]) {
  if (!offsets || !limits) return RPA_ERR_INVALID_ARGUMENT;
  rpa_status st = validate(cfg);
  if (st != RPA_OK) return st;
  int cus = 0;
  if (!device_cus(&cus)) return RPA_ERR_HIP;
  Layout L;
  if (!make_layout(cfg, cus, &L)) return RPA_ERR_INVALID_ARGUMENT;
  offsets[0] = L.hdr;
  offsets[1] = L.dseq;
  offsets[2] = L.pu;
  offsets[3] = 0;
  offsets[4] = L.pi;
  offsets[5] = L.qlist;
  offsets[6] = 0;
  offsets[7] = 0;
  limits[0] = L.max_du;
  limits[1] = L.max_pu;
  limits[2] = L.dec_slots;
  limits[3] = L.max_pi;
  limits[4] = kDecRows;
  limits[5] = L.pf_rows;
  limits[6] = L.dec_waves;
  limits[7] = 0;
  return RPA_OK;
}

rpa_status rpa_kv_append(const rpa_config* cfg, const void* k_new, const void* v_new, void* kv_pages,
                         const int32_t* kv_lens, const int32_t* page_indices, const int32_t* cu_q_lens,
                         const int32_t* num_seqs, void* stream) {
  rpa_status st = validate(cfg);
  if (st != RPA_OK) return st;
  if (!k_new || !v_new || !kv_pages || !kv_lens || !page_indices || !cu_q_lens || !num_seqs)
    return RPA_ERR_INVALID_ARGUMENT;
  for (const void* a : {k_new, v_new, (const void*)kv_pages})
    if ((reinterpret_cast<uintptr_t>(a) & 15u) != 0) return RPA_ERR_INVALID_ARGUMENT;
  if (!(cfg->k_scale > 0.f) || !(cfg->v_scale > 0.f)) return RPA_ERR_INVALID_ARGUMENT;
  if (cfg->num_q_tokens == 0) return RPA_OK;
  int cus = 0;
  if (!device_cus(&cus)) return RPA_ERR_HIP;
  AppendParams p;
  p.k_new = k_new;
  p.v_new = v_new;
  p.kv = kv_pages;
  p.kv_lens = kv_lens;
  p.page_indices = page_indices;
  p.cu_q_lens = cu_q_lens;
  p.num_seqs = num_seqs;
  p.T = cfg->num_q_tokens;
  p.Hkv = cfg->num_kv_heads;
  p.P = cfg->total_num_pages;
  p.page_size = cfg->page_size;
  p.max_num_seqs = cfg->max_num_seqs;
  p.pps = cfg->pages_per_seq;
  p.k_scale = cfg->k_scale;
  p.v_scale = cfg->v_scale;
  // the new rows' type is the q type
  const int in = cfg->q_dtype == RPA_DTYPE_F16 ? kInF16 : cfg->q_dtype == RPA_DTYPE_F32 ? kInF32 : kInBf16;
  const int mode = cfg->kv_dtype == RPA_DTYPE_FP8_E4M3FN                                   ? kApFp8
                   : cfg->kv_dtype == RPA_DTYPE_FP8_E5M2                                   ? kApE5M2
                   : cfg->kv_dtype == RPA_DTYPE_INT8                                       ? kApI8
                   : (in != kInF32 && cfg->k_scale == 1.f && cfg->v_scale == 1.f) ? kApCopy
                   : in == kInF16                                                          ? kApF16
                                                                                           : kApBf16;
  // a wave per token, grid-stride beyond 8 workgroups per compute unit
  int grid = (cfg->num_q_tokens + kApWaves - 1) / kApWaves;
  if (grid > cus * 8) grid = cus * 8;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TraceRange r("rpa_kv_append");
  switch (cfg->head_dim) {
    case 64: launch_append<64>(mode, in, grid, s, p); break;
    case 128: launch_append<128>(mode, in, grid, s, p); break;
    case 256: launch_append<256>(mode, in, grid, s, p); break;
    default: return RPA_ERR_UNSUPPORTED;
  }
  return check_launch();
}

rpa_status rpa_debug_decode_fp8(const uint8_t* codes, float* values, int32_t n, void* stream) {
  if (!codes || !values || n < 0) return RPA_ERR_INVALID_ARGUMENT;
  if (n == 0) return RPA_OK;
  const int threads = (n + 3) / 4;
  hipLaunchKernelGGL(decode_fp8_kernel, dim3((threads + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), codes, values, n);
  return check_launch();
}

}  // extern "C"
