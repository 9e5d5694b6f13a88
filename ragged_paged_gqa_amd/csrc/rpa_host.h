// Host-side logic of the C ABI that touches no device: configuration checks,
// the choice of prefill kernel, the decode launch size and the workspace
// layout. Plain C++ (rpa_host.cpp), so that it is also built, without HIP,
// under the address and undefined-behaviour sanitizers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "rpa.h"
#include "rpa_layout.h"

// Prefill-class work items the planner aims for per compute unit.
#ifndef RPA_PF_ITEMS_PER_CU
#define RPA_PF_ITEMS_PER_CU 3
#endif
// head_dims whose 16-bit prefill runs on the two-group (ping-pong) kernel;
// the others, an f32 q and one-byte K/V run on the 4-wave kernel.
#ifndef RPA_PP_MIN_D
#define RPA_PP_MIN_D 256
#endif
#ifndef RPA_PP_MAX_D
#define RPA_PP_MAX_D 256
#endif

namespace rpa {
namespace host {

// A configuration the library serves, or the status that refuses it.
rpa_status validate(const rpa_config* c);

// Byte offsets of the workspace regions and the record counts they bound.
struct Layout {
  size_t hdr, dseq, pu, pi, qlist, done, dpart, dplse, ppart, pplse, total;
  // decode units (S_max * Hkv), prefill units and items, decode partial slots
  int32_t max_du, max_pu, max_pi, dec_slots, tgt_p, pf_rows, dec_waves;
};

// The prefill class of `c` runs on the two-group tiles (tiles_pp_kernel).
bool uses_pp(const rpa_config* c);

// Workgroups of the decode launch on a device with `cus` compute units.
int dec_grid_for(const rpa_config* c, int cus);

// Workspace layout of `c` (validated) on a device with `cus` compute units;
// false when a count would overflow.
bool make_layout(const rpa_config* c, int cus, Layout* L);

}  // namespace host
}  // namespace rpa
