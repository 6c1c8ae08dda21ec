// Top-k lists over one wavefront: entry i of a sorted list (score descending, then row
// ascending) in lane i, or in LDS slot i.
#pragma once

#include "tq_device.h"

namespace tq {

// a better than b: higher score, then smaller row
__device__ __forceinline__ bool better(float as, int32_t ai, float bs, int32_t bi) {
  return as > bs || (as == bs && ai < bi);
}

// Shift a value up by one lane across the wavefront (DPP wave_shr:1; lane 0 gets 0).
__device__ __forceinline__ int32_t wave_shr1(int32_t x) {
  return __builtin_amdgcn_update_dpp(0, x, 0x138, 0xF, 0xF, false);
}

// Insert the wave-uniform candidate (cs, ci) into the lane-distributed sorted list (ls, li)
// of length k (lanes >= k are unused).
__device__ __forceinline__ void list_insert(float &ls, int32_t &li, float cs, int32_t ci, int k) {
  const int lane = lane_id();
  const bool b = lane < k && better(ls, li, cs, ci);
  const int pos = __popcll(__ballot(b));
  if (pos >= k) return;
  const float us = __int_as_float(wave_shr1(__float_as_int(ls)));
  const int32_t ui = wave_shr1(li);
  if (lane > pos) {
    ls = us;
    li = ui;
  } else if (lane == pos) {
    ls = cs;
    li = ci;
  }
}

// Insert the wave-uniform candidate (cs, ci) into the sorted list of length k held in LDS
// (entry i at ls[i], li[i]); returns the list's k-th score afterwards.
__device__ __forceinline__ float list_insert_lds(float *lsp, int32_t *lip, float cs, int32_t ci, int k) {
  const int lane = lane_id();
  float ls = lane < k ? lsp[lane] : -INFINITY;
  int32_t li = lane < k ? lip[lane] : 0x7FFFFFFF;
  const int pos = __popcll(__ballot(lane < k && better(ls, li, cs, ci)));
  if (pos < k) {
    const float us = __int_as_float(wave_shr1(__float_as_int(ls)));
    const int32_t ui = wave_shr1(li);
    if (lane > pos) {
      ls = us;
      li = ui;
    } else if (lane == pos) {
      ls = cs;
      li = ci;
    }
    if (lane >= pos && lane < k) {
      lsp[lane] = ls;
      lip[lane] = li;
    }
  }
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), k - 1));
}

}  // namespace tq
