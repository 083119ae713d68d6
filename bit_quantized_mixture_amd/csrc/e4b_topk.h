// Per-token top-k routing by one wave (gfx950): shared by the router kernels and the
// single-launch decode step, so both produce bit-identical expert ids and weights.
// Order: higher logit first, equal logits by the lower expert index; weights are the softmax
// over the chosen k logits (renormalised) or the full softmax probabilities.
#pragma once

#include "e4b_device.h"

namespace e4b {

constexpr int kMaxExpertsPerLane = 16;  // E <= 1024

// a beats b: higher value, or equal value and lower index.  Invalid entries carry
// index INT_MAX and value -inf; logits are finite, so any valid entry beats them.
__device__ __forceinline__ bool beats(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// One step of the wave-wide arg-max: combine (v, i) with the pair DPP control `ctrl` moves
// in (lanes outside row_mask keep theirs).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v),
                                                              kCtrl, kRowMask, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(i, i, kCtrl, kRowMask, 0xF, false);
  if (beats(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// Wave-wide arg-max under `beats`, with DPP lane moves (quad swaps, half-row and row
// mirrors, then the row broadcasts of lanes 15 and 31), which lands the result in lane 63;
// returned to every lane through a scalar read.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<0xB1, 0xF>(v, i);   // quad_perm [1,0,3,2]
  argmax_step<0x4E, 0xF>(v, i);   // quad_perm [2,3,0,1]
  argmax_step<0x141, 0xF>(v, i);  // row_half_mirror
  argmax_step<0x140, 0xF>(v, i);  // row_mirror: every lane holds its row's result
  argmax_step<0x142, 0xA>(v, i);  // row_bcast:15 into rows 1 and 3
  argmax_step<0x143, 0xC>(v, i);  // row_bcast:31 into rows 2 and 3
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

// Wave-wide sum in a fixed order (same lane moves as wave_argmax), returned to every lane.
__device__ __forceinline__ float wave_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xC, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Top-k of one token's logits `row` by one wave; lane j < k gets the j-th pick and its
// weight.  PL = logits per lane (E <= 64 * PL), a compile-time bound so the per-lane scans
// are short.
template <int PL>
__device__ __forceinline__ void topk_token(const float* __restrict__ row, int E, int k, int renorm,
                                           int lane, int& id, float& wt) {
  float v[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? row[e] : -INFINITY;
  }
  uint32_t taken = 0;  // bit i: my entry i already chosen
  int my_id = 0;
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && beats(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      my_id = bi;
      my_v = bv;
    }
  }
  const float vmax = __shfl(my_v, 0);  // the first pick is the largest logit
  float ex = lane < k ? expf(my_v - vmax) : 0.f;
  float denom;
  if (renorm) {
    denom = ex;
  } else {
    denom = 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) denom += expf(v[i] - vmax);
    }
  }
  denom = wave_sum(denom);
  id = my_id;
  wt = ex / denom;
}

}  // namespace e4b
