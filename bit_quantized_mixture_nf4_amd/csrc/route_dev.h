// route_dev.h -- top-k selection and softmax of one token's router logits by
// one wavefront (shared by the router kernel and the decode prep kernel).
#pragma once

#include "device.h"
#include "plan.h"

namespace e4b {

// Best (value, id) of lane and its DPP partner: larger value, then lower id.
template <int CTRL>
__device__ __forceinline__ void route_dpp_best(float &bv, int &bi) {
  const float ov = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, bv), __builtin_bit_cast(int, bv),
                                         CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(bi, bi, CTRL, 0xF, 0xF, false);
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

// One wavefront routes token t: selection compares the stored fp32 logits
// exactly (larger value first, equal values -> lower expert id); the weights
// are the softmax over the k selected logits (fp32, summed in slot order).
// Lane j < k writes slot j to idx[t * k + j] / wts[t * k + j] (and to
// lds_idx[t * k + j] when lds_idx is not null).
__device__ __forceinline__ void route_token(const float *__restrict__ logits, int64_t t, int E,
                                            int k, int lane, int32_t *__restrict__ idx,
                                            float *__restrict__ wts, int32_t *lds_idx) {
  constexpr int kMaxPer = kMaxE / 64;
  float v[kMaxPer];
  const int per = (E + 63) / 64;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int e = i * 64 + lane;
    v[i] = (i < per && e < E) ? logits[t * E + e] : -INFINITY;
  }
  uint32_t taken = 0;  // bit i: entry i of this lane already selected
  float sel0 = 0.0f, mysel = 0.0f;
  int myid = 0;
  for (int j = 0; j < k; ++j) {
    // lane-local best among untaken (lower index wins ties: ascending scan, strict >)
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int e = i * 64 + lane;
      if (i < per && e < E && !(taken & (1u << i)) && (v[i] > bv || bi == 0x7fffffff)) {
        bv = v[i];
        bi = e;
      }
    }
    // row (16-lane) reduction with DPP moves, then the four row winners by
    // readlane (no LDS round trips on the per-slot critical path)
    route_dpp_best<0xB1>(bv, bi);   // quad_perm [1,0,3,2]
    route_dpp_best<0x4E>(bv, bi);   // quad_perm [2,3,0,1]
    route_dpp_best<0x141>(bv, bi);  // row_half_mirror
    route_dpp_best<0x140>(bv, bi);  // row_mirror
    {
      float best = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 0));
      int besti = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
      for (int row = 1; row < 4; ++row) {
        const float ov =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), row * 16));
        const int oi = __builtin_amdgcn_readlane(bi, row * 16);
        if (ov > best || (ov == best && oi < besti)) {
          best = ov;
          besti = oi;
        }
      }
      bv = best;
      bi = besti;
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (j == 0) sel0 = bv;
    if (lane == j) {
      mysel = bv;
      myid = bi;
    }
  }
  // softmax over the selected logits, lane j holds slot j
  const float z = lane < k ? expf(mysel - sel0) : 0.0f;
  float s = 0.0f;
  for (int j = 0; j < k; ++j)
    s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, z), j));
  if (lane < k) {
    idx[t * k + lane] = myid;
    wts[t * k + lane] = z / s;
    if (lds_idx) lds_idx[t * k + lane] = myid;
  }
}

}  // namespace e4b
