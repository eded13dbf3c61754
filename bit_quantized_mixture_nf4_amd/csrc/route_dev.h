// route_dev.h -- top-k selection and softmax of one token's router logits by
// one wavefront (shared by the router kernel and the decode gate_up launch).
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

// Serial form: k rounds of a wave-wide argmax (any k). PER >= ceil(E / 64)
// logits per lane (the register arrays and unrolled loops are sized by it).
template <int PER>
__device__ __forceinline__ void route_token_serial(const float *__restrict__ logits, int64_t t, int E,
                                            int k, int lane, int32_t *__restrict__ idx,
                                            float *__restrict__ wts, int32_t *lds_idx) {
  constexpr int kMaxPer = PER;
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


constexpr int kRouteCand = 256;  // candidate list of the parallel form

// Per-wavefront LDS scratch of route_token.
struct alignas(16) RouteLds {
  float m[64];               // lane maxima
  float cv[kRouteCand + 4];  // candidate values (padded to a multiple of 4)
  int ci[kRouteCand + 4];    // candidate expert ids
  float sv[64];              // selected value by slot
  int si[64];                // selected id by slot
  float sz[64];              // exp(value - slot-0 value) by slot
};

// One wavefront routes token t: selection compares the stored fp32 logits
// exactly (larger value first, equal values -> lower expert id); the weights
// are the softmax over the k selected logits (fp32, summed in slot order).
// Lane j < k writes slot j to idx[t * k + j] / wts[t * k + j] (and to
// lds_idx[t * k + j] when lds_idx is not null).
//
// Parallel form (no serial chain of k wave reductions):
//  1. tau = the k-th largest lane maximum. The k lanes whose maxima are
//     >= tau hold k distinct logits >= tau, so every logit of the top k is
//     >= tau: the logits >= tau are the candidates.
//  2. The candidates are compacted into LDS (ballot prefix counts) and each
//     takes as its slot the number of candidates ordered before it.
// More than kRouteCand candidates (massive ties) or k > 64 take the serial form.
template <int PER>
__device__ __forceinline__ void route_token_per(const float *__restrict__ logits, int64_t t, int E,
                                                int k, int lane, int32_t *__restrict__ idx,
                                                float *__restrict__ wts, int32_t *lds_idx,
                                                RouteLds &sc) {
  if (k > 64) {
    route_token_serial<PER>(logits, t, E, k, lane, idx, wts, lds_idx);
    return;
  }
  constexpr int kMaxPer = PER;
  float v[kMaxPer];
  const int per = (E + 63) / 64;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int e = i * 64 + lane;
    v[i] = (i < per && e < E) ? logits[t * E + e] : -INFINITY;
    m = fmaxf(m, v[i]);
  }
  // 1. tau: the largest lane maximum with at least k maxima >= it
  sc.m[lane] = m;
  __builtin_amdgcn_wave_barrier();
  int ge = 0;
#pragma unroll
  for (int q = 0; q < 64; q += 4) {
    const float4 u = *reinterpret_cast<const float4 *>(&sc.m[q]);
    ge += (u.x >= m) + (u.y >= m) + (u.z >= m) + (u.w >= m);
  }
  float tau = ge >= k ? m : -INFINITY;
  tau = fmaxf(tau, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                 __builtin_bit_cast(int, tau), __builtin_bit_cast(int, tau), 0xB1, 0xF, 0xF, false)));
  tau = fmaxf(tau, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                 __builtin_bit_cast(int, tau), __builtin_bit_cast(int, tau), 0x4E, 0xF, 0xF, false)));
  tau = fmaxf(tau, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                 __builtin_bit_cast(int, tau), __builtin_bit_cast(int, tau), 0x141, 0xF, 0xF, false)));
  tau = fmaxf(tau, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                 __builtin_bit_cast(int, tau), __builtin_bit_cast(int, tau), 0x140, 0xF, 0xF, false)));
  {
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tau), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tau), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tau), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tau), 48));
    tau = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
  }
  // 2. compact the candidates (ascending expert id: entry i of every lane,
  //    lanes in order, then entry i + 1)
  const uint64_t below = (1ull << lane) - 1;
  int pos[kMaxPer];
  int C = 0;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const bool c = i < per && i * 64 + lane < E && v[i] >= tau;
    const uint64_t bal = __ballot(c);
    pos[i] = c ? C + __popcll(bal & below) : -1;
    C += __popcll(bal);
  }
  if (C > kRouteCand) {
    route_token_serial<PER>(logits, t, E, k, lane, idx, wts, lds_idx);
    return;
  }
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i)
    if (pos[i] >= 0) {
      sc.cv[pos[i]] = v[i];
      sc.ci[pos[i]] = i * 64 + lane;
    }
  // pad entries never precede a candidate
  if (lane < 4) {
    sc.cv[C + lane] = -INFINITY;
    sc.ci[C + lane] = 0x7fffffff;
  }
  __builtin_amdgcn_wave_barrier();
  // slot = candidates before this one (larger value, or equal value and lower id)
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i)
    if (pos[i] >= 0) {
      const int e = i * 64 + lane;
      int r = 0;
      for (int c = 0; c < C; c += 4) {
        const float4 u = *reinterpret_cast<const float4 *>(&sc.cv[c]);
        const int4 ui = *reinterpret_cast<const int4 *>(&sc.ci[c]);
        r += ((u.x > v[i]) | ((u.x == v[i]) & (ui.x < e))) + ((u.y > v[i]) | ((u.y == v[i]) & (ui.y < e))) +
             ((u.z > v[i]) | ((u.z == v[i]) & (ui.z < e))) + ((u.w > v[i]) | ((u.w == v[i]) & (ui.w < e)));
      }
      if (r < k) {
        sc.sv[r] = v[i];
        sc.si[r] = e;
      }
    }
  __builtin_amdgcn_wave_barrier();
  // softmax over the selected logits, lane j holds slot j
  const float z = lane < k ? expf(sc.sv[lane] - sc.sv[0]) : 0.0f;
  if (lane < k) sc.sz[lane] = z;
  __builtin_amdgcn_wave_barrier();
  float ssum = 0.0f;
  for (int j = 0; j < k; ++j) ssum += sc.sz[j];
  if (lane < k) {
    const int id = sc.si[lane];
    idx[t * k + lane] = id;
    wts[t * k + lane] = z / ssum;
    if (lds_idx) lds_idx[t * k + lane] = id;
  }
  __builtin_amdgcn_wave_barrier();
}

// route_token_per sized for E: entries per lane rounded up to 1, 2, 4, 8 or
// kMaxE / 64, so a small expert count runs no loop iterations sized for the
// largest (E is uniform across the grid: every wave takes the same branch).
__device__ __forceinline__ void route_token(const float *__restrict__ logits, int64_t t, int E,
                                            int k, int lane, int32_t *__restrict__ idx,
                                            float *__restrict__ wts, int32_t *lds_idx,
                                            RouteLds &sc) {
  static_assert(kMaxE / 64 == 16, "dispatch covers 1..16 logits per lane");
  if (E <= 64) route_token_per<1>(logits, t, E, k, lane, idx, wts, lds_idx, sc);
  else if (E <= 128) route_token_per<2>(logits, t, E, k, lane, idx, wts, lds_idx, sc);
  else if (E <= 256) route_token_per<4>(logits, t, E, k, lane, idx, wts, lds_idx, sc);
  else if (E <= 512) route_token_per<8>(logits, t, E, k, lane, idx, wts, lds_idx, sc);
  else route_token_per<16>(logits, t, E, k, lane, idx, wts, lds_idx, sc);
}

}  // namespace e4b
