// decode.hip -- forward for T <= 8 tokens as bandwidth-bound dequant-GEMVs.
//
// The 0.4.0 README ("Inference" section) describes the decode fast path: a
// single-token forward skips the one-hot grouping and its per-expert host
// syncs, and single-row projections read the packed 4-bit weight directly
// instead of materializing a dequantized expert. Here, for T <= 8, two
// launches and no host sync. In both, a workgroup owns a block of output rows
// for every expert the tokens touch, so the grid is fixed by the shape, every
// workgroup does the same work, and what is reduced across experts or K parts
// meets in LDS in a fixed order:
//   gate_up  every workgroup routes the tokens (when given logits) and groups
//            the <= 256 routed pairs by expert in LDS; a block is
//            kGuUnits gate rows and the matching up rows, and the workgroup
//            writes a = silu(g) * u of those units for every pair. Workgroup
//            0 also leaves the grouping in the workspace for the down launch.
//   down     a block is kDnRows rows of H; the workgroup computes each pair's
//            down projection of those rows (fp32, in LDS) and sums them into
//            y over each token's pairs in slot order: the combine needs no
//            launch of its own.
// Every packed byte of a touched expert is read once for all pairs routed to
// it. No MFMA: each code byte is expanded through an LDS table into two bf16
// codebook values and contracted with bf16 inputs by v_dot2_f32_bf16 in fp32;
// a 32-element chunk's partial sum is multiplied by its block scale.
#include <algorithm>
#include <utility>

#include "device.h"
#include "kernels.h"
#include "route_dev.h"

namespace e4b {

// f(std::integral_constant<int, i>) for i = 0 .. N - 1 (register sets
// indexed by constants)
template <typename F, int... Is>
__device__ __forceinline__ void dec_static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void dec_static_for(F &&f) {
  dec_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kDecThreads = 256;
constexpr int kTblCopies = 32;   // LDS table copies (lane l reads copy l % kTblCopies)
constexpr int kDecVec = 2;       // input vectors per GEMV pass (more pairs of an expert: passes of 2)
constexpr int kGuRows = 2;       // gate_up: weight rows per workgroup block (one unit's gate and up rows)
constexpr int kGuUnits = kGuRows / 2;
constexpr int kDnRows = 4;       // down: rows of H per workgroup block
constexpr int kPartFloats = 2048;    // LDS partial sums: K parts x pairs x rows
constexpr int kDecWgPerCu = 3;       // resident workgroups per CU the launch grid is sized for
constexpr int kRouteWaves = kDecThreads / 64;

// The grouping that the gate_up launch leaves in the workspace.
struct DecodePlan {
  int32_t n;                        // distinct experts
  int32_t pad[3];
  int32_t expert[kDecMaxPairs];     // distinct experts, ascending
  int32_t first[kDecMaxPairs + 1];  // first sorted position of each; first[n] = P
  float weight[kDecMaxPairs];       // routing weight of each sorted position
  int32_t pos[kDecMaxPairs];        // sorted position of flat pair t * k + j
};
static_assert(sizeof(DecodePlan) <= kDecPlanBytes, "the grouping fits its workspace slot");

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                                   false));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over an aligned group of G lanes (G a power of two, 4 <= G <= 64),
// every lane of the group getting the same bits: within a 16-lane row by DPP
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror),
// across rows by reading lanes 0, 16, 32, 48 (the rows' sums, added in row
// order). No LDS round trips, so the sums of many values overlap.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G >= 4 && G <= 64 && (G & (G - 1)) == 0, "group of 4..64 lanes");
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  if (G >= 8) v = dpp_add<0x141>(v);
  if (G >= 16) v = dpp_add<0x140>(v);
  if (G == 32) {
    const float lo = lane_value(v, 0) + lane_value(v, 16), hi = lane_value(v, 32) + lane_value(v, 48);
    v = (threadIdx.x & 32) ? hi : lo;
  } else if (G == 64) {
    v = (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
  }
  return v;
}

// The layer's 16 codebook values rounded to bf16 (to nearest, ties to
// even): code 2 i in the low half of pair[i], code 2 i + 1 in the high half.
// A kernel argument, so filling the table needs no memory load.
struct DecCodebook {
  uint32_t pair[8];
};

// byte -> (bf16 code of the high nibble | bf16 code of the low nibble << 16),
// the element order in memory (the even element sits in the high nibble).
// Entry (byte, copy) at byte * kTblCopies + copy. The copies of a byte are
// equal: thread tid writes four with each 16-byte store u = tid + 256 i
// (i < kTblCopies / 4), whose byte is u >> S (S = log2(kTblCopies / 4)):
// low nibble (tid >> S) & 15, high nibble i * (256 >> (S + 4)) + (tid >> (S +
// 4)). Values are picked from the pairs by select trees on those bits (no
// register array indexed at run time).
__device__ __forceinline__ void fill_code_table(uint32_t *tbl, const DecCodebook &cb) {
  static_assert((kTblCopies == 16 || kTblCopies == 32) && kDecThreads == 256, "fill layout");
  constexpr int S = kTblCopies == 32 ? 3 : 2;
  const int tid = threadIdx.x;
  const uint32_t q = (tid >> S) & 15;
  const uint32_t a0 = (q & 2) ? cb.pair[1] : cb.pair[0], a1 = (q & 2) ? cb.pair[3] : cb.pair[2];
  const uint32_t a2 = (q & 2) ? cb.pair[5] : cb.pair[4], a3 = (q & 2) ? cb.pair[7] : cb.pair[6];
  const uint32_t b0 = (q & 4) ? a1 : a0, b1 = (q & 4) ? a3 : a2;
  const uint32_t c = (q & 8) ? b1 : b0;
  const uint32_t lo = (q & 1) ? (c >> 16) : (c & 0xFFFFu);
  const uint32_t t = tid >> (S + 4);  // high nibble within the store's group of codes
#pragma unroll
  for (int i = 0; i < kTblCopies / 4; ++i) {
    uint32_t pr;
    if constexpr (kTblCopies == 32) {
      pr = cb.pair[i];  // codes 2 i, 2 i + 1
    } else {
      pr = (t & 2) ? cb.pair[2 * i + 1] : cb.pair[2 * i];  // codes 4 i .. 4 i + 3
    }
    const uint32_t hi = (t & 1) ? (pr >> 16) : (pr & 0xFFFFu);
    const uint32_t v = hi | (lo << 16);
    reinterpret_cast<u32x4 *>(tbl)[tid + kDecThreads * i] = u32x4{v, v, v, v};
  }
}

// The 16 bf16 code pairs of one 16-byte chunk of codes (word w, byte y at
// index 4 w + y), looked up in the lane's copy of the table.
__device__ __forceinline__ void lookup_chunk(const uint32_t *tl, const u32x4 &cw, uint32_t (&v)[16]) {
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int y = 0; y < 4; ++y) v[4 * w + y] = tl[((cw[w] >> (8 * y)) & 255u) * kTblCopies];
}

// Codebook value i (0..15) in bf16, by a select tree on the bits of i (no
// register array indexed at run time).
__device__ __forceinline__ uint32_t code_bf16(const DecCodebook &cb, uint32_t i) {
  const uint32_t h = i >> 1;
  const uint32_t a0 = (h & 1) ? cb.pair[1] : cb.pair[0], a1 = (h & 1) ? cb.pair[3] : cb.pair[2];
  const uint32_t a2 = (h & 1) ? cb.pair[5] : cb.pair[4], a3 = (h & 1) ? cb.pair[7] : cb.pair[6];
  const uint32_t b0 = (h & 2) ? a1 : a0, b1 = (h & 2) ? a3 : a2;
  const uint32_t c = (h & 4) ? b1 : b0;
  return (i & 1) ? (c >> 16) : (c & 0xFFFFu);
}

// The byte table with one copy per lane of a wave: entry (byte b, lane l) at
// u32 index 64 b + l, so the byte address of lane l's entry for byte b is
// 256 b + 4 l, which one byte permute builds from the code word (byte b into
// bits 8..15) and the lane's 4 l (bits 0..7). Filled by NT threads.
template <int NT>
__device__ __forceinline__ void fill_code_table64(uint32_t *tbl, const DecCodebook &cb) {
  static_assert((256 * 64 / 4) % NT == 0, "whole 16-byte units per thread");
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 256 * 64 / 4 / NT; ++i) {
    const int u = tid + NT * i;  // 16-byte unit: byte u / 16, lanes 4 (u % 16) ..
    const uint32_t b = uint32_t(u) >> 4;
    const uint32_t v = code_bf16(cb, b >> 4) | (code_bf16(cb, b & 15) << 16);
    reinterpret_cast<u32x4 *>(tbl)[u] = u32x4{v, v, v, v};
  }
}

// lookup_chunk for the 64-copy table: lane4 = 4 * lane (byte 0 of the permute
// source), one v_perm per code byte for the address.
__device__ __forceinline__ void lookup_chunk64(const uint32_t *tbl, uint32_t lane4, const u32x4 &cw,
                                               uint32_t (&v)[16]) {
  const char *tb = reinterpret_cast<const char *>(tbl);
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int y = 0; y < 4; ++y)
      v[4 * w + y] =
          *reinterpret_cast<const uint32_t *>(tb + __builtin_amdgcn_perm(lane4, cw[w], 0x0C0C0004u | (uint32_t(y) << 8)));
}

// Lanes per weight row for a reduction length of K: one 32-element chunk per
// lane and pass, the chunks of a row spread over up to 64 lanes.
__host__ __device__ inline int lanes_per_row(int K) {
  const int cpr = K >> 5;
  return cpr > 32 ? 64 : (cpr > 16 ? 32 : (cpr > 8 ? 16 : (cpr > 4 ? 8 : 4)));
}

// The grouping every workgroup reads: distinct experts d < n (ascending id)
// and their first sorted position first[d] (first[n] = P).
struct DecodeGroups {
  int32_t n;
  int32_t expert[kDecMaxPairs];
  int32_t first[kDecMaxPairs + 1];
};

// Weights of one projection stack.
struct DecStack {
  const uint8_t *packed;  // [E, out, in / 2]
  const float *absmax;    // [E, out, in / 64] (NF4/FP4)
  const uint8_t *scales;  // [E, out, in / 32] (MXFP4)
  int64_t e_bytes, e_blocks;
};

// The operands of one step: ROWS weight rows' 16 code bytes of chunk c and
// their block scales, and the chunk of up to kDecVec input vectors.
template <int ROWS>
struct WChunk {
  u32x4 cw[ROWS];
  float sc[ROWS];
  u32x4 xv[kDecVec][4];
};

template <int ROWS, bool MX>
__device__ __forceinline__ void load_wchunk(const DecStack &W, int e, int K, const int64_t (&wrow)[ROWS], int c,
                                            const uint16_t *__restrict__ vin, const int64_t (&vr)[kDecVec], int np,
                                            WChunk<ROWS> &o) {
  const uint8_t *wp = W.packed + int64_t(e) * W.e_bytes;
  const int64_t row_bytes = K >> 1;
  const int CPR = K >> 5;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    o.cw[r] = *reinterpret_cast<const u32x4 *>(wp + wrow[r] * row_bytes + c * 16);
    o.sc[r] = MX ? e8m0_value(W.scales[int64_t(e) * W.e_blocks + wrow[r] * CPR + c])
                 : W.absmax[int64_t(e) * W.e_blocks + wrow[r] * (K >> 6) + (c >> 1)];
  }
#pragma unroll
  for (int q = 0; q < kDecVec; ++q) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(vin + vr[q] + c * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) o.xv[q][i] = q < np ? src[i] : u32x4{0u, 0u, 0u, 0u};
  }
}

// K parts per expert: the groups of a workgroup split one expert's chunks
// when there are fewer experts than groups (a power of two, at least one
// chunk per lane, and the partial sums fit kPartFloats).
template <int ROWS>
__device__ __forceinline__ int k_parts(int n, int P, int groups, int cpr, int lpr) {
  int kp = 1;
  while (2 * kp * n <= groups && 2 * kp * lpr <= cpr && 2 * kp * P * ROWS <= kPartFloats) kp *= 2;
  return kp;
}

// A lane group's position in its work: item i (expert d = i >> kps, K part
// kp = i & (KP - 1), KP = 1 << kps), the pass over the expert's pairs
// starting at pair q0 (passes of kDecVec), and the step j over the part's
// chunks (the lane's chunk c_lo + li + j * LPR).
struct DecCursor {
  int i, q0, j;
};

struct DecItem {
  int e, s0, cnt, c_lo, c_hi, steps;
};

template <int LPR>
__device__ __forceinline__ DecItem dec_item(const DecodeGroups &G, int i, int kps, int CPR) {
  const int d = i >> kps, kp = i & ((1 << kps) - 1);
  DecItem it;
  it.e = G.expert[d];
  it.s0 = G.first[d];
  it.cnt = G.first[d + 1] - it.s0;
  it.c_lo = (kp * CPR) >> kps;
  it.c_hi = ((kp + 1) * CPR) >> kps;
  it.steps = (it.c_hi - it.c_lo + LPR - 1) / LPR;
  return it;
}

// Input vector rows (times K) of the pairs q0 .. q0 + np - 1 of item it.
template <typename VRow>
__device__ __forceinline__ void vec_rows(const DecItem &it, int q0, int K, VRow vrow, int64_t (&vr)[kDecVec],
                                         int &np) {
  np = min(kDecVec, it.cnt - q0);
#pragma unroll
  for (int q = 0; q < kDecVec; ++q) vr[q] = int64_t(vrow(it.s0 + q0 + (q < np ? q : 0))) * K;
}

// One pass (item it, pairs q0 .. q0 + np - 1, np <= NPB) over all of its
// steps. The operands of the current step arrive in w (loaded one step
// ahead); each step first issues the loads of the cursor's next step (the
// next chunk, or the first chunk of the next pass or item) into w, then
// computes. Lane 0 of the group writes the pass's sums of its K part:
// part_out[q * ROWS + r].
template <int LPR, int ROWS, int NPB, bool MX, typename VRow>
__device__ __forceinline__ void gemv_pass(const DecStack &W, int K, const int64_t (&wrow)[ROWS],
                                          const DecodeGroups &G, int kps, int total, int CPR, const DecItem &it,
                                          DecCursor &cur, WChunk<ROWS> &w, int np,
                                          const uint16_t *__restrict__ vin, VRow vrow, int li, const uint32_t *tl,
                                          float *part_out) {
  constexpr int kGroups = kDecThreads / LPR;
  float part[ROWS][NPB];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int q = 0; q < NPB; ++q) part[r][q] = 0.0f;
  for (int j = 0; j < it.steps; ++j) {
    const bool valid = it.c_lo + li + j * LPR < it.c_hi;
    // the next step's operands
    DecCursor nx = cur;
    if (j + 1 < it.steps) {
      nx.j = j + 1;
    } else if (cur.q0 + kDecVec < it.cnt) {
      nx.q0 = cur.q0 + kDecVec;
      nx.j = 0;
    } else {
      nx.i = cur.i + kGroups;
      nx.q0 = 0;
      nx.j = 0;
    }
    const WChunk<ROWS> cw = w;
    if (nx.i < total) {
      const DecItem ni = nx.i == cur.i ? it : dec_item<LPR>(G, nx.i, kps, CPR);
      const int cn = ni.c_lo + li + nx.j * LPR;
      int64_t vr[kDecVec];
      int nnp;
      vec_rows(ni, nx.q0, K, vrow, vr, nnp);
      load_wchunk<ROWS, MX>(W, ni.e, K, wrow, cn < ni.c_hi ? cn : ni.c_lo, vin, vr, nnp, w);
    }
    if (valid) {
      // a row's 16 lookups are issued together, the next row's under this
      // row's products (the scheduler would otherwise wait on each lookup)
      uint32_t v[2][16];
      lookup_chunk(tl, cw.cw[0], v[0]);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        if (r + 1 < ROWS) lookup_chunk(tl, cw.cw[r + 1], v[(r + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < NPB; ++q) {
          float acc = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc = dot2_bf16(v[r & 1][i], cw.xv[q][i >> 2][i & 3], acc);
          part[r][q] += acc * cw.sc[r];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (j + 1 == it.steps) cur = nx;
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int q = 0; q < NPB; ++q) part[r][q] = group_sum<LPR>(part[r][q]);
  if (li == 0) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
      for (int q = 0; q < NPB; ++q)
        if (q < np) part_out[q * ROWS + r] = part[r][q];
  }
}

// The block's GEMV for every distinct expert: ROWS weight rows (tile row r is
// weight row row_of(r), or none when row_of(r) < 0) of each expert against
// its pairs' input vectors (pair at sorted position s: vin + vrow(s) * K).
// Items (expert d, K part kp) go to lane group i % groups; each group walks
// its items, passes and chunk steps with the next step's operands in flight.
// Partial sums go to part[(kp * P + s) * ROWS + r].
template <int LPR, int ROWS, bool MX, typename RowOf, typename VRow>
__device__ __forceinline__ void gemv_block(const DecStack &W, int K, int P, const DecodeGroups &G, RowOf row_of,
                                           const uint16_t *__restrict__ vin, VRow vrow, const uint32_t *tbl,
                                           float *part, int KP) {
  const int tid = threadIdx.x, g = tid / LPR, li = tid % LPR;
  const int CPR = K >> 5;
  const int total = G.n * KP;
  const int kps = __builtin_ctz(KP);
  const uint32_t *tl = tbl + (tid & (kTblCopies - 1));
  int64_t wrow[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int w = row_of(r);
    wrow[r] = w < 0 ? 0 : w;  // a row without weights reads row 0; its sum is not kept
  }
  DecCursor cur{g, 0, 0};
  if (cur.i >= total) return;
  WChunk<ROWS> w;
  {
    const DecItem it = dec_item<LPR>(G, cur.i, kps, CPR);
    const int c = it.c_lo + li;
    int64_t vr[kDecVec];
    int np;
    vec_rows(it, 0, K, vrow, vr, np);
    load_wchunk<ROWS, MX>(W, it.e, K, wrow, c < it.c_hi ? c : it.c_lo, vin, vr, np, w);
  }
  while (cur.i < total) {
    const DecItem it = dec_item<LPR>(G, cur.i, kps, CPR);
    const int kp = cur.i & (KP - 1);
    const int np = min(kDecVec, it.cnt - cur.q0);
    float *out = part + (kp * P + it.s0 + cur.q0) * ROWS;
    static_assert(kDecVec == 2, "buckets 1, 2");
    if (np <= 1)
      gemv_pass<LPR, ROWS, 1, MX>(W, K, wrow, G, kps, total, CPR, it, cur, w, np, vin, vrow, li, tl, out);
    else
      gemv_pass<LPR, ROWS, 2, MX>(W, K, wrow, G, kps, total, CPR, it, cur, w, np, vin, vrow, li, tl, out);
  }
}

// Sum of the K parts of sorted position s, tile row r (fixed order).
template <int ROWS>
__device__ __forceinline__ float part_sum(const float *part, int KP, int P, int s, int r) {
  float v = part[s * ROWS + r];
  for (int kp = 1; kp < KP; ++kp) v += part[(kp * P + s) * ROWS + r];
  return v;
}

// LDS of the gate_up launch. The routing scratch shares space with the
// sorting arrays and the partial sums, which are written once the routing is
// done.
struct DecodeGuLds {
  uint32_t tbl[256 * kTblCopies];
  DecodeGroups groups;
  int32_t vrow[kDecMaxPairs];  // the token of the pair at each sorted position
  int32_t idx[kDecMaxPairs];  // routed expert of flat pair t * k + j
  float w[kDecMaxPairs];      // its weight
  int32_t sp[kDecMaxPairs];   // pair at sorted position
  union {
    RouteLds route[kRouteWaves];
    struct {
      float part[kPartFloats];
      int32_t key[kDecMaxPairs];
      int32_t se[kDecMaxPairs];   // expert at sorted position
      int32_t pos[kDecMaxPairs];  // sorted position of pair
      int32_t wsum[kDecThreads / 64];
    };
  };
};

// Routing (when given logits) and grouping of the P <= kDecMaxPairs pairs:
// pairs sorted by (expert, flat pair id). NT threads (a multiple of 256):
// wave t routes token t, thread p < kDecMaxPairs handles pair p, and every
// thread takes part in the barriers.
// MAXE: the largest expert count the caller routes (E <= MAXE); at most 256
// keeps only the router instances of up to four logits per lane.
template <int NT, int MAXE, typename Lds>
__device__ __forceinline__ void decode_group(const float *__restrict__ logits, int E, int k, int T,
                                             const int32_t *__restrict__ idx_in, const float *__restrict__ w_in,
                                             Lds &L) {
  static_assert(NT % kDecMaxPairs == 0 && kDecMaxPairs % 64 == 0, "every pair has a thread");
  constexpr int kWaves = NT / 64, kPairWaves = kDecMaxPairs / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int P = T * k;
  if (logits) {
    for (int t = wv; t < T; t += kWaves) {
      if constexpr (MAXE <= 256) {
        if (E <= 64)
          route_token_per<1>(logits, t, E, k, lane, L.idx, L.w, nullptr, L.route[wv]);
        else if (E <= 128)
          route_token_per<2>(logits, t, E, k, lane, L.idx, L.w, nullptr, L.route[wv]);
        else
          route_token_per<4>(logits, t, E, k, lane, L.idx, L.w, nullptr, L.route[wv]);
      } else {
        route_token(logits, t, E, k, lane, L.idx, L.w, nullptr, L.route[wv]);
      }
    }
  } else if (tid < P) {
    L.idx[tid] = safe_expert(idx_in[tid], E);
    L.w[tid] = w_in[tid];
  }
  __syncthreads();
  const int p = tid;
  // unique sort key: expert, then pair id (stable)
  const int key = p < P ? L.idx[p] * kDecMaxPairs + p : 0x7FFFFFFF;
  if (NT == kDecMaxPairs || p < kDecMaxPairs) L.key[p] = key;
  __syncthreads();
  int pos = 0;
  const int4 *k4 = reinterpret_cast<const int4 *>(L.key);
  for (int q = 0; q < (P + 3) / 4; ++q) {
    const int4 v = k4[q];
    pos += (v.x < key) + (v.y < key) + (v.z < key) + (v.w < key);
  }
  if (p < P) {
    L.sp[pos] = p;
    L.se[pos] = key / kDecMaxPairs;
    L.pos[p] = pos;
    L.vrow[pos] = p / k;
  }
  __syncthreads();
  // distinct experts: sorted position p starts a segment
  const bool starts = p < P && (p == 0 || L.se[p - 1] != L.se[p]);
  const uint64_t fm = __ballot(starts);
  int d = __popcll(fm & ((1ull << lane) - 1));
  if (lane == 0 && wv < kPairWaves) L.wsum[wv] = __popcll(fm);
  __syncthreads();
  int n = 0;
  for (int v = 0; v < kPairWaves; ++v) {
    d += v < wv ? L.wsum[v] : 0;
    n += L.wsum[v];
  }
  if (starts) {
    L.groups.first[d] = p;
    L.groups.expert[d] = L.se[p];
  }
  if (p == 0) {
    L.groups.first[n] = P;
    L.groups.n = n;
  }
  __syncthreads();
}

// Workgroup 0's copy of the grouping for the down launch, and the routing
// outputs (ids and weights by flat pair) when the launch routed.
template <typename Lds>
__device__ __forceinline__ void decode_write_plan(const Lds &L, int P, int n, bool routed, int32_t *__restrict__ idx_io,
                                                  float *__restrict__ w_io, DecodePlan *__restrict__ plan) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    plan->n = n;
    plan->first[n] = P;
  }
  if (tid < n) {
    plan->expert[tid] = L.groups.expert[tid];
    plan->first[tid] = L.groups.first[tid];
  }
  if (tid < P) {
    plan->weight[tid] = L.w[L.sp[tid]];
    plan->pos[tid] = L.pos[tid];
    if (routed) {
      idx_io[tid] = L.idx[tid];
      w_io[tid] = L.w[tid];
    }
  }
}

template <int LPR, bool MX>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(kDecWgPerCu))) void decode_gate_up_kernel(const float *__restrict__ logits, int E, int k,
                                                                     int T, int32_t *__restrict__ idx_io,
                                                                     float *__restrict__ w_io, DecStack W, int H,
                                                                     int I, const uint16_t *__restrict__ x, DecCodebook cb,
                                                                     DecodePlan *__restrict__ plan,
                                                                     uint16_t *__restrict__ a) {
  __shared__ DecodeGuLds L;
  fill_code_table(L.tbl, cb);  // its stores overlap the routing's loads
  decode_group<kDecThreads, kMaxE>(logits, E, k, T, logits ? nullptr : idx_io, w_io, L);
  const int tid = threadIdx.x, P = T * k, n = L.groups.n;
  if (blockIdx.x == 0) {
    decode_write_plan(L, P, n, logits != nullptr, idx_io, w_io, plan);
    __syncthreads();  // pos is read above; the partial sums share its space
  }
  const int KP = k_parts<kGuRows>(n, P, kDecThreads / LPR, H >> 5, LPR);
  const int nblk = (I + kGuUnits - 1) / kGuUnits;
  for (int b = int(blockIdx.x); b < nblk; b += int(gridDim.x)) {
    const int u0 = b * kGuUnits;
    // tile row r: gate row u0 + r, then (r >= kGuUnits) up row I + u0 + r - kGuUnits
    auto row_of = [&](int r) {
      const int u = u0 + (r % kGuUnits);
      return u < I ? (r < kGuUnits ? u : I + u) : -1;
    };
    gemv_block<LPR, kGuRows, MX>(W, H, P, L.groups, row_of, x, [&](int s) { return L.vrow[s]; }, L.tbl, L.part,
                                 KP);
    __syncthreads();
    if (tid < P * kGuUnits) {
      const int s = tid / kGuUnits, i = tid % kGuUnits;
      if (u0 + i < I) {
        const float g = part_sum<kGuRows>(L.part, KP, P, s, i), u = part_sum<kGuRows>(L.part, KP, P, s, kGuUnits + i);
        a[int64_t(s) * I + u0 + i] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
      }
    }
    __syncthreads();
  }
}

// ---- gate_up for rows of H = 2048: one 32-element chunk per lane of a wave ----
// One workgroup of 1024 threads per CU instead of three of 256: one code
// table (a copy per lane, so one byte permute per code byte builds its
// address), and the tokens' x rows staged in LDS once, so a step loads only
// the two weight rows' codes and scales (into one of kRingDepth register sets,
// statically indexed: the sets are reloaded in place, not copied). A
// workgroup block is `units` gate/up units; item (expert d, unit u) of a
// block goes to wave i % 16. Per pair the arithmetic is the 256-thread
// kernel's with 64 lanes per row (the same products, chunk scaling and
// lane sums), so both give the same bits.
constexpr int kRingThreads = 1024;
constexpr int kRingWaves = kRingThreads / 64;
constexpr int kRingH = 2048;       // the row length (H) this kernel covers
constexpr int kRingX4 = kRingH / 8;  // 16-byte units of an x row
constexpr int kRingMaxUnits = 4;   // units per workgroup block
constexpr int kRingDepth = 4;      // weight register sets per wave
constexpr int kRingMaxE = 256;     // expert counts this kernel routes

struct DecodeRingLds {
  uint32_t tbl[256 * 64];  // one copy per lane (fill_code_table64)
  // x of token t: unit g (elements 8 g .. 8 g + 7) of the row at
  // t * kRingX4 + (g % 4) * 64 + g / 4, so lane l reads its chunk's four
  // units at l, l + 64, l + 128, l + 192 (consecutive lanes, no conflicts)
  u32x4 xs[kDecodeMaxT * kRingX4];
  DecodeGroups groups;
  int32_t vrow[kDecMaxPairs];
  int32_t idx[kDecMaxPairs];
  float w[kDecMaxPairs];
  int32_t sp[kDecMaxPairs];
  int32_t pos[kDecMaxPairs];
  union {
    RouteLds route[kDecodeMaxT];  // wave t routes token t
    struct {
      float part[kDecMaxPairs * 2 * kRingMaxUnits];  // [sorted pair][gate units | up units]
      int32_t key[kDecMaxPairs];
      int32_t se[kDecMaxPairs];
      int32_t wsum[kDecMaxPairs / 64];
    };
  };
};

// The codes and block scales of an item: gate row u and up row I + u of
// expert e, the lane's 16 bytes (chunk lane) of each.
struct RingSet {
  u32x4 cw[2];
  float sc[2];
};

// Offsets are 32-bit: the launch takes these kernels only for stacks below
// 2^31 bytes, so each address is the stack's base plus one unsigned offset.
// MX: the chunk's E8M0 scale byte (one per 32 elements) instead of the fp32
// absmax of its 64-element block.
template <bool MX>
__device__ __forceinline__ void ring_load(const DecStack &W, int I, int e, int u, int lane, RingSet &o) {
  const uint32_t eb = uint32_t(W.e_bytes), ea = uint32_t(W.e_blocks);
  const uint32_t w0 = uint32_t(e) * eb + uint32_t(u) * (kRingH / 2) + uint32_t(lane) * 16;
  const uint32_t wd = uint32_t(I) * (kRingH / 2);  // gate -> up row
  o.cw[0] = *reinterpret_cast<const u32x4 *>(W.packed + w0);
  o.cw[1] = *reinterpret_cast<const u32x4 *>(W.packed + (w0 + wd));
  if constexpr (MX) {
    const uint32_t s0 = uint32_t(e) * ea + uint32_t(u) * (kRingH / kMxBlock) + uint32_t(lane);
    const uint32_t sd = uint32_t(I) * (kRingH / kMxBlock);
    o.sc[0] = e8m0_value(W.scales[s0]);
    o.sc[1] = e8m0_value(W.scales[s0 + sd]);
  } else {
    const uint32_t a0 = uint32_t(e) * ea + uint32_t(u) * (kRingH / kBlock) + (uint32_t(lane) >> 1);
    const uint32_t ad = uint32_t(I) * (kRingH / kBlock);
    o.sc[0] = W.absmax[a0];
    o.sc[1] = W.absmax[a0 + ad];
  }
}

template <bool MX>
__global__ __launch_bounds__(kRingThreads) void decode_gate_up_ring_kernel(
    const float *__restrict__ logits, int E, int k, int T, int32_t *__restrict__ idx_io, float *__restrict__ w_io,
    DecStack W, int I, int units, const uint16_t *__restrict__ x, DecCodebook cb, DecodePlan *__restrict__ plan,
    uint16_t *__restrict__ a) {
  static_assert(kRingH / 32 == 64 && kBlock == 64, "one chunk per lane, two chunks per block");
  static_assert(kDecMaxPairs * kRingMaxUnits <= 1024 && kRingMaxUnits <= 4, "item / ub by multiply and shift");
  __shared__ DecodeRingLds L;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  fill_code_table64<kRingThreads>(L.tbl, cb);
  {
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(x);
    for (int j = tid; j < T * kRingX4; j += kRingThreads) {
      const int t = j / kRingX4, g = j % kRingX4;
      L.xs[t * kRingX4 + (g & 3) * 64 + (g >> 2)] = xg[int64_t(t) * kRingX4 + g];
    }
  }
  decode_group<kRingThreads, kRingMaxE>(logits, E, k, T, logits ? nullptr : idx_io, w_io, L);
  const int P = T * k, n = L.groups.n;
  if (blockIdx.x == 0) decode_write_plan(L, P, n, logits != nullptr, idx_io, w_io, plan);
  const uint32_t lane4 = uint32_t(lane) * 4;
  const u32x4 *xl = L.xs + lane;
  const int nblk = (I + units - 1) / units;
  for (int b = int(blockIdx.x); b < nblk; b += int(gridDim.x)) {
    const int u0 = b * units, ub = min(units, I - u0);
    const int items = n * ub;
    // this wave's items wv, wv + 16, ...: q-th at i = wv + 16 q
    const int nq = wv < items ? (items - wv + kRingWaves - 1) / kRingWaves : 0;
    // i / ub as (i * m) >> 16, m = ceil(2^16 / ub): exact for ub <= 4 and
    // i < 1024 (the error stays below 1024 * 2 / (3 * 2^16) of a unit)
    const uint32_t m = (65536u + uint32_t(ub) - 1) / uint32_t(ub);
    auto item_d = [&](int q) { return int((uint32_t(wv + q * kRingWaves) * m) >> 16); };
    auto item_u = [&](int q, int d) { return u0 + (wv + q * kRingWaves) - d * ub; };
    RingSet ring[kRingDepth];
    dec_static_for<kRingDepth>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      if (r < nq) {
        const int d = item_d(r);
        ring_load<MX>(W, I, L.groups.expert[d], item_u(r, d), lane, ring[r]);
      }
    });
    for (int q0 = 0; q0 < nq; q0 += kRingDepth) {
      dec_static_for<kRingDepth>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const int q = q0 + r;
        if (q < nq) {
          const int d = item_d(q), u = item_u(q, d);
          const int s0 = L.groups.first[d], cnt = L.groups.first[d + 1] - s0;
          uint32_t v[2][16];
          lookup_chunk64(L.tbl, lane4, ring[r].cw[0], v[0]);
          lookup_chunk64(L.tbl, lane4, ring[r].cw[1], v[1]);
          const float sg = ring[r].sc[0], su = ring[r].sc[1];
          __builtin_amdgcn_sched_barrier(0);
          // this set's next item, loaded under the products
          if (q + kRingDepth < nq) {
            const int d2 = item_d(q + kRingDepth);
            ring_load<MX>(W, I, L.groups.expert[d2], item_u(q + kRingDepth, d2), lane, ring[r]);
          }
          __builtin_amdgcn_sched_barrier(0);
          for (int pp = 0; pp < cnt; ++pp) {
            const int sp = s0 + pp;
            const u32x4 *xr = xl + L.vrow[sp] * kRingX4;
            u32x4 xq[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xq[i] = xr[i * 64];
            float ag = 0.0f, au = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              ag = dot2_bf16(v[0][i], xq[i >> 2][i & 3], ag);
              au = dot2_bf16(v[1][i], xq[i >> 2][i & 3], au);
            }
            float pg = 0.0f, pu = 0.0f;
            pg += ag * sg;
            pu += au * su;
            pg = group_sum<64>(pg);
            pu = group_sum<64>(pu);
            if (lane == 0) {
              L.part[sp * (2 * kRingMaxUnits) + (u - u0)] = pg;
              L.part[sp * (2 * kRingMaxUnits) + kRingMaxUnits + (u - u0)] = pu;
            }
          }
        }
      });
    }
    __syncthreads();
    for (int j = tid; j < P * ub; j += kRingThreads) {
      const int sp = j / ub, i = j % ub;
      const float g = L.part[sp * (2 * kRingMaxUnits) + i], uu = L.part[sp * (2 * kRingMaxUnits) + kRingMaxUnits + i];
      a[int64_t(sp) * I + u0 + i] = f32_to_bf16(g / (1.0f + __expf(-g)) * uu);
    }
    __syncthreads();
  }
}

struct DecodeDnLds {
  uint32_t tbl[256 * kTblCopies];
  float part[kPartFloats];
  DecodeGroups groups;
  float weight[kDecMaxPairs];
  int32_t pos[kDecMaxPairs];
};

template <int LPR, bool MX>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(kDecWgPerCu))) void decode_down_kernel(DecStack W, int H, int I, int T, int k, DecCodebook cb,
                                                                  const DecodePlan *__restrict__ plan,
                                                                  const uint16_t *__restrict__ a,
                                                                  uint16_t *__restrict__ y) {
  __shared__ DecodeDnLds L;
  const int tid = threadIdx.x, P = T * k;
  // the grouping's loads are issued before the table fill's stores
  const int n = plan->n;
  const bool pt = tid < P;
  const float wt = pt ? plan->weight[tid] : 0.0f;
  const int ps = pt ? plan->pos[tid] : 0;
  const int ex = tid < n ? plan->expert[tid] : 0, fs = tid < n ? plan->first[tid] : 0;
  fill_code_table(L.tbl, cb);
  if (tid < n) {
    L.groups.expert[tid] = ex;
    L.groups.first[tid] = fs;
  }
  if (tid == 0) {
    L.groups.n = n;
    L.groups.first[n] = P;
  }
  if (pt) {
    L.weight[tid] = wt;
    L.pos[tid] = ps;
  }
  __syncthreads();
  const int KP = k_parts<kDnRows>(n, P, kDecThreads / LPR, I >> 5, LPR);
  const int nblk = (H + kDnRows - 1) / kDnRows;
  for (int b = int(blockIdx.x); b < nblk; b += int(gridDim.x)) {
    const int r0 = b * kDnRows;
    auto row_of = [&](int r) { return r0 + r < H ? r0 + r : -1; };
    gemv_block<LPR, kDnRows, MX>(W, I, P, L.groups, row_of, a, [](int s) { return s; }, L.tbl, L.part, KP);
    __syncthreads();
    // y rows of this block: each token's pairs in slot order
    if (tid < T * kDnRows) {
      const int t = tid / kDnRows, r = tid % kDnRows;
      if (r0 + r < H) {
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) {
          const int s = L.pos[t * k + j];
          acc += L.weight[s] * part_sum<kDnRows>(L.part, KP, P, s, r);
        }
        y[int64_t(t) * H + r0 + r] = f32_to_bf16(acc);
      }
    }
    __syncthreads();
  }
}

// ---- down for rows of I <= 1024 whose routed inputs fit in LDS ----
// The same workgroup shape as the gate_up launch above: 1024 threads per
// CU, one code table, the P rows of a staged in LDS once, and a static ring
// of weight register sets per wave. A workgroup block is kDnRingRows rows of
// H; item (expert d, quarter q) is rows 4 q .. 4 q + 3 of the block, and the
// two 32-lane halves of a wave take two rows each (lane c < I / 32 holds
// chunk c). Per pair the arithmetic is the 256-thread kernel's with 32 lanes
// per row, and the combine follows in the same workgroup in slot order, so
// both give the same bits.
constexpr int kDnRingRows = 8;                // rows of H per workgroup block
constexpr int kDnRingA = 48 * 1024;           // a elements (P * I) staged in LDS at most
constexpr int kDnRingMaxI = 1024;             // one chunk per lane of a 32-lane half

struct DecodeDnRingLds {
  uint32_t tbl[256 * kTblCopies];
  // a of sorted pair s: unit g (elements 8 g .. 8 g + 7, g < 4 C with C = I / 32
  // chunks) at s * 4 C + (g % 4) * C + g / 4, so lane c reads its chunk's units
  // at c, c + C, c + 2 C, c + 3 C (consecutive lanes, no conflicts)
  u32x4 as[kDnRingA / 8];
  float part[kDecMaxPairs * kDnRingRows];
  DecodeGroups groups;
  float weight[kDecMaxPairs];
  int32_t pos[kDecMaxPairs];
};

template <bool MX>
__global__ __launch_bounds__(kRingThreads) void decode_down_ring_kernel(DecStack W, int H, int I, int T, int k,
                                                                        DecCodebook cb,
                                                                        const DecodePlan *__restrict__ plan,
                                                                        const uint16_t *__restrict__ a,
                                                                        uint16_t *__restrict__ y) {
  __shared__ DecodeDnRingLds L;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int P = T * k, C = I >> 5, U4 = I >> 3;  // chunks per row, 16-byte units per row
  // the grouping's loads are issued before the table fill's stores
  const int n = plan->n;
  const bool pt = tid < P;
  const float wt = pt ? plan->weight[tid] : 0.0f;
  const int ps = pt ? plan->pos[tid] : 0;
  const int ex = tid < n ? plan->expert[tid] : 0, fs = tid < n ? plan->first[tid] : 0;
  if (tid < kDecThreads) fill_code_table(L.tbl, cb);
  {
    const u32x4 *ag = reinterpret_cast<const u32x4 *>(a);
    for (int j = tid; j < P * U4; j += kRingThreads) {
      const int sp = j / U4, g = j - sp * U4;
      L.as[sp * U4 + (g & 3) * C + (g >> 2)] = ag[j];
    }
  }
  if (tid < n) {
    L.groups.expert[tid] = ex;
    L.groups.first[tid] = fs;
  }
  if (tid == 0) {
    L.groups.n = n;
    L.groups.first[n] = P;
  }
  if (pt) {
    L.weight[tid] = wt;
    L.pos[tid] = ps;
  }
  __syncthreads();
  const uint32_t *tl = L.tbl + (lane & (kTblCopies - 1));
  const int half = lane >> 5, c = lane & 31;
  const bool act = c < C;
  const int cc = act ? c : 0;  // idle lanes load chunk 0 and contribute nothing
  const u32x4 *al = L.as + cc;
  const int nblk = (H + kDnRingRows - 1) / kDnRingRows;
  constexpr int kQ = kDnRingRows / 4;  // items per expert and block
  for (int b = int(blockIdx.x); b < nblk; b += int(gridDim.x)) {
    const int r0 = b * kDnRingRows;
    const int items = n * kQ;
    const int nq = wv < items ? (items - wv + kRingWaves - 1) / kRingWaves : 0;
    // item i = wv + 16 q: expert d = i / kQ, rows r0 + 4 (i % kQ) + 2 half + {0, 1}
    auto item_row = [&](int q) { return r0 + 4 * ((wv + q * kRingWaves) % kQ) + 2 * half; };
    auto load = [&](int q, RingSet &o) {
      const int d = (wv + q * kRingWaves) / kQ, row = item_row(q);
      const uint32_t e = uint32_t(L.groups.expert[d]);
      const uint32_t wb = e * uint32_t(W.e_bytes) + uint32_t(cc) * 16;
      const uint32_t ab = e * uint32_t(W.e_blocks) + (MX ? uint32_t(cc) : uint32_t(cc) >> 1);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t rr = uint32_t(min(row + j, H - 1));
        o.cw[j] = *reinterpret_cast<const u32x4 *>(W.packed + (wb + rr * uint32_t(I >> 1)));
        if constexpr (MX)
          o.sc[j] = e8m0_value(W.scales[ab + rr * uint32_t(I / kMxBlock)]);
        else
          o.sc[j] = W.absmax[ab + rr * uint32_t(I / kBlock)];
      }
    };
    RingSet ring[kRingDepth];
    dec_static_for<kRingDepth>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      if (r < nq) load(r, ring[r]);
    });
    for (int q0 = 0; q0 < nq; q0 += kRingDepth) {
      dec_static_for<kRingDepth>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const int q = q0 + r;
        if (q < nq) {
          const int d = (wv + q * kRingWaves) / kQ, row = item_row(q);
          const int s0 = L.groups.first[d], cnt = L.groups.first[d + 1] - s0;
          uint32_t v[2][16];
          lookup_chunk(tl, ring[r].cw[0], v[0]);
          lookup_chunk(tl, ring[r].cw[1], v[1]);
          const float s_0 = ring[r].sc[0], s_1 = ring[r].sc[1];
          __builtin_amdgcn_sched_barrier(0);
          if (q + kRingDepth < nq) load(q + kRingDepth, ring[r]);
          __builtin_amdgcn_sched_barrier(0);
          for (int pp = 0; pp < cnt; ++pp) {
            const int sp = s0 + pp;
            const u32x4 *ar = al + sp * U4;
            u32x4 xq[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xq[i] = ar[i * C];
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              a0 = dot2_bf16(v[0][i], xq[i >> 2][i & 3], a0);
              a1 = dot2_bf16(v[1][i], xq[i >> 2][i & 3], a1);
            }
            float p0 = 0.0f, p1 = 0.0f;
            if (act) {
              p0 += a0 * s_0;
              p1 += a1 * s_1;
            }
            p0 = group_sum<32>(p0);
            p1 = group_sum<32>(p1);
            if (c == 0) {
              L.part[sp * kDnRingRows + (row - r0)] = p0;
              L.part[sp * kDnRingRows + (row - r0) + 1] = p1;
            }
          }
        }
      });
    }
    __syncthreads();
    // y rows of this block: each token's pairs in slot order
    for (int j = tid; j < T * kDnRingRows; j += kRingThreads) {
      const int t = j / kDnRingRows, rr = j % kDnRingRows;
      if (r0 + rr < H) {
        float acc = 0.0f;
        for (int jj = 0; jj < k; ++jj) {
          const int sp = L.pos[t * k + jj];
          acc += L.weight[sp] * L.part[sp * kDnRingRows + rr];
        }
        y[int64_t(t) * H + r0 + rr] = f32_to_bf16(acc);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_decode_forward(const MoePlan &p, const e4b_moe_layer *L, const uint16_t *x,
                                 const float *logits, int32_t *idx, float *wts, uint16_t *y,
                                 char *ws, hipStream_t s, const e4b_kernel_events *ev) {
  static_assert(kDecMaxPairs * kGuRows <= kPartFloats && kDecMaxPairs * kDnRows <= kPartFloats,
                "one K part always fits");
  DecodePlan *plan = reinterpret_cast<DecodePlan *>(ws + p.off_dmap);
  uint16_t *a = reinterpret_cast<uint16_t *>(ws + p.off_a);
  const int H = int(p.H), I = int(p.I), T = int(p.T), k = int(p.k), E = int(p.E);
  const e4b_stack &gu = L->gate_up, &dn = L->down;
  const bool mx = gu.codebook == E4B_CB_MXFP4;
  const int blk = mx ? kMxBlock : kBlock;
  const DecStack Wgu{gu.packed, gu.absmax, gu.scales, gu.out * gu.in / 2, gu.out * gu.in / blk};
  const DecStack Wdn{dn.packed, dn.absmax, dn.scales, dn.out * dn.in / 2, dn.out * dn.in / blk};
  // the codebook in bf16 (round to nearest even; the tables hold no NaN)
  DecCodebook cbk;
  auto bf16_rne = [](uint32_t f) { return (f + 0x7FFFu + ((f >> 16) & 1u)) >> 16; };
  for (int i = 0; i < 8; ++i)
    cbk.pair[i] = bf16_rne(kCodebookBits[p.codebook][2 * i]) | (bf16_rne(kCodebookBits[p.codebook][2 * i + 1]) << 16);
  // one round of workgroups: at most kDecWgPerCu per compute unit
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  const int64_t cap = int64_t(cus > 0 ? cus : 1) * kDecWgPerCu;
  auto grid_of = [cap](int64_t blocks) { return dim3(uint32_t(blocks < cap ? blocks : cap)); };
  const dim3 grid_gu = grid_of((I + kGuUnits - 1) / kGuUnits), grid_dn = grid_of((H + kDnRows - 1) / kDnRows);
  const dim3 block(kDecThreads);
  // the kernels for the lanes per row that H (gate_up) and I (down) take
  auto with_lpr = [](int K, auto f) {
    switch (lanes_per_row(K)) {
      case 4: return f(std::integral_constant<int, 4>());
      case 8: return f(std::integral_constant<int, 8>());
      case 16: return f(std::integral_constant<int, 16>());
      case 32: return f(std::integral_constant<int, 32>());
      default: return f(std::integral_constant<int, 64>());
    }
  };
  // the 1024-thread launches address a stack with 32-bit offsets
  auto small = [](const e4b_stack &st) { return st.E * st.out * st.in / 2 < (int64_t(1) << 31); };
  if (H == kRingH && E <= kRingMaxE && small(gu)) {
    // one 1024-thread workgroup per CU, blocks of up to kRingMaxUnits units
    const int units = int(std::min<int64_t>(kRingMaxUnits, std::max<int64_t>(1, (I + cus - 1) / std::max(cus, 1))));
    const int64_t nblk = (I + units - 1) / units;
    const dim3 grid(uint32_t(std::min<int64_t>(nblk, std::max(cus, 1))));
    err = mx ? launch_k(ev, E4B_K_DECODE_GATE_UP, decode_gate_up_ring_kernel<true>, grid, dim3(kRingThreads), s, logits,
                        E, k, T, idx, wts, Wgu, I, units, x, cbk, plan, a)
             : launch_k(ev, E4B_K_DECODE_GATE_UP, decode_gate_up_ring_kernel<false>, grid, dim3(kRingThreads), s,
                        logits, E, k, T, idx, wts, Wgu, I, units, x, cbk, plan, a);
  } else {
    err = with_lpr(H, [&](auto lpr) {
    constexpr int LPR = decltype(lpr)::value;
    return mx ? launch_k(ev, E4B_K_DECODE_GATE_UP, decode_gate_up_kernel<LPR, true>, grid_gu, block, s, logits, E, k,
                         T, idx, wts, Wgu, H, I, x, cbk, plan, a)
              : launch_k(ev, E4B_K_DECODE_GATE_UP, decode_gate_up_kernel<LPR, false>, grid_gu, block, s, logits, E,
                         k, T, idx, wts, Wgu, H, I, x, cbk, plan, a);
    });
  }
  if (err != hipSuccess) return err;
  if (I <= kDnRingMaxI && int64_t(T) * k * I <= kDnRingA && small(dn)) {
    const dim3 grid(uint32_t(std::min<int64_t>((H + kDnRingRows - 1) / kDnRingRows, std::max(cus, 1))));
    return mx ? launch_k(ev, E4B_K_DECODE_DOWN, decode_down_ring_kernel<true>, grid, dim3(kRingThreads), s, Wdn, H, I,
                         T, k, cbk, plan, a, y)
              : launch_k(ev, E4B_K_DECODE_DOWN, decode_down_ring_kernel<false>, grid, dim3(kRingThreads), s, Wdn, H, I,
                         T, k, cbk, plan, a, y);
  }
  return with_lpr(I, [&](auto lpr) {
    constexpr int LPR = decltype(lpr)::value;
    return mx ? launch_k(ev, E4B_K_DECODE_DOWN, decode_down_kernel<LPR, true>, grid_dn, block, s, Wdn, H, I, T, k,
                         cbk, plan, a, y)
              : launch_k(ev, E4B_K_DECODE_DOWN, decode_down_kernel<LPR, false>, grid_dn, block, s, Wdn, H, I, T, k,
                         cbk, plan, a, y);
  });
}

}  // namespace e4b
