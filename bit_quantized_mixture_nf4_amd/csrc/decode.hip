// decode.hip -- forward for T <= 8 tokens as bandwidth-bound dequant-GEMVs.
//
// The 0.4.0 README ("Inference" section) describes the decode fast path: a
// single-token forward skips the one-hot grouping and its per-expert host
// syncs, and single-row projections read the packed 4-bit weight directly
// instead of materializing a dequantized expert. Here, for T <= 8:
//   prep     one workgroup groups the <= 8*k routed pairs by expert (stable)
//            and writes one self-contained work item per GEMV workgroup;
//   gate_up  one workgroup per (distinct expert, block of gate/up row pairs):
//            every packed byte is read once for all tokens routed to that
//            expert; a = silu(g) * u is written as bf16;
//   down     one workgroup per (distinct expert, block of rows of H);
//   combine  the shared deterministic gather-combine.
// No MFMA: the decode projections are bandwidth-bound GEMVs on the vector
// ALU. Each code byte is expanded through an LDS table into two bf16 codebook
// values and contracted with bf16 inputs by v_dot2_f32_bf16 in fp32; the block
// absmax scales each lane's partial sum.
#include "device.h"
#include "kernels.h"
#include "route_dev.h"

namespace e4b {

constexpr int kDecWaves = 8;  // waves of a decode workgroup: one K eighth each
constexpr int kDecThreads = 64 * kDecWaves;

// Workspace layout of the decode path (inside the permutation region, plus a
// work map after the forward buffers).
struct DecodeWs {
  int32_t *sorted;      // [P] pair id at sorted position
  int32_t *pos;         // [P] sorted position of pair id
  int32_t *map_count;   // [2] workgroups with work: gate_up, down
  int4 *map_gu;         // [min(E, P) * I / 16] work item of gate_up workgroup b
  int4 *map_dn;         // [min(E, P) * H / 16] work item of down workgroup b
                        // (sized for tiles of 16 units; tiles are kDecTile)
};

// A work item is everything a GEMV workgroup needs before its loads:
//   x: expert | token count << 16     y: first tile | tile count << 16
//   z: first sorted position          w: token of sorted position z + q in
//                                        bits [4q, 4q + 4) (q < 8; T <= 8)
__host__ __device__ inline int4 dec_item(int e, int np, int tile0, int nt, int s0, int toks) {
  return int4{e | (np << 16), tile0 | (nt << 16), s0, toks};
}

// Relative cost of a tile of an expert with np tokens, in eighths of the cost
// of a one-token tile (measured: the ALU work per byte grows with the token
// bucket; faster for gate_up, whose rows are longer).
__device__ __forceinline__ int dec_tile_cost8(int np, bool gate_up) {
  const int npb = np <= 1 ? 1 : (np <= 2 ? 2 : (np <= 4 ? 4 : 8));
  return gate_up ? 8 + 2 * (npb - 1) : 8 + 4 * (npb - 1) / 3;
}

// v shifted right by N lanes inside each 16-lane row, zero at the row start.
template <int N>
__device__ __forceinline__ int row_shr(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x110 + N, 0xF, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes: DPP shifts inside each row, then
// the row totals (read from lanes 15, 31, 47) added to the rows after them.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
  v += row_shr<1>(v);
  v += row_shr<2>(v);
  v += row_shr<4>(v);
  v += row_shr<8>(v);
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31),
            t2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row > 0 ? t0 : 0) + (row > 1 ? t1 : 0) + (row > 2 ? t2 : 0);
}

__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_inclusive_scan(v, threadIdx.x & 63), 63);
}

// One workgroup: routes the tokens when router logits are given (one
// wavefront per token, the same selection as the router kernel), groups the
// P <= 256 routed pairs by expert (stable), lists the distinct experts in
// ascending order and writes the work maps of the two GEMV launches (chunks
// of tiles of kDecTile units per distinct expert). Ranks come from
// comparisons of unique (expert, pair) keys, segment starts and the chunk
// offsets from wave ballots and scans.
// One wave per token routes (kDecodeMaxT waves); the waves past the first
// kDecMaxPairs threads then exit, and the rest of the kernel runs one thread
// per routed pair (a barrier waits only for the waves still running).
constexpr int kPrepThreads = 64 * kDecodeMaxT;
__global__ __launch_bounds__(kPrepThreads) void decode_prep_kernel(const float *__restrict__ logits, int E,
                                                          int32_t *__restrict__ idx,
                                                          float *__restrict__ wts, int P,
                                                          int k_route, int tiles_gu, int tiles_dn,
                                                          int target_gu, int target_dn,
                                                          DecodeWs w) {
  static_assert(kDecMaxPairs == 256, "one thread per routed pair");
  __shared__ __attribute__((aligned(16))) int32_t s_key[kDecMaxPairs];
  __shared__ int32_t s_sorted_e[kDecMaxPairs];
  __shared__ int32_t s_sorted_p[kDecMaxPairs];
  __shared__ int32_t s_dseg[kDecMaxPairs + 1];
  __shared__ int32_t s_wsum[5][4];
  __shared__ RouteLds s_route[kDecodeMaxT];
  __shared__ int4 s_item[kDecMaxPairs];          // distinct expert: id, pairs, segment, tokens
  __shared__ int32_t s_first[2][kDecMaxPairs + 1];  // its first work item per map
  __shared__ int32_t s_tpw[2][kDecMaxPairs];        // its tiles per work item per map
  const int p = threadIdx.x, lane = p & 63, wv = p >> 6;
  int e_p = 0;
  if (logits) {
    // s_sorted_e doubles as the routed ids until the keys are built
    const int T = P / k_route;
    for (int t = wv; t < T; t += kDecodeMaxT)
      route_token(logits, t, E, k_route, lane, idx, wts, s_sorted_e, s_route[wv]);
    __syncthreads();
    if (p >= kDecMaxPairs) return;
    if (p < P) e_p = s_sorted_e[p];
    __syncthreads();
  } else {
    if (p >= kDecMaxPairs) return;
    if (p < P) e_p = safe_expert(idx[p], E);
  }
  // unique sort key: expert, then pair id (stable)
  const int key = p < P ? e_p * kDecMaxPairs + p : 0x7FFFFFFF;
  s_key[p] = key;
  __syncthreads();
  int pos = 0;
  const int4 *k4 = reinterpret_cast<const int4 *>(s_key);
#pragma unroll 4
  for (int q = 0; q < (P + 3) / 4; ++q) {
    const int4 v = k4[q];
    pos += (v.x < key) + (v.y < key) + (v.z < key) + (v.w < key);
  }
  if (p < P) {
    s_sorted_e[pos] = key / kDecMaxPairs;
    s_sorted_p[pos] = p;
    w.sorted[pos] = p;
    w.pos[p] = pos;
  }
  __syncthreads();
  // distinct experts: position p starts a segment
  const bool first = p < P && (p == 0 || s_sorted_e[p - 1] != s_sorted_e[p]);
  const uint64_t fm = __ballot(first);
  int d = __popcll(fm & ((1ull << lane) - 1));
  if (lane == 0) s_wsum[0][wv] = __popcll(fm);
  __syncthreads();
  for (int v = 0; v < wv; ++v) d += s_wsum[0][v];
  const int n = s_wsum[0][0] + s_wsum[0][1] + s_wsum[0][2] + s_wsum[0][3];
  if (first) s_dseg[d] = p;
  if (p == 0) s_dseg[n] = P;
  __syncthreads();
  // Tiles per workgroup (thread = distinct expert): the total cost of all
  // tiles is split into about target workgroups of equal cost (target = the
  // workgroups the GEMV kernel keeps resident), then an inclusive scan over
  // the experts gives each expert's work items.
  const int tiles[2] = {tiles_gu, tiles_dn};
  const int target[2] = {target_gu, target_dn};
  const int np_d = p < n ? s_dseg[p + 1] - s_dseg[p] : 0;
  int c8[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    c8[j] = dec_tile_cost8(np_d, j == 0);
    const int tot = wave_sum(p < n ? tiles[j] * c8[j] : 0);
    if (lane == 0) s_wsum[3 + j][wv] = tot;
  }
  __syncthreads();
  int tpw[2], incl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int total = s_wsum[3 + j][0] + s_wsum[3 + j][1] + s_wsum[3 + j][2] + s_wsum[3 + j][3];
    tpw[j] = 1;
    int c = 0;
    if (p < n) {
      // chunks in proportion to the expert's share of the cost, rounded down,
      // so that the workgroups never exceed the resident set (one more would
      // start a second round and double the kernel's span)
      const int want = max(1, min(tiles[j], int(int64_t(tiles[j]) * c8[j] * target[j] / total)));
      tpw[j] = (tiles[j] + want - 1) / want;
      c = (tiles[j] + tpw[j] - 1) / tpw[j];
    }
    incl[j] = wave_inclusive_scan(c, lane);
    if (lane == 63) s_wsum[1 + j][wv] = incl[j];
  }
  __syncthreads();
  // this expert's id, segment and tokens (np <= 8: one token per expert
  // slot, T <= 8) and its first work item in each map go to LDS; then all
  // threads write the items, item b by thread b % 256 (its expert found by a
  // binary search over the first items)
  if (p < n) {
    const int s0 = s_dseg[p];
    int toks = 0;
    for (int q = 0; q < min(np_d, 8); ++q) toks |= (s_sorted_p[s0 + q] / k_route) << (4 * q);
    s_item[p] = make_int4(s_sorted_e[s0], np_d, s0, toks);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int base = 0;
    for (int v = 0; v < wv; ++v) base += s_wsum[1 + j][v];
    if (p < n) {
      s_first[j][p] = base + incl[j] - (tiles[j] + tpw[j] - 1) / tpw[j];
      s_tpw[j][p] = tpw[j];
    }
    if (p == 0)
      s_first[j][n] = s_wsum[1 + j][0] + s_wsum[1 + j][1] + s_wsum[1 + j][2] + s_wsum[1 + j][3];
  }
  __syncthreads();
  int4 *maps[2] = {w.map_gu, w.map_dn};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int count = s_first[j][n];
    for (int b = p; b < count; b += kDecMaxPairs) {
      int lo = 0, hi = n - 1;  // the last expert whose first item is <= b
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_first[j][mid] <= b) lo = mid;
        else hi = mid - 1;
      }
      const int4 it = s_item[lo];
      const int tile0 = (b - s_first[j][lo]) * s_tpw[j][lo];
      maps[j][b] = dec_item(it.x, it.y, tile0, min(s_tpw[j][lo], tiles[j] - tile0), it.z, it.w);
    }
    if (p == 0) w.map_count[j] = count;
  }
}

// Dequant-GEMV of the (at most 8) tokens of one expert against a block of its
// weight rows, on the vector ALU (no MFMA): every packed byte is read once and
// used for all the expert's tokens.
//
// A workgroup owns a chunk of consecutive tiles of kDecTile output units of one
// expert, read from the work map of the prep kernel (the grid holds one
// workgroup per (expert slot, tile); the surplus exits at once).
// The eight waves split the K blocks in eighths. Inside a wave, 16 lanes share
// a weight row (lane kl holds bytes [kl * BPL, kl * BPL + BPL) of the wave's
// K part, inside one absmax block) and a pass covers 4 rows, so a load
// instruction reads 4 runs of 16 * BPL contiguous bytes. Each lane keeps its
// K slice of every token's input in registers for all tiles. A code byte is
// expanded through an LDS table (replicated kTblCopies times, lanes of a
// half-wave hit distinct banks) into two bf16 codebook values, contracted
// with the inputs by v_dot2_f32_bf16 in fp32; the lane's partial is scaled by
// its block absmax and the 16 lanes of a row are summed with DPP row
// permutes. Per tile the eight K parts meet in a double-buffered LDS slot and
// are summed in a fixed order (one barrier per tile). GATE_UP runs gate row u
// and up row I + u in the same lanes and writes a = silu(g) * up.
constexpr int kTblCopies = 32;
constexpr int kDecPass = 4;             // passes of 4 rows per tile
constexpr int kDecTile = 4 * kDecPass;  // output units per tile

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same bits.
__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);  // row_half_mirror
  v = dpp_add<0x140>(v);  // row_mirror
  return v;
}

template <int BPL>
struct DecLoad;
template <>
struct DecLoad<4> {
  typedef uint32_t T;
  static __device__ __forceinline__ uint32_t word(const T &v, int i) { return v; }
};
template <>
struct DecLoad<8> {
  typedef u32x2 T;
  static __device__ __forceinline__ uint32_t word(const T &v, int i) { return v[i]; }
};
template <>
struct DecLoad<16> {
  typedef u32x4 T;
  static __device__ __forceinline__ uint32_t word(const T &v, int i) { return v[i]; }
};

struct DecCtx {
  const uint8_t *wp;   // this expert's packed rows, at the lane's byte offset
  const float *wa;     // this expert's absmax, at the lane's block
  const uint8_t *ws;   // MXFP4: this expert's E8M0 scales, at the lane's block
  int sstride;         // scale entries per weight row
  int row_bytes, nblk, I, tile0, nt, s0, np, kl, rq, wave, tid;
  int n_active;        // waves with K blocks (the others only meet the barriers)
  bool kvalid, active; // lane holds K bytes; this wave has K blocks
};

template <bool GATE_UP, int NP, int BPL, bool MX>
__device__ __forceinline__ void decode_tiles(const DecCtx &c, const uint32_t *tl,
                                             const uint16_t *__restrict__ xin, int64_t (&xrow)[NP],
                                             int K_in, float (*s_red)[GATE_UP ? 2 : 1][kDecWaves][kDecTile][8],
                                             uint16_t *__restrict__ out, int ldo, int xoff) {
  constexpr int NR = GATE_UP ? 2 : 1;
  constexpr int WPL = BPL / 4;  // packed words per lane
  typedef typename DecLoad<BPL>::T LT;
  // the tokens' inputs: 2 * BPL elements each, zero past the wave's K part
  uint32_t xr[NP][BPL];
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(xin + xrow[q] * K_in + xoff);
#pragma unroll
    for (int i = 0; i < BPL / 4; ++i) {
      const u32x4 v = src[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) xr[q][4 * i + j] = c.kvalid ? v[j] : 0u;
    }
  }
  LT wv[kDecPass][NR];
  float am[kDecPass][NR];
  const bool active = c.active;
  auto load_tile = [&](int t) {
#pragma unroll
    for (int ps = 0; ps < kDecPass; ++ps) {
      const int u = (c.tile0 + t) * kDecTile + 4 * ps + c.rq;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int64_t row = u + r * c.I;
        wv[ps][r] = *reinterpret_cast<const LT *>(c.wp + row * c.row_bytes);
        am[ps][r] = MX ? e8m0_value(c.ws[row * c.sstride]) : c.wa[row * c.sstride];
      }
    }
  };
  if (active) load_tile(0);
  __syncthreads();  // lookup table ready
  for (int t = 0; t < c.nt; ++t) {
    const int slot = t & 1;
    // the next tile's loads are issued once this tile's bytes are expanded;
    // past the last tile the last one is reloaded (uniform wait counts)
    const int tn = min(t + 1, c.nt - 1);
    // waves without K blocks (small K) skip the work and only meet the barrier
    if (active) {
#pragma unroll
    for (int ps = 0; ps < kDecPass; ++ps) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        uint32_t codes[BPL];
#pragma unroll
        for (int i = 0; i < WPL; ++i) {
          const uint32_t word = DecLoad<BPL>::word(wv[ps][r], i);
#pragma unroll
          for (int y = 0; y < 4; ++y) codes[4 * i + y] = tl[((word >> (8 * y)) & 255u) * kTblCopies];
        }
        const float a = am[ps][r];
        {
          const int u = (c.tile0 + tn) * kDecTile + 4 * ps + c.rq;
          const int64_t row = u + r * c.I;
          wv[ps][r] = *reinterpret_cast<const LT *>(c.wp + row * c.row_bytes);
          am[ps][r] = MX ? e8m0_value(c.ws[row * c.sstride]) : c.wa[row * c.sstride];
        }
        float acc[NP];
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          float sacc = 0.0f;
#pragma unroll
          for (int i = 0; i < BPL; ++i) sacc = dot2_bf16(codes[i], xr[q][i], sacc);
          acc[q] = row16_sum(sacc * a);
        }
        float v = acc[0];
#pragma unroll
        for (int q = 1; q < NP; ++q) v = c.kl == q ? acc[q] : v;
        if (c.kl < NP) s_red[slot][r][c.wave][4 * ps + c.rq][c.kl] = v;
      }
    }
    }
    __syncthreads();
    // sum the K parts of tile t: thread (token qq, unit mm)
    if (c.tid < kDecTile * c.np) {
      const int qq = c.tid / kDecTile, mm = c.tid % kDecTile;
      float v[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float sum = s_red[slot][r][0][mm][qq];
        for (int k = 1; k < c.n_active; ++k) sum += s_red[slot][r][k][mm][qq];
        v[r] = sum;
      }
      const float val = GATE_UP ? v[0] / (1.0f + __expf(-v[0])) * v[NR - 1] : v[0];
      out[int64_t(c.s0 + qq) * ldo + (c.tile0 + t) * kDecTile + mm] = f32_to_bf16(val);
    }
  }
}

template <bool GATE_UP, int BPL, bool MX>
__global__ __launch_bounds__(kDecThreads) void decode_gemv_kernel(
    const uint8_t *__restrict__ Wp, const float *__restrict__ Wa, const uint8_t *__restrict__ Ws,
    int64_t w_e_bytes,
    int64_t w_e_blocks, int K_in, int n_units, int I, const uint16_t *__restrict__ vin,
    int k_route, DecodeWs w, int cb, uint16_t *__restrict__ out, int ldo) {
  constexpr int NR = GATE_UP ? 2 : 1;
  __shared__ uint32_t tbl[256 * kTblCopies];
  __shared__ float s_red[2][NR][kDecWaves][kDecTile][8];
  static_assert(kDecTile * 8 <= kDecThreads, "one reducing thread per (token, unit)");
  const int count = w.map_count[GATE_UP ? 0 : 1];
  const int4 item = (GATE_UP ? w.map_gu : w.map_dn)[blockIdx.x];
  if (int(blockIdx.x) >= count) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // entry (byte, copy) at byte * kTblCopies + copy: high nibble's code in the
  // low half, low nibble's code in the high half (element order in memory);
  // thread tid fills entries tid + 512 k (low nibble tid / 32, high nibble k)
  static_assert(kDecThreads == 16 * kTblCopies, "table fill layout");
  {
    const float lo = codebook_value(cb, tid / kTblCopies);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      tbl[tid + kDecThreads * k] = pack_bf16x2(codebook_value(cb, k), lo);
  }
  const uint32_t *tl = tbl + (lane & (kTblCopies - 1));

  DecCtx c;
  c.tid = tid;
  c.wave = wave;
  c.kl = lane & 15;
  c.rq = lane >> 4;
  const int e = item.x & 0xFFFF;
  c.np = min(item.x >> 16, 8);  // <= T <= 8 when the ids are distinct per token
  c.tile0 = item.y & 0xFFFF;
  c.nt = item.y >> 16;
  c.s0 = item.z;
  c.nblk = K_in >> 6;
  c.I = I;
  c.row_bytes = K_in >> 1;
  // this wave's K blocks [b0, b0 + nb); lanes past them (kvalid false) read
  // the row's first bytes and carry zero inputs
  const int bpw = (c.nblk + kDecWaves - 1) / kDecWaves;
  const int b0 = wave * bpw;
  const int nb = max(0, min(bpw, c.nblk - b0));
  c.n_active = (c.nblk + bpw - 1) / bpw;
  c.active = nb > 0;
  c.kvalid = c.kl * BPL < nb * 32;
  const int kbyte = c.kvalid ? b0 * 32 + c.kl * BPL : 0;
  c.wp = Wp + int64_t(e) * w_e_bytes + kbyte;
  // a lane's BPL <= 16 bytes lie inside one 64-element absmax block and,
  // 16-byte aligned, inside one 32-element MXFP4 block
  c.sstride = MX ? K_in >> 5 : c.nblk;
  c.wa = MX ? nullptr : Wa + int64_t(e) * w_e_blocks + (kbyte >> 5);
  c.ws = MX ? Ws + int64_t(e) * w_e_blocks + (kbyte >> 4) : nullptr;
  const int xoff = 2 * kbyte;  // element offset of the lane's input slice

#define E4B_DEC_NP(N)                                                                        \
  {                                                                                          \
    int64_t xrow[N];                                                                         \
    for (int q = 0; q < N; ++q) {                                                            \
      const int qc = min(q, c.np - 1);                                                       \
      xrow[q] = GATE_UP ? int64_t((item.w >> (4 * qc)) & 15) : int64_t(c.s0 + qc);         \
    }                                                                                        \
    decode_tiles<GATE_UP, N, BPL, MX>(c, tl, vin, xrow, K_in, s_red, out, ldo, xoff);        \
  }
  if (c.np <= 1) E4B_DEC_NP(1)
  else if (c.np <= 2) E4B_DEC_NP(2)
  else if (c.np <= 4) E4B_DEC_NP(4)
  else E4B_DEC_NP(8)
#undef E4B_DEC_NP
}

template <bool GATE_UP, bool MX>
static const void *dec_kernel_fn(int bpl) {
  return bpl == 4   ? reinterpret_cast<const void *>(&decode_gemv_kernel<GATE_UP, 4, MX>)
         : bpl == 8 ? reinterpret_cast<const void *>(&decode_gemv_kernel<GATE_UP, 8, MX>)
                    : reinterpret_cast<const void *>(&decode_gemv_kernel<GATE_UP, 16, MX>);
}

// Workgroups of one decode GEMV variant resident on the current device at
// once (occupancy x compute units), cached per device; 0 if the query fails.
static int dec_resident_workgroups(bool gate_up, int bpl, bool mx) {
  constexpr int kMaxDev = 64;
  static int cache[kMaxDev][2][2][3];  // 0: not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  const int vi = bpl == 4 ? 0 : (bpl == 8 ? 1 : 2);
  int &slot = cache[dev][gate_up ? 1 : 0][mx ? 1 : 0][vi];
  if (slot > 0) return slot;
  const void *fn = gate_up ? (mx ? dec_kernel_fn<true, true>(bpl) : dec_kernel_fn<true, false>(bpl))
                           : (mx ? dec_kernel_fn<false, true>(bpl) : dec_kernel_fn<false, false>(bpl));
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kDecThreads, 0) != hipSuccess)
    return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  slot = per_cu * cus;
  return slot;
}

hipError_t launch_decode_forward(const MoePlan &p, const e4b_moe_layer *L, const uint16_t *x,
                                 const float *logits, int32_t *idx, float *wts, uint16_t *y,
                                 char *ws, hipStream_t s, const e4b_kernel_events *ev) {
  DecodeWs w;
  // the decode path reuses the sorted / pos slots of the permutation region
  w.sorted = reinterpret_cast<int32_t *>(ws + p.off_sorted);
  w.pos = reinterpret_cast<int32_t *>(ws + p.off_pos);
  uint16_t *a_buf = reinterpret_cast<uint16_t *>(ws + p.off_a);
  uint16_t *o_buf = reinterpret_cast<uint16_t *>(ws + p.off_o);
  const int P = int(p.P);
  w.map_count = reinterpret_cast<int32_t *>(ws + p.off_dmap);
  w.map_gu = reinterpret_cast<int4 *>(w.map_count + 4);
  w.map_dn = w.map_gu + (p.P < p.E ? p.P : p.E) * (p.I / 16);
  const int ymax = int(p.P < p.E ? p.P : p.E);
  const int H = int(p.H), I = int(p.I);
  const e4b_stack &gu = L->gate_up, &dn = L->down;
  // bytes per lane: 16 lanes cover the wave's bpw blocks (32 bytes each)
  auto bpl_of = [](int K_in) {
    const int bpw = (K_in / kBlock + kDecWaves - 1) / kDecWaves;
    return bpw <= 2 ? 4 : (bpw <= 4 ? 8 : 16);
  };
  const int bpl_gu = bpl_of(H), bpl_dn = bpl_of(I);
  // the workgroups each GEMV kernel keeps resident on the device
  const int target_gu = dec_resident_workgroups(true, bpl_gu, gu.codebook == E4B_CB_MXFP4);
  const int target_dn = dec_resident_workgroups(false, bpl_dn, dn.codebook == E4B_CB_MXFP4);
  if (target_gu <= 0 || target_dn <= 0) return hipErrorInvalidDeviceFunction;
  hipError_t perr = launch_k(ev, E4B_K_DECODE_PREP, decode_prep_kernel, dim3(1), dim3(kPrepThreads), s,
                             logits, int(p.E), idx, wts, P, int(p.k), I / kDecTile, H / kDecTile,
                             target_gu, target_dn, w);
  if (perr != hipSuccess) return perr;

  auto launch = [&](bool gate_up, int K_in, int n_units, const e4b_stack &st,
                    const uint16_t *vin, uint16_t *dst, int ldo, int kernel_id) {
    const int bpl = bpl_of(K_in);
    const int tiles = n_units / kDecTile;
    const dim3 grid(uint32_t(tiles * ymax));
    const bool mx = st.codebook == E4B_CB_MXFP4;
    const int64_t eb = st.out * st.in / 2, ea = st.out * st.in / (mx ? kMxBlock : kBlock);
#define E4B_DEC_LAUNCH(GU, B, MX)                                                             \
  (void)launch_k(ev, kernel_id, decode_gemv_kernel<GU, B, MX>, grid, dim3(kDecThreads), s, st.packed, \
                 st.absmax, st.scales, eb, ea, K_in, n_units, I, vin, int(p.k), w, int(p.codebook), \
                 dst, ldo)
#define E4B_DEC_BPL(GU, MX)                                                                   \
  {                                                                                           \
    if (bpl == 4) E4B_DEC_LAUNCH(GU, 4, MX);                                                  \
    else if (bpl == 8) E4B_DEC_LAUNCH(GU, 8, MX);                                             \
    else E4B_DEC_LAUNCH(GU, 16, MX);                                                          \
  }
    if (gate_up) {
      if (mx) E4B_DEC_BPL(true, true) else E4B_DEC_BPL(true, false)
    } else {
      if (mx) E4B_DEC_BPL(false, true) else E4B_DEC_BPL(false, false)
    }
#undef E4B_DEC_BPL
#undef E4B_DEC_LAUNCH
  };
  // gate_up: I units (gate row u, up row I + u) over K_in = H
  launch(true, H, I, gu, x, a_buf, I, E4B_K_DECODE_GATE_UP);
  // down: H rows over K_in = I
  launch(false, I, H, dn, a_buf, o_buf, H, E4B_K_DECODE_DOWN);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine_rows(o_buf, w.pos, wts, p.T, int(p.k), H, y, s, ev);
}

}  // namespace e4b
