// decode.hip -- forward for T <= 8 tokens as bandwidth-bound dequant-GEMVs.
//
// The 0.4.0 README ("Inference" section) describes the decode fast path: a
// single-token forward skips the one-hot grouping and its per-expert host
// syncs, and single-row projections read the packed 4-bit weight directly
// instead of materializing a dequantized expert. Here, for T <= 8:
//   prep     one workgroup groups the <= 8*k routed pairs by expert (stable)
//            and lists the distinct experts in ascending order;
//   gate_up  one workgroup per (distinct expert, block of gate/up row pairs):
//            every packed byte is read once for all tokens routed to that
//            expert; a = silu(g) * u is written as bf16;
//   down     one workgroup per (distinct expert, block of rows of H);
//   combine  the shared deterministic gather-combine.
// The projections of the (at most 8) tokens of one expert form a skinny GEMM:
// it runs on the 16x16x32 bf16 MFMA with the tokens as the 16-row A operand
// (rows past the expert's token count are computed and dropped), so the cost
// per weight byte does not grow with the number of tokens. Each code byte is
// expanded through a 256-entry LDS table into two bf16 codebook values; the
// block absmax scales the fp32 partial of each 64-element block.
#include "device.h"
#include "kernels.h"

namespace e4b {

constexpr int kDecWaves = 8;  // waves of a decode workgroup: one K eighth each
constexpr int kDecThreads = 64 * kDecWaves;

// Workspace layout of the decode path (inside the permutation region).
struct DecodeWs {
  int32_t *n_distinct;  // [1]
  int32_t *dexp;        // [kDecMaxPairs] expert id of distinct expert d (ascending)
  int32_t *dseg;        // [kDecMaxPairs + 1] sorted-pair offsets of distinct expert d
  int32_t *sorted;      // [P] pair id at sorted position
  int32_t *pos;         // [P] sorted position of pair id
};

__global__ __launch_bounds__(256) void decode_prep_kernel(const int32_t *__restrict__ idx, int P,
                                                          DecodeWs w) {
  __shared__ int32_t s_e[kDecMaxPairs];
  __shared__ int32_t s_sorted[kDecMaxPairs];
  __shared__ int32_t s_first[kDecMaxPairs];
  const int p = threadIdx.x;
  if (p < P) s_e[p] = idx[p];
  __syncthreads();
  int pos = 0;
  if (p < P) {
    const int e = s_e[p];
    for (int q = 0; q < P; ++q) {
      const int eq = s_e[q];
      pos += (eq < e || (eq == e && q < p)) ? 1 : 0;
    }
    s_sorted[pos] = p;
    w.sorted[pos] = p;
    w.pos[p] = pos;
  }
  __syncthreads();
  if (p < P) s_first[p] = (p == 0 || s_e[s_sorted[p - 1]] != s_e[s_sorted[p]]) ? 1 : 0;
  __syncthreads();
  if (p < P && s_first[p]) {
    int d = 0;
    for (int q = 0; q < p; ++q) d += s_first[q];
    w.dexp[d] = s_e[s_sorted[p]];
    w.dseg[d] = p;
  }
  if (p == 0) {
    int n = 0;
    for (int q = 0; q < P; ++q) n += s_first[q];
    w.n_distinct[0] = n;
    w.dseg[n] = P;
  }
}

// Skinny-GEMM form of the projection of one expert's np <= 8 tokens, on the
// 16x16x32 bf16 MFMA: the tokens' inputs are the A operand (16 rows, rows past
// np repeat the last token and are not stored), 16 weight rows of the expert
// are the B operand, the reduction runs over in_features.
//
// A workgroup owns a chunk of consecutive tiles of 16 output units of one
// expert: the chunk length is chosen on the device from the number of
// distinct experts, so that about wg_target workgroups have work (the grid
// holds one workgroup per (expert slot, tile) and the surplus exits at once); its eight waves split the K blocks in eighths, so each wave holds
// its eighth of the token inputs in registers for all tiles. Per tile and
// 64-element absmax block, lane (g = l / 16, m = l % 16) loads the 8 code bytes
// [8g, 8g + 8) of weight row m, expands each byte into two bf16 codebook
// values through an LDS table (replicated kTblCopies times so that the lanes
// of a half-wave read distinct banks), and two MFMAs contract the block; the
// block's absmax (weight row m is the lane's output column) scales the fp32
// partial before it joins the accumulator. Weight bytes and absmax of the
// next tile are in flight while a tile is contracted. Per tile
// the eight K partials meet in a double-buffered LDS slot and are summed in a
// fixed order (one barrier per tile). GATE_UP runs the gate and up tiles of
// the same units in the same lanes and writes a = silu(g) * up.
constexpr int kTblCopies = 32;

// AM_VEC: every wave owns 0 or MAXB blocks and MAXB divides the blocks per row,
// so a wave's absmax run is one aligned vector load.
template <bool GATE_UP, int MAXB, bool AM_VEC>
__global__ __launch_bounds__(kDecThreads) void decode_mfma_kernel(
    const uint8_t *__restrict__ Wp, const float *__restrict__ Wa, int64_t w_e_bytes,
    int64_t w_e_blocks, int K_in, int n_units, int I, const uint16_t *__restrict__ vin,
    int k_route, DecodeWs w, int cb, uint16_t *__restrict__ out, int ldo, int wg_target) {
  constexpr int NR = GATE_UP ? 2 : 1;
  __shared__ uint32_t tbl[256 * kTblCopies];
  __shared__ f32x4 s_red[2][NR][kDecWaves][64];
  const int n_tiles = n_units >> 4;
  const int n_dist = w.n_distinct[0];
  const int tiles_per_wg = min(n_tiles, max(1, (n_dist * n_tiles + wg_target - 1) / wg_target));
  const int chunks = (n_tiles + tiles_per_wg - 1) / tiles_per_wg;
  const int d = blockIdx.x / chunks;
  if (d >= n_dist) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, m = lane & 15;
  // entry (byte, copy) at byte * kTblCopies + copy: high nibble's code in the
  // low half, low nibble's code in the high half (element order in memory)
  // (thread tid fills entries tid + 512 k: low nibble tid / 32, high nibble k)
  static_assert(kDecThreads == 16 * kTblCopies, "table fill layout");
  {
    const float lo = codebook_value(cb, tid / kTblCopies);
#pragma unroll
    for (int k = 0; k < 16; ++k) tbl[tid + kDecThreads * k] = pack_bf16x2(codebook_value(cb, k), lo);
  }
  const uint32_t *tl = tbl + (lane & (kTblCopies - 1));

  const int e = w.dexp[d];
  const int s0 = w.dseg[d];
  const int np = w.dseg[d + 1] - s0;
  const int nblk = K_in >> 6;
  const int tile0 = (blockIdx.x - d * chunks) * tiles_per_wg;
  const int nt = min(tiles_per_wg, n_tiles - tile0);
  const uint8_t *wp = Wp + int64_t(e) * w_e_bytes;
  const float *wa = Wa + int64_t(e) * w_e_blocks;

  // this wave's K blocks [b0, b0 + nb); loads of blocks past nb read a valid
  // block of the row instead (their products are never formed), so every load
  // is unconditional and the wait counts stay exact
  const int bpw = (nblk + kDecWaves - 1) / kDecWaves;
  const int b0 = wave * bpw;
  const int nb = max(0, min(bpw, nblk - b0));
  const int row_bytes = K_in >> 1;
  int bcl[MAXB];
#pragma unroll
  for (int b = 0; b < MAXB; ++b) bcl[b] = min(b0 + b, nblk - 1);

  // the tokens' inputs for this wave's blocks (registers, all tiles)
  const int q = min(m, np - 1);
  const int64_t xrow = GATE_UP ? int64_t(w.sorted[s0 + q] / k_route) : int64_t(s0 + q);
  const uint16_t *xp = vin + xrow * K_in + 16 * g;
  u32x4 xr[MAXB][2];
#pragma unroll
  for (int b = 0; b < MAXB; ++b) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(xp + bcl[b] * 64);
    xr[b][0] = src[0];
    xr[b][1] = src[1];
  }

  struct Stage {
    u32x2 wv[NR][MAXB];
    float am[NR][MAXB];
  };
  auto load_tile = [&](int t, Stage &st) {
    const int u = (tile0 + t) * 16 + m;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int64_t row = u + r * I;
      const uint8_t *src = wp + row * row_bytes + 8 * g;
      const float *ap = wa + row * nblk;
#pragma unroll
      for (int b = 0; b < MAXB; ++b)
        st.wv[r][b] = *reinterpret_cast<const u32x2 *>(src + bcl[b] * 32);
      if constexpr (AM_VEC) {
        const float *av = ap + min(b0, nblk - MAXB);
        if constexpr (MAXB == 2) {
          const f32x2 v = *reinterpret_cast<const f32x2 *>(av);
          st.am[r][0] = v[0];
          st.am[r][1] = v[1];
        } else {
#pragma unroll
          for (int c = 0; c < MAXB / 4; ++c) {
            const f32x4 v = reinterpret_cast<const f32x4 *>(av)[c];
#pragma unroll
            for (int i = 0; i < 4; ++i) st.am[r][4 * c + i] = v[i];
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < MAXB; ++b) st.am[r][b] = ap[bcl[b]];
      }
    }
  };
  Stage st0, st1;
  load_tile(0, st0);
  if (nt == 1) {
    __syncthreads();
  } else {
    load_tile(1, st1);
    __syncthreads();
  }

  auto contract = [&](const Stage &st, int slot) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int b = 0; b < MAXB; ++b) {
        if (b < nb) {
          u32x4 c0, c1;
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            c0[y] = tl[((st.wv[r][b][0] >> (8 * y)) & 255u) * kTblCopies];
            c1[y] = tl[((st.wv[r][b][1] >> (8 * y)) & 255u) * kTblCopies];
          }
          f32x4 part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, xr[b][0]), __builtin_bit_cast(bf16x8, c0),
              f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xr[b][1]),
                                                         __builtin_bit_cast(bf16x8, c1), part,
                                                         0, 0, 0);
          const float am = st.am[r][b];
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j] += part[j] * am;
        }
      }
      s_red[slot][r][wave][lane] = acc;
    }
  };
  // sum the K parts of tile t: thread (token row qq, unit mm)
  auto reduce_store = [&](int t, int slot) {
    if (tid < 16 * np) {
      const int qq = tid >> 4, mm = tid & 15;
      const int src_lane = 16 * (qq >> 2) + mm, comp = qq & 3;
      float v[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float sum = s_red[slot][r][0][src_lane][comp];
#pragma unroll
        for (int k = 1; k < kDecWaves; ++k) sum += s_red[slot][r][k][src_lane][comp];
        v[r] = sum;
      }
      const float val = GATE_UP ? v[0] / (1.0f + __expf(-v[0])) * v[NR - 1] : v[0];
      out[int64_t(s0 + qq) * ldo + (tile0 + t) * 16 + mm] = f32_to_bf16(val);
    }
  };
  if (nt == 1) {
    contract(st0, 0);
    __syncthreads();
    reduce_store(0, 0);
    return;
  }
  // two tiles in flight; prefetch ids past the last tile are clamped to it
  // (a redundant load keeps the wait counts of every iteration identical)
  for (int t = 0; t < nt; t += 2) {
    contract(st0, 0);
    load_tile(min(t + 2, nt - 1), st0);
    __syncthreads();
    reduce_store(t, 0);
    if (t + 1 < nt) contract(st1, 1);
    load_tile(min(t + 3, nt - 1), st1);
    __syncthreads();
    if (t + 1 < nt) reduce_store(t + 1, 1);
  }
}


hipError_t launch_decode_forward(const MoePlan &p, const e4b_moe_layer *L, const uint16_t *x,
                                 const int32_t *idx, const float *wts, uint16_t *y, char *ws,
                                 hipStream_t s) {
  DecodeWs w;
  // the decode path reuses slots of the permutation region:
  // dexp <= min(E, P) entries, dseg <= min(E, P) + 1 entries
  w.n_distinct = reinterpret_cast<int32_t *>(ws + p.off_tile_offsets);
  w.dexp = reinterpret_cast<int32_t *>(ws + p.off_counts);
  w.dseg = reinterpret_cast<int32_t *>(ws + p.off_offsets);
  w.sorted = reinterpret_cast<int32_t *>(ws + p.off_sorted);
  w.pos = reinterpret_cast<int32_t *>(ws + p.off_pos);
  uint16_t *a_buf = reinterpret_cast<uint16_t *>(ws + p.off_a);
  uint16_t *o_buf = reinterpret_cast<uint16_t *>(ws + p.off_o);
  const int P = int(p.P);
  hipLaunchKernelGGL(decode_prep_kernel, dim3(1), dim3(256), 0, s, idx, P, w);

  const int ymax = int(p.P < p.E ? p.P : p.E);
  const int H = int(p.H), I = int(p.I);
  const e4b_stack &gu = L->gate_up, &dn = L->down;
  // two workgroups of the decode kernel fit one CU (LDS); aim at one wave of them
  const int wg_target = 512;
  auto launch = [&](bool gate_up, int K_in, int n_units, const e4b_stack &st,
                    const uint16_t *vin, uint16_t *dst, int ldo, int kernel_id) {
    const int nblk = K_in / kBlock;
    const int bpw = (nblk + kDecWaves - 1) / kDecWaves;
    const int tiles = n_units / 16;
    const dim3 grid(uint32_t(tiles * ymax));
    const int64_t eb = st.out * st.in / 2, ea = st.out * st.in / kBlock;
    timer_before(kernel_id, s);
#define E4B_DEC_LAUNCH(GU, MB, AV)                                                            \
  hipLaunchKernelGGL((decode_mfma_kernel<GU, MB, AV>), grid, dim3(kDecThreads), 0, s,          \
                     st.packed, st.absmax, eb, ea, K_in, n_units, I, vin, int(p.k), w,         \
                     p.codebook, dst, ldo, wg_target)
#define E4B_DEC_LAUNCH_MB(GU)                                                                 \
  do {                                                                                        \
    const int mb = bpw <= 2 ? 2 : (bpw <= 4 ? 4 : 8);                                         \
    const bool av = bpw == mb && nblk % mb == 0;                                              \
    if (mb == 2) {                                                                            \
      if (av) E4B_DEC_LAUNCH(GU, 2, true); else E4B_DEC_LAUNCH(GU, 2, false);                 \
    } else if (mb == 4) {                                                                     \
      if (av) E4B_DEC_LAUNCH(GU, 4, true); else E4B_DEC_LAUNCH(GU, 4, false);                 \
    } else {                                                                                  \
      if (av) E4B_DEC_LAUNCH(GU, 8, true); else E4B_DEC_LAUNCH(GU, 8, false);                 \
    }                                                                                         \
  } while (0)
    if (gate_up)
      E4B_DEC_LAUNCH_MB(true);
    else
      E4B_DEC_LAUNCH_MB(false);
#undef E4B_DEC_LAUNCH_MB
#undef E4B_DEC_LAUNCH
    timer_after(kernel_id, s);
  };
  // gate_up: I units (gate row u, up row I + u) over K_in = H
  launch(true, H, I, gu, x, a_buf, I, E4B_K_DECODE_GATE_UP);
  // down: H rows over K_in = I
  launch(false, I, H, dn, a_buf, o_buf, H, E4B_K_DECODE_DOWN);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine_rows(o_buf, w.pos, wts, p.T, int(p.k), H, y, s);
}

}  // namespace e4b
