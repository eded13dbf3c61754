// gemm.hip -- grouped GEMM over routed pairs with the 4-bit weight dequantized
// on the fly (bf16 MFMA, fp32 accumulation).
//
// One launch covers every expert (the grouped-nf4-gemm design the 0.31.1
// project page describes: one launch over the packed stacks, decode in the
// kernel, fp32 accumulation). Rows of a tile are routed pairs of one expert in
// sorted order; the tile schedule is read from device-side offsets, so the
// host never synchronizes.
//
// Operand modes
//   A_GATHER : A[m] = src[token(sorted_pair[row])]   (x or grad_y, [T, lda])
//   A_DIRECT : A[m] = src[row]                       (a or dGU, sorted rows)
//   B_NT     : B[n][k] = W[n][k]   weight rows are output columns (forward)
//   B_NN     : B[n][k] = W[k][n]   weight rows are the reduction (dgrad:
//              grad_output @ W, bitsandbytes PR #1965 recompute bullet)
// Epilogues
//   EPI_SWIGLU  : columns are gate/up pairs; a = silu(g) * u -> bf16, and the
//                 bf16 g, u are optionally stored for the backward
//                 (0.1.0 sdist, Experts4bit.forward: chunk into gate | up).
//   EPI_STORE   : bf16 store.
//   EPI_DSWIGLU : dgrad of act(gate) * up scaled by the routing weight, plus
//                 this tile's share of d y / d routing weight.
//   EPI_ACT / EPI_DACT : the same for an ungated layer (has_gate=False in
//                 Experts4bit.__init__: a plain up projection h, a = act(h)).
//
// Tile: 256 (pairs) x 128 * WN (columns) x 64 (one quantization block per
// K-step); 4 x WN waves, each 64 x 128 = 2 x 4 MFMA 32x32x16 tiles. WN = 2
// (both gate_up GEMMs and the down forward): 512 threads, one workgroup per
// CU, double-buffered LDS. WN = 1 (down dgrad): 256 threads, one LDS stage,
// two workgroups per CU. A and the dequantized B are staged in LDS; B is
// dequantized once per workgroup (codebook in LDS, fp32 multiply by the block
// absmax, round-to-nearest-even bf16), i.e. exactly the bf16 view that
// e4b_dequantize_nf4 returns.
#include "codebook8.h"
#include "gemm_dev.h"

namespace e4b {

// Waves are laid out 4 (M) x 2 (N); wave w -> (wm = w / 2, wn = w % 2), so the
// waves holding the first 128 rows sit on all four SIMDs and a tile whose
// rows end early frees whole SIMDs. Each wave owns 64 x 128 outputs
// (2 x 4 MFMA 32x32x16 tiles, 128 fp32 accumulators per lane).
// WN waves along N (4 along M): the tile has 128 * WN columns. WN = 2: 512
// threads, two LDS stages (one workgroup per CU; the two waves of a SIMD run
// the halves of a K-step in opposite order). WN = 1: 256 threads, one LDS
// stage, two workgroups per CU hide each other's staging and epilogues.
// QB = 1: the bf16 passthrough lane (B is stored bf16 and staged as is).
// QB = 2: the int8 / fp8 lanes (one code byte per weight, fp32 absmax per 64,
// decoded through a 256-entry table like the 4-bit codes).
template <int AMODE, int BMODE, int EPI, int WN, int QB>
__global__ __launch_bounds__(256 * WN, WN == 1 ? 2 : 1) void grouped_gemm_kernel(GemmArgs g) {
  constexpr int kGemmWavesN = WN;
  constexpr int kThreads = 256 * WN;
  constexpr int kBN = 128 * WN;
  constexpr int kStages = WN == 1 ? 1 : 2;
  constexpr int kAPass = kBM * 8 / kThreads;  // A rows per thread per K-step
  // B_NN with 4-bit codes: the dequantized tile is stored [k][n] (64 rows of
  // kBN columns, row stride kSBn elements = 32 bytes past a multiple of 128,
  // 16-byte units of a row XOR-swizzled by nn_unit) and the MFMA operand
  // (8 consecutive k of one n per lane) is read with the LDS transpose read
  // ds_read_b64_tr_b16, which hands each lane of a 16-lane group 4
  // consecutive rows of one column of a 4 x 16 block.
  constexpr bool kNNq = BMODE == B_NN && QB != 1;
  constexpr bool kC8 = QB == 2;
  constexpr int kSBn = kBN + 16;
  static_assert(kBK * kSBn <= kBN * kLds, "B_NN tile fits the B stage");
  // the codebook first: its LDS address fits a ds_read's immediate offset
  __shared__ __attribute__((aligned(64))) float sCode[kC8 ? 256 : 16];
  __shared__ __attribute__((aligned(16))) uint16_t sA[kStages][kBM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kStages][kBN * kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kGemmWavesN, wn = wave % kGemmWavesN;

  // ---- tile -> (expert, m-tile, n-tile). The grid is sized for the most
  // m-tiles any routing can produce; the W tiles this routing has are split
  // into eight contiguous ranges of equal length, one per XCD (dispatch puts
  // block b on XCD b % 8), so every XCD gets the same share of real tiles
  // and the n-tiles of one m-tile share that XCD's L2. Blocks past the
  // ranges exit at once. ----
  const int n_mt = g.tile_offsets[g.E];
  const uint32_t W = uint32_t(n_mt) * uint32_t(g.n_tiles);
  const uint32_t per_xcd = (W + 7) / 8, xi = blockIdx.x / 8;
  const uint32_t L = (blockIdx.x % 8) * per_xcd + xi;
  if (xi >= per_xcd || L >= W) return;
  const int mt = int(L / uint32_t(g.n_tiles));
  const int nt = int(L % uint32_t(g.n_tiles));
  const int4 tm = g.tile_map[mt];
  const int e = tm.x, seg = tm.y, row0 = tm.z, valid_rows = tm.w;

  if (!QB && tid < 16) sCode[tid] = codebook_value(g.cb, tid);
  if (kC8 && tid < 256) {
    const float mg = kMag8[g.cb - E4B_CB_INT8].v[tid & 127];
    sCode[tid] = tid < 128 ? mg : -mg;  // code byte = sign bit 7 | magnitude index
  }

  // ---- A rows: column chunk (tid & 7) of rows (tid >> 3) + (kThreads / 8) i.
  // Rows past the segment read the last valid row: their outputs are never
  // stored. ----
  const int a_cc = tid & 7;
  uint32_t a_off[kAPass];
#pragma unroll
  for (int i = 0; i < kAPass; ++i) {
    const int r = min((tid >> 3) + (kThreads / 8) * i, valid_rows - 1);
    const int srow = seg + row0 + r;
    const int src = AMODE == A_GATHER ? g.sorted_pair[srow] / g.topk : srow;
    a_off[i] = uint32_t(src) * uint32_t(g.lda) + uint32_t(a_cc * 8);
  }

  // ---- B source; columns past N read a valid weight row/column instead
  // (their outputs are never stored) ----
  const uint8_t *wp = g.Wp + int64_t(e) * g.w_e_bytes;
  // block scales: fp32 absmax per 64 elements, or (MXFP4) an E8M0 byte per 32
  const float *wa = g.mx ? nullptr : g.Wa + int64_t(e) * g.w_e_blocks;
  const uint8_t *ws8 = g.mx ? g.Ws + int64_t(e) * g.w_e_blocks : nullptr;
  const int row_bytes = QB == 1 ? g.w_in * 2 : (kC8 ? g.w_in : g.w_in >> 1), row_blocks = g.w_in >> 6;
  const int row_mx = g.w_in >> 5;
  // B_NT: thread owns half (32 elements) of one tile column = one weight row
  const int b_c = tid >> 1, b_half = tid & 1;
  int b_row = 0;
  if (BMODE == B_NT) {
    if (EPI == EPI_SWIGLU) {
      const int cw = b_c >> 7, j = (b_c & 127) >> 5, ll = b_c & 31;
      const int pair = nt * (kBN / 2) + cw * 64 + (j & 1) * 32 + ll;
      b_row = pair < g.I ? pair + (j >= 2 ? g.I : 0) : 0;
    } else {
      b_row = nt * kBN + b_c;
      b_row = b_row < g.N ? b_row : 0;
    }
  }
  const uint8_t *b_src_nt = wp + int64_t(b_row) * row_bytes + b_half * (QB == 1 ? 64 : (kC8 ? 32 : 16));
  const float *b_am_nt = g.mx ? nullptr : wa + int64_t(b_row) * row_blocks;
  // MXFP4: the thread's 32 elements of K-step ks are the MX block 2 ks + b_half
  const uint8_t *b_sc_nt = g.mx ? ws8 + int64_t(b_row) * row_mx + b_half : nullptr;
  // B_NN, bf16 lane: thread owns a 4 (k) x 8 (n) patch: n group cg, k group kg (16)
  const int b_cg = tid >> 4, b_kg = tid & 15;
  int b_n = nt * kBN + b_cg * 8;
  b_n = b_n < g.N ? b_n : 0;
  const uint8_t *b_src_nn = wp + int64_t(b_kg * 4) * row_bytes + b_n * 2;
  // B_NN, 4-bit codes: thread owns 32 consecutive columns (16 bytes, inside
  // one absmax block) of one of the K-step's 64 weight rows; the tile is
  // kept in LDS in the weights' own [k][n] order (row stride kSBn)
  const int q_row = tid / (kBN / 32), q_c = tid % (kBN / 32);
  int q_col = nt * kBN + q_c * 32;
  q_col = q_col < g.N ? q_col : 0;
  const uint8_t *b_src_q = wp + int64_t(q_row) * row_bytes + (kC8 ? q_col : q_col >> 1);
  const float *b_am_q = g.mx ? nullptr : wa + int64_t(q_row) * row_blocks + (q_col >> 6);
  const uint8_t *b_sc_q = g.mx ? ws8 + int64_t(q_row) * row_mx + (q_col >> 5) : nullptr;

  u32x4 ra[kAPass];
  u32x4 rb, rb2;  // codes of the thread's 32 weights (8-bit: 32 bytes)
  float ram;
  u32x4 rbq[QB == 1 ? 4 : 1];  // bf16 lane: B_NT 32 elements of a row, B_NN 4 rows x 8 columns

  auto load = [&](int ks) {
#pragma unroll
    for (int i = 0; i < kAPass; ++i)
      ra[i] = *reinterpret_cast<const u32x4 *>(g.A + a_off[i] + uint32_t(ks * kBK));
    if (QB == 1) {
#pragma unroll
      for (int d = 0; d < 4; ++d)
        rbq[d] = BMODE == B_NT
                     ? *reinterpret_cast<const u32x4 *>(b_src_nt + ks * (kBK * 2) + d * 16)
                     : *reinterpret_cast<const u32x4 *>(b_src_nn +
                                                        (int64_t(ks) * kBK + d) * row_bytes);
    } else if (BMODE == B_NT) {
      rb = *reinterpret_cast<const u32x4 *>(b_src_nt + ks * (kC8 ? kBK : kBK / 2));
      if (kC8) rb2 = *reinterpret_cast<const u32x4 *>(b_src_nt + ks * kBK + 16);
      ram = g.mx ? e8m0_value(b_sc_nt[2 * ks]) : b_am_nt[ks];
    } else {
      rb = *reinterpret_cast<const u32x4 *>(b_src_q + int64_t(ks) * kBK * row_bytes);
      if (kC8) rb2 = *reinterpret_cast<const u32x4 *>(b_src_q + int64_t(ks) * kBK * row_bytes + 16);
      ram = g.mx ? e8m0_value(b_sc_q[int64_t(ks) * kBK * row_mx])
                 : b_am_q[int64_t(ks) * kBK * row_blocks];
    }
  };

  auto store = [&](int buf) {
    uint16_t *a_dst = sA[buf];
#pragma unroll
    for (int i = 0; i < kAPass; ++i)
      *reinterpret_cast<u32x4 *>(a_dst + ((tid >> 3) + (kThreads / 8) * i) * kLds + a_cc * 8) =
          ra[i];
    uint16_t *b_dst = sB[buf];
    if (QB == 1) {
      if (BMODE == B_NT) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
          *reinterpret_cast<u32x4 *>(b_dst + b_c * kLds + b_half * 32 + d * 8) = rbq[d];
      } else {
        // column c of the 4 x 8 patch: the 16-bit halves of rows 0..3
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
          *reinterpret_cast<u32x2 *>(b_dst + (b_cg * 8 + c) * kLds + b_kg * 4) =
              u32x2{__builtin_amdgcn_perm(rbq[1][c >> 1], rbq[0][c >> 1], sel),
                    __builtin_amdgcn_perm(rbq[3][c >> 1], rbq[2][c >> 1], sel)};
        }
      }
    } else if (BMODE == B_NT || kNNq) {
      // all 32 codebook reads are issued before the first product; each
      // byte of hi4 / lo4 is the byte offset (4 * nibble) of a table entry
      float c[32];
      const char *tbl = reinterpret_cast<const char *>(sCode);
      if (kC8) {
        // byte j of the 32 is weight j: its table offset is 4 * byte
#pragma unroll
        for (int d = 0; d < 8; ++d)
#pragma unroll
          for (int b = 0; b < 4; ++b)
            c[4 * d + b] = *reinterpret_cast<const float *>(
                tbl + (__builtin_amdgcn_perm(0u, d < 4 ? rb[d] : rb2[d - 4], 0x0C0C0C00u | uint32_t(b)) << 2));
      }
#pragma unroll
      for (int d = 0; d < 4 && !kC8; ++d) {
        const uint32_t hi4 = (rb[d] >> 2) & 0x3C3C3C3Cu, lo4 = (rb[d] << 2) & 0x3C3C3C3Cu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          // v_perm: byte b of the source into byte 0, zeros above
          const uint32_t sel = 0x0C0C0C00u | uint32_t(b);
          c[8 * d + 2 * b] =
              *reinterpret_cast<const float *>(tbl + __builtin_amdgcn_perm(0u, hi4, sel));
          c[8 * d + 2 * b + 1] =
              *reinterpret_cast<const float *>(tbl + __builtin_amdgcn_perm(0u, lo4, sel));
        }
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __fmul_rn(c[8 * d + e], ram);
        const u32x4 q{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7])};
        if (BMODE == B_NT)
          *reinterpret_cast<u32x4 *>(b_dst + b_c * kLds + b_half * 32 + d * 8) = q;
        else
          *reinterpret_cast<u32x4 *>(b_dst + q_row * kSBn + nn_unit(4 * q_c + d) * 8) = q;
      }
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // a wave whose 64 rows all lie past the segment skips its MFMAs
  const bool wave_active = wm * 64 < valid_rows;

  const int nK = g.K / kBK;
  __syncthreads();  // sCode visible
  load(0);
  store(0);
  if (nK > 1) load(1);
  __syncthreads();

  // The two waves sharing a SIMD (w and w + 4) run the two halves of a K-step
  // in opposite order, so one issues MFMAs while the other dequantizes and
  // stores the next stage. Within one barrier interval both orders are safe:
  // the compute reads buffer `cur` (filled before the previous barrier) and
  // the stores fill buffer `cur ^ 1` (last read before the previous barrier).
  // kNNq fragment addresses: lane (group qg = lane / 16, qs = lane % 16)
  // reads rows 8 (qg / 2) + qs / 4 (+ 16 kk + 4 r) and the 4 columns
  // wn * 128 + 32 j + 16 (qg % 2) + 4 (qs % 4) of the [k][n] tile
  int q_off[4];
  {
    const int qg = lane >> 4, qs = lane & 15;
    const int rrow = 8 * (qg >> 1) + (qs >> 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 128 + 32 * j + 16 * (qg & 1) + 4 * (qs & 3);
      q_off[j] = rrow * kSBn + nn_unit(col >> 3) * 8 + (col & 7);
    }
  }
  auto compute = [&](int cur) {
    if (!wave_active) return;
    const uint16_t *a_src = sA[cur] + (wm * 64 + (lane & 31)) * kLds + (lane >> 5) * 8;
    const uint16_t *b_src = sB[cur] + (wn * 128 + (lane & 31)) * kLds + (lane >> 5) * 8;
    // fragments of k-slice kk + 1 are read while the MFMAs of kk run (the
    // one-workgroup-per-CU tiles; the narrow tile has no registers to spare)
    constexpr bool kPrefetch = WN == 2;
    bf16x8 af[2][2], bfr[2][4];
    auto frag = [&](int kk, int slot) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[slot][i] = *reinterpret_cast<const bf16x8 *>(a_src + i * 32 * kLds + kk * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (kNNq) {
          const uint16_t *p = sB[cur] + q_off[j] + kk * 16 * kSBn;
          const s16x4 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * kSBn);
          bfr[slot][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          bfr[slot][j] = *reinterpret_cast<const bf16x8 *>(b_src + j * 32 * kLds + kk * 16);
        }
      }
    };
    if (kPrefetch) frag(0, 0);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int slot = kPrefetch ? kk & 1 : 0;
      if (!kPrefetch)
        frag(kk, 0);
      else if (kk + 1 < kBK / 16)
        frag(kk + 1, (kk + 1) & 1);
      // weights are the MFMA A-operand: acc[i][j] holds D[tile col][tile row]
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[slot][j], af[slot][i],
                                                              acc[i][j], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
    }
  };
  if constexpr (kStages == 1) {
    // one stage: contract it, then refill it from the registers loaded one
    // K-step earlier and start the loads of the step after
    for (int ks = 0; ks < nK; ++ks) {
      compute(0);
      __syncthreads();
      if (ks + 1 < nK) {
        store(0);
        if (ks + 2 < nK) load(ks + 2);
      }
      __syncthreads();
    }
  } else {
    const bool store_first = wave >= 4;
    for (int ks = 0; ks < nK; ++ks) {
      const int cur = ks & 1;
      if (store_first) {
        if (ks + 1 < nK) store(cur ^ 1);
        if (ks + 2 < nK) load(ks + 2);
        compute(cur);
      } else {
        compute(cur);
        if (ks + 1 < nK) store(cur ^ 1);
        if (ks + 2 < nK) load(ks + 2);
      }
      __syncthreads();
    }
  }

  // ---- LoRA: one more 16-deep slice, pair side = the per-pair projection
  // (fp32 [P, 16], rounded to bf16 here), weight side = the bf16 pack of the
  // scaled adapter [E, rows, 16] at the weight row of each tile column ----
  if (g.lora_p != nullptr && wave_active) {
    const int kh = lane >> 5;
    bf16x8 pf[2], wf[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = min(wm * 64 + i * 32 + (lane & 31), valid_rows - 1);
      const float4 *src =
          reinterpret_cast<const float4 *>(g.lora_p + int64_t(seg + row0 + r) * kLoraK + 8 * kh);
      const float4 v0 = src[0], v1 = src[1];
      const u32x4 q{pack_bf16x2(v0.x, v0.y), pack_bf16x2(v0.z, v0.w), pack_bf16x2(v1.x, v1.y),
                    pack_bf16x2(v1.z, v1.w)};
      pf[i] = __builtin_bit_cast(bf16x8, q);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = wn * 128 + j * 32 + (lane & 31);
      int row;
      if (BMODE == B_NT && EPI == EPI_SWIGLU) {
        const int pair = nt * (kBN / 2) + wn * 64 + (j & 1) * 32 + (lane & 31);
        row = pair < g.I ? pair + (j >= 2 ? g.I : 0) : 0;
      } else {
        row = nt * kBN + c;
        row = row < g.N ? row : 0;
      }
      wf[j] = *reinterpret_cast<const bf16x8 *>(g.lora_w + (int64_t(e) * g.lora_rows + row) * kLoraK +
                                                8 * kh);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], pf[i], acc[i][j], 0, 0, 0);
  }

  // ---- epilogue ----
  // acc[i][j][4q + t]: tile row  = wm*64 + i*32 + lane%32,
  //                    tile col  = wn*128 + j*32 + 8q + 4*(lane/32) + t   (t = 0..3)
  // so each lane holds runs of 4 consecutive columns of one row.
  const int lrow = wm * 64 + (lane & 31);
  const int lcol = wn * 128 + 4 * (lane >> 5);
  if (EPI == EPI_STORE && WN == 2) {
    // Through LDS, so that the stores are whole row segments: rows 0..127 of
    // the tile go to the A stages, rows 128..255 to the B stages (bf16, row
    // stride kOut), then every thread writes 16 contiguous bytes, a wave two
    // 512-byte row segments. The K loop's last barrier has retired every read
    // of both stages.
    constexpr int kOut = kBN + 8;
    static_assert(WN != 2 || (128 * kOut <= kStages * kBM * kLds && 128 * kOut <= kStages * kBN * kLds),
                  "half a tile fits each stage pair");
    uint16_t *half = wm < 2 ? sA[0] : sB[0];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (lrow + i * 32) & 127;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16 &a = acc[i][j];
          *reinterpret_cast<u32x2 *>(half + r * kOut + lcol + j * 32 + 8 * q) =
              u32x2{pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
        }
    }
    __syncthreads();
    const int cc = (tid & 31) * 8, col = nt * kBN + cc;
#pragma unroll 4
    for (int pass = 0; pass < kBM / 16; ++pass) {
      const int row = pass * 16 + (tid >> 5);
      const uint16_t *src = (row < 128 ? sA[0] : sB[0]) + (row & 127) * kOut + cc;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(src);
      if (row < valid_rows && col < g.N)
        *reinterpret_cast<u32x4 *>(g.C + int64_t(seg + row0 + row) * g.ldc + col) = v;
    }
  } else if (EPI == EPI_STORE) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = lrow + i * 32;
      if (row < valid_rows) {
        uint16_t *crow = g.C + int64_t(seg + row0 + row) * g.ldc;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = nt * kBN + lcol + j * 32 + 8 * q;
            const f32x16 &a = acc[i][j];
            if (col < g.N)
              *reinterpret_cast<u32x2 *>(crow + col) =
                  u32x2{pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
          }
      }
    }
  } else if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = lrow + i * 32;
      if (row < valid_rows) {
        const int64_t grow = seg + row0 + row;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int pair = nt * (kBN / 2) + wn * 64 + jj * 32 + 8 * q + 4 * (lane >> 5);
            if (pair < g.I) {
              float gv[4], uv[4], av[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                gv[t] = acc[i][jj][4 * q + t];
                uv[t] = acc[i][jj + 2][4 * q + t];
                av[t] = gv[t] * sigmoidf_(gv[t]) * uv[t];
              }
              if (g.C)
                *reinterpret_cast<u32x2 *>(g.C + grow * g.ldc + pair) =
                    u32x2{pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3])};
              static_assert(EPI != EPI_SWIGLU || kBN / 2 == kGuBlockPairs, "one g|u block per tile");
              if (g.GU) {
                // the tile's 128 pairs are block nt of the blocked g|u
                const int64_t ch = gu_chunk(mt, nt, g.n_tiles, row, pair - nt * (kBN / 2));
                *reinterpret_cast<u32x4 *>(g.GU + ch * 8) =
                    u32x4{pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3]),
                          pack_bf16x2(uv[0], uv[1]), pack_bf16x2(uv[2], uv[3])};
              }
            }
          }
      }
    }
  } else if (EPI == EPI_ACT) {
    // ungated: h = this tile's columns of the up projection, a = silu(h)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = lrow + i * 32;
      if (row < valid_rows) {
        const int64_t grow = seg + row0 + row;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = nt * kBN + lcol + j * 32 + 8 * q;
            if (col < g.N) {
              float hv[4], av[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                hv[t] = acc[i][j][4 * q + t];
                av[t] = hv[t] * sigmoidf_(hv[t]);
              }
              if (g.C)
                *reinterpret_cast<u32x2 *>(g.C + grow * g.ldc + col) =
                    u32x2{pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3])};
              if (g.GU)
                *reinterpret_cast<u32x2 *>(g.GU + grow * g.ldgu + col) =
                    u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
            }
          }
      }
    }
  } else if (EPI == EPI_DACT) {
    // ungated dgrad: grad_a = w * G2, dh = grad_a * silu'(h), partial sum of G2 * silu(h)
    float *red = reinterpret_cast<float *>(sA[0]);
    float part[2] = {0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = lrow + i * 32;
      const int64_t grow = seg + row0 + min(row, valid_rows - 1);
      const float wr = g.topk_w[g.sorted_pair[grow]];
      const uint16_t *hrow = g.GU + grow * g.ldgu;
      uint16_t *crow = g.C + grow * g.ldc;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nt * kBN + lcol + j * 32 + 8 * q;
          const u32x2 hq = *reinterpret_cast<const u32x2 *>(hrow + min(n, g.N - 4));
          const float hv[4] = {bf16_lo(hq[0]), bf16_hi(hq[0]), bf16_lo(hq[1]), bf16_hi(hq[1])};
          float dh[4], pq = 0.0f;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float sg = sigmoidf_(hv[t]);
            const float G2 = acc[i][j][4 * q + t];
            pq += G2 * (hv[t] * sg);
            dh[t] = wr * G2 * sg * (1.0f + hv[t] * (1.0f - sg));
          }
          if (row < valid_rows && n < g.N) {
            part[i] += pq;
            *reinterpret_cast<u32x2 *>(crow + n) =
                u32x2{pack_bf16x2(dh[0], dh[1]), pack_bf16x2(dh[2], dh[3])};
          }
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float pr = part[i] + __shfl_xor(part[i], 32);
      if (lane < 32) red[wn * kBM + lrow + i * 32] = pr;
    }
    __syncthreads();
    for (int r = tid; r < valid_rows; r += kThreads) {
      const int64_t grow = seg + row0 + r;
      float sum = red[r];
#pragma unroll
      for (int c = 1; c < kGemmWavesN; ++c) sum += red[c * kBM + r];
      g.partial[grow * g.n_tiles + nt] = sum;
    }
  } else {  // EPI_DSWIGLU
    float *red = reinterpret_cast<float *>(sB[0]);  // [kGemmWavesN][kBM] partial row sums
    static_assert(EPI != EPI_DSWIGLU || kGemmWavesN * kBM * 2 <= kStages * kBN * kLds,
                  "the partial sums fit the B stage");
    // dGU goes out through LDS in four rounds (row half i, column half jh of
    // the tile): the four waves' 32 rows each x 64 pairs of dg then du (bf16,
    // row stride kSt) in the A stage, then 128-byte row segments per store
    constexpr int kSt = 128 + 8;
    static_assert(EPI != EPI_DSWIGLU || 128 * kSt <= kStages * kBM * kLds, "a round fits the A stage");
    uint16_t *stg = sA[0];
    // The saved g|u of the lane's 2 x 4 x 4 column runs (one 16-byte chunk of
    // the tile's g|u block each) are fetched in eight batches (row half i,
    // column group j), one batch ahead of its use, with rows and columns
    // clamped to chunks the forward wrote (out-of-range results are not
    // stored), so the loads of a batch overlap the arithmetic of the previous.
    static_assert(EPI != EPI_DSWIGLU || kBN == kGuBlockPairs, "one g|u block per tile");
    int64_t grow[2];
    int rrow[2];
    float wr[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rrow[i] = min(lrow + i * 32, valid_rows - 1);
      grow[i] = seg + row0 + rrow[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) wr[i] = g.topk_w[g.sorted_pair[grow[i]]];
    u32x2 gg[2][4], uu[2][4];
    // the forward wrote the chunks of pairs 0, 4, ..., cmax of this block
    const int cmax = min(kBN, g.N - nt * kBN) - 4;
    auto fetch = [&](int b, int slot) {
      const int i = b >> 2, j = b & 3;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = min(lcol + j * 32 + 8 * q, cmax);
        const u32x4 v = *reinterpret_cast<const u32x4 *>(
            g.GU + gu_chunk(mt, nt, g.n_tiles, rrow[i], c) * 8);
        gg[slot][q] = u32x2{v[0], v[1]};
        uu[slot][q] = u32x2{v[2], v[3]};
      }
    };
    float part[2] = {0.0f, 0.0f};
    fetch(0, 0);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (b + 1 < 8) fetch(b + 1, (b + 1) & 1);
      const int i = b >> 2, j = b & 3, slot = b & 1;
      const bool row_ok = lrow + i * 32 < valid_rows;
      uint16_t *srow = stg + (wm * 32 + (lane & 31)) * kSt;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nt * kBN + lcol + j * 32 + 8 * q;
        const u32x2 gq = gg[slot][q], uq = uu[slot][q];
        const float gv[4] = {bf16_lo(gq[0]), bf16_hi(gq[0]), bf16_lo(gq[1]), bf16_hi(gq[1])};
        const float uv[4] = {bf16_lo(uq[0]), bf16_hi(uq[0]), bf16_lo(uq[1]), bf16_hi(uq[1])};
        float dg[4], du[4], pq = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float s = sigmoidf_(gv[t]);
          const float silu = gv[t] * s;
          const float G2 = acc[i][j][4 * q + t];
          pq += G2 * (silu * uv[t]);
          const float ga = wr[i] * G2;
          dg[t] = ga * uv[t] * s * (1.0f + gv[t] * (1.0f - s));
          du[t] = ga * silu;
        }
        if (row_ok && n < g.N) part[i] += pq;
        const int pr_ = (j & 1) * 32 + 8 * q + 4 * (lane >> 5);  // pair within the round
        *reinterpret_cast<u32x2 *>(srow + pr_) = u32x2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
        *reinterpret_cast<u32x2 *>(srow + 64 + pr_) =
            u32x2{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
      }
      if (j & 1) {
        // round (i, j / 2) staged: 128 rows x 16 chunks of 16 bytes
        __syncthreads();
        const int jh = j >> 1;
#pragma unroll
        for (int pass = 0; pass < 128 * 16 / kThreads; ++pass) {
          const int id = pass * kThreads + tid, R = id >> 4, c = id & 15;
          const int trow = (R >> 5) * 64 + i * 32 + (R & 31);
          const int n = nt * kBN + jh * 64 + (c & 7) * 8;
          const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + R * kSt + c * 8);
          if (trow < valid_rows && n < g.N)
            *reinterpret_cast<u32x4 *>(g.C + (seg + row0 + trow) * int64_t(g.ldc) + (c < 8 ? 0 : g.I) + n) = v;
        }
        __syncthreads();
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      // the two half-waves hold the two column halves of the same rows
      const float pr = part[i] + __shfl_xor(part[i], 32);
      if (lane < 32) red[wn * kBM + lrow + i * 32] = pr;
    }
    __syncthreads();
    for (int r = tid; r < valid_rows; r += kThreads) {
      const int64_t grow = seg + row0 + r;
      float sum = red[r];
#pragma unroll
      for (int c = 1; c < kGemmWavesN; ++c) sum += red[c * kBM + r];
      g.partial[grow * g.n_tiles + nt] = sum;
    }
  }
}

hipError_t launch_grouped_gemm(GemmVariant v, const GemmArgs &a, hipStream_t s,
                               const e4b_kernel_events *ev) {
  if (a.grid == 0) return hipSuccess;
  // a multiple of 8 blocks: each XCD then has at least ceil(W / 8) of them
  const dim3 grid((a.grid + 7) / 8 * 8);
  const int qb = a.cb == E4B_CB_BF16 ? 1 : (a.cb == E4B_CB_INT8 || a.cb == E4B_CB_FP8 ? 2 : 0);
  const int kid = int(v);  // GemmVariant ids are the e4b_kernel ids of the four GEMMs
#define E4B_GEMM(AM, BM, EP, WNV)                                                              \
  return qb == 1   ? launch_k(ev, kid, grouped_gemm_kernel<AM, BM, EP, WNV, 1>, grid, dim3(256 * (WNV)), s, a) \
         : qb == 2 ? launch_k(ev, kid, grouped_gemm_kernel<AM, BM, EP, WNV, 2>, grid, dim3(256 * (WNV)), s, a) \
                   : launch_k(ev, kid, grouped_gemm_kernel<AM, BM, EP, WNV, 0>, grid, dim3(256 * (WNV)), s, a)
  switch (v) {
    case GEMM_GATE_UP_FWD:
    case GEMM_DOWN_FWD:
    case GEMM_GATE_UP_DGRAD: return launch_gemm_wide(v, a, s, ev);
    case GEMM_DOWN_DGRAD:
      if (a.gated) {
        // 256-column tiles: the same m-tiles, half as many n-tiles; the
        // partials keep one entry per 128-pair block
        GemmArgs w = a;
        w.n_tiles = (a.N + 2 * kGuBlockPairs - 1) / (2 * kGuBlockPairs);
        w.grid = a.grid / uint32_t(a.n_tiles) * uint32_t(w.n_tiles);
        return launch_gemm_wide(v, w, s, ev);
      }
      E4B_GEMM(A_GATHER, B_NN, EPI_DACT, kBNNarrow / 128);
  }
#undef E4B_GEMM
  return hipErrorInvalidValue;
}

}  // namespace e4b
