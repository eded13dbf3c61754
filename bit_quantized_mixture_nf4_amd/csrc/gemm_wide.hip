// gemm_wide.hip -- the grouped GEMMs over routed pairs, with the stored
// weight decoded on the fly (bf16 MFMA, fp32 accumulation): the gate_up and
// down forward projections and both dgrad projections.
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
//                 the tile's share of d y / d routing weight.
//   EPI_ACT / EPI_DACT : the same for an ungated layer (has_gate=False in
//                 Experts4bit.__init__: a plain up projection h, a = act(h)).
//
// Tile: 256 pairs x 256 columns x 64 (one quantization block per K-step).
// * 8 waves of 64 x 128 (two per SIMD, 2 x 4 MFMA 32x32x16 bf16 tiles and
//   128 fp32 accumulators per lane), so one wave's MFMAs run while the other
//   waits for memory; the 4-wave shape (128 x 128 per wave, a third fewer LDS
//   fragment bytes per MFMA) is kept as Shape<2>. The dequantized weight is
//   the MFMA A operand, so a lane's accumulators hold runs of 4 consecutive
//   output columns of one pair.
// * The K loop is software-pipelined inside each wave. While the MFMAs of
//   K-step ks run from LDS stage ks & 1, the wave stages K-step ks + 1 into
//   the other stage -- LDS stores of the A rows it loaded one step earlier,
//   and the B tile's dequantization (codebook lookups in LDS, one fp32
//   multiply by the block scale, round to bf16, LDS stores) -- and issues
//   the global loads of later K-steps (A: ks + 2; B: ks + 3, two register
//   sets). The instruction stream of a K-step is cut into slots of one MFMA
//   each (32 per wave and K-step); every slot carries a fixed share of that
//   work and a scheduling barrier closes it, so the compiler keeps the work
//   between the MFMAs instead of clustering it, and the lookups' LDS latency
//   elapses under the MFMAs that follow.
// * B is dequantized once per workgroup: bf16(fl32(code value * block
//   scale)), the bf16 view that e4b_dequantize_nf4 returns. For B_NN the
//   dequantized tile is kept in the weights' own [k][n] order (16-byte units
//   of a row XOR-swizzled by nn_unit) and the MFMA operand (8 consecutive k
//   of one n per lane) is read with the LDS transpose read ds_read_b64_tr_b16,
//   which hands each lane of a 16-lane group 4 consecutive rows of one column
//   of a 4 x 16 block.
// * LoRA: one more 16-deep MFMA slice after the K loop, pair side = the
//   per-pair rank projection (fp32 [P, 16], rounded to bf16), weight side =
//   the bf16 pack of the scaled adapter [E, rows, 16] at the weight row of
//   each tile column; the epilogues then see the adapted product.
#include <type_traits>

#include "codebook8.h"
#include "gemm_dev.h"

namespace e4b {

// storage of the weight operand
// SK_CODE8: one code byte per weight (the int8 / fp8 lanes) and an fp32
// absmax per 64, decoded through a 256-entry table exactly like the 4-bit codes
enum { SK_ABSMAX = 0, SK_MX = 1, SK_BF16 = 2, SK_CODE8 = 3 };

// the tile shape the launches use (waves along M; see wide::Shape)
constexpr int kWideWM = 4;

namespace wide {

constexpr int kBN = 256;
// B_NN [k][n] tile row stride (elements): 576 bytes, 16 banks past a multiple
// of 64, so that the four rows x 16 columns of the two 16-lane groups that a
// transpose read serves in one pass fall on distinct banks (a 272-element
// stride put their rows 8 banks apart: 2-way conflicts)
constexpr int kSBn = kBN + 32;
constexpr uint32_t kGroupM = 4;  // m-tiles per group of the tile order

// The two shapes of the 256 x 256 tile: WM waves along M (2 along N).
//   WM = 2: 4 waves of 128 x 128 (one per SIMD), 64 MFMAs per wave per K-step;
//   WM = 4: 8 waves of 64 x 128 (two per SIMD), 32 MFMAs per wave per K-step,
//           so one wave's MFMAs run while the other waits for memory.
// Per thread: kAP A rows (16 bytes each), kNU B units (32 weights: half of
// a B_NT weight row's 64-step, or 32 columns of one B_NN row), kNE weights.
//
// Slot schedule of a K-step (staging of K-step ks + 1 into the other stage),
// one MFMA per slot:
// * fragments of k-slice kk + 1 are read in the first kNF slots of segment
//   kk, in the order the MFMAs of kk + 1 use them (A0, B0..B3, A1..);
// * 4-bit B: the two weights of pair p are looked up in slot p, the pair
//   multiplied by its block scale and rounded to bf16 kMulLag slots later,
//   group q (pairs 4q..4q+3) stored in slot bw(q);
// * A rows are stored in slots kAStore.. and reloaded (K-step ks + 2) kAP
//   slots later; the B loads of ks + 3 follow the A loads, so that the
//   in-order vmcnt counter never makes an A store wait for a B load two
//   steps ahead;
// * after slot kBarrier every wave has written its share of the next stage
//   and read its last fragment of this one: one barrier there, then the next
//   K-step's k-slice 0 fragments are read under the last MFMAs.
template <int WM>
struct Shape {
  static constexpr int kThreads = 128 * WM;
  static constexpr int kMI = 8 / WM;             // 32-row MFMA tiles per wave
  static constexpr int kSlots = 16 * kMI;        // MFMAs per wave per K-step
  static constexpr int kSeg = 4 * kMI;           // slots per k-slice
  static constexpr int kNF = kMI + 4;            // fragments per k-slice
  static constexpr int kAP = 2048 / kThreads;    // A rows per thread
  static constexpr int kNU = 512 / kThreads;     // B units per thread
  static constexpr int kNE = 32 * kNU;           // B weights per thread
  static constexpr int kNP = kNE / 2;            // their pairs
  static constexpr int kMulLag = WM == 2 ? 8 : 6;
  static constexpr int mul_slot(int p) { return p + kMulLag; }
  static constexpr int bw(int q) { return mul_slot(4 * q + 3) + 1; }
  static constexpr int kNextFrag = kSlots - kNF;
  static constexpr int kBarrier = kNextFrag - 1;
  static constexpr int kAStore = kBarrier + 1 - 2 * kAP;
  static constexpr int kALoad = kAStore + kAP;
  static constexpr int kBLoad = kALoad + kAP;
  static_assert(bw(kNE / 8 - 1) <= kBarrier && kAStore >= 0, "next-stage stores end before the barrier");
  static_assert(mul_slot(kNP - 1) < kBLoad && kBLoad < kSlots, "B reloaded after the last use of its registers");
  static_assert(2 * kSeg + kNF - 1 < kBarrier, "the last fragment read of this stage precedes the barrier");
  static_assert(kNP <= kSlots, "one pair looked up per slot");
};

__device__ __forceinline__ void slot_end() { __builtin_amdgcn_sched_barrier(0); }

// f(std::integral_constant<int, i>) for i = 0 .. N - 1, each index a constant
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace wide

template <int AMODE, int BMODE, int EPI, int SK, bool LORA, int WM>
__global__ __launch_bounds__(wide::Shape<WM>::kThreads, 1) void gemm_wide_kernel(GemmArgs g) {
  using namespace wide;
  using S = Shape<WM>;
  constexpr int kThreads = S::kThreads, kMI = S::kMI, kSlots = S::kSlots, kAP = S::kAP, kNU = S::kNU;
  constexpr int kNE = S::kNE, kNP = S::kNP, kRowsW = 32 * kMI;
  constexpr bool kQ = SK != SK_BF16;
  constexpr bool kMX = SK == SK_MX;
  constexpr bool kC8 = SK == SK_CODE8;
  constexpr bool kNN = BMODE == B_NN;
  static_assert(EPI == EPI_SWIGLU || EPI == EPI_ACT || EPI == EPI_STORE || EPI == EPI_DSWIGLU ||
                    EPI == EPI_DACT,
                "forward / dgrad epilogues");
  // the codebook first: its LDS address fits a ds_read's immediate offset
  __shared__ __attribute__((aligned(64))) float sCode[kC8 ? 256 : 16];
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kLds];
  static_assert(kBK * kSBn <= kBN * kLds, "B_NN tile fits the B stage");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave rows wm * kRowsW, columns wn * 128

  // ---- tile -> (expert, m-tile, n-tile): the W tiles of this routing split
  // into eight contiguous ranges of equal length, one per XCD (dispatch puts
  // block b on XCD b % 8); blocks past the ranges exit at once. Tile L runs
  // through groups of kGroupM consecutive m-tiles (the same expert, mostly),
  // n-tile by n-tile, so the CUs of one XCD work on a few m-tiles times a
  // few n-tiles at once and share both operands' lines in its L2 ----
  const int n_mt = g.tile_offsets[g.E];
  const uint32_t W = uint32_t(n_mt) * uint32_t(g.n_tiles);
  const uint32_t per_xcd = (W + 7) / 8, xi = blockIdx.x / 8;
  const uint32_t L = (blockIdx.x % 8) * per_xcd + xi;
  if (xi >= per_xcd || L >= W) return;
  const uint32_t grp = L / (kGroupM * uint32_t(g.n_tiles)), rem = L % (kGroupM * uint32_t(g.n_tiles));
  const uint32_t m0 = grp * kGroupM, gm = min(kGroupM, uint32_t(n_mt) - m0);
  const int mt = int(m0 + rem % gm);
  const int nt = int(rem / gm);
  const int4 tm = g.tile_map[mt];
  const int e = tm.x, seg = tm.y, row0 = tm.z, valid_rows = tm.w;

  if (kQ && !kC8 && tid < 16) sCode[tid] = codebook_value(g.cb, tid);
  if (kC8 && tid < 256) {
    const float mg = kMag8[g.cb - E4B_CB_INT8].v[tid & 127];
    sCode[tid] = tid < 128 ? mg : -mg;  // code byte = sign bit 7 | magnitude index
  }

  // ---- A: column chunk tid & 7 of rows (tid >> 3) + (kThreads / 8) i; rows
  // past the segment read the last valid row (their outputs are never stored) ----
  const int a_cc = tid & 7;
  uint32_t a_off[kAP];
#pragma unroll
  for (int i = 0; i < kAP; ++i) {
    const int r = min((tid >> 3) + (kThreads / 8) * i, valid_rows - 1);
    const int srow = seg + row0 + r;
    const int src = AMODE == A_GATHER ? g.sorted_pair[srow] / g.topk : srow;
    a_off[i] = uint32_t(src) * uint32_t(g.lda) + uint32_t(a_cc * 8);
  }

  // ---- B source; columns past N read a valid weight row / column instead ----
  const uint8_t *wp = g.Wp + int64_t(e) * g.w_e_bytes;
  const float *wa = SK == SK_ABSMAX || kC8 ? g.Wa + int64_t(e) * g.w_e_blocks : nullptr;
  const uint8_t *ws8 = kMX ? g.Ws + int64_t(e) * g.w_e_blocks : nullptr;
  const int row_bytes = kC8 ? g.w_in : (kQ ? g.w_in >> 1 : g.w_in * 2);
  const int row_blocks = g.w_in >> 6, row_mx = g.w_in >> 5;
  // B_NT: the thread owns tile column b_c = one weight row; its kNU units
  // are the 32-weight halves b_h0 .. b_h0 + kNU - 1 of the row's 64-step
  const int b_c = kNU == 2 ? tid : tid >> 1, b_h0 = kNU == 2 ? 0 : tid & 1;
  int b_row = 0;
  if (!kNN) {
    if (EPI == EPI_SWIGLU) {
      // tile column c: wave column half c >> 7 holds 64 gate rows then the
      // 64 up rows of the same pairs
      const int cw = b_c >> 7, j = (b_c & 127) >> 5, ll = b_c & 31;
      const int pair = nt * (kBN / 2) + cw * 64 + (j & 1) * 32 + ll;
      b_row = pair < g.I ? pair + (j >= 2 ? g.I : 0) : 0;
    } else {
      b_row = nt * kBN + b_c;
      b_row = b_row < g.N ? b_row : 0;
    }
  }
  const uint8_t *b_nt = wp + int64_t(b_row) * row_bytes;
  // B_NN, 4-bit: unit h of the thread = 32 consecutive columns (16 code
  // bytes inside one scale block) of one of the K-step's 64 weight rows
  // (q_row), kept in the weights' own [k][n] order in LDS
  int q_row[kNU], q_c[kNU];
  const uint8_t *b_nnq[kNU];
  const float *b_nna[kNU];
  const uint8_t *b_nns[kNU];
  // B_NN, bf16: unit h = a 4 (k) x 8 (n) patch
  int p_cg[kNU], p_kg[kNU];
  const uint8_t *b_nnb[kNU];
#pragma unroll
  for (int h = 0; h < kNU; ++h) {
    const int u = tid + kThreads * h;
    q_row[h] = u >> 3;
    q_c[h] = u & 7;
    int col = nt * kBN + q_c[h] * 32;
    col = col < g.N ? col : 0;
    b_nnq[h] = wp + int64_t(q_row[h]) * row_bytes + (kC8 ? col : col >> 1);
    b_nna[h] = SK == SK_ABSMAX || kC8 ? wa + int64_t(q_row[h]) * row_blocks + (col >> 6) : nullptr;
    b_nns[h] = kMX ? ws8 + int64_t(q_row[h]) * row_mx + (col >> 5) : nullptr;
    p_cg[h] = u >> 4;
    p_kg[h] = u & 15;
    int n = nt * kBN + p_cg[h] * 8;
    n = n < g.N ? n : 0;
    b_nnb[h] = wp + int64_t(p_kg[h] * 4) * row_bytes + n * 2;
  }

  const int nK = g.K / kBK;

  // ---- registers of the staging pipeline ----
  u32x4 ra[kAP];                    // A rows of K-step ks + 1
  u32x4 rb[2][kNU];                 // 4-bit B: codes of two K-steps (sets by parity)
  u32x4 rb2[2][kNU];                // 8-bit B: the second 16 code bytes of each unit
  float rs[2][kNU];                 // their block scales (per unit)
  u32x4 rq[4 * kNU];                // bf16 B of K-step ks + 1

  auto load_a = [&](int ks) {
#pragma unroll
    for (int i = 0; i < kAP; ++i)
      ra[i] = *reinterpret_cast<const u32x4 *>(g.A + a_off[i] + uint32_t(ks * kBK));
  };
  auto load_a_one = [&](int ks, int i) {
    ra[i] = *reinterpret_cast<const u32x4 *>(g.A + a_off[i] + uint32_t(ks * kBK));
  };
  // 4-bit B of K-step ks into register set st
  auto load_b = [&](int ks, int st) {
    if (!kNN) {
      const u32x4 *src = reinterpret_cast<const u32x4 *>(b_nt + ks * (kC8 ? kBK : kBK / 2));
#pragma unroll
      for (int h = 0; h < kNU; ++h) {
        if (kC8) {
          rb[st][h] = src[2 * (b_h0 + h)];
          rb2[st][h] = src[2 * (b_h0 + h) + 1];
        } else {
          rb[st][h] = src[b_h0 + h];
        }
        // a 64-step is one absmax block, or two MX blocks (one per half)
        rs[st][h] = kMX ? e8m0_value(ws8[int64_t(b_row) * row_mx + 2 * ks + b_h0 + h])
                        : wa[int64_t(b_row) * row_blocks + ks];
      }
    } else {
#pragma unroll
      for (int h = 0; h < kNU; ++h) {
        rb[st][h] = *reinterpret_cast<const u32x4 *>(b_nnq[h] + int64_t(ks) * kBK * row_bytes);
        if (kC8) rb2[st][h] = *reinterpret_cast<const u32x4 *>(b_nnq[h] + int64_t(ks) * kBK * row_bytes + 16);
        rs[st][h] = kMX ? e8m0_value(b_nns[h][int64_t(ks) * kBK * row_mx])
                        : b_nna[h][int64_t(ks) * kBK * row_blocks];
      }
    }
  };
  auto load_q = [&](int ks) {
#pragma unroll
    for (int d = 0; d < 4 * kNU; ++d) {
      if (!kNN)
        rq[d] = *reinterpret_cast<const u32x4 *>(b_nt + ks * (kBK * 2) + b_h0 * 64 + d * 16);
      else
        rq[d] = *reinterpret_cast<const u32x4 *>(b_nnb[d >> 2] + (int64_t(ks) * kBK + (d & 3)) * row_bytes);
    }
  };

  auto store_a_one = [&](int buf, int i) {
    *reinterpret_cast<u32x4 *>(sA[buf] + ((tid >> 3) + (kThreads / 8) * i) * kLds + a_cc * 8) = ra[i];
  };
  // bf16 B: group q (B_NT, q < 4 kNU: 8 k of the thread's column; B_NN,
  // q < 2 kNU: 4 columns of a 4 x 8 patch, transposed by byte permutes)
  auto store_q_one = [&](int buf, int q) {
    uint16_t *dst = sB[buf];
    if (!kNN) {
      if (q < 4 * kNU) *reinterpret_cast<u32x4 *>(dst + b_c * kLds + b_h0 * 32 + q * 8) = rq[q];
    } else if (q < 2 * kNU) {
      const int h = q >> 1, c0 = (q & 1) * 4;
#pragma unroll
      for (int c = c0; c < c0 + 4; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        *reinterpret_cast<u32x2 *>(dst + (p_cg[h] * 8 + c) * kLds + p_kg[h] * 4) =
            u32x2{__builtin_amdgcn_perm(rq[4 * h + 1][c >> 1], rq[4 * h][c >> 1], sel),
                  __builtin_amdgcn_perm(rq[4 * h + 3][c >> 1], rq[4 * h + 2][c >> 1], sel)};
      }
    }
  };

  // 4-bit B dequantization: element el of the thread's kNE (unit el >> 5;
  // B_NT: k of its column; B_NN: column el & 31); the byte offset
  // (4 * nibble) of its table entry, then the entry
  const char *tbl = reinterpret_cast<const char *>(sCode);
  float cv[kNE];
  auto lookup = [&](int st, int el) {
    if constexpr (kC8) {
      // byte el & 31 of the unit: the table offset 4 * byte
      const int b = el & 31;
      const uint32_t word = (b < 16 ? rb[st][el >> 5] : rb2[st][el >> 5])[(b >> 2) & 3];
      const uint32_t off = __builtin_amdgcn_perm(0u, word, 0x0C0C0C00u | uint32_t(b & 3)) << 2;
      cv[el] = *reinterpret_cast<const float *>(tbl + off);
    } else {
      const uint32_t word = rb[st][el >> 5][(el >> 3) & 3];
      const uint32_t sh = (el & 1) ? (word << 2) : (word >> 2);
      const uint32_t off = __builtin_amdgcn_perm(0u, sh & 0x3C3C3C3Cu, 0x0C0C0C00u | uint32_t((el >> 1) & 3));
      cv[el] = *reinterpret_cast<const float *>(tbl + off);
    }
  };
  uint32_t bq[kNP];
  auto mul_pair = [&](int st, int p) {
    const float s = rs[st][p >> 4];
    bq[p] = pack_bf16x2(__fmul_rn(cv[2 * p], s), __fmul_rn(cv[2 * p + 1], s));
  };
  auto store_b_group = [&](int buf, int q) {
    const u32x4 v{bq[4 * q], bq[4 * q + 1], bq[4 * q + 2], bq[4 * q + 3]};
    if (!kNN)
      *reinterpret_cast<u32x4 *>(sB[buf] + b_c * kLds + b_h0 * 32 + q * 8) = v;
    else
      *reinterpret_cast<u32x4 *>(sB[buf] + q_row[q >> 2] * kSBn + nn_unit(4 * q_c[q >> 2] + (q & 3)) * 8) = v;
  };

  // ---- fragments: A rows wm * kRowsW + 32 i, B columns wn * 128 + 32 j ----
  // B_NN transpose-read addresses: lane (group qg = lane / 16, qs = lane % 16)
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
  bf16x8 af[2][kMI], bfr[2][4];
  // fragment f of k-slice kk: f < 4 B column tile f, f >= 4 A row tile f - 4
  auto frag_one = [&](int buf, int kk, int slot, int f) {
    if (f >= 4) {
      af[slot][f - 4] = *reinterpret_cast<const bf16x8 *>(sA[buf] + (wm * kRowsW + (f - 4) * 32 + (lane & 31)) * kLds +
                                                         (lane >> 5) * 8 + kk * 16);
    } else if (kNN && kQ) {
      const uint16_t *p = sB[buf] + q_off[f] + kk * 16 * kSBn;
      const s16x4 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * kSBn);
      bfr[slot][f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      bfr[slot][f] = *reinterpret_cast<const bf16x8 *>(sB[buf] + (wn * 128 + f * 32 + (lane & 31)) * kLds +
                                                      (lane >> 5) * 8 + kk * 16);
    }
  };
  // the order in which the MFMAs of a k-slice first use them: A0, B0..B3, A1..
  auto frag_in_order = [&](int buf, int kk, int slot, int w) {
    frag_one(buf, kk, slot, w == 0 ? 4 : (w <= 4 ? w - 1 : w));
  };

  f32x16 acc[kMI][4];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- prologue: stage 0 <- K-step 0; registers <- K-step 1 (A, B set 1)
  // and K-step 2 (B set 0) ----
  __syncthreads();  // sCode visible
  const int k1 = min(1, nK - 1), k2 = min(2, nK - 1);
  load_a(0);
  if (kQ) {
    load_b(0, 0);
    load_b(k1, 1);
#pragma unroll
    for (int el = 0; el < kNE; ++el) lookup(0, el);
#pragma unroll
    for (int p = 0; p < kNP; ++p) mul_pair(0, p);
#pragma unroll
    for (int q = 0; q < kNE / 8; ++q) store_b_group(0, q);
    load_b(k2, 0);
  } else {
    load_q(0);
#pragma unroll
    for (int q = 0; q < 4 * kNU; ++q) store_q_one(0, q);
    load_q(k1);
  }
#pragma unroll
  for (int i = 0; i < kAP; ++i) store_a_one(0, i);
  load_a(k1);
  __syncthreads();
  static_for<S::kNF>([&](auto f) { frag_in_order(0, 0, 0, f); });

  // ---- one K-step: compute stage CUR (K-step ks) while staging K-step
  // ks + 1 into stage CUR ^ 1 from register set CUR ^ 1 ----
  auto kstep = [&](auto cur_c, int ks) {
    constexpr int CUR = decltype(cur_c)::value, NXT = CUR ^ 1;
    const int ka = min(ks + 2, nK - 1), kb = min(ks + 3, nK - 1);
    static_for<kSlots>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      constexpr int kk = s / S::kSeg, w = s % S::kSeg, fs = kk & 1;
      // the MFMA of this slot: tile (i, j) = (w >> 2, w & 3) of k-slice kk;
      // weights are the MFMA A-operand, so acc[i][j] holds D[col][row]
      acc[w >> 2][w & 3] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[fs][w & 3], af[fs][w >> 2], acc[w >> 2][w & 3], 0, 0, 0);
      if constexpr (kk < 3 && w < S::kNF) frag_in_order(CUR, kk + 1, fs ^ 1, w);
      if constexpr (kQ) {
        if constexpr (s < kNP) {
          lookup(NXT, 2 * s);
          lookup(NXT, 2 * s + 1);
        }
        if constexpr (s >= S::kMulLag && s < S::kMulLag + kNP) mul_pair(NXT, s - S::kMulLag);
        static_for<kNE / 8>([&](auto qc) {
          if constexpr (S::bw(decltype(qc)::value) == s) store_b_group(NXT, decltype(qc)::value);
        });
        if constexpr (s == S::kBLoad) load_b(kb, NXT);
      } else {
        if constexpr (s >= 2 && s < 2 + 4 * kNU) store_q_one(NXT, s - 2);
        if constexpr (s == 2 + 4 * kNU) load_q(ka);
      }
      if constexpr (s >= S::kAStore && s < S::kAStore + kAP) store_a_one(NXT, s - S::kAStore);
      if constexpr (s >= S::kALoad && s < S::kALoad + kAP) load_a_one(ka, s - S::kALoad);
      if constexpr (s == S::kBarrier) {
        slot_end();
        __syncthreads();
      }
      // the next K-step's k-slice 0 from the stage just written (buffer 0:
      // k-slice 3 of this step reads buffer 1)
      if constexpr (s >= S::kNextFrag) frag_in_order(NXT, 0, 0, s - S::kNextFrag);
      slot_end();
    });
  };
  // pairs of K-steps (a branch-free loop body), then an odd last step
  int ks = 0;
  for (; ks + 1 < nK; ks += 2) {
    kstep(std::integral_constant<int, 0>{}, ks);
    kstep(std::integral_constant<int, 1>{}, ks + 1);
  }
  if (ks < nK) kstep(std::integral_constant<int, 0>{}, ks);

  // ---- LoRA: one more 16-deep slice ----
  if constexpr (LORA) {
    const int kh = lane >> 5;
    bf16x8 pf[kMI], wf[4];
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
      const int r = min(wm * kRowsW + i * 32 + (lane & 31), valid_rows - 1);
      const float4 *src =
          reinterpret_cast<const float4 *>(g.lora_p + int64_t(seg + row0 + r) * kLoraK + 8 * kh);
      const float4 v0 = src[0], v1 = src[1];
      const u32x4 q{pack_bf16x2(v0.x, v0.y), pack_bf16x2(v0.z, v0.w), pack_bf16x2(v1.x, v1.y),
                    pack_bf16x2(v1.z, v1.w)};
      pf[i] = __builtin_bit_cast(bf16x8, q);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int row;
      if (!kNN && EPI == EPI_SWIGLU) {
        const int pair = nt * (kBN / 2) + wn * 64 + (j & 1) * 32 + (lane & 31);
        row = pair < g.I ? pair + (j >= 2 ? g.I : 0) : 0;
      } else {
        row = nt * kBN + wn * 128 + j * 32 + (lane & 31);
        row = row < g.N ? row : 0;
      }
      wf[j] = *reinterpret_cast<const bf16x8 *>(g.lora_w + (int64_t(e) * g.lora_rows + row) * kLoraK + 8 * kh);
    }
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], pf[i], acc[i][j], 0, 0, 0);
  }

  // ---- epilogue ----
  // acc[i][j][4q + t]: tile row = wm*kRowsW + i*32 + lane%32,
  //                    tile col = wn*128 + j*32 + 8q + 4*(lane/32) + t   (t = 0..3)
  const int lrow = wm * kRowsW + (lane & 31);
  const int lcol = wn * 128 + 4 * (lane >> 5);
  if (EPI == EPI_STORE) {
    // Through LDS, so that the stores are whole row segments: rows 0..127 of
    // the tile go to the A stages, rows 128..255 to the B stages (bf16, row
    // stride kOut), then every thread writes 16 contiguous bytes, a wave two
    // 512-byte row segments. The barrier retires the last K-step's reads of
    // the next-step fragments.
    constexpr int kOut = kBN + 8;
    __syncthreads();
    static_assert(128 * kOut <= 2 * kBM * kLds && 128 * kOut <= 2 * kBN * kLds, "half a tile fits each stage pair");
    uint16_t *half = wm * kRowsW < 128 ? sA[0] : sB[0];
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
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
    for (int pass = 0; pass < kBM / (kThreads / 32); ++pass) {
      const int row = pass * (kThreads / 32) + (tid >> 5);
      const uint16_t *src = (row < 128 ? sA[0] : sB[0]) + (row & 127) * kOut + cc;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(src);
      if (row < valid_rows && col < g.N)
        *reinterpret_cast<u32x4 *>(g.C + int64_t(seg + row0 + row) * g.ldc + col) = v;
    }
  } else if (EPI == EPI_SWIGLU) {
    // a = silu(g) u of the wave's 64 pairs goes out through the wave's own LDS
    // rows (one row tile of 32 rows at a time) as 128-byte row segments; the
    // g|u chunks are stored directly (a wave writes 1 KB per instruction)
    constexpr int kASt = 64 + 8;  // staging row: 64 pairs of a (bf16) + pad
    static_assert(4 * 32 * kASt <= 2 * kBM * kLds, "four waves' staging rows fit a stage pair");
    if (g.C) __syncthreads();  // uniform: every wave has read its last fragments of the stages
    uint16_t *stg = (wave < 4 ? sA[0] : sB[0]) + (wave & 3) * 32 * kASt;
    uint16_t *srow = stg + (lane & 31) * kASt;
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
      const int row = lrow + i * 32;
      if (row < valid_rows) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int pw = jj * 32 + 8 * q + 4 * (lane >> 5);  // pair within the wave's 64
            const int pair = nt * (kBN / 2) + wn * 64 + pw;
            if (pair < g.I) {
              float gv[4], uv[4], av[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                gv[t] = acc[i][jj][4 * q + t];
                uv[t] = acc[i][jj + 2][4 * q + t];
                av[t] = gv[t] * sigmoidf_(gv[t]) * uv[t];
              }
              if (g.C)
                *reinterpret_cast<u32x2 *>(srow + pw) = u32x2{pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3])};
              static_assert(EPI != EPI_SWIGLU || kBN / 2 == kGuBlockPairs, "one g|u block per tile");
              if (g.GU) {
                // the tile's 128 pairs are block nt of the blocked g|u
                const int64_t ch = gu_chunk(mt, nt, g.n_tiles, row, pair - nt * (kBN / 2));
                *reinterpret_cast<u32x4 *>(g.GU + ch * 8) =
                    u32x4{pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3]), pack_bf16x2(uv[0], uv[1]),
                          pack_bf16x2(uv[2], uv[3])};
              }
            }
          }
      }
      if (g.C) {
        // row tile i staged (the wave's own rows: LDS keeps one wave's
        // operations in order): eight rows of 128 bytes per instruction
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int r = 8 * it + (lane >> 3), ch = lane & 7;
          const int trow = wm * kRowsW + i * 32 + r;
          const int pair0 = nt * (kBN / 2) + wn * 64 + ch * 8;
          const u32x4 o = *reinterpret_cast<const u32x4 *>(stg + r * kASt + ch * 8);
          if (trow < valid_rows && pair0 < g.I)
            *reinterpret_cast<u32x4 *>(g.C + (seg + row0 + trow) * int64_t(g.ldc) + pair0) = o;
        }
      }
    }
  } else if (EPI == EPI_DSWIGLU) {
    // down dgrad of a gated layer: the wave's 128 columns are the pairs of
    // g|u block blk = 2 nt + wn. Per pair, from the saved g|u and the routing
    // weight w: grad_a = w G2, dg = grad_a u silu'(g), du = grad_a silu(g)
    // (bf16 into dGU [row, g | u]); per row, the block's share of
    // d y / d w = sum of G2 silu(g) u over its pairs. Each row tile of the
    // wave (32 rows x 128 dg | 128 du) is staged in the wave's own LDS rows
    // and leaves as 256-byte row segments.
    static_assert(EPI != EPI_DSWIGLU || kBN == 2 * kGuBlockPairs, "two g|u blocks per tile");
    constexpr int kDgSt = 2 * kGuBlockPairs + 8;  // staging row: dg | du of 128 pairs (bf16) + pad
    static_assert(4 * 32 * kDgSt <= 2 * kBM * kLds && 4 * 32 * kDgSt <= 2 * kBN * kLds,
                  "four waves' staging rows fit each stage pair");
    const int npb = (g.I + kGuBlockPairs - 1) / kGuBlockPairs;
    const int blk = 2 * nt + wn;
    const int nvalid = min(kGuBlockPairs, g.I - blk * kGuBlockPairs);  // pairs of this block (a multiple of 64)
    const int cmax = nvalid - 4;                                        // last chunk the forward wrote
    // every wave has read its last fragments of the stages before they are reused
    __syncthreads();
    uint16_t *stg = (wave < 4 ? sA[0] : sB[0]) + (wave & 3) * 32 * kDgSt;
    if (cmax >= 0) {  // uniform over the wave
      // the lane's 4 chunks of batch b = (row tile i, column tile j) = (b / 4, b % 4)
      // (g[4], u[4] of 4 consecutive pairs each), clamped to chunks the forward
      // wrote (results past I are not stored); batch b + 1 is in flight while
      // batch b is used
      int rr[kMI];
      float wr[kMI];
#pragma unroll
      for (int i = 0; i < kMI; ++i) rr[i] = min(lrow + i * 32, valid_rows - 1);
#pragma unroll
      for (int i = 0; i < kMI; ++i) wr[i] = g.topk_w[g.sorted_pair[seg + row0 + rr[i]]];
      u32x4 v[2][4];
      auto fetch = [&](int b, int slot) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = min((b & 3) * 32 + 8 * q + 4 * (lane >> 5), cmax);
          v[slot][q] = *reinterpret_cast<const u32x4 *>(g.GU + gu_chunk(mt, blk, npb, rr[b >> 2], c) * 8);
        }
      };
      float part[kMI];
#pragma unroll
      for (int i = 0; i < kMI; ++i) part[i] = 0.0f;
      uint16_t *srow = stg + (lane & 31) * kDgSt;
      fetch(0, 0);
#pragma unroll
      for (int b = 0; b < 4 * kMI; ++b) {
        if (b + 1 < 4 * kMI) fetch(b + 1, (b + 1) & 1);
        const int i = b >> 2, j = b & 3;
        const int row = lrow + i * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = j * 32 + 8 * q + 4 * (lane >> 5);
          const u32x4 cv4 = v[b & 1][q];
          const float gv[4] = {bf16_lo(cv4[0]), bf16_hi(cv4[0]), bf16_lo(cv4[1]), bf16_hi(cv4[1])};
          const float uv[4] = {bf16_lo(cv4[2]), bf16_hi(cv4[2]), bf16_lo(cv4[3]), bf16_hi(cv4[3])};
          float dg[4], du[4], pq = 0.0f;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float sg = sigmoidf_(gv[t]);
            const float silu = gv[t] * sg;
            const float G2 = acc[i][j][4 * q + t];
            pq += G2 * (silu * uv[t]);
            const float ga = wr[i] * G2;
            dg[t] = ga * uv[t] * sg * (1.0f + gv[t] * (1.0f - sg));
            du[t] = ga * silu;
          }
          if (row < valid_rows && c <= cmax) part[i] += pq;
          *reinterpret_cast<u32x2 *>(srow + c) = u32x2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
          *reinterpret_cast<u32x2 *>(srow + kGuBlockPairs + c) =
              u32x2{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
        }
        if (j == 3) {
          // row tile i staged (the wave's own rows: LDS keeps one wave's
          // operations in order): two rows per instruction, each as a
          // 256-byte dg segment and a 256-byte du segment
#pragma unroll 4
          for (int it = 0; it < 16; ++it) {
            const int r = 2 * it + (lane >> 5), half = (lane >> 4) & 1, ch = lane & 15;
            const int trow = wm * kRowsW + i * 32 + r;
            const u32x4 o = *reinterpret_cast<const u32x4 *>(stg + r * kDgSt + half * kGuBlockPairs + ch * 8);
            if (trow < valid_rows && ch * 8 < nvalid)
              *reinterpret_cast<u32x4 *>(g.C + (seg + row0 + trow) * int64_t(g.ldc) + (half ? g.I : 0) +
                                         blk * kGuBlockPairs + ch * 8) = o;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kMI; ++i) {
        // the two half-waves hold the two column halves of the same rows
        const float pr = part[i] + __shfl_xor(part[i], 32);
        if (lane < 32 && lrow + i * 32 < valid_rows) g.partial[(seg + row0 + rr[i]) * int64_t(npb) + blk] = pr;
      }
    }
  } else if (EPI == EPI_DACT) {
    // down dgrad of an ungated layer: the wave's 128 columns are the
    // intermediate units of block blk = 2 nt + wn. Per unit, from the saved h
    // and the routing weight w: dh = w G2 silu'(h) (bf16 into dH [row, unit]);
    // per row, the block's share of d y / d w = sum of G2 silu(h). Each row
    // tile of the wave (32 rows x 128 units) is staged in the wave's own LDS
    // rows and leaves as 256-byte row segments.
    constexpr int kDhSt = kGuBlockPairs + 8;  // staging row: 128 units of dh (bf16) + pad
    static_assert(4 * 32 * kDhSt <= 2 * kBM * kLds, "four waves' staging rows fit a stage pair");
    const int npb = (g.I + kGuBlockPairs - 1) / kGuBlockPairs;
    const int blk = 2 * nt + wn;
    const int nvalid = min(kGuBlockPairs, g.I - blk * kGuBlockPairs);  // units of this block (a multiple of 64)
    __syncthreads();  // every wave has read its last fragments of the stages
    uint16_t *stg = (wave < 4 ? sA[0] : sB[0]) + (wave & 3) * 32 * kDhSt;
    if (nvalid > 0) {  // uniform over the wave
      int rr[kMI];
      float wr[kMI];
#pragma unroll
      for (int i = 0; i < kMI; ++i) rr[i] = min(lrow + i * 32, valid_rows - 1);
#pragma unroll
      for (int i = 0; i < kMI; ++i) wr[i] = g.topk_w[g.sorted_pair[seg + row0 + rr[i]]];
      // h of batch b = (row tile i, column tile j): the lane's 4 runs of 4
      // units, clamped to units below I; batch b + 1 is in flight while b is used
      u32x2 v[2][4];
      auto fetch = [&](int b, int slot) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = min((b & 3) * 32 + 8 * q + 4 * (lane >> 5), nvalid - 4);
          v[slot][q] = *reinterpret_cast<const u32x2 *>(g.GU + (seg + row0 + rr[b >> 2]) * int64_t(g.ldgu) +
                                                        blk * kGuBlockPairs + c);
        }
      };
      float part[kMI];
#pragma unroll
      for (int i = 0; i < kMI; ++i) part[i] = 0.0f;
      uint16_t *srow = stg + (lane & 31) * kDhSt;
      fetch(0, 0);
#pragma unroll
      for (int b = 0; b < 4 * kMI; ++b) {
        if (b + 1 < 4 * kMI) fetch(b + 1, (b + 1) & 1);
        const int i = b >> 2, j = b & 3;
        const int row = lrow + i * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = j * 32 + 8 * q + 4 * (lane >> 5);
          const u32x2 hq = v[b & 1][q];
          const float hv[4] = {bf16_lo(hq[0]), bf16_hi(hq[0]), bf16_lo(hq[1]), bf16_hi(hq[1])};
          float dh[4], pq = 0.0f;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float sg = sigmoidf_(hv[t]);
            const float G2 = acc[i][j][4 * q + t];
            pq += G2 * (hv[t] * sg);
            dh[t] = wr[i] * G2 * sg * (1.0f + hv[t] * (1.0f - sg));
          }
          if (row < valid_rows && c < nvalid) part[i] += pq;
          *reinterpret_cast<u32x2 *>(srow + c) = u32x2{pack_bf16x2(dh[0], dh[1]), pack_bf16x2(dh[2], dh[3])};
        }
        if (j == 3) {
          // row tile i staged (the wave's own rows: LDS keeps one wave's
          // operations in order): four rows of 256 bytes per instruction
#pragma unroll
          for (int it = 0; it < 8; ++it) {
            const int r = 4 * it + (lane >> 4), ch = lane & 15;
            const int trow = wm * kRowsW + i * 32 + r;
            const u32x4 o = *reinterpret_cast<const u32x4 *>(stg + r * kDhSt + ch * 8);
            if (trow < valid_rows && ch * 8 < nvalid)
              *reinterpret_cast<u32x4 *>(g.C + (seg + row0 + trow) * int64_t(g.ldc) + blk * kGuBlockPairs + ch * 8) = o;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kMI; ++i) {
        // the two half-waves hold the two column halves of the same rows
        const float pr = part[i] + __shfl_xor(part[i], 32);
        if (lane < 32 && lrow + i * 32 < valid_rows) g.partial[(seg + row0 + rr[i]) * int64_t(npb) + blk] = pr;
      }
    }
  } else {  // EPI_ACT: ungated, h = this tile's columns of the up projection, a = silu(h)
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
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
  }
}

namespace {
hipError_t launch_gemm_wide(GemmVariant v, const GemmArgs &a, hipStream_t s, const e4b_kernel_events *ev) {
  if (a.grid == 0) return hipSuccess;
  // a multiple of 8 blocks: each XCD then has at least ceil(W / 8) of them
  const dim3 grid((a.grid + 7) / 8 * 8), block(wide::Shape<kWideWM>::kThreads);
  const int kid = int(v);
  const bool c8 = a.cb == E4B_CB_INT8 || a.cb == E4B_CB_FP8;
  const int sk = a.cb == E4B_CB_BF16 ? SK_BF16 : (a.mx ? SK_MX : (c8 ? SK_CODE8 : SK_ABSMAX));
#define E4B_WIDE_SK(AM, BM, EP, LO)                                                                          \
  return sk == SK_BF16    ? launch_k(ev, kid, gemm_wide_kernel<AM, BM, EP, SK_BF16, LO, kWideWM>, grid, block, s, a)  \
         : sk == SK_CODE8 ? launch_k(ev, kid, gemm_wide_kernel<AM, BM, EP, SK_CODE8, LO, kWideWM>, grid, block, s, a) \
         : sk == SK_MX    ? launch_k(ev, kid, gemm_wide_kernel<AM, BM, EP, SK_MX, LO, kWideWM>, grid, block, s, a)    \
                       : launch_k(ev, kid, gemm_wide_kernel<AM, BM, EP, SK_ABSMAX, LO, kWideWM>, grid, block, s, a)
#define E4B_WIDE(AM, BM, EP)                     \
  do {                                           \
    if (a.lora_p) E4B_WIDE_SK(AM, BM, EP, true); \
    E4B_WIDE_SK(AM, BM, EP, false);              \
  } while (0)
  switch (v) {
    case GEMM_GATE_UP_FWD:
      if (a.gated) E4B_WIDE(A_GATHER, B_NT, EPI_SWIGLU);
      E4B_WIDE(A_GATHER, B_NT, EPI_ACT);
    case GEMM_DOWN_FWD: E4B_WIDE(A_DIRECT, B_NT, EPI_STORE);
    case GEMM_GATE_UP_DGRAD: E4B_WIDE(A_DIRECT, B_NN, EPI_STORE);
    case GEMM_DOWN_DGRAD:
      if (a.gated) E4B_WIDE(A_GATHER, B_NN, EPI_DSWIGLU);
      E4B_WIDE(A_GATHER, B_NN, EPI_DACT);
    default: break;
  }
#undef E4B_WIDE_SK
#undef E4B_WIDE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_grouped_gemm(GemmVariant v, const GemmArgs &a, hipStream_t s, const e4b_kernel_events *ev) {
  if (v != GEMM_DOWN_DGRAD) return launch_gemm_wide(v, a, s, ev);
  // the down dgrad arrives planned per 128-unit block (the routing-weight
  // partials keep one entry per block); its tiles are 256 columns wide: the
  // same m-tiles, half as many n-tiles
  GemmArgs w = a;
  w.n_tiles = (a.N + 2 * kGuBlockPairs - 1) / (2 * kGuBlockPairs);
  w.grid = a.n_tiles > 0 ? a.grid / uint32_t(a.n_tiles) * uint32_t(w.n_tiles) : 0;
  return launch_gemm_wide(v, w, s, ev);
}

}  // namespace e4b
