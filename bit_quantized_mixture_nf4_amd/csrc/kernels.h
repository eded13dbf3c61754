// kernels.h -- host-side launchers of the library's kernels (internal).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace e4b {

// Chunk index (16 bytes: g[4] then u[4], bf16, of 4 consecutive pairs) of row
// r of m-tile mt and pair c of 128-pair column block pb (npb blocks per
// m-tile) in a gated layer's saved / recomputed g|u. Within a block, lane
// r % 32 + 32 ((c % 8) / 4) of run ((r / 32, c / 32), (c % 32) / 8): a wave
// of the GEMM epilogues that write and read it moves 1 KB per instruction.
__device__ __forceinline__ int64_t gu_chunk(int mt, int pb, int npb, int r, int c) {
  return (int64_t(mt) * npb + pb) * kGuBlockChunks +
         ((((r >> 5) * 4 + (c >> 5)) * 4 + ((c & 31) >> 3)) * 64 + ((c & 7) >> 2) * 32 + (r & 31));
}

enum GemmVariant {
  GEMM_GATE_UP_FWD = 0,   // A gathered x,      B = W_gu rows,    SiLU*up (or SiLU) epilogue
  GEMM_DOWN_FWD = 1,      // A sorted a,        B = W_dn rows,    bf16 store
  GEMM_DOWN_DGRAD = 2,    // A gathered grad_y, B = W_dn^T,       SiLU-backward epilogue
  GEMM_GATE_UP_DGRAD = 3  // A sorted dGU,      B = W_gu^T,       bf16 store
};

struct GemmArgs {
  const uint16_t *A;
  int32_t lda;
  const int32_t *sorted_pair;
  int32_t topk;
  const uint8_t *Wp;   // packed stack
  const float *Wa;     // absmax stack (NF4, FP4)
  const uint8_t *Ws;   // E8M0 scale stack (MXFP4, one byte per 32 elements)
  int32_t mx;          // 1: MXFP4 (scales in Ws), 0: absmax in Wa
  int64_t w_e_bytes;   // packed bytes per expert
  int64_t w_e_blocks;  // absmax (or MXFP4 scale) entries per expert
  int32_t w_in;        // stored in_features
  int32_t N;           // output columns (gate/up: number of gate-up pairs = I)
  int32_t K;           // reduction length (multiple of 64)
  int32_t I;           // intermediate size
  const int32_t *offsets;
  const int32_t *tile_offsets;
  const int4 *tile_map;  // per m-tile: expert, segment start, first row, rows
  int32_t E;
  int32_t n_tiles;
  uint32_t grid;
  int32_t cb;
  uint16_t *C;  // STORE: C[row, col]; gate_up fwd: a[row, pair] (may be null); down dgrad: dGU
  int32_t ldc;
  uint16_t *GU;  // gate_up fwd: out g|u [row, 2I] (may be null); down dgrad: in g|u
  const float *topk_w;
  float *partial;  // down dgrad: [P, n_tiles]
  int32_t gated;   // gate_up fwd / down dgrad: 1 SwiGLU pairs, 0 a plain activation of the up rows
  int32_t ldgu;    // row stride of the saved g|u (gated, 2I) or h (ungated, I)
  // LoRA slice (null: none): per-pair projection fp32 [P, kLoraK] in sorted
  // order, and the bf16 pack of the scaled adapter [E, lora_rows, kLoraK]
  // indexed by the weight row of each output column
  const float *lora_p;
  const uint16_t *lora_w;
  int32_t lora_rows;
};

// Launch of `kernel` on `s`, bracketed by the call's events for kernel id
// `kid` when the caller passed both (e4b_kernel_events): hipExtLaunchKernelGGL
// records them at the dispatch's start and end.
template <typename F, typename... Args>
inline hipError_t launch_k(const e4b_kernel_events *ev, int kid, F kernel, dim3 grid, dim3 block,
                           hipStream_t s, Args... args) {
  hipEvent_t e0 = ev ? ev->start[kid] : nullptr, e1 = ev ? ev->stop[kid] : nullptr;
  if (e0 && e1)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError();
}

// An expert id as the kernels use it: ids outside [0, E) read as expert 0,
// so no index derived from a bad id leaves its buffer.
__device__ __forceinline__ int safe_expert(int32_t id, int E) {
  return uint32_t(id) < uint32_t(E) ? id : 0;
}

hipError_t launch_route(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w,
                        hipStream_t s, const e4b_kernel_events *ev = nullptr);

// Where the routing permutation lives: in the workspace, or in the saved
// buffer when the forward keeps it for the dgrad.
struct PermView {
  int32_t *offsets;       // [E + 1] first sorted position of each expert
  int32_t *tile_offsets;  // [E + 1] first m-tile of each expert
  int4 *tile_map;         // [m_tiles_bound] expert, segment start, first row, rows
  int32_t *sorted;        // [P] pair id at sorted position
  int32_t *pos;           // [P] sorted position of pair id
};
PermView perm_in_workspace(const MoePlan &p, char *ws);
PermView perm_in_saved(const MoePlan &p, char *saved);

// Fills the permutation (histogram scratch and counts in the workspace).
hipError_t launch_permute(const MoePlan &p, const int32_t *idx, char *ws, const PermView &v,
                          hipStream_t s, const e4b_kernel_events *ev = nullptr);

// The MX forward's grouped GEMM (csrc/mx.hip): MXFP4 weights against MXFP8
// activation rows (codes with the bytes of each element pair swapped, E8M0
// scale per 32), K a multiple of 128.
struct MxGemmArgs {
  const int32_t *sorted_pair;  // gate_up: activation row = token of the sorted pair
  int32_t topk;
  const uint8_t *Wp;  // packed E2M1 stack
  const uint8_t *Ws;  // E8M0 scales of the stack
  int64_t w_e_bytes, w_e_blocks;
  const uint8_t *A;   // activation codes [rows, K]
  const uint8_t *As;  // activation scales [rows, K / 32]
  int32_t K, N, I, E;
  const int32_t *tile_offsets;
  const int4 *tile_map;
  int32_t n_tiles;
  uint32_t grid;
  uint16_t *C;    // down: o [P, H] bf16
  int32_t ldc;
  uint8_t *Cq;    // gate_up: a = bf16(silu(g) * u) as MXFP8 codes [P, I], element pairs swapped
  uint8_t *Cs;    // gate_up: the E8M0 scales of a [P, I / 32]
};
hipError_t launch_mx8_rows(const uint16_t *x, int64_t rows, int64_t K, uint8_t *codes,
                           uint8_t *scales, hipStream_t s);
hipError_t launch_mx_gemm(bool gate_up, const MxGemmArgs &a, hipStream_t s,
                          const e4b_kernel_events *ev = nullptr);

// The grouped GEMMs (gemm_wide.hip, 256 x 256 tiles). grid = m_tiles_bound *
// n_tiles; the launch rounds it up to a multiple of 8. The down dgrad is given
// n_tiles over 128-unit blocks (the routing-weight partials' granularity).
hipError_t launch_grouped_gemm(GemmVariant v, const GemmArgs &a, hipStream_t s,
                               const e4b_kernel_events *ev = nullptr);

// y[t] = sum_j w[t, j] * rows[pos(t, j)] in fp32, slot order.
hipError_t launch_combine_rows(const uint16_t *rows, const int32_t *pos_of_pair, const float *w,
                               int64_t T, int k, int H, uint16_t *out, hipStream_t s,
                               const e4b_kernel_events *ev = nullptr);
// grad_x[t] = sum_j rows[pos(t, j)], and (gw not null) gw[t, j] = the sum of
// partial[pos(t, j)][0 .. n_tiles) in ascending order.
hipError_t launch_combine_dgrad(const uint16_t *rows, const int32_t *pos_of_pair, int64_t T, int k,
                                int H, uint16_t *out, const float *partial, int n_tiles,
                                float *gw, hipStream_t s, const e4b_kernel_events *ev = nullptr);

// An INT8 / FP8 stack dequantized to bf16 (bf16 == true) or fp32 [E, out, in]
// (quant.hip).
hipError_t launch_dequantize8(const e4b_stack &st, bool bf16, void *out, hipStream_t s);

// The decode forward for T <= 8 (decode.hip): two launches, gate_up (routing
// when logits is not null, grouping, GEMV, SiLU*up) and down (GEMV and the
// weighted combine). With logits null the ids and weights in idx / w are
// used; otherwise the gate_up launch routes the tokens and writes them there.
hipError_t launch_decode_forward(const MoePlan &p, const e4b_moe_layer *L, const uint16_t *x,
                                 const float *logits, int32_t *idx, float *w, uint16_t *y,
                                 char *ws, hipStream_t s, const e4b_kernel_events *ev);

// ---- LoRA (lora.hip) ----
// Operand packs of the adapters, with zeros for r <= j < kLoraK:
//   LP_COLS   : out[e, n, :] = bf16(s * B[e, n, j])   (B [E, N, r]; GEMM slice)
//   LP_COLS_T : out[e, n, :] = bf16(s * A[e, j, n])   (A [E, r, N]; GEMM slice)
//   LP_JK_A   : out[e, j, k] = bf16(A[e, j, k])       (A [E, r, K]; projection, N = K)
//   LP_JK_B   : out[e, j, k] = bf16(B[e, k, j])       (B [E, K, r]; projection, N = K)
enum LoraPackType { LP_COLS = 0, LP_COLS_T = 1, LP_JK_A = 2, LP_JK_B = 3 };
struct LoraPackJob {
  const float *M;
  uint16_t *out;
  int64_t E;
  int64_t items;  // set by the launcher
  int32_t N;
  int32_t type;
  float s;
};
constexpr int kLoraPackJobs = 8;
struct LoraPackJobs {
  LoraPackJob j[kLoraPackJobs];
  int64_t first_block[kLoraPackJobs];  // set by the launcher
  int32_t n;
  int32_t r;
};
// All packs of one call in one launch (jobs.n <= kLoraPackJobs).
hipError_t launch_lora_packs(LoraPackJobs jobs, hipStream_t st);

// Source rows of a per-pair projection / of an adapter gradient.
enum LoraSrc {
  LS_X_GATHER = 0,  // src[token(sorted pair)]           (x or grad_y, [T, ld])
  LS_ROWS = 1,      // src[sorted position]               (a or dGU, [P, ld])
  LS_GU_ACT = 2,    // silu(g) * u from g|u [P, 2I] rows  (the activation a; gradients only)
  LS_WX_GATHER = 3  // topk_w[pair] * src[token(pair)]    (the weighted grad_y; gradients only)
};
// out[s, j] = sum_k src(s)[k] M(e(s), k, j) (j < r, zero up to kLoraK), fp32
// [P, kLoraK], on MFMA over the m-tiles of the permutation (rows of a tile
// share one expert); Mj is the j-major pack [E, kLoraK, K] of the adapter
// (LP_JK_A / LP_JK_B). src_mode LS_X_GATHER or LS_ROWS; K % 64 == 0.
hipError_t launch_lora_proj(int src_mode, const uint16_t *src, int64_t ld, int K,
                            const int32_t *sorted, int topk, const PermView &v, int E,
                            int64_t m_tiles_bound, const uint16_t *Mj, float *out, hipStream_t st);
// Adapter gradient of expert e: G[n, j] = s * sum over e's sorted pairs of
// U(pair)[n] * V(pair)[j] (* topk_w[pair] when v_weighted), written as
// [E, N, r] (a B-shaped gradient) or [E, r, N] (A-shaped, out_trans); U
// comes from src in `mode` (LoraSrc). Up to four gradients per launch.
struct LoraWgJob {
  const uint16_t *src;
  const float *V;
  float *out;
  int64_t ld;
  int32_t N;
  int32_t mode;
  int32_t v_weighted;
  int32_t out_trans;
};
struct LoraWgJobs {
  LoraWgJob j[4];
  int32_t n;
};
hipError_t launch_lora_wgrads(const LoraWgJobs &jobs, int I, const int32_t *sorted,
                              const int32_t *offsets, const int32_t *tile_offsets, int topk,
                              const float *topk_w, int64_t E, int r, float s, hipStream_t st);

}  // namespace e4b
