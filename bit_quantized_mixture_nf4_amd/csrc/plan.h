// plan.h -- host-side argument validation and workspace planning.
//
// This translation unit makes no HIP call, so every status code of the C ABI
// can be forced and checked on a machine without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/e4b.h"

namespace e4b {

// Tile shape shared by every grouped GEMM of the forward and dgrad.
constexpr int kBM = 256;   // rows (routed pairs) per tile
// the saved / recomputed g|u of a gated layer is blocked per (m-tile, 128
// pairs): 256 x 128 pairs of g and u, 128 KB (layout in kernels.h, gu_chunk)
constexpr int kGuBlockPairs = 128;
constexpr int kGuBlockChunks = kBM * kGuBlockPairs / 4;  // 16-byte chunks per block
// output columns per tile of every grouped GEMM (8 waves, one workgroup per CU)
constexpr int kBNWide = 256;
constexpr int kBK = 64;    // reduction step = one quantization block
constexpr int kBlock = 64; // quantization block (elements along `in`)
constexpr int kMxBlock = 32;  // MXFP4 scale block (elements along `in`)
constexpr int kPermChunk = 256;  // pairs per histogram / scatter chunk
constexpr int kMaxE = 1024;
constexpr int kMaxTopK = 32;
constexpr int kDecodeMaxT = 8;
constexpr int kDecMaxPairs = kDecodeMaxT * kMaxTopK;
constexpr int kDecodeMaxK = 16384; // max(H, I) on the decode path
constexpr size_t kDecPlanBytes = 5376;  // decode: the grouping the gate_up launch leaves for the down launch
constexpr int kLoraK = 16;         // LoRA rank slot: one 16-deep MFMA slice (r <= 16)

struct MoePlan {
  int64_t E, H, I, T, k, P;
  int32_t codebook;
  int32_t gated;    // 1: gate_up holds gate | up (2I rows); 0: a plain up projection (I rows)
  int64_t gu_cols;  // rows of the first stack: 2I or I
  size_t gu_bytes;  // the saved / recomputed g|u (gated: blocked) or h
  int64_t nchunks;        // permutation chunks of kPermChunk pairs
  int64_t m_tiles_bound;  // upper bound of sum_e ceil(count_e / kBM)
  int64_t n_tiles_gu;     // gate_up forward tiles: kBNWide/2 gate-up pairs per tile
  int64_t n_tiles_h;      // down forward tiles over H (kBNWide)
  int64_t n_tiles_i;      // down dgrad: blocks of kGuBlockPairs units over I (one partial each)
  int64_t n_tiles_h_gud;  // gate_up dgrad tiles over H (kBNWide)
  int nbits_e;            // bits needed for an expert id
  // workspace byte offsets
  size_t off_hist, off_chunk_base, off_counts, off_offsets, off_tile_offsets;
  size_t off_sorted, off_pos;
  size_t off_tile_map;  // int4 per m-tile: expert, segment start, first row, rows
  size_t off_a, off_o;                          // forward
  size_t off_dmap;  // forward, decode path: the grouping the gate_up launch leaves for the down launch
  size_t off_mx_xq, off_mx_xs, off_mx_aq, off_mx_as;  // forward, MX path (MXFP4 layers)
  size_t off_gu, off_dgu, off_partial, off_gx;  // dgrad
  size_t ws_bytes;
  // LoRA calls: after the base workspace, fp32 [P, kLoraK] per-pair
  // projections (x A_gu^T, a A_dn^T, grad_y B_dn, dGU B_gu) and bf16
  // [E, rows, kLoraK] operand packs (s B_gu, s B_dn, s A_gu^T, s A_dn^T)
  size_t off_l_xa, off_l_aa, off_l_gb, off_l_hb;
  size_t off_l_a;  // bf16 a [P, I] of the backward's recomputed forward
  size_t off_pk_bgu, off_pk_bdn, off_pk_agu, off_pk_adn;
  // j-major bf16 [E, kLoraK, K] packs for the projections: A_gu, A_dn, B_dn^T, B_gu^T
  size_t off_pj_agu, off_pj_adn, off_pj_bdn, off_pj_bgu;
  size_t lora_ws_bytes;
  // saved buffer: bf16 g|u (blocked), then the forward's permutation (tile
  // map, tile offsets, offsets, sorted pairs, pair positions), then the LoRA
  // forward's fp32 [P, kLoraK] rank projections x A_gu^T and a A_dn^T
  size_t sv_tile_map, sv_tile_offsets, sv_offsets, sv_sorted, sv_pos, sv_xa, sv_aa;
  size_t saved_bytes;
};

// Validates a layer descriptor; fills E, H, I, codebook.
e4b_status check_layer(const e4b_moe_layer *L, MoePlan *p);

// Validates (L, T, top_k) and computes the workspace layout.
e4b_status plan_moe(const e4b_moe_layer *L, int64_t T, int32_t top_k, MoePlan *p);

e4b_status check_stack(const e4b_stack *st);
e4b_status check_quantize(const float *w, int64_t E, int64_t out, int64_t in,
                          int32_t blocksize, int32_t codebook, const uint8_t *packed,
                          const float *absmax);
e4b_status check_quantize_mx(const float *w, int64_t E, int64_t out, int64_t in,
                             const uint8_t *packed, const uint8_t *scales);

// True when (T, H, I, k) fit the decode GEMV path: T <= 8 and a weight row
// spans at most 64 lanes of 64 (T <= 2) or 32 (T <= 8) elements.
bool decode_fits(const MoePlan &p);

e4b_status check_forward(const MoePlan &p, const void *x, const float *logits,
                         const int32_t *idx, const float *w, const void *y,
                         const void *saved, const void *ws, size_t ws_bytes,
                         int32_t path, int *use_decode);
// Validates a LoRA descriptor against the plan (pointers, alignment, 1 <= r <= kLoraK).
e4b_status check_lora(const e4b_lora *lora);

e4b_status check_dgrad(const MoePlan &p, const int32_t *idx, const float *w,
                       const void *x, const void *saved, const void *gy,
                       const void *gx, const float *gw, const void *ws,
                       size_t ws_bytes);

inline bool aligned16(const void *ptr) {
  return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0;
}

}  // namespace e4b
