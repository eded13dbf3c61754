// plan.cpp -- host-side validation and workspace planning (no HIP calls).
#include "plan.h"

namespace e4b {

namespace {

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Every element offset inside one activation-sized buffer is computed in
// 32 bits by the kernels.
constexpr int64_t kMaxElems32 = (int64_t(1) << 31) - 1;

int bits_for(int64_t n) {
  int b = 0;
  while ((int64_t(1) << b) < n) ++b;
  return b;
}

}  // namespace

e4b_status check_stack(const e4b_stack *st) {
  if (!st || !st->packed) return E4B_ERR_NULL;
  if (st->codebook < E4B_CB_NF4 || st->codebook > E4B_CB_FP8) return E4B_ERR_CODEBOOK;
  const bool mx = st->codebook == E4B_CB_MXFP4;
  if (st->blocksize != (mx ? kMxBlock : kBlock)) return E4B_ERR_BLOCKSIZE;
  // the scale buffer of the mode: fp32 absmax (NF4, FP4), E8M0 bytes (MXFP4), none (BF16)
  const void *scale = mx ? static_cast<const void *>(st->scales)
                         : st->codebook == E4B_CB_BF16 ? nullptr : st->absmax;
  if (st->codebook != E4B_CB_BF16 && !scale) return E4B_ERR_NULL;
  // rows are whole 64-element K-steps of the GEMMs in every mode
  if (st->E <= 0 || st->out <= 0 || st->in <= 0 || st->in % kBlock != 0) return E4B_ERR_SHAPE;
  if (st->out * st->in > kMaxElems32 * 2) return E4B_ERR_SHAPE;
  if (!aligned16(st->packed) || (scale && !aligned16(scale))) return E4B_ERR_ALIGN;
  return E4B_OK;
}

e4b_status check_quantize_mx(const float *w, int64_t E, int64_t out, int64_t in,
                             const uint8_t *packed, const uint8_t *scales) {
  if (!w || !packed || !scales) return E4B_ERR_NULL;
  if (E <= 0 || out <= 0 || in <= 0 || in % kMxBlock != 0) return E4B_ERR_SHAPE;
  if (out * in > kMaxElems32 * 2) return E4B_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(scales)) return E4B_ERR_ALIGN;
  return E4B_OK;
}

e4b_status check_quantize(const float *w, int64_t E, int64_t out, int64_t in,
                          int32_t blocksize, int32_t codebook, const uint8_t *packed,
                          const float *absmax) {
  const bool bf16 = codebook == E4B_CB_BF16;
  if (!w || !packed || (!bf16 && !absmax)) return E4B_ERR_NULL;
  if (blocksize != kBlock) return E4B_ERR_BLOCKSIZE;
  if (codebook != E4B_CB_NF4 && codebook != E4B_CB_FP4 && codebook != E4B_CB_INT8 &&
      codebook != E4B_CB_FP8 && !bf16)
    return E4B_ERR_CODEBOOK;
  if (E <= 0 || out <= 0 || in <= 0 || in % kBlock != 0) return E4B_ERR_SHAPE;
  if (out * in > kMaxElems32 * 2) return E4B_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(packed) || (!bf16 && !aligned16(absmax))) return E4B_ERR_ALIGN;
  return E4B_OK;
}

e4b_status check_layer(const e4b_moe_layer *L, MoePlan *p) {
  if (!L) return E4B_ERR_NULL;
  e4b_status s = check_stack(&L->gate_up);
  if (s != E4B_OK) return s;
  s = check_stack(&L->down);
  if (s != E4B_OK) return s;
  const e4b_stack &gu = L->gate_up, &dn = L->down;
  if (gu.codebook != dn.codebook) return E4B_ERR_CODEBOOK;
  if (gu.E != dn.E || gu.E > kMaxE) return E4B_ERR_SHAPE;
  // gated (SwiGLU: gate | up, 2I rows) or ungated (a plain up projection, I rows)
  if ((gu.out != 2 * dn.in && gu.out != dn.in) || gu.in != dn.out) return E4B_ERR_SHAPE;
  p->E = gu.E;
  p->H = gu.in;
  p->I = dn.in;
  p->gated = gu.out == 2 * dn.in ? 1 : 0;
  p->gu_cols = gu.out;
  p->codebook = gu.codebook;
  return E4B_OK;
}

e4b_status plan_moe(const e4b_moe_layer *L, int64_t T, int32_t top_k, MoePlan *p) {
  if (!p) return E4B_ERR_NULL;
  *p = MoePlan{};
  e4b_status s = check_layer(L, p);
  if (s != E4B_OK) return s;
  if (T < 0) return E4B_ERR_SHAPE;
  if (top_k < 1 || top_k > kMaxTopK || top_k > p->E) return E4B_ERR_SHAPE;
  p->T = T;
  p->k = top_k;
  p->P = T * top_k;
  const int64_t P = p->P, H = p->H, I = p->I, E = p->E;
  if (P > kMaxElems32 / 4) return E4B_ERR_SHAPE;
  if (P * 2 * I > kMaxElems32 || P * H > kMaxElems32 || T * E > kMaxElems32) return E4B_ERR_SHAPE;

  p->nchunks = (P + kPermChunk - 1) / kPermChunk;
  const int64_t busy = P < E ? P : E;  // at most P experts have a pair
  p->m_tiles_bound = (P + busy * (kBM - 1)) / kBM;
  // gated: kBNWide / 2 gate-up pairs per tile; ungated: kBNWide columns of the up projection
  const int64_t bn_gu = p->gated ? kBNWide / 2 : kBNWide;
  p->n_tiles_gu = (I + bn_gu - 1) / bn_gu;
  p->n_tiles_h = (H + kBNWide - 1) / kBNWide;
  p->n_tiles_i = (I + kGuBlockPairs - 1) / kGuBlockPairs;
  // saved / recomputed g|u: gated, blocked per (m-tile, 128 pairs); ungated h [P, I]
  p->gu_bytes = p->gated ? size_t(p->m_tiles_bound) * size_t((I + kGuBlockPairs - 1) / kGuBlockPairs) *
                               size_t(kGuBlockChunks) * 16
                         : size_t(P) * size_t(I) * 2;
  p->n_tiles_h_gud = (H + kBNWide - 1) / kBNWide;
  p->nbits_e = bits_for(E);

  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t n_ec = size_t(E) * size_t(p->nchunks);
  p->off_hist = take(n_ec * 4);
  p->off_chunk_base = take(n_ec * 4);
  p->off_counts = take(size_t(E) * 4);
  p->off_offsets = take(size_t(E + 1) * 4);
  p->off_tile_offsets = take(size_t(E + 1) * 4);
  p->off_sorted = take(size_t(P) * 4);
  p->off_pos = take(size_t(P) * 4);
  p->off_tile_map = take(size_t(p->m_tiles_bound) * 16);
  const size_t base = off;
  // forward region
  p->off_a = take(size_t(P) * I * 2);
  p->off_o = take(size_t(P) * H * 2);
  p->off_dmap = T <= kDecodeMaxT ? take(kDecPlanBytes) : 0;
  // the MX forward's activation rows (MXFP4 layers): x and a as E4M3 codes + E8M0 scales
  const bool mx = p->codebook == E4B_CB_MXFP4;
  p->off_mx_xq = mx ? take(size_t(T) * H) : 0;
  p->off_mx_xs = mx ? take(size_t(T) * H / kMxBlock) : 0;
  p->off_mx_aq = mx ? take(size_t(P) * I) : 0;
  p->off_mx_as = mx ? take(size_t(P) * I / kMxBlock) : 0;
  const size_t fwd_end = off;
  // dgrad region (overlaps the forward region: the two calls never run at once
  // on one workspace)
  off = base;
  p->off_gu = take(p->gu_bytes);
  p->off_dgu = take(size_t(P) * p->gu_cols * 2);
  p->off_partial = take(size_t(P) * p->n_tiles_i * 4);
  p->off_gx = take(size_t(P) * H * 2);
  const size_t dgrad_end = off;
  p->ws_bytes = fwd_end > dgrad_end ? fwd_end : dgrad_end;
  off = p->ws_bytes;
  p->off_l_xa = take(size_t(P) * kLoraK * 4);
  p->off_l_aa = take(size_t(P) * kLoraK * 4);
  p->off_l_gb = take(size_t(P) * kLoraK * 4);
  p->off_l_hb = take(size_t(P) * kLoraK * 4);
  p->off_l_a = take(size_t(P) * I * 2);
  p->off_pk_bgu = take(size_t(E) * 2 * I * kLoraK * 2);
  p->off_pk_bdn = take(size_t(E) * H * kLoraK * 2);
  p->off_pk_agu = take(size_t(E) * H * kLoraK * 2);
  p->off_pk_adn = take(size_t(E) * I * kLoraK * 2);
  p->off_pj_agu = take(size_t(E) * kLoraK * H * 2);
  p->off_pj_adn = take(size_t(E) * kLoraK * I * 2);
  p->off_pj_bdn = take(size_t(E) * kLoraK * H * 2);
  p->off_pj_bgu = take(size_t(E) * kLoraK * 2 * I * 2);
  p->lora_ws_bytes = off;
  p->sv_tile_map = align_up(p->gu_bytes, 256);
  p->sv_tile_offsets = p->sv_tile_map + size_t(p->m_tiles_bound) * 16;
  p->sv_offsets = p->sv_tile_offsets + size_t(E + 1) * 4;
  p->sv_sorted = p->sv_offsets + size_t(E + 1) * 4;
  p->sv_pos = p->sv_sorted + size_t(P) * 4;
  p->sv_xa = align_up(p->sv_pos + size_t(P) * 4, 256);
  p->sv_aa = p->sv_xa + size_t(P) * kLoraK * 4;
  p->saved_bytes = p->sv_aa + size_t(P) * kLoraK * 4;
  return E4B_OK;
}

bool decode_fits(const MoePlan &p) {
  const int64_t kmax = p.H > p.I ? p.H : p.I;
  const bool four_bit = p.codebook == E4B_CB_NF4 || p.codebook == E4B_CB_FP4 || p.codebook == E4B_CB_MXFP4;
  return four_bit && p.gated && p.T <= kDecodeMaxT && p.P <= kDecMaxPairs &&
         kmax <= kDecodeMaxK;
}

e4b_status check_forward(const MoePlan &p, const void *x, const float *logits,
                         const int32_t *idx, const float *w, const void *y,
                         const void *saved, const void *ws, size_t ws_bytes,
                         int32_t path, int *use_decode) {
  if (path != E4B_PATH_AUTO && path != E4B_PATH_GROUPED && path != E4B_PATH_DECODE &&
      path != E4B_PATH_MX8)
    return E4B_ERR_PATH;
  // the MX forward: an MXFP4 gated layer, K-steps of 128 on both GEMMs, no saved state
  if (path == E4B_PATH_MX8 && (p.codebook != E4B_CB_MXFP4 || !p.gated || p.H % 128 != 0 ||
                               p.I % 128 != 0 || saved != nullptr))
    return E4B_ERR_PATH;
  const bool fits = decode_fits(p);
  if (path == E4B_PATH_DECODE && (!fits || saved != nullptr)) return E4B_ERR_PATH;
  *use_decode = path == E4B_PATH_DECODE || (path == E4B_PATH_AUTO && fits && saved == nullptr);
  if (p.T == 0) return E4B_OK;
  if (!x || !idx || !w || !y) return E4B_ERR_NULL;
  if (!ws) return E4B_ERR_NULL;
  if (ws_bytes < p.ws_bytes) return E4B_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(idx) || !aligned16(w) || !aligned16(y) || !aligned16(ws))
    return E4B_ERR_ALIGN;
  if (logits && !aligned16(logits)) return E4B_ERR_ALIGN;
  if (saved && !aligned16(saved)) return E4B_ERR_ALIGN;
  return E4B_OK;
}

e4b_status check_lora(const e4b_lora *lora) {
  if (!lora || !lora->A_gu || !lora->B_gu || !lora->A_dn || !lora->B_dn) return E4B_ERR_NULL;
  if (lora->r < 1 || lora->r > kLoraK) return E4B_ERR_SHAPE;
  if (!aligned16(lora->A_gu) || !aligned16(lora->B_gu) || !aligned16(lora->A_dn) ||
      !aligned16(lora->B_dn))
    return E4B_ERR_ALIGN;
  return E4B_OK;
}

e4b_status check_dgrad(const MoePlan &p, const int32_t *idx, const float *w,
                       const void *x, const void *saved, const void *gy,
                       const void *gx, const float *gw, const void *ws,
                       size_t ws_bytes) {
  if (p.T == 0) return E4B_OK;
  if (!idx || !w || !gy || !gx) return E4B_ERR_NULL;
  if (!saved && !x) return E4B_ERR_NULL;
  if (!ws) return E4B_ERR_NULL;
  if (ws_bytes < p.ws_bytes) return E4B_ERR_WORKSPACE;
  if (!aligned16(idx) || !aligned16(w) || !aligned16(gy) || !aligned16(gx) || !aligned16(ws))
    return E4B_ERR_ALIGN;
  if (x && !aligned16(x)) return E4B_ERR_ALIGN;
  if (saved && !aligned16(saved)) return E4B_ERR_ALIGN;
  if (gw && !aligned16(gw)) return E4B_ERR_ALIGN;
  return E4B_OK;
}

}  // namespace e4b

extern "C" const char *e4b_status_string(e4b_status s) {
  switch (s) {
    case E4B_OK: return "ok";
    case E4B_ERR_NULL: return "a required pointer is NULL";
    case E4B_ERR_SHAPE: return "invalid shape (dims <= 0, in % 64 != 0, top_k out of range, E > 1024, mismatched stacks or too large)";
    case E4B_ERR_BLOCKSIZE: return "blocksize must be 64 (MXFP4: 32)";
    case E4B_ERR_CODEBOOK: return "unknown codebook or gate_up/down codebooks differ";
    case E4B_ERR_DTYPE: return "unknown output dtype";
    case E4B_ERR_WORKSPACE: return "workspace missing or too small";
    case E4B_ERR_ALIGN: return "device buffer not 16-byte aligned";
    case E4B_ERR_PATH: return "invalid path (decode path needs a gated 4-bit layer (NF4, FP4, MXFP4), T <= 8, saved == NULL and max(H, I) <= 16384)";
    case E4B_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

extern "C" size_t e4b_moe_workspace_bytes(const e4b_moe_layer *L, int64_t T, int32_t top_k) {
  e4b::MoePlan p;
  return e4b::plan_moe(L, T, top_k, &p) == E4B_OK ? p.ws_bytes : 0;
}

extern "C" size_t e4b_moe_lora_workspace_bytes(const e4b_moe_layer *L, int64_t T, int32_t top_k) {
  e4b::MoePlan p;
  return e4b::plan_moe(L, T, top_k, &p) == E4B_OK ? p.lora_ws_bytes : 0;
}

extern "C" size_t e4b_moe_saved_bytes(const e4b_moe_layer *L, int64_t T, int32_t top_k) {
  e4b::MoePlan p;
  return e4b::plan_moe(L, T, top_k, &p) == E4B_OK ? p.saved_bytes : 0;
}
