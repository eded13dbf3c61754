// api.hip -- e4b_moe_forward / e4b_moe_dgrad: validate, then enqueue the
// kernels of the routed expert MLP on the caller's stream (no host sync).
//
// Forward (experts4bit-qlora 0.1.0 sdist, Experts4bit.forward):
//   route (optional) -> permute -> gate_up GEMM + SiLU*up -> down GEMM
//   -> weighted gather-combine.
// dgrad (bitsandbytes PR #1965, recompute-in-backward bullet):
//   [permute + gate_up GEMM again if nothing was saved] -> down GEMM on
//   W_dn^T with the SiLU-backward epilogue -> gate_up GEMM on W_gu^T
//   -> gather-combine of grad_x and of the routing-weight gradient.
#include "device.h"
#include "kernels.h"

using namespace e4b;

namespace e4b {

namespace {

GemmArgs base_args(const MoePlan &p, const e4b_stack &st, const PermView &v) {
  GemmArgs a{};
  a.sorted_pair = v.sorted;
  a.topk = int32_t(p.k);
  a.Wp = st.packed;
  a.mx = st.codebook == E4B_CB_MXFP4;
  a.Wa = a.mx ? nullptr : st.absmax;
  a.Ws = a.mx ? st.scales : nullptr;
  const bool bf16 = st.codebook == E4B_CB_BF16;
  const bool c8 = st.codebook == E4B_CB_INT8 || st.codebook == E4B_CB_FP8;
  a.w_e_bytes = bf16 ? st.out * st.in * 2 : (c8 ? st.out * st.in : st.out * st.in / 2);
  a.w_e_blocks = bf16 ? 0 : st.out * st.in / (a.mx ? kMxBlock : kBlock);  // BF16: none
  a.w_in = int32_t(st.in);
  a.I = int32_t(p.I);
  a.offsets = v.offsets;
  a.tile_offsets = v.tile_offsets;
  a.tile_map = v.tile_map;
  a.E = int32_t(p.E);
  a.cb = p.codebook;
  a.gated = p.gated;
  a.ldgu = int32_t(p.gu_cols);
  return a;
}

// gate_up projection of every routed pair: writes a = silu(g)*u (if a_out) and
// the bf16 g|u (if gu_out).
hipError_t run_gate_up(const MoePlan &p, const e4b_moe_layer *L, const uint16_t *x,
                       uint16_t *a_out, uint16_t *gu_out, const PermView &v, hipStream_t s,
                       const e4b_kernel_events *ev) {
  GemmArgs a = base_args(p, L->gate_up, v);
  a.A = x;
  a.lda = int32_t(p.H);
  a.N = int32_t(p.I);
  a.K = int32_t(p.H);
  a.n_tiles = int32_t(p.n_tiles_gu);
  a.grid = uint32_t(p.m_tiles_bound * p.n_tiles_gu);
  a.C = a_out;
  a.ldc = int32_t(p.I);
  a.GU = gu_out;
  return launch_grouped_gemm(GEMM_GATE_UP_FWD, a, s, ev);
}

}  // namespace
}  // namespace e4b

#define E4B_TRY(expr)                                   \
  do {                                                  \
    if ((expr) != hipSuccess) return E4B_ERR_HIP;       \
  } while (0)

extern "C" e4b_status e4b_moe_forward_timed(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                                            const void *x_bf16, const float *router_logits,
                                            int32_t *topk_idx, float *topk_w, void *y_bf16,
                                            void *saved, void *ws, size_t ws_bytes, int32_t path,
                                            hipStream_t stream, const e4b_kernel_events *ev) {
  MoePlan p;
  e4b_status st = plan_moe(L, T, top_k, &p);
  if (st != E4B_OK) return st;
  int use_decode = 0;
  st = check_forward(p, x_bf16, router_logits, topk_idx, topk_w, y_bf16, saved, ws, ws_bytes,
                     path, &use_decode);
  if (st != E4B_OK || T == 0) return st;
  char *w = static_cast<char *>(ws);
  const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
  uint16_t *y = static_cast<uint16_t *>(y_bf16);

  if (use_decode) {
    E4B_TRY(launch_decode_forward(p, L, x, router_logits, topk_idx, topk_w, y, w, stream, ev));
    return E4B_OK;
  }
  if (router_logits)
    E4B_TRY(launch_route(router_logits, T, int(p.E), top_k, topk_idx, topk_w, stream, ev));
  if (path == E4B_PATH_MX8) {
    const PermView v = perm_in_workspace(p, w);
    E4B_TRY(launch_permute(p, topk_idx, w, v, stream, ev));
    uint8_t *xq = reinterpret_cast<uint8_t *>(w + p.off_mx_xq);
    uint8_t *xs = reinterpret_cast<uint8_t *>(w + p.off_mx_xs);
    uint8_t *aq = reinterpret_cast<uint8_t *>(w + p.off_mx_aq);
    uint8_t *as = reinterpret_cast<uint8_t *>(w + p.off_mx_as);
    uint16_t *o_buf = reinterpret_cast<uint16_t *>(w + p.off_o);
    E4B_TRY(launch_mx8_rows(x, T, int(p.H), xq, xs, stream));
    MxGemmArgs a{};
    a.sorted_pair = v.sorted;
    a.topk = top_k;
    a.Wp = L->gate_up.packed;
    a.Ws = L->gate_up.scales;
    a.w_e_bytes = L->gate_up.out * L->gate_up.in / 2;
    a.w_e_blocks = L->gate_up.out * L->gate_up.in / kMxBlock;
    a.A = xq;
    a.As = xs;
    a.K = int32_t(p.H);
    a.N = int32_t(p.I);
    a.I = int32_t(p.I);
    a.E = int32_t(p.E);
    a.tile_offsets = v.tile_offsets;
    a.tile_map = v.tile_map;
    a.n_tiles = int32_t(p.n_tiles_gu);
    a.grid = uint32_t(p.m_tiles_bound * p.n_tiles_gu);
    a.Cq = aq;
    a.Cs = as;
    E4B_TRY(launch_mx_gemm(true, a, stream, ev));
    MxGemmArgs d = a;
    d.Wp = L->down.packed;
    d.Ws = L->down.scales;
    d.w_e_bytes = L->down.out * L->down.in / 2;
    d.w_e_blocks = L->down.out * L->down.in / kMxBlock;
    d.A = aq;
    d.As = as;
    d.K = int32_t(p.I);
    d.N = int32_t(p.H);
    d.n_tiles = int32_t(p.n_tiles_h);
    d.grid = uint32_t(p.m_tiles_bound * p.n_tiles_h);
    d.C = o_buf;
    d.ldc = int32_t(p.H);
    E4B_TRY(launch_mx_gemm(false, d, stream, ev));
    E4B_TRY(launch_combine_rows(o_buf, v.pos, topk_w, T, top_k, int(p.H), y, stream, ev));
    return E4B_OK;
  }
  // with a saved buffer the permutation is written there for the dgrad
  const PermView v = saved ? perm_in_saved(p, static_cast<char *>(saved)) : perm_in_workspace(p, w);
  E4B_TRY(launch_permute(p, topk_idx, w, v, stream, ev));

  uint16_t *a_buf = reinterpret_cast<uint16_t *>(w + p.off_a);
  uint16_t *o_buf = reinterpret_cast<uint16_t *>(w + p.off_o);
  E4B_TRY(run_gate_up(p, L, x, a_buf, static_cast<uint16_t *>(saved), v, stream, ev));

  GemmArgs d = base_args(p, L->down, v);
  d.A = a_buf;
  d.lda = int32_t(p.I);
  d.N = int32_t(p.H);
  d.K = int32_t(p.I);
  d.n_tiles = int32_t(p.n_tiles_h);
  d.grid = uint32_t(p.m_tiles_bound * p.n_tiles_h);
  d.C = o_buf;
  d.ldc = int32_t(p.H);
  E4B_TRY(launch_grouped_gemm(GEMM_DOWN_FWD, d, stream, ev));

  E4B_TRY(launch_combine_rows(o_buf, v.pos, topk_w, T, top_k, int(p.H), y, stream, ev));
  return E4B_OK;
}

extern "C" e4b_status e4b_moe_forward(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                                      const void *x_bf16, const float *router_logits,
                                      int32_t *topk_idx, float *topk_w, void *y_bf16,
                                      void *saved, void *ws, size_t ws_bytes, int32_t path,
                                      hipStream_t stream) {
  return e4b_moe_forward_timed(L, T, top_k, x_bf16, router_logits, topk_idx, topk_w, y_bf16, saved,
                               ws, ws_bytes, path, stream, nullptr);
}

extern "C" e4b_status e4b_moe_dgrad_timed(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                                          const int32_t *topk_idx, const float *topk_w,
                                          const void *x_bf16, const void *saved,
                                          const void *grad_y_bf16, void *grad_x_bf16,
                                          float *grad_topk_w, void *ws, size_t ws_bytes,
                                          hipStream_t stream, const e4b_kernel_events *ev) {
  MoePlan p;
  e4b_status st = plan_moe(L, T, top_k, &p);
  if (st != E4B_OK) return st;
  st = check_dgrad(p, topk_idx, topk_w, x_bf16, saved, grad_y_bf16, grad_x_bf16, grad_topk_w, ws,
                   ws_bytes);
  if (st != E4B_OK || T == 0) return st;
  char *w = static_cast<char *>(ws);
  // the saved buffer holds the forward's permutation; without it the
  // permutation and the gate_up projection are recomputed
  const uint16_t *gu = static_cast<const uint16_t *>(saved);
  PermView v;
  if (saved) {
    v = perm_in_saved(p, static_cast<char *>(const_cast<void *>(saved)));
  } else {
    v = perm_in_workspace(p, w);
    E4B_TRY(launch_permute(p, topk_idx, w, v, stream, ev));
    uint16_t *gu_ws = reinterpret_cast<uint16_t *>(w + p.off_gu);
    E4B_TRY(run_gate_up(p, L, static_cast<const uint16_t *>(x_bf16), nullptr, gu_ws, v, stream, ev));
    gu = gu_ws;
  }
  uint16_t *dgu = reinterpret_cast<uint16_t *>(w + p.off_dgu);
  float *partial = reinterpret_cast<float *>(w + p.off_partial);
  uint16_t *gx = reinterpret_cast<uint16_t *>(w + p.off_gx);

  GemmArgs d = base_args(p, L->down, v);
  d.A = static_cast<const uint16_t *>(grad_y_bf16);
  d.lda = int32_t(p.H);
  d.N = int32_t(p.I);
  d.K = int32_t(p.H);
  d.n_tiles = int32_t(p.n_tiles_i);
  d.grid = uint32_t(p.m_tiles_bound * p.n_tiles_i);
  d.C = dgu;
  d.ldc = int32_t(p.gu_cols);
  d.GU = const_cast<uint16_t *>(gu);
  d.topk_w = topk_w;
  d.partial = partial;
  E4B_TRY(launch_grouped_gemm(GEMM_DOWN_DGRAD, d, stream, ev));

  GemmArgs u = base_args(p, L->gate_up, v);
  u.A = dgu;
  u.lda = int32_t(p.gu_cols);
  u.N = int32_t(p.H);
  u.K = int32_t(p.gu_cols);
  u.n_tiles = int32_t(p.n_tiles_h_gud);
  u.grid = uint32_t(p.m_tiles_bound * p.n_tiles_h_gud);
  u.C = gx;
  u.ldc = int32_t(p.H);
  E4B_TRY(launch_grouped_gemm(GEMM_GATE_UP_DGRAD, u, stream, ev));

  E4B_TRY(launch_combine_dgrad(gx, v.pos, T, top_k, int(p.H), static_cast<uint16_t *>(grad_x_bf16),
                               partial, int(p.n_tiles_i), grad_topk_w, stream, ev));
  return E4B_OK;
}

extern "C" e4b_status e4b_moe_dgrad(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                                    const int32_t *topk_idx, const float *topk_w,
                                    const void *x_bf16, const void *saved,
                                    const void *grad_y_bf16, void *grad_x_bf16,
                                    float *grad_topk_w, void *ws, size_t ws_bytes,
                                    hipStream_t stream) {
  return e4b_moe_dgrad_timed(L, T, top_k, topk_idx, topk_w, x_bf16, saved, grad_y_bf16,
                             grad_x_bf16, grad_topk_w, ws, ws_bytes, stream, nullptr);
}

extern "C" e4b_status e4b_moe_perm_layout(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                                          e4b_perm_layout *out) {
  if (!out) return E4B_ERR_NULL;
  MoePlan p;
  const e4b_status st = plan_moe(L, T, top_k, &p);
  if (st != E4B_OK) return st;
  out->counts = p.off_counts;
  out->offsets = p.off_offsets;
  out->tile_offsets = p.off_tile_offsets;
  out->sorted_pair = p.off_sorted;
  out->pos_of_pair = p.off_pos;
  out->tile_map = p.off_tile_map;
  out->m_tiles_bound = p.m_tiles_bound;
  return E4B_OK;
}

// ---- LoRA over the frozen base ----
namespace e4b {
namespace {

struct LoraWs {
  float *xa, *aa, *gb, *hb;
  uint16_t *a;                                  // recomputed a [P, I] (backward without saved state)
  uint16_t *pk_bgu, *pk_bdn, *pk_agu, *pk_adn;  // GEMM slices: scaled, by output column
  uint16_t *pj_agu, *pj_adn, *pj_bdn, *pj_bgu;  // projections: j-major
};

LoraWs lora_ws(const MoePlan &p, char *w) {
  LoraWs l;
  l.xa = reinterpret_cast<float *>(w + p.off_l_xa);
  l.aa = reinterpret_cast<float *>(w + p.off_l_aa);
  l.gb = reinterpret_cast<float *>(w + p.off_l_gb);
  l.hb = reinterpret_cast<float *>(w + p.off_l_hb);
  l.a = reinterpret_cast<uint16_t *>(w + p.off_l_a);
  l.pk_bgu = reinterpret_cast<uint16_t *>(w + p.off_pk_bgu);
  l.pk_bdn = reinterpret_cast<uint16_t *>(w + p.off_pk_bdn);
  l.pk_agu = reinterpret_cast<uint16_t *>(w + p.off_pk_agu);
  l.pk_adn = reinterpret_cast<uint16_t *>(w + p.off_pk_adn);
  l.pj_agu = reinterpret_cast<uint16_t *>(w + p.off_pj_agu);
  l.pj_adn = reinterpret_cast<uint16_t *>(w + p.off_pj_adn);
  l.pj_bdn = reinterpret_cast<uint16_t *>(w + p.off_pj_bdn);
  l.pj_bgu = reinterpret_cast<uint16_t *>(w + p.off_pj_bgu);
  return l;
}

float lora_scale(const e4b_lora *lo) { return lo->alpha / float(lo->r); }

void add_pack(LoraPackJobs &jobs, const float *M, int64_t E, int N, int type, float s,
              uint16_t *out) {
  LoraPackJob &J = jobs.j[jobs.n++];
  J.M = M;
  J.out = out;
  J.E = E;
  J.items = 0;
  J.N = N;
  J.type = type;
  J.s = s;
}

void add_wgrad(LoraWgJobs &jobs, int mode, const uint16_t *src, int64_t ld, int N, const float *V,
               bool v_weighted, bool out_trans, float *out) {
  LoraWgJob &J = jobs.j[jobs.n++];
  J.src = src;
  J.V = V;
  J.out = out;
  J.ld = ld;
  J.N = N;
  J.mode = mode;
  J.v_weighted = v_weighted;
  J.out_trans = out_trans;
}

// x A_gu^T per pair into xa, then the gate_up GEMM with the s B_gu slice.
hipError_t lora_gate_up(const MoePlan &p, const e4b_moe_layer *L, const uint16_t *x,
                        uint16_t *a_out, uint16_t *gu_out, const PermView &v, const LoraWs &l,
                        float *xa, hipStream_t s) {
  hipError_t err = launch_lora_proj(LS_X_GATHER, x, p.H, int(p.H), v.sorted, int(p.k), v, int(p.E),
                                    p.m_tiles_bound, l.pj_agu, xa, s);
  if (err != hipSuccess) return err;
  GemmArgs a = base_args(p, L->gate_up, v);
  a.A = x;
  a.lda = int32_t(p.H);
  a.N = int32_t(p.I);
  a.K = int32_t(p.H);
  a.n_tiles = int32_t(p.n_tiles_gu);
  a.grid = uint32_t(p.m_tiles_bound * p.n_tiles_gu);
  a.C = a_out;
  a.ldc = int32_t(p.I);
  a.GU = gu_out;
  a.lora_p = xa;
  a.lora_w = l.pk_bgu;
  a.lora_rows = int32_t(2 * p.I);
  return launch_grouped_gemm(GEMM_GATE_UP_FWD, a, s);
}

}  // namespace
}  // namespace e4b

extern "C" e4b_status e4b_moe_lora_forward(const e4b_moe_layer *L, const e4b_lora *lora,
                                           int64_t T, int32_t top_k, const void *x_bf16,
                                           const float *router_logits, int32_t *topk_idx,
                                           float *topk_w, void *y_bf16, void *saved, void *ws,
                                           size_t ws_bytes, hipStream_t stream) {
  MoePlan p;
  e4b_status st = plan_moe(L, T, top_k, &p);
  if (st != E4B_OK) return st;
  st = check_lora(lora);
  if (st != E4B_OK) return st;
  if (!p.gated) return E4B_ERR_SHAPE;  // adapters are defined for gated layers
  int use_decode = 0;
  st = check_forward(p, x_bf16, router_logits, topk_idx, topk_w, y_bf16, saved, ws, ws_bytes,
                     E4B_PATH_GROUPED, &use_decode);
  if (st != E4B_OK || T == 0) return st;
  if (ws_bytes < p.lora_ws_bytes) return E4B_ERR_WORKSPACE;
  char *w = static_cast<char *>(ws);
  const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
  const LoraWs l = lora_ws(p, w);
  const float sc = lora_scale(lora);

  if (router_logits)
    E4B_TRY(launch_route(router_logits, T, int(p.E), top_k, topk_idx, topk_w, stream));
  const PermView v = saved ? perm_in_saved(p, static_cast<char *>(saved)) : perm_in_workspace(p, w);
  E4B_TRY(launch_permute(p, topk_idx, w, v, stream));
  LoraPackJobs packs{};
  packs.r = lora->r;
  add_pack(packs, lora->B_gu, p.E, int(2 * p.I), LP_COLS, sc, l.pk_bgu);
  add_pack(packs, lora->B_dn, p.E, int(p.H), LP_COLS, sc, l.pk_bdn);
  add_pack(packs, lora->A_gu, p.E, int(p.H), LP_JK_A, 1.0f, l.pj_agu);
  add_pack(packs, lora->A_dn, p.E, int(p.I), LP_JK_A, 1.0f, l.pj_adn);
  E4B_TRY(launch_lora_packs(packs, stream));

  // with saved state, the two forward rank projections are kept for the backward
  char *sv = static_cast<char *>(saved);
  float *xa = saved ? reinterpret_cast<float *>(sv + p.sv_xa) : l.xa;
  float *aa = saved ? reinterpret_cast<float *>(sv + p.sv_aa) : l.aa;
  uint16_t *a_buf = reinterpret_cast<uint16_t *>(w + p.off_a);
  uint16_t *o_buf = reinterpret_cast<uint16_t *>(w + p.off_o);
  E4B_TRY(lora_gate_up(p, L, x, a_buf, static_cast<uint16_t *>(saved), v, l, xa, stream));
  E4B_TRY(launch_lora_proj(LS_ROWS, a_buf, p.I, int(p.I), v.sorted, int(p.k), v, int(p.E),
                           p.m_tiles_bound, l.pj_adn, aa, stream));
  GemmArgs d = base_args(p, L->down, v);
  d.A = a_buf;
  d.lda = int32_t(p.I);
  d.N = int32_t(p.H);
  d.K = int32_t(p.I);
  d.n_tiles = int32_t(p.n_tiles_h);
  d.grid = uint32_t(p.m_tiles_bound * p.n_tiles_h);
  d.C = o_buf;
  d.ldc = int32_t(p.H);
  d.lora_p = aa;
  d.lora_w = l.pk_bdn;
  d.lora_rows = int32_t(p.H);
  E4B_TRY(launch_grouped_gemm(GEMM_DOWN_FWD, d, stream));
  E4B_TRY(launch_combine_rows(o_buf, v.pos, topk_w, T, top_k, int(p.H),
                              static_cast<uint16_t *>(y_bf16), stream));
  return E4B_OK;
}

extern "C" e4b_status e4b_moe_lora_backward(const e4b_moe_layer *L, const e4b_lora *lora,
                                            int64_t T, int32_t top_k, const int32_t *topk_idx,
                                            const float *topk_w, const void *x_bf16,
                                            const void *saved, const void *grad_y_bf16,
                                            void *grad_x_bf16, float *grad_topk_w, float *dA_gu,
                                            float *dB_gu, float *dA_dn, float *dB_dn, void *ws,
                                            size_t ws_bytes, hipStream_t stream) {
  MoePlan p;
  e4b_status st = plan_moe(L, T, top_k, &p);
  if (st != E4B_OK) return st;
  st = check_lora(lora);
  if (st != E4B_OK) return st;
  if (!p.gated) return E4B_ERR_SHAPE;
  st = check_dgrad(p, topk_idx, topk_w, x_bf16, saved, grad_y_bf16, grad_x_bf16, grad_topk_w, ws,
                   ws_bytes);
  if (st != E4B_OK || T == 0) return st;
  if (!dA_gu || !dB_gu || !dA_dn || !dB_dn || !x_bf16) return E4B_ERR_NULL;
  if (!aligned16(dA_gu) || !aligned16(dB_gu) || !aligned16(dA_dn) || !aligned16(dB_dn))
    return E4B_ERR_ALIGN;
  if (ws_bytes < p.lora_ws_bytes) return E4B_ERR_WORKSPACE;
  char *w = static_cast<char *>(ws);
  const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
  const uint16_t *gy = static_cast<const uint16_t *>(grad_y_bf16);
  const LoraWs l = lora_ws(p, w);
  const float sc = lora_scale(lora);
  const int r = lora->r;

  LoraPackJobs packs{};
  packs.r = r;
  add_pack(packs, lora->B_dn, p.E, int(p.H), LP_JK_B, 1.0f, l.pj_bdn);
  add_pack(packs, lora->B_gu, p.E, int(2 * p.I), LP_JK_B, 1.0f, l.pj_bgu);
  add_pack(packs, lora->A_dn, p.E, int(p.I), LP_COLS_T, sc, l.pk_adn);
  add_pack(packs, lora->A_gu, p.E, int(p.H), LP_COLS_T, sc, l.pk_agu);
  if (!saved) {  // the recomputed forward's operands
    add_pack(packs, lora->B_gu, p.E, int(2 * p.I), LP_COLS, sc, l.pk_bgu);
    add_pack(packs, lora->A_gu, p.E, int(p.H), LP_JK_A, 1.0f, l.pj_agu);
    add_pack(packs, lora->A_dn, p.E, int(p.I), LP_JK_A, 1.0f, l.pj_adn);
  }
  E4B_TRY(launch_lora_packs(packs, stream));
  const uint16_t *gu = static_cast<const uint16_t *>(saved);
  const float *xa, *aa;
  PermView v;
  if (saved) {
    // the permutation, g|u and the forward's rank projections x A_gu^T, a A_dn^T
    const char *sv = static_cast<const char *>(saved);
    v = perm_in_saved(p, const_cast<char *>(sv));
    xa = reinterpret_cast<const float *>(sv + p.sv_xa);
    aa = reinterpret_cast<const float *>(sv + p.sv_aa);
  } else {
    // recompute them exactly as the forward does
    v = perm_in_workspace(p, w);
    E4B_TRY(launch_permute(p, topk_idx, w, v, stream));
    uint16_t *gu_ws = reinterpret_cast<uint16_t *>(w + p.off_gu);
    E4B_TRY(lora_gate_up(p, L, x, l.a, gu_ws, v, l, l.xa, stream));
    E4B_TRY(launch_lora_proj(LS_ROWS, l.a, p.I, int(p.I), v.sorted, int(p.k), v, int(p.E),
                             p.m_tiles_bound, l.pj_adn, l.aa, stream));
    gu = gu_ws;
    xa = l.xa;
    aa = l.aa;
  }
  uint16_t *dgu = reinterpret_cast<uint16_t *>(w + p.off_dgu);
  float *partial = reinterpret_cast<float *>(w + p.off_partial);
  uint16_t *gx = reinterpret_cast<uint16_t *>(w + p.off_gx);

  // grad_y B_dn per pair, then the down dgrad GEMM with the s A_dn^T slice
  E4B_TRY(launch_lora_proj(LS_X_GATHER, gy, p.H, int(p.H), v.sorted, int(p.k), v, int(p.E),
                           p.m_tiles_bound, l.pj_bdn, l.gb, stream));
  GemmArgs d = base_args(p, L->down, v);
  d.A = gy;
  d.lda = int32_t(p.H);
  d.N = int32_t(p.I);
  d.K = int32_t(p.H);
  d.n_tiles = int32_t(p.n_tiles_i);
  d.grid = uint32_t(p.m_tiles_bound * p.n_tiles_i);
  d.C = dgu;
  d.ldc = int32_t(2 * p.I);
  d.GU = const_cast<uint16_t *>(gu);
  d.topk_w = topk_w;
  d.partial = partial;
  d.lora_p = l.gb;
  d.lora_w = l.pk_adn;
  d.lora_rows = int32_t(p.I);
  E4B_TRY(launch_grouped_gemm(GEMM_DOWN_DGRAD, d, stream));

  // dGU B_gu per pair, then the gate_up dgrad GEMM with the s A_gu^T slice
  E4B_TRY(launch_lora_proj(LS_ROWS, dgu, 2 * p.I, int(2 * p.I), v.sorted, int(p.k), v, int(p.E),
                           p.m_tiles_bound, l.pj_bgu, l.hb, stream));
  GemmArgs u = base_args(p, L->gate_up, v);
  u.A = dgu;
  u.lda = int32_t(2 * p.I);
  u.N = int32_t(p.H);
  u.K = int32_t(2 * p.I);
  u.n_tiles = int32_t(p.n_tiles_h_gud);
  u.grid = uint32_t(p.m_tiles_bound * p.n_tiles_h_gud);
  u.C = gx;
  u.ldc = int32_t(p.H);
  u.lora_p = l.hb;
  u.lora_w = l.pk_agu;
  u.lora_rows = int32_t(p.H);
  E4B_TRY(launch_grouped_gemm(GEMM_GATE_UP_DGRAD, u, stream));

  E4B_TRY(launch_combine_dgrad(gx, v.pos, T, top_k, int(p.H), static_cast<uint16_t *>(grad_x_bf16),
                               partial, int(p.n_tiles_i), grad_topk_w, stream));

  // the four per-expert outer-product sums, one launch
  LoraWgJobs g{};
  add_wgrad(g, LS_ROWS, dgu, 2 * p.I, int(2 * p.I), xa, false, false, dB_gu);
  add_wgrad(g, LS_X_GATHER, x, p.H, int(p.H), l.hb, false, true, dA_gu);
  add_wgrad(g, LS_WX_GATHER, gy, p.H, int(p.H), aa, false, false, dB_dn);
  add_wgrad(g, LS_GU_ACT, gu, 2 * p.I, int(p.I), l.gb, true, true, dA_dn);
  E4B_TRY(launch_lora_wgrads(g, int(p.I), v.sorted, v.offsets, v.tile_offsets, int(p.k), topk_w,
                             p.E, r, sc, stream));
  return E4B_OK;
}
