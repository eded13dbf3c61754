"""GPU parity of the routed expert forward and dgrad against the oracle.

Bar: routing ids and the permutation exact; routing weights within 1e-6; y,
grad_x and grad_topk_w within 1e-2 * max|oracle| per tensor; dgrad with the
saved gate/up equal bit for bit to dgrad that recomputes them; every output
bitwise identical across runs.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import bit_quantized_mixture_nf4_amd as e4b
from workloads import MoEConfig, get_config
from gpu_util import DEV, Problem, announce, tol_check, to_np, bf16_tensor

pytestmark = pytest.mark.gpu


def _read_i32(ws, off, n):
    return ws[off : off + 4 * n].view(torch.int32).cpu().numpy()


def _check_permutation(layer, ws, idx, E, P):
    """Every array of the permutation in the workspace equals the oracle's, as
    exact integers, at the offsets the library reports (e4b_moe_perm_layout)."""
    T, k = idx.shape
    lay = e4b.perm_layout(layer, T, k)
    counts, offsets, sp, pos = oracle.permute(idx, E)
    assert np.array_equal(_read_i32(ws, lay["counts"], E), counts)
    assert np.array_equal(_read_i32(ws, lay["offsets"], E + 1), offsets)
    assert np.array_equal(_read_i32(ws, lay["sorted_pair"], P), sp)
    assert np.array_equal(_read_i32(ws, lay["pos_of_pair"], P), pos)
    mt = (counts + 255) // 256
    tiles = np.concatenate([[0], np.cumsum(mt)])
    assert np.array_equal(_read_i32(ws, lay["tile_offsets"], E + 1), tiles)
    # m-tile map: (expert, segment start, first row, rows) per real m-tile, zero past them
    want = np.zeros((lay["m_tiles_bound"], 4), np.int64)
    for e in range(E):
        for t in range(mt[e]):
            want[tiles[e] + t] = (e, offsets[e], 256 * t, min(256, counts[e] - 256 * t))
    got = _read_i32(ws, lay["tile_map"], 4 * lay["m_tiles_bound"]).reshape(-1, 4)
    assert np.array_equal(got, want)


def _oracle_fwd(pb, idx, w, tokens=None):
    wgu, wdn = pb.oracle_weights()
    x = pb.x if tokens is None else pb.x[tokens]
    return oracle.moe_forward(x, idx, w, wgu, wdn)


def _oracle_dgrad(pb, idx, w, tokens=None):
    wgu, wdn = pb.oracle_weights()
    sel = slice(None) if tokens is None else tokens
    return oracle.moe_dgrad(pb.x[sel], idx, w, wgu, wdn, pb.grad_y[sel])


@pytest.fixture(scope="module")
def tiny():
    announce("tiny layer E8 H256 I128 k2 T64")
    return Problem(get_config("tiny"), seed=0)


def test_route_exact(tiny):
    cfg = tiny.cfg
    y, idx, w, _ = e4b.moe_forward(tiny.layer, tiny.x_d, cfg.k, logits=tiny.logits_d, path="grouped")
    idx_ref, w_ref = oracle.route(tiny.logits, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    wg = w.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(wg - w_ref)) <= 1e-6
    assert np.max(np.abs(wg.sum(1) - 1.0)) <= 1e-6


@pytest.mark.parametrize("name,T", [("qwen3_prefill", None), ("olmoe", None), ("qwen3_decode", 8)])
def test_route_exact_workload_logits(name, T):
    from workloads import gen_logits

    cfg = get_config(name, T)
    lg = gen_logits(cfg, 1)
    announce(f"route {name} T={cfg.T} E={cfg.E}")
    lib = e4b.load()
    idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=DEV)
    w = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=DEV)
    # route through a forward on a tiny stand-in layer with the same E and k
    small = MoEConfig("s", E=cfg.E, H=64, I=64, k=cfg.k, T=cfg.T, routing=cfg.routing)
    pb = Problem(small, seed=0, with_grad=False)
    idx_ref, w_ref = oracle.route(lg, cfg.k)
    # decode-sized batches are also routed inside the decode gate_up launch
    paths = ["grouped", "decode"] if cfg.T <= 8 else ["grouped"]
    for path in paths:
        idx.fill_(-1)
        w.fill_(0.0)
        e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=torch.from_numpy(lg).to(DEV),
                        topk_idx=idx, topk_w=w, path=path)
        assert np.array_equal(idx.cpu().numpy(), idx_ref), path
        assert np.max(np.abs(w.cpu().numpy() - w_ref)) <= 1e-6, path
    del lib


@pytest.mark.parametrize("E,k,levels", [(8, 2, 2), (64, 32, 2), (128, 8, 4), (1024, 32, 1)])
def test_route_ties(E, k, levels):
    # logits drawn from a few values: the order among equal logits (lower
    # expert id first) decides the selection; with one level every logit
    # ties (more candidates than the parallel form holds: the serial form)
    rng = np.random.default_rng(E + k)
    announce(f"route ties E={E} k={k} levels={levels}")
    small = MoEConfig("s", E=E, H=64, I=64, k=k, T=8, routing="uniform")
    pb = Problem(small, seed=0, with_grad=False)
    for T, paths in ((8, ["grouped", "decode"]), (48, ["grouped"])):
        lg = rng.integers(0, levels, size=(T, E)).astype(np.float32) * 0.5
        x = torch.zeros(T, 64, dtype=torch.bfloat16, device=DEV)
        idx_ref, w_ref = oracle.route(lg, k)
        for path in paths:
            idx = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
            w = torch.zeros(T, k, dtype=torch.float32, device=DEV)
            e4b.moe_forward(pb.layer, x, k, logits=torch.from_numpy(lg).to(DEV), topk_idx=idx,
                            topk_w=w, path=path)
            assert np.array_equal(idx.cpu().numpy(), idx_ref), (T, path)
            assert np.max(np.abs(w.cpu().numpy() - w_ref)) <= 1e-6, (T, path)


def test_permutation_exact(tiny):
    cfg = tiny.cfg
    ws = torch.zeros(e4b.workspace_bytes(tiny.layer, cfg.T, cfg.k), dtype=torch.uint8, device=DEV)
    _, idx, _, _ = e4b.moe_forward(tiny.layer, tiny.x_d, cfg.k, logits=tiny.logits_d,
                                   path="grouped", workspace=ws)
    torch.cuda.synchronize()
    _check_permutation(tiny.layer, ws, idx.cpu().numpy(), cfg.E, cfg.P)


@pytest.mark.parametrize("name,T", [("tiny", 700), ("olmoe", None), ("qwen3_prefill", None),
                                    ("mixtral", None)])
def test_permutation_exact_multi_chunk(name, T):
    """Many 256-pair chunks (the per-chunk histogram, the carried scan and the
    per-chunk scatter base), up to the Zipf-routed Qwen3 prefill batch
    (P = 131072, its hottest expert spanning dozens of m-tiles)."""
    from workloads import gen_logits

    cfg = get_config(name, T)
    lg = gen_logits(cfg, 0)
    announce(f"permutation {name} E={cfg.E} k={cfg.k} T={cfg.T} P={cfg.P}")
    # routed through a forward on a small stand-in layer with the same E, k and T
    small = MoEConfig("s", E=cfg.E, H=64, I=64, k=cfg.k, T=cfg.T, routing=cfg.routing)
    pb = Problem(small, seed=0, with_grad=False)
    ws = torch.zeros(e4b.workspace_bytes(pb.layer, cfg.T, cfg.k), dtype=torch.uint8, device=DEV)
    _, idx, _, _ = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=torch.from_numpy(lg).to(DEV),
                                   path="grouped", workspace=ws)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    assert np.array_equal(idx_np, oracle.route(lg, cfg.k)[0])
    _check_permutation(pb.layer, ws, idx_np, cfg.E, cfg.P)
    # given ids (no logits): the same permutation from the caller's buffer
    ws.zero_()
    e4b.moe_forward(pb.layer, pb.x_d, cfg.k, topk_idx=idx, topk_w=torch.full_like(idx, 0.5, dtype=torch.float32),
                    path="grouped", workspace=ws)
    torch.cuda.synchronize()
    _check_permutation(pb.layer, ws, idx_np, cfg.E, cfg.P)


def test_forward_tiny_grouped(tiny):
    cfg = tiny.cfg
    y, idx, w, _ = e4b.moe_forward(tiny.layer, tiny.x_d, cfg.k, logits=tiny.logits_d, path="grouped")
    idx_ref, w_ref = oracle.route(tiny.logits, cfg.k)
    tol_check(to_np(y), _oracle_fwd(tiny, idx_ref, w_ref), "y")


@pytest.mark.parametrize("T", [1, 3, 8])
def test_forward_tiny_decode_path(tiny, T):
    cfg = tiny.cfg
    x = tiny.x_d[:T].contiguous()
    lg = tiny.logits_d[:T].contiguous()
    y, idx, w, _ = e4b.moe_forward(tiny.layer, x, cfg.k, logits=lg, path="decode")
    idx_ref, w_ref = oracle.route(tiny.logits[:T], cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    tol_check(to_np(y), _oracle_fwd(tiny, idx_ref, w_ref, tokens=slice(0, T)), f"y decode T={T}")
    y2, _, _, _ = e4b.moe_forward(tiny.layer, x, cfg.k, logits=lg, path="grouped")
    tol_check(to_np(y), to_np(y2).astype(np.float64), f"decode vs grouped T={T}", rel=2e-2)


def test_dgrad_tiny_recompute_equals_saved(tiny):
    cfg = tiny.cfg
    y, idx, w, saved = e4b.moe_forward(tiny.layer, tiny.x_d, cfg.k, logits=tiny.logits_d, save=True)
    gx_s, gw_s = e4b.moe_dgrad(tiny.layer, idx, w, tiny.grad_y_d, saved=saved)
    gx_r, gw_r = e4b.moe_dgrad(tiny.layer, idx, w, tiny.grad_y_d, x=tiny.x_d)
    torch.cuda.synchronize()
    assert torch.equal(gx_s.view(torch.int16), gx_r.view(torch.int16))
    assert torch.equal(gw_s.view(torch.int32), gw_r.view(torch.int32))
    idx_ref, w_ref = oracle.route(tiny.logits, cfg.k)
    gx_ref, gw_ref = _oracle_dgrad(tiny, idx_ref, w_ref)
    tol_check(to_np(gx_s), gx_ref, "grad_x")
    tol_check(to_np(gw_s), gw_ref, "grad_topk_w")
    # forward with save=True gives the same y as without
    y2, _, _, _ = e4b.moe_forward(tiny.layer, tiny.x_d, cfg.k, logits=tiny.logits_d, path="grouped")
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_runs_are_bitwise_deterministic(tiny):
    cfg = tiny.cfg
    outs = []
    for _ in range(2):
        y, idx, w, saved = e4b.moe_forward(tiny.layer, tiny.x_d, cfg.k, logits=tiny.logits_d, save=True)
        gx, gw = e4b.moe_dgrad(tiny.layer, idx, w, tiny.grad_y_d, saved=saved)
        torch.cuda.synchronize()
        # the outputs; the saved buffer's padding is never written, so only
        # what the dgrad reads from it enters the comparison (through gx, gw)
        outs.append([t.clone() for t in (y, idx, w, gx, gw)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_ragged_multi_tile_and_empty_experts():
    """I not a multiple of 128 (masked columns), an expert with > 3 m-tiles, idle experts."""
    cfg = MoEConfig("ragged", E=6, H=192, I=320, k=2, T=700, routing="normal")
    announce("ragged E6 H192 I320 k2 T700")
    pb = Problem(cfg, seed=3)
    T, k = cfg.T, cfg.k
    rng = np.random.default_rng(0)
    idx = np.zeros((T, k), np.int32)
    idx[:, 0] = 0  # expert 0: 700 pairs -> 3 m-tiles, ragged tail
    idx[:, 1] = rng.choice([1, 2, 4], size=T, p=[0.6, 0.3, 0.1])  # experts 3 and 5 idle
    w = rng.random((T, k)).astype(np.float32)
    idx_d = torch.from_numpy(idx).to(DEV)
    w_d = torch.from_numpy(w).to(DEV)
    y, _, _, saved = e4b.moe_forward(pb.layer, pb.x_d, k, topk_idx=idx_d, topk_w=w_d, save=True)
    tol_check(to_np(y), _oracle_fwd(pb, idx, w.astype(np.float64)), "y ragged")
    gx, gw = e4b.moe_dgrad(pb.layer, idx_d, w_d, pb.grad_y_d, saved=saved)
    gx_ref, gw_ref = _oracle_dgrad(pb, idx, w.astype(np.float64))
    tol_check(to_np(gx), gx_ref, "grad_x ragged")
    tol_check(to_np(gw), gw_ref, "grad_w ragged")


@pytest.mark.parametrize("kind", ["fp4", "nf4"])
def test_forward_dgrad_small_both_codebooks(kind):
    cfg = MoEConfig("small", E=4, H=256, I=256, k=2, T=300, routing="uniform")
    announce(f"small {kind} E4 H256 I256 k2 T300")
    pb = Problem(cfg, seed=5, codebook=kind)
    y, idx, w, _ = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d)
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    tol_check(to_np(y), _oracle_fwd(pb, idx_ref, w_ref), f"y {kind}")
    gx, gw = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, x=pb.x_d)
    gx_ref, gw_ref = _oracle_dgrad(pb, idx_ref, w_ref)
    tol_check(to_np(gx), gx_ref, f"grad_x {kind}")
    tol_check(to_np(gw), gw_ref, f"grad_w {kind}")


def test_zero_tokens_noop(tiny):
    x = torch.empty(0, tiny.cfg.H, dtype=torch.bfloat16, device=DEV)
    idx = torch.empty(0, 2, dtype=torch.int32, device=DEV)
    w = torch.empty(0, 2, dtype=torch.float32, device=DEV)
    y, _, _, _ = e4b.moe_forward(tiny.layer, x, 2, topk_idx=idx, topk_w=w)
    assert y.shape == (0, tiny.cfg.H)
    gx, gw = e4b.moe_dgrad(tiny.layer, idx, w, x, x=x)
    assert gx.shape == (0, tiny.cfg.H) and gw.shape == (0, 2)


def test_single_expert_top1_is_dense_swiglu():
    """E=1, k=1, weight 1: the routed path reduces to one dense SwiGLU MLP."""
    cfg = MoEConfig("dense", E=1, H=128, I=192, k=1, T=260, routing="normal")
    announce("dense E1 H128 I192 k1 T260")
    pb = Problem(cfg, seed=2)
    idx = torch.zeros(cfg.T, 1, dtype=torch.int32, device=DEV)
    w = torch.ones(cfg.T, 1, dtype=torch.float32, device=DEV)
    y, _, _, _ = e4b.moe_forward(pb.layer, pb.x_d, 1, topk_idx=idx, topk_w=w, path="grouped")
    wgu, wdn = pb.oracle_weights()
    x = pb.x.astype(np.float64)
    g = x @ wgu[0, : cfg.I].T.astype(np.float64)
    u = x @ wgu[0, cfg.I :].T.astype(np.float64)
    ref = (g / (1 + np.exp(-g)) * u) @ wdn[0].T.astype(np.float64)
    tol_check(to_np(y), ref, "dense y")


def _decode_case(cfg, idx, seed=1, kind="nf4", path="decode"):
    """One forward path vs the oracle with given routing ids (weights drawn here)."""
    T, k = idx.shape
    # ids in range are a precondition the kernels do not check
    assert idx.min() >= 0 and idx.max() < cfg.E
    pb = Problem(cfg, seed=seed, codebook=kind, with_grad=False)
    w = np.random.default_rng(seed).random((T, k)).astype(np.float32) + 0.1
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(DEV)
    w_d = torch.from_numpy(w).to(DEV)
    y, _, _, _ = e4b.moe_forward(pb.layer, pb.x_d, k, topk_idx=idx_d, topk_w=w_d, path=path)
    tol_check(to_np(y), _oracle_fwd(pb, idx, w.astype(np.float64)), f"y {path} {cfg.name}")


@pytest.mark.parametrize("kind", ["nf4", "fp4"])
def test_decode_all_tokens_share_experts(kind):
    """Every token on the same k experts: the 8-token bucket of the GEMV."""
    cfg = MoEConfig("share", E=16, H=512, I=256, k=4, T=8, routing="normal")
    announce(f"decode share {kind} E16 H512 I256 k4 T8")
    idx = np.tile(np.array([[3, 9, 0, 14]], np.int32), (8, 1))
    _decode_case(cfg, idx, kind=kind)


def test_decode_mixed_token_counts():
    """Experts with 1, 2, 3, 5 and 8 tokens in one call (every vector bucket of the
    GEMV, and experts with more pairs than one pass takes)."""
    cfg = MoEConfig("mixed", E=32, H=1024, I=512, k=4, T=8, routing="normal")
    announce("decode mixed counts E32 H1024 I512 k4 T8")
    idx = np.zeros((8, 4), np.int32)
    for t in range(8):
        # expert 0: 8 tokens; 2: 5; 4: 3; 15-17: 2 each; the rest 1
        idx[t] = [0, 2 if t < 5 else 20 + t, 4 if t < 3 else 12 + t, 10 + t]
    _decode_case(cfg, idx)


@pytest.mark.parametrize("H,I", [(16384, 64), (64, 16384)])
@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_longest_and_shortest_rows(path, H, I):
    """in_features 16384 (the decode limit) and 64 (one block), on either projection."""
    cfg = MoEConfig("long", E=4, H=H, I=I, k=2, T=5, routing="normal")
    announce(f"{path} long rows E4 H{H} I{I} k2 T5")
    idx = np.array([[0, 1], [1, 2], [3, 0], [2, 3], [0, 2]], np.int32)
    _decode_case(cfg, idx, path=path)


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_expert_repeated_within_tokens(path):
    """Given ids may repeat an expert within a token: each slot is its own pair
    (here 16 pairs on expert 5, more than one GEMV pass takes, and 3 on 1)."""
    cfg = MoEConfig("repeat", E=8, H=512, I=320, k=3, T=8, routing="normal")
    announce(f"{path} repeated experts E8 H512 I320 k3 T8")
    idx = np.array([[5, 5, t % 3] for t in range(8)], np.int32)
    _decode_case(cfg, idx, path=path)


def _ids_with_repeats(E, T, k, rng):
    """Routing ids drawn from a few experts (shared by several tokens, repeated
    within tokens) plus the last expert id."""
    idx = rng.integers(0, min(E, 5), size=(T, k)).astype(np.int32)
    idx[0, 0] = E - 1
    return idx


@pytest.mark.parametrize("E,I,T,k,kind", [(8, 1088, 8, 4, "nf4"), (256, 64, 8, 8, "fp4"), (6, 640, 3, 2, "nf4"),
                                          (16, 640, 8, 8, "mxfp4")])
def test_decode_rows_of_2048(E, I, T, k, kind):
    """H = 2048 (one 32-element chunk per lane of a wave) and E <= 256 take the
    one-workgroup-per-CU gate_up launch: blocks of ceil(I / CUs) units, at most
    4 (on 256 CUs: I = 1088 gives 272 blocks of 4, so some workgroups take two;
    I = 640 blocks of 3 with a last block of one unit), experts with up to T
    tokens and repeated within a token, and 256 experts."""
    cfg = MoEConfig("rows2048", E=E, H=2048, I=I, k=k, T=T, routing="normal")
    announce(f"decode rows of 2048 {kind} E{E} I{I} k{k} T{T}")
    _decode_case(cfg, _ids_with_repeats(E, T, k, np.random.default_rng(E + I + T)), kind=kind)


@pytest.mark.parametrize("E,T", [(128, 1), (64, 5), (257, 2)])
def test_decode_rows_of_2048_routed(E, T):
    """The same launch routing from logits (one wave per token): ids exact, weights
    within 1e-6, y against the oracle. E = 257 takes the 256-thread launch."""
    cfg = MoEConfig("rows2048r", E=E, H=2048, I=64, k=8, T=T, routing="normal")
    announce(f"decode rows of 2048 routed E{E} I64 k8 T{T}")
    pb = Problem(cfg, seed=3, with_grad=False)
    y, idx, w, _ = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, path="decode")
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.max(np.abs(w.cpu().numpy() - w_ref)) <= 1e-6
    tol_check(to_np(y), _oracle_fwd(pb, idx_ref, w_ref), f"y rows2048 routed E{E}")


@pytest.mark.parametrize("kind", ["nf4", "mxfp4"])
def test_decode_gate_up_launches_agree_bitwise(kind):
    """The 1024-thread gate_up launch (E <= 256) and the 256-thread one (E = 257)
    compute each pair with the same products, chunk scaling and lane sums: the
    same 256 experts routed the same way give the same y bits, whether or not
    the layer holds a 257th (never routed) expert."""
    cfg = MoEConfig("agree", E=257, H=2048, I=64, k=8, T=8, routing="normal")
    announce(f"decode gate_up launches agree bitwise {kind} E256 vs E257 H2048 I64 k8 T8")
    pb = Problem(cfg, seed=5, codebook=kind, with_grad=False)
    st = [pb.layer.gate_up, pb.layer.down]

    def first(t):
        return None if t is None else t[:256].contiguous()

    sub = e4b.MoELayer(*(e4b.QuantStack(first(q.packed), first(q.absmax), 256, q.out, q.inn, q.codebook,
                                        first(q.scales)) for q in st))
    idx = _ids_with_repeats(256, cfg.T, cfg.k, np.random.default_rng(5))
    idx[1] = np.arange(8) * 31  # experts spread over the stack
    w = (np.random.default_rng(6).random((cfg.T, cfg.k)) + 0.1).astype(np.float32)
    idx_d, w_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)
    y256, _, _, _ = e4b.moe_forward(sub, pb.x_d, cfg.k, topk_idx=idx_d, topk_w=w_d, path="decode")
    y257, _, _, _ = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, topk_idx=idx_d, topk_w=w_d, path="decode")
    torch.cuda.synchronize()
    assert torch.equal(y256.view(torch.int16), y257.view(torch.int16))
    tol_check(to_np(y256), _oracle_fwd(pb, idx, w.astype(np.float64)), "y agree")


def test_decode_down_launches_agree_bitwise():
    """The 1024-thread down launch (P * I <= 48K: P = 64 here) and the 256-thread
    one (P = 72: a ninth slot per token, routed with weight 0) compute each pair
    and each combine the same way: the same y bits."""
    cfg = MoEConfig("agree_dn", E=16, H=2048, I=768, k=8, T=8, routing="normal")
    announce("decode down launches agree bitwise P64 vs P72 E16 H2048 I768 T8")
    pb = Problem(cfg, seed=7, with_grad=False)
    rng = np.random.default_rng(7)
    idx8 = np.stack([rng.permutation(16)[:8] for _ in range(cfg.T)]).astype(np.int32)
    w8 = (rng.random((cfg.T, 8)) + 0.1).astype(np.float32)
    idx9 = np.concatenate([idx8, idx8[:, :1]], axis=1)
    w9 = np.concatenate([w8, np.zeros((cfg.T, 1), np.float32)], axis=1)
    ys = []
    for idx, w in ((idx8, w8), (idx9, w9)):
        y, _, _, _ = e4b.moe_forward(pb.layer, pb.x_d, idx.shape[1], topk_idx=torch.from_numpy(idx).to(DEV),
                                     topk_w=torch.from_numpy(w).to(DEV), path="decode")
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))


def test_grouped_topk_equals_E():
    """Every token routed to every expert (top_k = E)."""
    cfg = MoEConfig("allE", E=4, H=256, I=128, k=4, T=96, routing="normal")
    announce("grouped top_k = E E4 H256 I128 T96")
    pb = Problem(cfg, seed=4)
    y, idx, w, saved = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, save=True)
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    tol_check(to_np(y), _oracle_fwd(pb, idx_ref, w_ref), "y top_k=E")
    gx, gw = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, saved=saved)
    gx_ref, gw_ref = _oracle_dgrad(pb, idx_ref, w_ref)
    tol_check(to_np(gx), gx_ref, "grad_x top_k=E")
    tol_check(to_np(gw), gw_ref, "grad_w top_k=E")


@pytest.mark.parametrize("kind", ["nf4", "mxfp4", "bf16", "int8", "fp8"])
@pytest.mark.parametrize("I", [256, 320])
def test_down_dgrad_wide_tile(kind, I):
    """H = 4096 puts the down dgrad on the 256-column tile: two g|u blocks per
    tile (I = 256), and a tile whose second block lies past I (I = 320)."""
    cfg = MoEConfig("wide_dgrad", E=4, H=4096, I=I, k=2, T=300, routing="uniform")
    announce(f"wide down dgrad {kind} E4 H4096 I{I} k2 T300")
    pb = Problem(cfg, seed=7, codebook=kind)
    y, idx, w, saved = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, save=True,
                                       path="grouped")
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    gx, gw = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, saved=saved)
    gx2, gw2 = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, x=pb.x_d)
    assert torch.equal(gx.view(torch.uint8), gx2.view(torch.uint8)) and torch.equal(gw, gw2)
    gx_ref, gw_ref = _oracle_dgrad(pb, idx_ref, w_ref)
    tol_check(to_np(gx), gx_ref, f"grad_x wide {kind}")
    tol_check(to_np(gw), gw_ref, f"grad_w wide {kind}")
