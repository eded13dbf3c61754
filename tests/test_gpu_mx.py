"""GPU parity of the MXFP4 storage lane (E2M1 codes, E8M0 scale per 32):
the conversion and dequantization bit-exact against the oracle, and the
grouped forward, dgrad, decode GEMV and LoRA step on MXFP4 layers against the
oracle evaluated on the same stored values."""

import numpy as np
import pytest
import torch

import oracle
import bit_quantized_mixture_nf4_amd as e4b
from workloads import MoEConfig, get_config, gen_weights
from gpu_util import DEV, Problem, announce, tol_check, to_np

pytestmark = pytest.mark.gpu


def _adversarial(rows=16, inn=128, seed=0):
    """Blocks with every E2M1 midpoint and its fp32 neighbours at several
    scales, saturating values, zero blocks, -0.0 and subnormals."""
    rng = np.random.default_rng(seed)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    pts = np.concatenate([mags, (mags[:-1] + mags[1:]) / 2, [6.5, 7.0, 7.99]]).astype(np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(9)), np.nextafter(pts, np.float32(-1))])
    pts = pts[pts >= 0]
    w = (rng.standard_normal((rows, inn)) * 0.02).astype(np.float32)
    for r in range(0, rows, 2):
        k = int(rng.integers(-20, 20))
        blk = rng.choice(pts, size=32) * rng.choice([-1, 1], size=32)
        blk[0] = 6.0  # pins the shared exponent at k
        w[r, :32] = (blk * 2.0 ** k).astype(np.float32)
    w[1, 32:64] = 0.0
    w[3, 32:64] = -0.0
    w[5, 40] = -1e-30
    w[7, 64:96] = np.float32(1e-40)  # subnormal block
    w[9, 96:] = np.float32(3.0e38) * rng.choice([-1, 1], size=32)
    return w[None]


def _check(w):
    announce(f"mxfp4 quantize shape={w.shape}")
    st = e4b.quantize(torch.from_numpy(w).to(DEV), "mxfp4")
    p_ref, s_ref = oracle.quantize_mx(w)
    assert np.array_equal(st.scales.cpu().numpy(), s_ref)
    assert np.array_equal(st.packed.cpu().numpy(), p_ref)
    E, out, inn = w.shape
    ref32 = oracle.dequantize_mx(p_ref, s_ref, out, inn)
    got32 = e4b.dequantize(st, torch.float32).cpu().numpy()
    assert np.array_equal(got32.view(np.uint32), ref32.view(np.uint32))
    got16 = e4b.dequantize(st, torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got16, oracle.bf16_rne_bits(ref32))
    # every stored value is exact in bf16 (the bit-identical dequantization)
    assert np.array_equal(oracle.bf16_bits_to_f32(got16), ref32)


def test_mx_quantize_dequantize_bit_exact():
    cfg = get_config("tiny")
    _check(gen_weights(cfg, 0, "gate_up"))
    _check(_adversarial())


@pytest.fixture(scope="module")
def tiny_mx():
    announce("tiny layer E8 H256 I128 k2 T64, mxfp4")
    return Problem(get_config("tiny"), seed=4, codebook="mxfp4")


def test_mx_forward_dgrad_grouped(tiny_mx):
    pb, cfg = tiny_mx, tiny_mx.cfg
    y, idx, w, saved = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, save=True)
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    wgu, wdn = pb.oracle_weights()
    tol_check(to_np(y), oracle.moe_forward(pb.x, idx_ref, w_ref, wgu, wdn), "y mxfp4")
    gx, gw = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, saved=saved)
    gx_ref, gw_ref = oracle.moe_dgrad(pb.x, idx_ref, w_ref, wgu, wdn, pb.grad_y)
    tol_check(to_np(gx), gx_ref, "grad_x mxfp4")
    tol_check(to_np(gw), gw_ref, "grad_topk_w mxfp4")


@pytest.mark.parametrize("T", [1, 8])
def test_mx_decode_path(tiny_mx, T):
    pb, cfg = tiny_mx, tiny_mx.cfg
    x = pb.x_d[:T].contiguous()
    lg = pb.logits_d[:T].contiguous()
    y, idx, w, _ = e4b.moe_forward(pb.layer, x, cfg.k, logits=lg, path="decode")
    idx_ref, w_ref = oracle.route(pb.logits[:T], cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    wgu, wdn = pb.oracle_weights()
    tol_check(to_np(y), oracle.moe_forward(pb.x[:T], idx_ref, w_ref, wgu, wdn), f"y mxfp4 decode T={T}")


def test_mx_ragged_dgrad_b_nn_blocks():
    # H and I not multiples of 128: the dgrad's K-strided tiles cover partial
    # column groups; every 32-column MX block of a row stays inside one tile
    cfg = MoEConfig("mx_ragged", E=4, H=192, I=320, k=2, T=300, routing="normal")
    announce("mxfp4 ragged E4 H192 I320 k2 T300")
    pb = Problem(cfg, seed=6, codebook="mxfp4")
    y, idx, w, saved = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, save=True)
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    wgu, wdn = pb.oracle_weights()
    tol_check(to_np(y), oracle.moe_forward(pb.x, idx_ref, w_ref, wgu, wdn), "y mxfp4 ragged")
    gx, gw = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, saved=saved)
    gx_ref, gw_ref = oracle.moe_dgrad(pb.x, idx_ref, w_ref, wgu, wdn, pb.grad_y)
    tol_check(to_np(gx), gx_ref, "grad_x mxfp4 ragged")
    tol_check(to_np(gw), gw_ref, "grad_topk_w mxfp4 ragged")


# ---- the MX forward (E4B_PATH_MX8): MXFP8 activations on the block-scaled MFMA ----

def _unswap(codes):
    c = np.asarray(codes).copy()
    c[:, 0::2], c[:, 1::2] = codes[:, 1::2], codes[:, 0::2]
    return c


def test_mx8_rows_bit_exact():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    # E4M3 midpoints, saturating values, a zero block, -0.0 and tiny values
    mids = np.array([1.0625, 1.1875, 432.0, 440.0, 464.0, 2.0 ** -10, 3 * 2.0 ** -10, 0.0], np.float32)
    x[0, :32] = 0.0
    x[1, :32] = np.concatenate([[448.0], mids, -mids, np.zeros(32 - 17)]).astype(np.float32)
    x[2, 32:64] = -0.0
    x[3, 64:96] = np.float32(1e-30)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    announce("mx8 rows 64 x 256")
    codes, scales = e4b.mx8_rows(xb.to(DEV))
    c_ref, s_ref = oracle.quantize_mx8_rows(xb.float().numpy())
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(_unswap(codes.cpu().numpy()), c_ref)


@pytest.mark.parametrize("name", ["tiny", "mx_mid"])
def test_mx8_forward_against_oracle(name, tiny_mx):
    if name == "tiny":
        pb = tiny_mx
    else:
        cfg = MoEConfig("mx_mid", E=6, H=256, I=384, k=2, T=300, routing="normal")
        announce("mxfp4 layer E6 H256 I384 k2 T300, mx8 path")
        pb = Problem(cfg, seed=12, codebook="mxfp4", with_grad=False)
    cfg = pb.cfg
    y, idx, w, _ = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, path="mx8")
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    wgu, wdn = pb.oracle_weights()
    # the oracle converts bf16-rounded x the same way (x is bf16 on the device)
    xb = torch.from_numpy(pb.x).to(torch.bfloat16).float().numpy()
    tol_check(to_np(y), oracle.mx8_forward(xb, idx_ref, w_ref, wgu, wdn), f"y mx8 {name}")
    # against the exact-activation MXFP4 forward: the activation rounding only
    y2, _, _, _ = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, path="grouped")
    tol_check(to_np(y), to_np(y2).astype(np.float64), f"mx8 vs grouped {name}", rel=0.1)
    # run to run: bitwise identical
    y3, _, _, _ = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, path="mx8")
    assert torch.equal(y.view(torch.int16), y3.view(torch.int16))


@pytest.mark.parametrize("T", [0, 1, 5])
def test_mx8_small_batches(tiny_mx, T):
    # one m-tile per expert with one to five valid rows (or no call at all)
    pb, cfg = tiny_mx, tiny_mx.cfg
    x, lg = pb.x_d[:T].contiguous(), pb.logits_d[:T].contiguous()
    announce(f"mx8 path T={T}")
    y, idx, w, _ = e4b.moe_forward(pb.layer, x, cfg.k, logits=lg, path="mx8")
    assert y.shape == (T, cfg.H)
    if T == 0:
        return
    idx_ref, w_ref = oracle.route(pb.logits[:T], cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    wgu, wdn = pb.oracle_weights()
    xb = torch.from_numpy(pb.x[:T]).to(torch.bfloat16).float().numpy()
    tol_check(to_np(y), oracle.mx8_forward(xb, idx_ref, w_ref, wgu, wdn), f"y mx8 T={T}")


def test_mx8_given_routing_top_k_equals_E():
    # routing passed in (no logits), every token on every expert
    cfg = MoEConfig("mx_allE", E=4, H=256, I=128, k=4, T=96, routing="normal")
    announce("mxfp4 top_k = E E4 H256 I128 T96, mx8 path with given routing")
    pb = Problem(cfg, seed=9, codebook="mxfp4", with_grad=False)
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    idx_d = torch.from_numpy(idx_ref).to(DEV)
    w_d = torch.from_numpy(w_ref.astype(np.float32)).to(DEV)
    y, _, _, _ = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, topk_idx=idx_d, topk_w=w_d, path="mx8")
    wgu, wdn = pb.oracle_weights()
    xb = torch.from_numpy(pb.x).to(torch.bfloat16).float().numpy()
    tol_check(to_np(y), oracle.mx8_forward(xb, idx_ref, w_d.cpu().numpy().astype(np.float64), wgu, wdn),
              "y mx8 top_k=E")
