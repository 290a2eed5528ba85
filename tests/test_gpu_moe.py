"""GPU parity of the mixture-of-experts decode FFN (qmoe_ffn_decode) against
the oracle, stage by stage.

For each slot z with a valid expert e = ids[z]: h_z must meet the FFN h
tolerance against act(g) * u, where g and u are the oracle's GEMVs of expert
e's gate and up over the oracle's RMS-normalised x; a slot with an invalid
id must hold h_z = 0.  Then y must meet
    |y - sum_z coef_z y_z| <= sum_z |coef_z| (1e-4 S_z + 1e-6) + 2^-22 sum_z |coef_z y_z|
with y_z, S_z the oracle's down GEMV of expert e over the GPU's own h_z (fp64)
and the last term the fp32 rounding of the weighted sum.  Repeated calls must
agree bit for bit (the slots are summed in slot order).

Rows of whole 256-weight superunits take the streaming kernel (the slots
share the CUs, and the last workgroup of a down row range sums the slots);
other rows, and any forced launch shape, take the register kernel, which the
`register_kernel` cases run on shapes the streaming kernel would take.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

SEED = 0x5EED


@pytest.fixture(scope="module")
def qd(gpu):
    import quantized_decode_q4k_amd as qd
    qd.lib()
    return qd


from helpers import dev, h_tolerance, say  # noqa: E402


@pytest.fixture
def register_kernel(qd):
    """A forced launch shape keeps the MoE launches on the register kernel."""
    qd.set_launch_override(2, 0, 0)
    yield
    qd.set_launch_override(0, 0, 0)


def check_moe(qd, fg, fd, hidden, ff, n_experts, ids, coef, act, with_norm=True, tag=""):
    n_sel = len(ids)
    Wg = synth.quant_weights(fg, n_experts * ff, hidden, SEED, tensor_id=91)
    Wu = synth.quant_weights(fg, n_experts * ff, hidden, SEED, tensor_id=92)
    Wd = synth.quant_weights(fd, n_experts * hidden, ff, SEED, tensor_id=93)
    x = synth.normal((hidden,), SEED, tensor_id=94)
    nw = synth.normal((hidden,), SEED, tensor_id=95, mean=1.0, std=0.1)
    say(f"moe {tag} {fg}/{fd} hidden={hidden} ff={ff} experts={n_experts} ids={list(ids)} act={act}")
    dW = [dev(a) for a in (Wg, Wu, Wd)]
    di = torch.tensor(np.asarray(ids, np.int32)).cuda()
    dc = torch.tensor(np.asarray(coef, np.float32)).cuda()
    outs = []
    for rep in range(2):
        h = torch.full((n_sel, ff), float("nan"), device="cuda")
        y = qd.qmoe_ffn_decode(fg, *dW[:2], fd, dW[2], n_experts, di, dc, dev(x),
                               dev(nw) if with_norm else None, 1e-6, act, h_out=h)
        outs.append((y.cpu().numpy(), h.cpu().numpy()))
    (y, h), (y2, h2) = outs
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"
    xn = oracle.rmsnorm(x, nw, 1e-6) if with_norm else x.astype(np.float64)[None]
    xn32 = xn.astype(np.float32)
    aid = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_SILU
    ref = np.zeros(hidden)
    bound = np.full(hidden, 0.0)
    mag = np.zeros(hidden)
    for z, (e, c) in enumerate(zip(ids, coef)):
        if not 0 <= e < n_experts:
            assert np.array_equal(h[z], np.zeros(ff, np.float32)), f"slot {z}: invalid id, h not zero"
            continue
        g64, Sg = oracle.gemv(fg, Wg, xn32, n_experts * ff, hidden, e * ff, (e + 1) * ff)
        u64, Su = oracle.gemv(fg, Wu, xn32, n_experts * ff, hidden, e * ff, (e + 1) * ff)
        sl = slice(e * ff, (e + 1) * ff)
        href = oracle.act_vec(aid, g64[0, sl]) * u64[0, sl]
        tol = h_tolerance(g64[0, sl], u64[0, sl], Sg[0, sl], Su[0, sl], aid)
        err = np.abs(h[z] - href)
        assert (err <= tol).all(), f"slot {z} h: worst {np.max(err / tol):.3f} of tolerance"
        yz, Sz = oracle.gemv(fd, Wd, h[z], n_experts * hidden, ff, e * hidden, (e + 1) * hidden)
        yz, Sz = yz[0, e * hidden:(e + 1) * hidden], Sz[0, e * hidden:(e + 1) * hidden]
        ref += c * yz
        bound += abs(c) * (1e-4 * Sz + 1e-6)
        mag += np.abs(c * yz)
    err = np.abs(y - ref)
    tot = bound + 2.0 ** -22 * mag + 1e-30
    assert (err <= tot).all(), f"{tag} y: worst {np.max(err / tot):.3f} of bound"


def test_moe_top8_of_16_gelu(qd):
    ids = [3, 15, 0, 7, 3, 11, 9, 1]   # a repeated expert is allowed
    coef = [0.31, 0.17, 0.12, 0.1, 0.09, 0.08, 0.07, 0.06]
    check_moe(qd, "q4_k", "q6_k", 2560, 1536, 16, ids, coef, "gelu_tanh", tag="top8")


def test_moe_single_slot_silu_no_norm(qd):
    check_moe(qd, "q4_k", "q4_k", 1024, 768, 4, [2], [0.75], "silu", with_norm=False, tag="top1")


def test_moe_invalid_id_contributes_nothing(qd):
    check_moe(qd, "q8_0", "q8_0", 512, 512, 6, [5, -1, 6, 0], [0.5, 9.0, 7.0, 0.25], "gelu_tanh",
              tag="invalid ids")


def test_moe_q6k_experts_many_slots(qd):
    ids = list(range(0, 24, 2)) + [1, 3, 5, 7]
    coef = list(np.linspace(0.02, 0.2, len(ids)))
    check_moe(qd, "q6_k", "q6_k", 768, 512, 24, ids, coef, "silu", tag="16 slots")


def test_moe_bench_configuration(qd):
    """The moe_decode bench workload's shape and launch configuration: 8 of 128
    experts, hidden 2560, expert FF 1024, Q4_K gate/up with GELU-tanh, Q6_K
    down, routing weights summing to one."""
    rng = np.random.default_rng(7)
    ids = [int(v) for v in rng.choice(128, 8, replace=False)]
    coef = [float(v) for v in rng.dirichlet(np.ones(8))]
    check_moe(qd, "q4_k", "q6_k", 2560, 1024, 128, ids, coef, "gelu_tanh", tag="bench config")


def test_moe_three_slots_ragged_ranges(qd):
    """Three slots: 85 workgroups per slot, row ranges of unequal length."""
    check_moe(qd, "q4_k", "q6_k", 2560, 1024, 32, [30, 2, 17], [0.5, 0.3, 0.2], "gelu_tanh",
              tag="3 slots")


def test_moe_sixty_four_slots(qd):
    """The most slots a call takes: four workgroups per slot."""
    rng = np.random.default_rng(11)
    ids = [int(v) for v in rng.integers(0, 40, 64)]
    ids[5] = 40       # out of range: contributes nothing
    coef = [float(v) for v in rng.uniform(-0.1, 0.2, 64)]
    check_moe(qd, "q4_k", "q6_k", 1024, 512, 40, ids, coef, "silu", tag="64 slots")


def test_moe_partial_superunit_rows(qd):
    """Q8_0 rows of 800 weights (not whole superunits): the register kernel."""
    check_moe(qd, "q8_0", "q8_0", 800, 512, 5, [4, 1, 1], [0.6, 0.3, 0.1], "gelu_tanh",
              tag="K % 256 != 0")


def test_moe_register_kernel_bench_configuration(qd, register_kernel):
    rng = np.random.default_rng(7)
    ids = [int(v) for v in rng.choice(128, 8, replace=False)]
    coef = [float(v) for v in rng.dirichlet(np.ones(8))]
    check_moe(qd, "q4_k", "q6_k", 2560, 1024, 128, ids, coef, "gelu_tanh", tag="register kernel")


def test_moe_register_kernel_invalid_id(qd, register_kernel):
    check_moe(qd, "q8_0", "q8_0", 512, 512, 6, [5, -1, 6, 0], [0.5, 9.0, 7.0, 0.25], "gelu_tanh",
              tag="register kernel, invalid ids")


def test_moe_long_rows_streaming(qd):
    """Hidden 16384: beyond the register kernel's staging (which would refuse
    it), on the streaming kernel."""
    check_moe(qd, "q4_k", "q6_k", 16384, 512, 3, [2, 0], [0.7, 0.3], "gelu_tanh", tag="hidden 16384")
