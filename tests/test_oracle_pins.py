"""Pins of the float64 oracle to facts other than itself (CPU only).

Each test names what fixes the expected value: a hand-worked example, a
closed form, a special case that reduces to plain round-to-nearest, brute
force, an independent least-squares solve, exact rational arithmetic, or a
number printed by the pages.
"""
import json
import os
from fractions import Fraction
import itertools
import struct

import numpy as np
import pytest

import oracle as O
from oracle import check as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _spd_from_x(rng, n, d, scales=None):
    X = rng.standard_normal((n, d))
    if scales is not None:
        X = X * scales[None, :]
    return X, 2.0 * X.T @ X


# --------------------------------------------------------------------------
# quantizer: hand-worked examples of the min-max reading (golden fixture)
# --------------------------------------------------------------------------
def test_quantizer_hand_examples():
    cases = json.load(open(os.path.join(GOLDEN, "quantizer_examples.json")))["cases"]
    for c in cases:
        maxq = (1 << c["bits"]) - 1
        w = np.array(c["w"])[None, :]
        s, z, _ = O.group_params(w, maxq)
        assert s[0] == pytest.approx(c["s"], rel=1e-15), c["name"]
        assert z[0] == c["z"], c["name"]
        q, wq, _ = O.quantize_values(w[0], s[0], z[0], maxq)
        assert q.tolist() == c["q"], c["name"]
        assert np.allclose(wq, c["w_hat"], rtol=0, atol=1e-15), c["name"]


def test_quantizer_properties():
    rng = _rng(1)
    for bits in (2, 3, 4, 8):
        maxq = (1 << bits) - 1
        x = rng.standard_normal((200, 37)) * rng.uniform(0.01, 3, size=(200, 1)) + rng.uniform(-1, 1, (200, 1))
        s, z, tz = O.group_params(x, maxq)
        assert np.all(s > 0)
        assert np.all((z >= 0) & (z <= maxq)) and np.all(z == np.rint(z))
        for k in range(x.shape[1]):
            q, wq, _ = O.quantize_values(x[:, k], s, z, maxq)
            assert np.all((q >= 0) & (q <= maxq))
            # on the grid s*(Z - z)
            assert np.allclose(wq / s - np.rint(wq / s), 0, atol=1e-9)
            # within half a step (values lie inside [xmin, xmax] of their own group)
            assert np.all(np.abs(x[:, k] - wq) <= s / 2 * (1 + 1e-9) + 1e-12)
        # zero is exactly representable: the code z dequantizes to 0
        assert np.all(s * (z - z) == 0)


# --------------------------------------------------------------------------
# damping constant and the timing of group parameters: hand-worked values
# (tests/golden/damping_and_group_timing.json holds the derivations)
# --------------------------------------------------------------------------
def _golden_dg():
    return json.load(open(os.path.join(GOLDEN, "damping_and_group_timing.json")))


def test_damping_hand_examples():
    f = _golden_dg()
    c = f["damping_diagonal"]
    H = np.diag(c["diag_H"])
    assert O.damping(H, c["damp"]) == pytest.approx(c["lambda"], rel=1e-15)
    W = np.zeros((1, 4))
    r = O.gptq(W, H, 4, -1, 4, c["damp"], False)
    assert r["lam"] == pytest.approx(c["lambda"], rel=1e-15)
    assert np.allclose(np.diag(r["U"]), c["U_diag"], rtol=1e-14, atol=0)
    c = f["damping_2x2"]
    H = np.array(c["H"])
    r = O.gptq(np.zeros((1, 2)), H, 4, -1, 2, c["damp"], False)
    assert r["lam"] == pytest.approx(c["lambda"], rel=1e-15)
    assert np.allclose(r["U"], c["U"], rtol=1e-14, atol=1e-16)
    # the same U from the second route on the hand-damped matrix
    Hd = H + c["lambda"] * np.eye(2)
    assert np.allclose(O.inverse_cholesky_upper_reverse(Hd), c["U"], rtol=1e-14, atol=1e-16)


@pytest.mark.parametrize("B", [2, 4])
def test_group_parameters_from_compensated_values(B):
    c = _golden_dg()["group_timing"]
    H = np.array(c["H"])
    W = np.array(c["W"])
    r = O.gptq(W, H, c["bits"], c["group_size"], B, c["damp"], False)
    assert np.allclose(r["U"], c["U_chosen"], rtol=0, atol=1e-13)
    assert r["codes"].tolist() == c["codes"]
    assert np.allclose(r["scales"], c["scales"], rtol=1e-12, atol=0)
    assert np.array_equal(r["zeros"], np.array(c["zeros"]))
    assert np.allclose(r["E"], c["E"], rtol=0, atol=1e-13)
    assert np.allclose(r["w_hat"], c["w_hat"], rtol=0, atol=1e-13)
    # the column-by-column form with explicit inverses of the remaining set
    nv = O.obq_naive(W, H, c["bits"], c["group_size"], c["damp"], False)
    assert nv["codes"].tolist() == c["codes"]
    assert np.allclose(nv["w_hat"], c["w_hat"], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# P1: H proportional to I  =>  no compensation  =>  plain per-group RTN
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bits,g,B", [(4, 8, 8), (4, 8, 16), (3, 4, 12), (2, -1, 5), (4, 16, 32)])
@pytest.mark.parametrize("c", [1.0, 37.5])
def test_identity_hessian_reduces_to_rtn(bits, g, B, c):
    rng = _rng(2)
    d_out, d_in = 40, 48
    W = rng.standard_normal((d_out, d_in)) * 0.02
    H = c * np.eye(d_in)
    r = O.gptq(W, H, bits, g, B, damp=0.01, act_order=False)
    # U is diagonal, so there is nothing to propagate
    assert np.count_nonzero(np.triu(r["U"], 1)) == 0
    # direct RTN written out here, independently of the oracle's loop
    maxq = (1 << bits) - 1
    ge = d_in if g == -1 else g
    for c0 in range(0, d_in, ge):
        grp = W[:, c0:c0 + ge]
        lo = np.minimum(grp.min(1), 0)
        hi = np.maximum(grp.max(1), 0)
        s = (hi - lo) / maxq
        z = np.rint(-lo / s)
        q = np.clip(np.rint(grp / s[:, None]) + z[:, None], 0, maxq)
        assert np.array_equal(r["codes"][:, c0:c0 + ge], q)
        assert np.array_equal(r["scales"][c0 // ge], s)
        assert np.array_equal(r["zeros"][c0 // ge], z)
    rt = O.rtn(W, bits, g)
    assert np.array_equal(rt["codes"], r["codes"])


# --------------------------------------------------------------------------
# P2: the blocked lazy loop equals naive OBQ (inverse over the remaining
#     columns recomputed every column) on tiny inputs
# --------------------------------------------------------------------------
def _codes_equal_except_ties(a, b, ta, tol):
    diff = a != b
    if not diff.any():
        return True
    frac = np.abs(ta - np.floor(ta) - 0.5)
    return bool(np.all(frac[diff] < tol))


@pytest.mark.parametrize("d_in", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("act_order", [False, True])
def test_blocked_equals_naive_obq(d_in, bits, act_order):
    rng = _rng(10 + d_in * 7 + bits)
    X, H = _spd_from_x(rng, 3 * d_in + 2, d_in, scales=np.exp(rng.standard_normal(d_in)))
    W = rng.standard_normal((64, d_in)) * 0.05
    naive = {}
    for g in sorted({1, 2, 4, d_in} & set(range(1, d_in + 1))):
        if d_in % g and g != d_in:
            pass
        ref = O.obq_naive(W, H, bits, g, 0.01, act_order)
        for B in range(g, d_in + g, g):
            r = O.gptq(W, H, bits, g, B, 0.01, act_order)
            assert np.array_equal(r["perm"], ref["perm"])
            assert _codes_equal_except_ties(r["codes"], ref["codes"], ref["t"], 1e-9), (g, B)
        naive[g] = ref
    assert naive


# --------------------------------------------------------------------------
# P3: the result does not depend on the block size beyond rounding
# --------------------------------------------------------------------------
def test_block_size_independence():
    rng = _rng(3)
    d_in = 96
    X, H = _spd_from_x(rng, 400, d_in, scales=np.exp(rng.standard_normal(d_in)))
    W = rng.standard_normal((80, d_in)) * 0.02
    base = O.gptq(W, H, 4, 8, 8, 0.01, True)
    for B in (16, 24, 48, 96, 200):
        r = O.gptq(W, H, 4, 8, B, 0.01, True)
        assert _codes_equal_except_ties(r["codes"], base["codes"], base["t"], 1e-9), B
        assert np.allclose(r["scales"], base["scales"], rtol=1e-10)
        assert np.array_equal(r["zeros"], base["zeros"])


# --------------------------------------------------------------------------
# P4: the inverse factor
# --------------------------------------------------------------------------
def test_inverse_factor_routes_and_reconstruction():
    rng = _rng(4)
    for d in (1, 2, 7, 64, 130):
        X, H = _spd_from_x(rng, 3 * d + 5, d, scales=np.exp(rng.standard_normal(d)))
        Hd = H + O.damping(H, 0.01) * np.eye(d)
        U = O.inverse_cholesky_upper(Hd)
        U2 = O.inverse_cholesky_upper_reverse(Hd)
        assert np.allclose(np.tril(U, -1), 0)
        assert np.all(np.diag(U) > 0)
        assert np.allclose(U.T @ U @ Hd, np.eye(d), atol=1e-8)
        assert np.max(np.abs(U - U2)) <= 1e-9 * np.max(np.abs(U))
        L = np.linalg.cholesky(Hd)
        assert np.linalg.norm(L @ L.T - Hd) <= 10 * d * np.finfo(float).eps * np.linalg.norm(Hd)


def test_indefinite_hessian_raises():
    H = -np.eye(5)
    W = np.ones((3, 5))
    with pytest.raises(np.linalg.LinAlgError):
        O.gptq(W, H, 4, -1, 5, damp=0.0, act_order=False)


# --------------------------------------------------------------------------
# P5: closed form of the whole loop:  W0 - W_hat = E U  and
#     proxy loss = 1/2 (||E||^2 - lambda ||dW||^2)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("act_order", [False, True])
def test_closed_form_of_loop(act_order):
    rng = _rng(5)
    d_in = 160
    X, H = _spd_from_x(rng, 600, d_in, scales=np.exp(rng.standard_normal(d_in)))
    W = rng.standard_normal((50, d_in)) * 0.02
    r = O.gptq(W, H, 3, 32, 64, 0.01, act_order)
    dW = W[:, r["perm"]] - r["w_hat"]
    assert np.max(np.abs(dW - r["E"] @ r["U"])) <= 1e-12 * max(1.0, np.max(np.abs(dW)))
    Wh = O.dequantize(r["codes"], r["scales"], r["zeros"], r["perm"], r["group"])
    loss = O.proxy_loss(W, Wh, H)
    dW_orig = W - Wh
    closed = 0.5 * (np.sum(r["E"] ** 2) - r["lam"] * np.sum(dW_orig ** 2))
    assert loss == pytest.approx(closed, rel=1e-9)
    # the loss is also ||dW X^T||^2 computed from X directly
    assert loss == pytest.approx(np.sum((dW_orig @ X.T) ** 2), rel=1e-9)


# --------------------------------------------------------------------------
# OBQ update = least-squares optimum of the remaining columns (independent
# solve with lstsq on the damped, augmented activations)
# --------------------------------------------------------------------------
def test_first_update_is_least_squares_optimum():
    rng = _rng(6)
    d_in, n = 7, 30
    X = rng.standard_normal((n, d_in)) * np.exp(rng.standard_normal(d_in))
    H = 2.0 * X.T @ X
    damp = 0.05
    lam = O.damping(H, damp)
    W = rng.standard_normal((5, d_in)) * 0.3
    snap = {}

    def obs(k, Wcur):
        if k == 0:
            snap["W"] = Wcur.copy()

    r = O.gptq(W, H, 3, -1, d_in, damp, False, on_column=obs)
    # minimize ||dW X^T||^2 + lam/2 ||dW||^2 over the remaining columns with
    # column 0 fixed at its quantized value
    Xa = np.vstack([X, np.sqrt(lam / 2.0) * np.eye(d_in)])
    for row in range(W.shape[0]):
        d0 = r["w_hat"][row, 0] - W[row, 0]
        sol, *_ = np.linalg.lstsq(Xa[:, 1:], -Xa[:, 0] * d0, rcond=None)
        assert np.allclose(snap["W"][row, 1:], W[row, 1:] + sol, rtol=1e-9, atol=1e-12)


# --------------------------------------------------------------------------
# P6: Hessian equals the exact rational sum on bf16 inputs
# --------------------------------------------------------------------------
def _bf16_to_fraction(bits16):
    v = struct.unpack("<f", struct.pack("<I", int(bits16) << 16))[0]
    return Fraction(v)


def test_hessian_exact_rational():
    rng = _rng(7)
    n, d = 9, 4
    bits = (rng.integers(0x3C00, 0x4100, size=(n, d)) | (rng.integers(0, 2, size=(n, d)) << 15)).astype(np.uint16)
    H = O.hessian([bits[:4], bits[4:]], "bf16", d)
    for i in range(d):
        for j in range(d):
            exact = 2 * sum(_bf16_to_fraction(bits[t, i]) * _bf16_to_fraction(bits[t, j]) for t in range(n))
            assert abs(Fraction(H[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
    assert np.array_equal(H, H.T)
    assert np.all(np.linalg.eigvalsh(H) > -1e-9 * np.abs(H).max())
    # chunk additivity
    H1 = O.hessian([bits], "bf16", d)
    assert np.allclose(H, H1, rtol=1e-15)


# --------------------------------------------------------------------------
# P8: scaling H leaves the result unchanged
# --------------------------------------------------------------------------
def test_hessian_scale_invariance():
    rng = _rng(8)
    d_in = 64
    X, H = _spd_from_x(rng, 200, d_in, scales=np.exp(rng.standard_normal(d_in)))
    W = rng.standard_normal((60, d_in)) * 0.02
    a = O.gptq(W, H, 4, 16, 32, 0.01, True)
    b = O.gptq(W, 4.0 * H, 4, 16, 32, 0.01, True)     # power of two: exact
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["perm"], b["perm"])
    assert np.array_equal(a["scales"], b["scales"]) and np.array_equal(a["zeros"], b["zeros"])
    c = O.gptq(W, 3.3 * H, 4, 16, 32, 0.01, True)
    assert np.array_equal(a["perm"], c["perm"])
    assert _codes_equal_except_ties(c["codes"], a["codes"], a["t"], 1e-9)


# --------------------------------------------------------------------------
# P9: activation order
# --------------------------------------------------------------------------
def test_act_order_perm():
    rng = _rng(9)
    d = 50
    X, H = _spd_from_x(rng, 200, d, scales=np.exp(rng.standard_normal(d)))
    p = O.act_order_perm(H)
    assert sorted(p.tolist()) == list(range(d))
    assert np.all(np.diff(np.diag(H)[p]) <= 0)
    # ties keep ascending index
    Ht = np.diag([3.0, 5.0, 3.0, 5.0, 1.0, 3.0])
    assert O.act_order_perm(Ht).tolist() == [1, 3, 0, 2, 5, 4]
    # constant diagonal -> identity -> same result as act_order off
    Hc = H / np.sqrt(np.outer(np.diag(H), np.diag(H))) * 7.0
    Hc[np.diag_indices(d)] = 7.0
    W = rng.standard_normal((30, d)) * 0.02
    a = O.gptq(W, Hc, 4, 10, 10, 0.01, True)
    b = O.gptq(W, Hc, 4, 10, 10, 0.01, False)
    assert np.array_equal(a["perm"], np.arange(d))
    assert np.array_equal(a["codes"], b["codes"])


# --------------------------------------------------------------------------
# P10: packing, storage sizes and the pages' arithmetic
# --------------------------------------------------------------------------
def test_pack_hand_words():
    # 4 bits: code k in bits [4k, 4k+4) -> codes 1..8 give 0x87654321
    w = O.pack(np.array([[1, 2, 3, 4, 5, 6, 7, 8]]), 4)
    assert w.shape == (1, 1) and int(w[0, 0]) == 0x87654321
    # 3 bits: codes 0..10 = [1,2,3,4,5,6,7,0,1,2,5]; code 10 (value 5 = 0b101)
    # straddles: its bits 0,1 land in word 0 bits 30,31 (1, 0) and bit 2 in word 1 bit 0
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 0, 1, 2, 5]])
    expect0 = sum(int(c) << (3 * k) for k, c in enumerate(codes[0])) & 0xFFFFFFFF
    w = O.pack(codes, 3)
    assert w.shape == (2, 1)
    assert int(w[0, 0]) == expect0 and (int(w[0, 0]) >> 30) == 0b01
    assert int(w[1, 0]) == 1
    # 3-bit words are word-aligned every 32 codes (3 words)
    assert O.packed_words(32, 3) == 3 and O.packed_words(33, 3) == 4


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_roundtrip(bits):
    rng = _rng(11)
    for d_in in (1, 10, 11, 32, 33, 97):
        c = rng.integers(0, 1 << bits, size=(13, d_in))
        w = O.pack(c, bits)
        assert w.shape == ((bits * d_in + 31) // 32, 13)
        assert np.array_equal(O.unpack(w, bits, d_in), c)


def test_page_storage_figures():
    f = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    gc = f["group_count"]
    rows, cols = gc["shape"]
    assert rows * O.n_groups(cols, gc["group_size"]) == gc["groups"]
    for key in ("memory_7b", "memory_70b"):
        m = f[key]
        # packed 4-bit payload bytes of params, metadata excluded
        assert m["params"] * 4 / 8 / 1e9 == pytest.approx(m["int4_GB"])
        assert m["params"] * 2 / 1e9 == pytest.approx(m["fp16_GB"])
    m = f["memory_175b"]
    assert m["params"] * 4 / 8 / 1e9 == pytest.approx(m["int4_GB"])
    assert m["params"] * 2 / 1e9 == pytest.approx(m["wide_GB"])
    # a d_out x d_in layer packs into exactly 1/4 of its fp16 bytes
    d_out, d_in = 4096, 4096
    assert O.packed_words(d_in, 4) * 4 * d_out * f["int4_vs_fp16"]["factor"] == d_out * d_in * 2


# --------------------------------------------------------------------------
# P11: brute force on tiny rows: GPTQ's greedy result is never better than
#      the exact optimum on the same grid, and it matches its own loss
# --------------------------------------------------------------------------
def test_brute_force_lower_bound():
    rng = _rng(12)
    d_in, bits = 4, 2
    maxq = 3
    X, H = _spd_from_x(rng, 12, d_in)
    W = rng.standard_normal((6, d_in)) * 0.5
    r = O.gptq(W, H, bits, -1, d_in, 0.0, False)
    Wh = O.dequantize(r["codes"], r["scales"], r["zeros"], r["perm"], r["group"])
    for row in range(W.shape[0]):
        s, z = r["scales"][0, row], r["zeros"][0, row]
        best = min(
            0.5 * (W[row] - s * (np.array(q) - z)) @ H @ (W[row] - s * (np.array(q) - z))
            for q in itertools.product(range(maxq + 1), repeat=d_in))
        got = 0.5 * (W[row] - Wh[row]) @ H @ (W[row] - Wh[row])
        assert got >= best - 1e-12


# --------------------------------------------------------------------------
# P12: GPTQ beats round-to-nearest on a realistic layer (expected, reported)
# --------------------------------------------------------------------------
def test_gptq_beats_rtn_small_layer():
    from post_weight_quantization_04_amd import synth
    wl = synth.WORKLOADS["toy"]
    W = O.widen(synth.make_w(wl), "f32")
    H = O.hessian([synth.make_x(wl)], "f32", wl.d_in)
    r = O.gptq(W, H, 4, 128, 128, 0.01, False)
    Wh = O.dequantize(r["codes"], r["scales"], r["zeros"], r["perm"], r["group"])
    rt = O.rtn(W, 4, 128)
    assert O.proxy_loss(W, Wh, H) < O.proxy_loss(W, rt["w_hat"], H)


# --------------------------------------------------------------------------
# the parity checker itself: mistakes planted on the CPU must be caught
# --------------------------------------------------------------------------
def test_checker_accepts_self_and_catches_planted_errors():
    rng = _rng(13)
    d_in = 64
    X, H = _spd_from_x(rng, 300, d_in, scales=np.exp(rng.standard_normal(d_in)))
    W = rng.standard_normal((40, d_in)) * 0.02
    r = O.gptq(W, H, 4, 16, 32, 0.01, True)
    qp = O.pack(r["codes"], 4)
    ok = C.check_layer(W, H, 4, 16, 32, 0.01, True, qp, r["scales"], r["zeros"], r["perm"])
    assert ok["ok"] and ok["exempt_codes"] == 0
    # a code off by one away from any tie -> mismatch
    frac = np.abs(r["t"] - np.floor(r["t"]) - 0.5)
    row, col = np.argwhere((frac > 0.2) & (r["codes"] > 0))[0]
    bad = r["codes"].copy()
    bad[row, col] -= 1
    res = C.check_layer(W, H, 4, 16, 32, 0.01, True, O.pack(bad, 4), r["scales"], r["zeros"], r["perm"])
    assert not res["ok"] and res["mismatch_codes"] >= 1
    # a perturbed scale -> fails the relative check
    sc = r["scales"].copy()
    sc[1, 3] *= 1.01
    res = C.check_layer(W, H, 4, 16, 32, 0.01, True, qp, sc, r["zeros"], r["perm"])
    assert not res["ok"]
    # an order that is not sorted by diag(H) -> rejected
    p = r["perm"].copy()
    p[[0, -1]] = p[[-1, 0]]
    res = C.check_layer(W, H, 4, 16, 32, 0.01, True, qp, r["scales"], r["zeros"], p)
    assert not res["ok"] and not res["perm"]["ok"]


def test_checker_follows_exact_ties():
    # a column whose pre-round value is exactly at a half-integer: either code is right
    H = np.eye(3) * 2.0
    W = np.array([[-1.5, 0.75, 3.0]])     # 2 bits, one group: s = 1.5, z = 1, t(0.75) = 0.5
    r = O.gptq(W, H, 2, -1, 3, 0.0, False)
    t = r["t"][0, 1]
    assert abs(t - np.floor(t) - 0.5) < 1e-12
    alt = r["codes"].copy()
    alt[0, 1] += 1 if np.rint(t) == np.floor(t) else -1
    res = C.check_layer(W, H, 2, -1, 3, 0.0, False, O.pack(alt, 2), r["scales"], r["zeros"], r["perm"],
                        exempt_frac=1.0)     # one exempt entry out of four on this tiny row
    assert res["ok"] and res["exempt_codes"] == 1 and res["loss_rel"] == 0.0


def test_hessian_check_rule():
    rng = _rng(14)
    X, H = _spd_from_x(rng, 100, 20)
    H32 = H.astype(np.float32).astype(np.float64)
    assert C.check_hessian(H32, H)["ok"]
    Hb = H.copy()
    Hb[3, 5] += 1e-3 * np.sqrt(H[3, 3] * H[5, 5])
    assert not C.check_hessian(Hb, H)["ok"]


# --------------------------------------------------------------------------
# dequantize-then-multiply on a packed layer: hand-worked products
# (tests/golden/dequant_matmul_examples.json), and the same product built
# from a quantized layer against the quantizer's own w_hat
# --------------------------------------------------------------------------
def test_dequant_matmul_hand_examples():
    cases = json.load(open(os.path.join(GOLDEN, "dequant_matmul_examples.json")))["cases"]
    for c in cases:
        qp = np.array(c["qpacked"], dtype=np.uint32)
        # the stored words are the hand-derived bit streams of the codes
        assert [int(v) for v in qp.reshape(-1)] == [int(h, 16) for h in c["qpacked_hex"]], c["name"]
        assert np.array_equal(O.unpack(qp, c["bits"], c["d_in"]), np.array(c["codes"])), c["name"]
        g = c["d_in"] if c["group_size"] == -1 else c["group_size"]
        Wh = O.dequantize(np.array(c["codes"]), c["scales"], c["zeros"], np.array(c["perm"]), g)
        assert np.array_equal(Wh, np.array(c["W_hat"])), c["name"]
        Y = O.dequant_matmul(np.array(c["A"], dtype=np.float64), qp, c["scales"], c["zeros"], np.array(c["perm"]),
                             c["bits"], c["group_size"], c["d_in"])
        assert np.array_equal(Y, np.array(c["Y"])), c["name"]


def test_dequant_matmul_reproduces_quantized_layer():
    rng = _rng(15)
    d_in, d_out = 96, 20
    X, H = _spd_from_x(rng, 300, d_in, scales=np.exp(rng.standard_normal(d_in)))
    W = rng.standard_normal((d_out, d_in)) * 0.02
    r = O.gptq(W, H, 3, 32, 32, 0.01, True)
    qp = O.pack(r["codes"], 3)
    A = rng.standard_normal((5, d_in))
    Y = O.dequant_matmul(A, qp, r["scales"], r["zeros"], r["perm"], 3, 32, d_in)
    # the quantizer's dequantized values, processing order, moved back by perm
    W_back = np.empty_like(r["w_hat"])
    W_back[:, r["perm"]] = r["w_hat"]
    assert np.allclose(Y, A @ W_back.T, rtol=1e-13, atol=1e-15)
