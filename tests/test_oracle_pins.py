"""Pins of the CPU oracle against what the pages print and what mathematics fixes.

Each test checks the oracle against something other than itself: a value printed on a
page (``tests/golden/pages_printed_values.json``), a closed form, an invariant, a
hand-worked rounding case, a library routine, or a brute-force loop on tiny inputs.
Together they are meant to fail on a plausible slip anywhere in the oracle (a dropped
term, a wrong sign or index, a transposed operand, a wrong rounding mode).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import roofline
from weight_only_int4_w4a16_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def printed():
    with open(os.path.join(GOLDEN, "pages_printed_values.json")) as f:
        return json.load(f)


def close_to_printed(value, printed_value, digits):
    """``value`` rounds to ``printed_value`` at ``digits`` decimals (half a unit of slack)."""
    return abs(value - printed_value) <= 0.5 * 10.0 ** (-digits) + 1e-12


# ---------------------------------------------------------------- levels and packing

def test_signed_int4_has_sixteen_levels_minus8_to_7():
    p = printed()["signed_int4_levels"]
    levels = np.arange(p["min"], p["max"] + 1)
    assert levels.size == p["count"] == 16
    stored = oracle.to_offset_binary(levels)
    assert sorted(stored.tolist()) == list(range(16))          # bijective onto nibbles
    for bad in (-9, 8):
        with pytest.raises(ValueError):
            oracle.to_offset_binary(np.array([bad]))
    # dequantizing every stored nibble with s = 1 and the implicit zero 8 gives -8..7
    q = stored.reshape(16, 1)
    qw = oracle.pack_codes(np.vstack([q[:8], q[8:]]).reshape(16, 1))
    w = oracle.dequant_sym(qw, np.ones((1, 1), np.float16), 16)
    assert w.astype(np.int64).ravel().tolist() == levels.tolist()


def test_sym_quantizer_stays_in_signed_range_and_reaches_both_ends():
    W = synth.gaussian_weight(256, 64, seed=11)
    q, s = oracle.quantize_rtn_sym(W, 128)
    assert q.min() >= -8 and q.max() <= 7
    assert q.min() == -7 or q.max() == 7                        # max|w| lands on +-7


def test_pack_every_code_at_every_nibble_position():
    for j in range(8):
        for v in range(16):
            col = np.zeros((8, 1), np.uint8)
            col[j, 0] = v
            word = oracle.pack_codes(col)
            assert word.shape == (1, 1) and word.dtype == np.int32
            assert int(word.view(np.uint32)[0, 0]) == v << (4 * j)
            assert np.array_equal(oracle.unpack_codes(word), col)


def test_pack_roundtrip_random_words_including_sign_bit():
    g = np.random.default_rng(3)
    w = g.integers(-2**31, 2**31, size=(64, 40), dtype=np.int64).astype(np.int32)
    assert np.array_equal(oracle.pack_codes(oracle.unpack_codes(w)), w)
    z = g.integers(-2**31, 2**31, size=(5, 7), dtype=np.int64).astype(np.int32)
    assert np.array_equal(oracle.pack_zeros(oracle.unpack_zeros(z)), z)


def test_two_codes_per_byte_low_nibble_first():
    q = np.random.default_rng(4).integers(0, 16, size=(32, 3), dtype=np.uint8)
    qw = oracle.pack_codes(q)
    b = qw.astype("<i4").view(np.uint8).reshape(4, 3, 4)          # (K/8, N, byte)
    for r in range(4):
        for n in range(3):
            for byte in range(4):
                assert b[r, n, byte] & 0xF == q[8 * r + 2 * byte, n]
                assert b[r, n, byte] >> 4 == q[8 * r + 2 * byte + 1, n]


def test_zero_points_pack_along_n():
    z = np.random.default_rng(5).integers(0, 16, size=(3, 24), dtype=np.uint8)
    qz = oracle.pack_zeros(z)
    assert qz.shape == (3, 3)
    u = qz.view(np.uint32)
    for gi in range(3):
        for n in range(24):
            assert (int(u[gi, n // 8]) >> (4 * (n % 8))) & 0xF == z[gi, n]


# ---------------------------------------------------------------- format arithmetic

def test_packed_layout_shapes_and_bytes_for_4096x11008():
    p = printed()["packed_layout_4096x11008_g128"]
    W = synth.gaussian_weight(p["K"], p["N"], seed=12)
    q, s, z = oracle.quantize_rtn_asym(W, p["group_size"], "f16")
    qw, qz = oracle.pack_codes(q), oracle.pack_zeros(z)
    assert qw.shape == tuple(p["qweight_shape"]) and qw.dtype == np.int32
    assert s.shape == tuple(p["scales_shape"]) and s.dtype == np.float16
    assert qz.shape == tuple(p["qzeros_shape"]) and qz.dtype == np.int32
    sb = oracle.storage_bytes(p["K"], p["N"], p["group_size"])
    assert (sb["qweight"], sb["scales"], sb["qzeros"]) == (qw.nbytes, s.nbytes, qz.nbytes)
    assert sb["total"] == 23_425_024 and sb["fp16"] == 90_177_536
    assert close_to_printed(sb["qweight"] / 1e6, p["qweight_MB"], 1)
    assert close_to_printed(sb["scales"] / 1e6, p["scales_MB"], 2)
    assert close_to_printed(sb["qzeros"] / 1e6, p["qzeros_MB"], 2)
    assert close_to_printed(sb["total"] / 1e6, p["total_MB"], 1)
    assert close_to_printed(sb["fp16"] / 1e6, p["fp16_MB"], 1)
    assert close_to_printed(sb["total"] / sb["fp16"], p["ratio"], 2)


def test_bits_per_weight_printed_values():
    p = printed()
    bpw = p["bits_per_weight"]
    assert oracle.bits_per_weight(128) == 4.15625
    assert oracle.bits_per_weight(32) == 4.625
    assert close_to_printed(oracle.bits_per_weight(128), bpw["g128_scale_and_zero"], 2)
    assert close_to_printed(oracle.bits_per_weight(32), bpw["g32_scale_and_zero"], 2)
    assert close_to_printed(oracle.bits_per_weight(128) / 16, bpw["g128_fraction_of_fp16"], 2)
    assert close_to_printed(oracle.bits_per_weight(32) / 16, bpw["g32_fraction_of_fp16"], 2)
    assert oracle.bytes_per_weight(128, zeros=False) == p["bytes_per_weight_g128_scale_only"]["value"]
    assert oracle.bits_per_weight(64, zeros=False) == 4.25          # NF4 with fp16 absmax / 64


def test_four_bit_tick_gap_is_17_times_eight_bit():
    ratio = printed()["tick_gap_4bit_over_8bit"]["value"]
    W = synth.gaussian_weight(128, 16, seed=13)
    _, s4, _ = oracle.quantize_rtn_asym(W, 128, scale_dtype=None, bits=4)
    _, s8, _ = oracle.quantize_rtn_asym(W, 128, scale_dtype=None, bits=8)
    np.testing.assert_allclose(s4 / s8, ratio, rtol=1e-12)


# ---------------------------------------------------------------- quantizer invariants

@pytest.mark.parametrize("g", [32, 128])
@pytest.mark.parametrize("sdt", ["f16", "bf16"])
def test_affine_quantizer_error_at_most_half_step(g, sdt):
    W = synth.gaussian_weight(512, 96, seed=14)
    W[5, :] = 0.0                                                  # exact zeros survive
    W[g:2 * g, 3] = np.abs(W[g:2 * g, 3]) + 0.01                   # one-signed groups
    W[2 * g:3 * g, 4] = -np.abs(W[2 * g:3 * g, 4]) - 0.01
    q, s, z = oracle.quantize_rtn_asym(W, g, sdt)
    sv = oracle.scale_values(s, sdt)
    assert q.max() <= 15 and z.max() <= 15
    rows = np.arange(512) // g
    err = np.abs(W.astype(np.float64) - (q.astype(np.float64) - z[rows]) * sv[rows])
    assert np.all(err <= 0.5 * sv[rows] * (1 + 1e-9))
    assert (err / sv[rows]).max() > 0.45                           # the bound is tight
    # the stored scale is the smallest storable value >= range / 15
    Wg = W.astype(np.float64).reshape(-1, g, 96)
    rng = np.maximum(Wg.max(1), 0) - np.minimum(Wg.min(1), 0)
    assert np.all(sv >= rng / 15)
    if sdt == "f16":
        below = np.nextafter(s, np.float16(0)).astype(np.float64)
    else:
        below = oracle.bf16_bits_to_f64(s - 1)
    assert np.all(below < rng / 15)
    w_hat = oracle.dequant_affine(oracle.pack_codes(q), s, oracle.pack_zeros(z), g, sdt)
    zero_bits = w_hat.view(np.uint16)[5, :] if sdt == "f16" else w_hat[5, :]
    assert np.all(zero_bits == 0)                                  # +0.0 exactly


def test_symmetric_quantizer_error_at_most_half_step():
    W = synth.gaussian_weight(256, 32, seed=15)
    q, s = oracle.quantize_rtn_sym(W, 128)
    sv = s.astype(np.float64)
    rows = np.arange(256) // 128
    err = np.abs(W - q.astype(np.float64) * sv[rows])
    assert np.all(err <= 0.5 * sv[rows] * (1 + 1e-9))
    amax = np.abs(W.astype(np.float64).reshape(2, 128, 32)).max(1)
    assert np.all(sv >= amax / 7) and np.all(np.nextafter(s, np.float16(0)) < amax / 7)


def test_degenerate_all_zero_group():
    W = np.zeros((64, 8), np.float32)
    q, s, z = oracle.quantize_rtn_asym(W, 32)
    assert np.all(s == 1) and np.all(z == 0) and np.all(q == 0)
    qs, ss = oracle.quantize_rtn_sym(W, 32)
    assert np.all(ss == 1) and np.all(qs == 0)


# ---------------------------------------------------------------- dequantization

def test_dequant_power_of_two_scale_is_exact():
    g = np.random.default_rng(6)
    q = g.integers(0, 16, size=(64, 16), dtype=np.uint8)
    z = g.integers(0, 16, size=(2, 16), dtype=np.uint8)
    k = g.integers(1, 10, size=(2, 16))
    s = (2.0 ** -k).astype(np.float16)
    w = oracle.dequant_affine(oracle.pack_codes(q), s, oracle.pack_zeros(z), 32)
    expect = (q.astype(np.int64) - np.repeat(z, 32, 0)) * np.repeat(2.0 ** -k, 32, 0)
    assert np.array_equal(w.astype(np.float64), expect)


def test_dequant_ties_round_to_even_hand_worked():
    # fp16: s = fp16(0.1) = 1638 * 2**-14; 3 s = 1228.5 * 2**-12 -> tie -> 1228 * 2**-12
    q = np.full((8, 8), 3, np.uint8)
    z = np.zeros((1, 8), np.uint8)
    s = np.full((1, 8), 0.1, np.float16)
    w = oracle.dequant_affine(oracle.pack_codes(q), s, oracle.pack_zeros(z), 8, "f16")
    assert np.all(w.astype(np.float64) == 1228 * 2.0 ** -12)
    # bf16: s = 1 + 2**-7; 3 s = 3.0234375 = 193.5 * 2**-6 -> tie -> 194 * 2**-6 = 0x4042
    sb = np.full((1, 8), 0x3F81, np.uint16)
    wb = oracle.dequant_affine(oracle.pack_codes(q), sb, oracle.pack_zeros(z), 8, "bf16")
    assert np.all(wb == 0x4042)


def test_dequant_q_equals_z_is_positive_zero_and_sign_is_q_minus_z():
    q = np.tile(np.arange(16, dtype=np.uint8), 8).reshape(8, 16).T.copy()   # (16, 8)
    z = np.full((1, 8), 5, np.uint8)
    s = np.full((1, 8), 0.25, np.float16)
    w = oracle.dequant_affine(oracle.pack_codes(q), s, oracle.pack_zeros(z), 16)
    assert np.all(w.view(np.uint16)[5] == 0)
    assert np.array_equal(w[:, 0].astype(np.float64), (np.arange(16) - 5) * 0.25)


def test_bf16_rounding_matches_torch_cast():
    torch = pytest.importorskip("torch")
    v = np.random.default_rng(7).standard_normal(100000).astype(np.float32)
    v = np.concatenate([v, np.float32([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 0.0])])
    ours = oracle.round_nearest_bf16_bits(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    up = oracle.round_up_bf16_bits(np.abs(v[:1000]).astype(np.float64))
    upv = oracle.bf16_bits_to_f64(up)
    assert np.all(upv >= np.abs(v[:1000])) and np.all(oracle.bf16_bits_to_f64(up - 1) < np.abs(v[:1000]))


def test_f16_rounding_matches_torch_cast():
    torch = pytest.importorskip("torch")
    v = (np.random.default_rng(8).standard_normal(100000) * 0.05).astype(np.float32)
    ours = oracle.round_nearest_f16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float16).numpy()
    assert np.array_equal(ours.view(np.uint16), ref.view(np.uint16))


# ---------------------------------------------------------------- GEMM

def _tiny_case(M, K, N, g, sym, dt, seed):
    W = synth.gaussian_weight(K, N, seed=seed)
    if sym:
        q, s = oracle.quantize_rtn_sym(W, g, dt)
        qw, qz, zv = oracle.pack_codes(oracle.to_offset_binary(q)), None, np.full((K // g, N), 8)
    else:
        q, s, z = oracle.quantize_rtn_asym(W, g, dt)
        qw, qz, zv = oracle.pack_codes(q), oracle.pack_zeros(z), z.astype(np.int64)
    x = synth.activations(M, K, seed + 1, dt)
    return x, qw, s, qz, zv


@pytest.mark.parametrize("M,K,N,g", [(1, 64, 8, 32), (3, 128, 16, 64), (2, 96, 8, 32)])
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_gemm_ref_equals_bruteforce_loops(M, K, N, g, sym, dt):
    x, qw, s, qz, zv = _tiny_case(M, K, N, g, sym, dt, seed=20 + M + K)
    w_hat = oracle.dequant_affine(qw, s, qz, g, dt)
    y = oracle.gemm_ref(x, w_hat, dt)
    xv = (x.astype(np.float64) if dt == "f16" else oracle.bf16_bits_to_f64(x)).tolist()
    sv = oracle.scale_values(s, dt).tolist()
    if dt == "f16":
        r16 = lambda v: float(np.float16(v))
    else:
        r16 = lambda v: float(oracle.bf16_bits_to_f64(oracle.round_nearest_bf16_bits(np.float64(v))))
    yb = np.array(oracle.gemm_bruteforce(xv, qw.tolist(), sv, zv.tolist(), g, r16))
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-12)


def test_gemm_one_hot_row_returns_the_dequantized_row():
    x, qw, s, qz, _ = _tiny_case(1, 256, 24, 128, False, "f16", seed=30)
    w_hat = oracle.dequant_affine(qw, s, qz, 128)
    for k in (0, 7, 128, 255):
        e = np.zeros((1, 256), np.float16)
        e[0, k] = 1
        assert np.array_equal(oracle.gemm_ref(e, w_hat)[0], w_hat[k].astype(np.float64))


def test_gemm_small_integers_and_power_of_two_scales_exact():
    g = np.random.default_rng(9)
    M, K, N, gs = 3, 128, 16, 32
    q = g.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = g.integers(0, 16, size=(K // gs, N), dtype=np.uint8)
    e = g.integers(2, 6, size=(K // gs, N))
    s = (2.0 ** -e).astype(np.float16)
    xi = g.integers(-4, 5, size=(M, K))
    y = oracle.gemm_ref(xi.astype(np.float16), oracle.dequant_affine(
        oracle.pack_codes(q), s, oracle.pack_zeros(z), gs))
    # exact integer arithmetic: y * 2**5 is an integer
    rows = np.arange(K) // gs
    wi = (q.astype(np.int64) - z[rows]) * (2 ** (5 - e[rows]))
    assert np.array_equal(y * 32, (xi @ wi).astype(np.float64))


def test_gemm_operand_orientation():
    # a transposed or mis-grouped weight changes the product: y[:, n] depends on column n only
    x, qw, s, qz, _ = _tiny_case(2, 128, 16, 32, False, "f16", seed=40)
    w_hat = oracle.dequant_affine(qw, s, qz, 32)
    y = oracle.gemm_ref(x, w_hat)
    y5 = oracle.gemm_ref_columns(x, w_hat[:, 5:6])
    assert np.array_equal(y[:, 5:6], y5)
    assert y.shape == (2, 16)


# ---------------------------------------------------------------- SwiGLU epilogue


def test_silu_closed_forms():
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4, so SiLU(ln 3) = 0.75 ln 3 and
    # SiLU(-ln 3) = -0.25 ln 3; SiLU(0) = 0; SiLU(a) -> a for large a, -> 0 for very negative a
    l3 = np.log(3.0)
    assert abs(oracle.silu(l3) - 0.75 * l3) < 1e-15
    assert abs(oracle.silu(-l3) + 0.25 * l3) < 1e-15
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(40.0) - 40.0) < 1e-15
    assert abs(oracle.silu(-40.0)) < 1e-15
    assert oracle.silu(-1000.0) == 0.0 and np.isfinite(oracle.silu(-1000.0))


def test_silu_odd_part_identity():
    # a*sigmoid(a) - (-a)*sigmoid(-a) = a (sigmoid(a) + sigmoid(-a)) = a, for any a
    a = np.random.default_rng(5).normal(0, 4, 200)
    np.testing.assert_allclose(oracle.silu(a) - oracle.silu(-a), a, rtol=0, atol=1e-12)


def test_swiglu_gate_columns_come_first():
    # one-hot x picks row k of W_hat: gate column = ln 3, up column = 2 -> h = 1.5 ln 3;
    # with the halves swapped it would be SiLU(2) ln 3 = 1.7616 ln 3
    w = np.zeros((4, 4), np.float16)
    w[2, 0], w[2, 2] = np.float16(np.log(3.0)), np.float16(2.0)
    w[1, 1], w[1, 3] = np.float16(0.0), np.float16(5.0)
    x = np.zeros((2, 4), np.float16)
    x[0, 2] = 1
    x[1, 1] = 1
    h = oracle.swiglu_ref(x, w)
    g3 = float(np.float16(np.log(3.0)))
    assert h.shape == (2, 2)
    assert abs(h[0, 0] - 2.0 * g3 / (1.0 + 1.0 / np.exp(g3))) < 1e-15   # 1.5 ln 3 up to fp16(ln 3)
    assert abs(h[0, 0] - 1.5 * np.log(3.0)) < 2e-3
    assert h[1, 1] == 0.0                                                 # gate 0 -> h = 0, up 5
    assert h[0, 1] == 0.0 and h[1, 0] == 0.0


def test_swiglu_bound_covers_first_order_perturbation():
    # perturbing g and u by up to eps*Y moves h by at most the stated bound
    rng = np.random.default_rng(6)
    y = rng.normal(0, 3, (4, 32))
    eps = 1e-3
    Y = np.abs(y).max()
    bound = oracle.swiglu_bound(y, eps)
    g, u = oracle.swiglu_split(y)
    for _ in range(20):
        dg = rng.uniform(-1, 1, g.shape) * eps * Y
        du = rng.uniform(-1, 1, u.shape) * eps * Y
        dh = oracle.silu(g + dg) * (u + du) - oracle.silu(g) * u
        assert np.abs(dh).max() <= bound


# ---------------------------------------------------------------- GPTQ


def test_gptq_pages_two_weight_example():
    # two nearly identical input columns: fixing w1 = 0.26 at 0.30 (0.04 over) moves the still
    # free w2 down by about 0.04 and leaves the output almost unchanged; with orthogonal
    # columns nothing moves ("4.3 Weight-only INT4", section 2.2)
    rng = np.random.default_rng(3)
    x1 = rng.normal(0, 1, 512)
    w = np.array([[0.26], [0.50]])
    for x2, expect in ((x1 + 1e-3 * rng.normal(0, 1, 512), -0.04), (None, 0.0)):
        if x2 is None:
            X = np.zeros((512, 2))
            X[:256, 0] = x1[:256]
            X[256:, 1] = x1[256:]
        else:
            X = np.stack([x1, x2], axis=1)
        Hinv = np.linalg.inv(oracle.hessian(X, damp=0.0))
        W_new, Hinv_next = oracle.compensate(w, np.array([0.30]), Hinv)
        assert W_new[0, 0] == 0.30
        assert abs((W_new[1, 0] - 0.50) - expect) < 1e-3
        assert Hinv_next.shape == (1, 1)
        if x2 is not None:
            # the output moved far less than the 0.04 overshoot alone would move it
            moved = np.linalg.norm(X @ (W_new - w)) / np.linalg.norm(x1)
            assert moved < 0.02 * 0.04


def test_gptq_with_uncorrelated_inputs_is_rtn():
    # diagonal H: no compensation reaches another row, so the codes are the RTN codes
    rng = np.random.default_rng(4)
    K, N = 64, 24
    W = rng.normal(0, 0.02, (K, N))
    X = np.diag(rng.uniform(0.5, 2.0, K))
    q, s, z = oracle.gptq_quantize(W, X, 32)
    qr, sr, zr = oracle.quantize_rtn_asym(W, 32)
    assert np.array_equal(q, qr) and np.array_equal(s, sr) and np.array_equal(z, zr)
    qs, ss = oracle.gptq_quantize(W, X, 32, symmetric=True)
    qsr, ssr = oracle.quantize_rtn_sym(W, 32)
    assert np.array_equal(qs, qsr) and np.array_equal(ss, ssr)


def _correlated_inputs(rng, n, K, rho=0.9):
    C = rho ** np.abs(np.subtract.outer(np.arange(K), np.arange(K)))
    return rng.normal(0, 1, (n, K)) @ np.linalg.cholesky(C).T


@pytest.mark.parametrize("sym", [False, True])
def test_gptq_lowers_the_output_error_against_rtn(sym):
    # the objective of section 2.1: ||X W - X W_hat|| on the calibration inputs
    rng = np.random.default_rng(7 + sym)
    K, N, g = 128, 32, 32
    W = rng.normal(0, 0.02, (K, N))
    X = _correlated_inputs(rng, 512, K)
    if sym:
        q, s = oracle.gptq_quantize(W, X, g, symmetric=True)
        qr, sr = oracle.quantize_rtn_sym(W, g)
        wh = oracle.dequant_sym(oracle.pack_codes(oracle.to_offset_binary(q)), s, g)
        whr = oracle.dequant_sym(oracle.pack_codes(oracle.to_offset_binary(qr)), sr, g)
    else:
        q, s, z = oracle.gptq_quantize(W, X, g)
        qr, sr, zr = oracle.quantize_rtn_asym(W, g)
        wh = oracle.dequant_affine(oracle.pack_codes(q), s, oracle.pack_zeros(z), g)
        whr = oracle.dequant_affine(oracle.pack_codes(qr), sr, oracle.pack_zeros(zr), g)
    e_gptq = np.linalg.norm(X @ (W - wh.astype(np.float64)))
    e_rtn = np.linalg.norm(X @ (W - whr.astype(np.float64)))
    assert e_gptq < 0.7 * e_rtn


def test_gptq_inverse_update_equals_direct_inverse():
    rng = np.random.default_rng(8)
    K, N = 64, 8
    W = rng.normal(0, 0.02, (K, N))
    X = _correlated_inputs(rng, 256, K)
    a = oracle.gptq_quantize(W, X, 32, scale_dtype="bf16")
    b = oracle.gptq_quantize(W, X, 32, scale_dtype="bf16", exact_inverse=True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ---------------------------------------------------------------- AWQ

def test_awq_scaled_activation_rounding_hand_worked():
    # fp16 in [2, 4) has a step of 2/1024. 3 * 1025/1024 = 3 + 1.5 steps: a tie between an
    # odd (1 step) and an even (2 steps) significand -> 3 + 4/1024. 3 * 1027/1024 = 3 + 4.5
    # steps -> the even 4 steps, 3 + 8/1024 (truncation would give the first 3 + 2/1024,
    # round-half-up the second 3 + 10/1024). A power of two is exact.
    x = np.array([[3.0, 3.0, 1.5, -0.75]], dtype=np.float16)
    s = np.array([1025 / 1024, 1027 / 1024, 0.5, 4.0], dtype=np.float16)
    got = oracle.awq.scale_activations(x, s, "f16").astype(np.float64)
    assert got.tolist() == [[3 + 4 / 1024, 3 + 8 / 1024, 0.75, -3.0]]
    # bf16 in [2, 4) has a step of 2/128: 3 * (1 + 1/128) = 3 + 1.5 steps -> 3 + 4/128
    xb = oracle.round_nearest_bf16_bits(np.array([[3.0, -5.0]]))
    sb = oracle.round_nearest_bf16_bits(np.array([1 + 1 / 128, 0.25]))
    gotb = oracle.bf16_bits_to_f64(oracle.awq.scale_activations(xb, sb, "bf16"))
    assert gotb.tolist() == [[3 + 4 / 128, -1.25]]


def test_awq_scaling_is_an_identity_before_quantization():
    # section 3.2: Y = (X S^-1)(S W). S scales the rows of W (input channels), so a slip to
    # columns, or S instead of S^-1 on one side, breaks the identity.
    rng = np.random.default_rng(21)
    K, N = 48, 24
    W = rng.normal(0, 1, (K, N))
    X = rng.normal(0, 1, (16, K))
    s_inv = oracle.round_nearest_f16(rng.uniform(0.2, 5.0, K))
    SW = oracle.awq.scale_weight(W, s_inv)
    XS = X * s_inv.astype(np.float64)[None, :]
    assert np.allclose(XS @ SW, X @ W, rtol=1e-12, atol=1e-12)
    assert not np.allclose(XS @ (W * (1.0 / s_inv.astype(np.float64))[None, :N]), X @ W)


def test_awq_alpha_zero_is_rtn_and_scales_normalised():
    rng = np.random.default_rng(22)
    K, N, g = 64, 16, 32
    W = rng.normal(0, 0.05, (K, N))
    X = rng.normal(0, 1, (128, K)) * rng.uniform(0.1, 10.0, K)[None, :]
    assert np.all(oracle.awq.candidate_scales(X, 0.0) == np.float16(1.0))
    quant, s_inv, alpha, errs = oracle.awq.awq_quantize(W, X, g, n_grid=1)
    assert alpha == 0.0
    for u, v in zip(quant, oracle.quantize_rtn_asym(W, g)):
        assert np.array_equal(u, v)
    # errs[0] is RTN's output error, computed here through the plain GEMM oracle
    q, s, z = oracle.quantize_rtn_asym(W, g)
    wh = oracle.dequant_affine(oracle.pack_codes(q), s, oracle.pack_zeros(z), g)
    X16 = oracle.round_nearest_f16(X)
    e = np.sum((oracle.gemm_ref(X16, W, "f64") - oracle.gemm_ref(X16, wh)) ** 2)
    assert errs[0] == pytest.approx(e, rel=1e-12)
    # s = a ** alpha with max(s) min(s) = 1; larger mean |x| -> larger s -> smaller s_inv
    a = np.mean(np.abs(X), axis=0)
    sv = 1.0 / oracle.awq.candidate_scales(X, 0.5).astype(np.float64)
    assert sv.max() * sv.min() == pytest.approx(1.0, rel=2e-3)
    order = np.argsort(a)
    assert np.all(np.diff(sv[order]) >= -1e-3 * sv[order][1:])
    assert sv[order[-1]] / sv[order[0]] == pytest.approx(np.sqrt(a.max() / a.min()), rel=2e-3)


def test_awq_silent_channel_keeps_a_finite_scale():
    # a channel whose calibration activations are all zero gets the floor 1e-8 of the largest
    # mean |x|, so its scale stays finite and the search still runs (its weight row is scaled
    # down, which costs nothing: it never meets a nonzero activation)
    rng = np.random.default_rng(25)
    X = rng.normal(0, 1, (64, 32))
    X[:, 5] = 0.0
    for alpha in (0.0, 0.5, 0.95):
        s_inv = oracle.awq.candidate_scales(X, alpha).astype(np.float64)
        assert np.all(np.isfinite(s_inv)) and np.all(s_inv > 0)
    assert s_inv[5] == s_inv.max()          # the smallest s, the largest S^-1
    W = rng.normal(0, 0.05, (32, 16))
    quant, s_inv, alpha, errs = oracle.awq.awq_quantize(W, X, 32, n_grid=4)
    assert np.all(np.isfinite(errs)) and min(errs) <= errs[0]


def test_awq_amplified_weight_has_a_smaller_effective_error():
    # section 3.2: with the group's step unchanged, a weight scaled by s before rounding and
    # divided by s after has at most half a step / s of error. The group's range is fixed
    # by two other weights (-1 and 1), so scaling the third by 2 leaves the step alone.
    rng = np.random.default_rng(23)
    w = rng.uniform(-0.45, 0.45, 4000)
    errs = {}
    for s in (1.0, 2.0):
        W = np.stack([np.full_like(w, -1.0), np.full_like(w, 1.0), s * w, np.zeros_like(w)])
        q, sc, z = oracle.quantize_rtn_asym(W, 4, None)
        step = sc[0]
        assert np.allclose(step, 2.0 / 15)
        w_hat = (q[2].astype(np.float64) - z[0]) * step
        errs[s] = np.abs(w_hat / s - w)
        assert np.all(errs[s] <= step / (2 * s) + 1e-12)
    assert errs[1.0].max() > 0.9 * (2.0 / 15) / 2
    assert errs[2.0].mean() < 0.6 * errs[1.0].mean()


@pytest.mark.parametrize("sym,dt", [(False, "f16"), (True, "bf16")])
def test_awq_lowers_the_output_error_against_rtn(sym, dt):
    # section 3.1: the channels with large activations carry the error; protecting them by
    # scaling (3.2) beats RTN on inputs where 1/32 of the channels run 10x larger
    rng = np.random.default_rng(24 + sym)
    K, N, g = 256, 64, 64
    X = rng.normal(0, 1, (256, K))
    X[:, rng.choice(K, K // 32, replace=False)] *= 10.0
    W = rng.normal(0, 0.05, (K, N))
    quant, s_inv, alpha, errs = oracle.awq.awq_quantize(W, X, g, dt, sym)
    assert alpha > 0 and min(errs) == errs[int(round(alpha * 20))]
    assert min(errs) < 0.7 * errs[0]
    # the returned codes reproduce the chosen error through the plain dequant + GEMM oracle
    if sym:
        q, s = quant
        wh = oracle.dequant_sym(oracle.pack_codes(oracle.to_offset_binary(q)), s, g, dt)
    else:
        q, s, z = quant
        wh = oracle.dequant_affine(oracle.pack_codes(q), s, oracle.pack_zeros(z), g, dt)
    Xq = oracle.round_nearest_f16(X) if dt == "f16" else oracle.round_nearest_bf16_bits(X)
    y = oracle.gemm_ref(oracle.awq.scale_activations(Xq, s_inv, dt), wh, dt)
    y0 = (Xq.astype(np.float64) if dt == "f16" else oracle.bf16_bits_to_f64(Xq)) @ W
    assert np.sum((y - y0) ** 2) == pytest.approx(min(errs), rel=1e-9)


# ---------------------------------------------------------------- W4A8

def test_w4a8_activation_codes_hand_worked():
    # a row whose largest magnitude is 127 has sx = 1 exactly, so the codes are rint(x):
    # 63.5 -> 64 and 2.5 -> 2 (ties to even), -0.5 -> -0, 127 -> 127
    x = np.array([[127.0, 63.5, -0.5, 2.5, -1.25], [0.0, 0.0, 0.0, 0.0, 0.0]], dtype=np.float16)
    xq, sx = oracle.w4a8.quantize_act_int8(x, "f16")
    assert sx.dtype == np.float32 and sx.tolist() == [1.0, 0.0]
    assert xq.tolist() == [[127, 64, 0, 2, -1], [0, 0, 0, 0, 0]]
    # a negative extreme maps to -127, and the scale is the fp32 quotient max|x| / 127
    xb = oracle.round_nearest_bf16_bits(np.array([[-3.0, 1.5, 0.75]]))
    xq, sx = oracle.w4a8.quantize_act_int8(xb, "bf16")
    assert sx[0] == np.float32(3.0) / np.float32(127.0)
    assert xq.tolist() == [[-127, 64, 32]]   # 1.5 / (3/127) = 63.5 -> 64; 31.75 -> 32


def test_w4a8_activation_error_at_most_half_a_step():
    x = synth.activations(8, 512, seed=41, dtype="f16")
    xq, sx = oracle.w4a8.quantize_act_int8(x, "f16")
    err = np.abs(x.astype(np.float64) - xq.astype(np.float64) * sx.astype(np.float64)[:, None])
    # half a step, plus the fp32 rounding of the quotient (half an ulp of |x| / sx, times sx)
    assert np.all(err <= 0.5 * sx[:, None] + 2.0 ** -24 * np.abs(x.astype(np.float64)) * (1 + 1e-9))
    assert (err / sx[:, None]).max() > 0.45
    assert np.all(np.abs(xq).max(axis=1) == 127)


def test_w4a8_integer_product_is_exact_bruteforce():
    rng = np.random.default_rng(42)
    M, K, N = 3, 16, 8
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    q = rng.integers(-8, 8, (K, N)).astype(np.int8)
    got = oracle.w4a8.int_gemm(xq, q)
    for m in range(M):
        for n in range(N):
            assert got[m, n] == sum(int(xq[m, k]) * int(q[k, n]) for k in range(K))
    # the extreme: every term 127 * -8 (or -127 * -8) over a long K stays exact
    big = oracle.w4a8.int_gemm(np.full((1, 4096), -127, np.int8), np.full((4096, 1), -8, np.int8))
    assert big[0, 0] == 4096 * 1016


def test_w4a8_signed_codes_from_offset_binary():
    u = np.arange(16, dtype=np.uint8).reshape(16, 1)
    q = oracle.w4a8.signed_codes(oracle.pack_codes(np.vstack([u, u])))
    assert q[:16, 0].tolist() == list(range(-8, 8))


def test_w4a8_reference_equals_python_loops():
    # the whole W4A8 reference (per-token codes, unpacked offset-binary weights, integer sum,
    # both scales) against plain Python arithmetic on a tiny case
    rng = np.random.default_rng(46)
    M, K, N = 3, 16, 8
    x = rng.normal(0, 1, (M, K)).astype(np.float16)
    u = rng.integers(0, 16, (K, N)).astype(np.uint8)
    sw = np.array(rng.uniform(0.01, 0.02, N), dtype=np.float16)
    y = oracle.w4a8.gemm_w4a8_ref(x, oracle.pack_codes(u), sw, "f16")
    for m in range(M):
        xs = [float(v) for v in x[m]]
        sx = float(np.float32(max(abs(v) for v in xs)) / np.float32(127))
        q = [max(-127, min(127, int(np.rint(np.float32(v) / np.float32(sx))))) for v in xs]
        for n in range(N):
            acc = sum(q[k] * (int(u[k, n]) - 8) for k in range(K))
            assert y[m, n] == acc * sx * float(sw[n])


def test_w4a8_reduces_to_w4a16_when_x_is_on_the_int8_grid():
    # x = sx * xq exactly (integers with max 127, sx = 1) and power-of-two weight scales:
    # the W4A8 result equals the W4A16 oracle on the per-channel-scaled weight
    rng = np.random.default_rng(43)
    K, N = 64, 16
    x = rng.integers(-127, 128, (4, K)).astype(np.float16)
    x[:, 0] = 127
    W = rng.normal(0, 0.05, (K, N))
    q, s = oracle.quantize_rtn_sym(W, K, "f16")
    s = np.float16(2.0) ** np.rint(np.log2(s.astype(np.float64))).astype(np.float16)
    qw = oracle.pack_codes(oracle.to_offset_binary(q))
    y8 = oracle.w4a8.gemm_w4a8_ref(x, qw, s, "f16")
    y16 = oracle.gemm_ref(x, oracle.dequant_sym(qw, s, K))
    assert np.array_equal(y8, y16)


def test_w4a8_error_within_the_activation_quantization_bound():
    # |y_w4a8 - x W_hat| <= sum_k |x - sx xq| |W_hat| <= sx / 2 * sum_k |W_hat[k, n]|
    x = synth.activations(6, 256, seed=44, dtype="bf16")
    W = synth.gaussian_weight(256, 32, seed=45)
    q, s = oracle.quantize_rtn_sym(W, 256, "bf16")
    qw = oracle.pack_codes(oracle.to_offset_binary(q))
    w_hat = oracle.bf16_bits_to_f64(oracle.dequant_sym(qw, s, 256, "bf16"))
    y8 = oracle.w4a8.gemm_w4a8_ref(x, qw, s, "bf16")
    y16 = oracle.bf16_bits_to_f64(x) @ w_hat
    _, sx = oracle.w4a8.quantize_act_int8(x, "bf16")
    bound = 0.5 * sx.astype(np.float64)[:, None] * np.abs(w_hat).sum(axis=0)[None, :]
    # the integer result times the stored scales is W_hat's own product up to the one rounding
    # of each W_hat entry to bf16 (relative 2**-9)
    slack = 2.0 ** -8 * np.abs(oracle.bf16_bits_to_f64(x)) @ np.abs(w_hat)
    assert np.all(np.abs(y8 - y16) <= bound + slack)
    assert np.max(np.abs(y8 - y16) / bound) > 0.02


# ---------------------------------------------------------------- NF4

def test_inverse_normal_matches_library():
    special = pytest.importorskip("scipy.special")
    for p in (0.5, 0.6, 0.75, 0.9, 0.96875, 0.01, 1e-6):
        assert abs(oracle.inverse_normal_cdf(p) - special.ndtri(p)) < 1e-12


def test_nf4_codebook_structure_and_quantiles():
    special = pytest.importorskip("scipy.special")
    c = oracle.nf4_codebook()
    assert c.dtype == np.float16 and c.shape == (16,)
    assert np.all(np.diff(c.astype(np.float64)) > 0)
    assert c[0] == -1 and c[15] == 1 and np.sum(c == 0) == 1 and c[7] == 0
    p_end = 1 - 1 / 32
    top = special.ndtri(p_end)
    pos = special.ndtri(np.linspace(0.5, p_end, 9)[1:]) / top
    neg = -special.ndtri(np.linspace(0.5, p_end, 8)[1:]) / top
    assert np.array_equal(c[8:], pos.astype(np.float16))
    assert np.array_equal(c[:7], np.sort(neg).astype(np.float16))


def test_nf4_codebook_matches_frozen_fixture():
    vals = np.loadtxt(os.path.join(GOLDEN, "nf4_codebook.txt"), dtype=np.float64)
    assert np.array_equal(oracle.nf4_codebook().astype(np.float64), vals)


def test_nf4_quantizer_picks_nearest_level_and_dequant():
    c = oracle.nf4_codebook()
    W = synth.gaussian_weight(128, 8, seed=16)
    codes, a = oracle.quantize_nf4(W, c, 64)
    cv = c.astype(np.float64)
    av = a.astype(np.float64)
    r = W.astype(np.float64) / np.repeat(av, 64, 0)
    assert np.all(np.abs(r) <= 1)
    for k in range(0, 128, 7):
        for n in range(8):
            d = np.abs(r[k, n] - cv)
            assert codes[k, n] == int(np.argmin(d))
    w = oracle.dequant_nf4(oracle.pack_codes(codes), np.ones((2, 8), np.float16), c, 64)
    assert np.array_equal(w, cv[codes].astype(np.float16))           # a = 1 -> the level
    w2 = oracle.dequant_nf4(oracle.pack_codes(codes), np.full((2, 8), 2, np.float16), c, 64)
    assert np.array_equal(w2.astype(np.float64), 2 * cv[codes])      # a = 2 -> exact double


def test_nf4_dequant_block_index_hand_worked():
    """"INT4 and Low-Bit Inference", section 5 (The formats): NF4 scales each block of 64
    consecutive weights by its own absmax. Hand-worked: one column, two blocks with absmax
    0.5 and 4; the codes at both ends of each block are the extreme levels (code 15 = +1,
    code 0 = -1) or the zero level (code 7)."""
    c = oracle.nf4_codebook()
    codes = np.full((128, 1), 7, np.uint8)
    codes[0, 0], codes[63, 0], codes[64, 0], codes[127, 0] = 15, 0, 15, 0
    a = np.array([[0.5], [4.0]], np.float16)
    w = oracle.dequant_nf4(oracle.pack_codes(codes), a, c, 64).astype(np.float64)[:, 0]
    assert (w[0], w[63], w[64], w[127]) == (0.5, -0.5, 4.0, -4.0)
    assert np.all(w[1:63] == 0) and np.all(w[65:127] == 0)


@pytest.mark.parametrize("block", [32, 64, 128])
def test_nf4_dequant_absmax_per_block_and_column(block):
    """Every (block, column) gets a distinct power-of-two absmax; with code 15 (level +1)
    everywhere, W_hat must repeat each absmax over exactly the `block` consecutive k of its
    block, in its own column (a power of two times +1 is exact)."""
    c = oracle.nf4_codebook()
    K, N = 4 * block, 8
    codes = np.full((K, N), 15, np.uint8)
    e = np.arange(4)[:, None] * N + np.arange(N)[None, :]           # 32 distinct exponents
    a = np.ldexp(1.0, e - 16).astype(np.float16)                    # 2^-16 .. 2^15
    assert len(np.unique(a)) == 4 * N
    w = oracle.dequant_nf4(oracle.pack_codes(codes), a, c, block).astype(np.float64)
    for b in range(4):
        for n in range(N):
            assert np.all(w[b * block:(b + 1) * block, n] == float(a[b, n])), (b, n)


# ---------------------------------------------------------------- roofline arithmetic

def test_naive_path_bytes_and_ceiling():
    p = printed()["naive_path"]
    assert roofline.naive_bytes_per_weight() == p["bytes_per_weight"]
    assert 2.0 / 0.5 == p["ceiling"]


def test_llama3_70b_decode_floors():
    rows = printed()["llama3_70b_decode_floor_h100"]["rows"]
    bw = rows[0]["weight_GB"] * 1e9 / (rows[0]["floor_ms"] * 1e-3)   # one bandwidth for all
    for r in rows:
        t = roofline.decode_floor(r["weight_GB"] * 1e9, 1.0, bw) * 1e3
        assert abs(t - r["floor_ms"]) / r["floor_ms"] < 0.01
    assert abs(rows[0]["floor_ms"] / 2 - rows[0]["floor_tp2_ms"]) < 1e-9
    # INT4 bytes are a quarter of BF16 bytes to the printed precision
    assert abs(rows[0]["weight_GB"] / 4 - rows[2]["weight_GB"]) / rows[2]["weight_GB"] < 0.01


def test_worked_example_8b_crossover():
    p = printed()["worked_example_8b"]
    P, bw, peak, peak8 = p["params"], p["bandwidth_Bps"], p["fp16_flops"], p["int8_ops"]
    bpw4 = oracle.bytes_per_weight(128, zeros=False)
    assert bpw4 * 8 == p["w4a16_bits"]
    assert close_to_printed(P * bpw4 / 1e9, p["w4a16_GB"], 1)
    floors = {k: roofline.decode_floor(P, b, bw) * 1e3 for k, b in
              (("fp16", 2.0), ("w8a8", 1.0), ("w4a16", bpw4))}
    for k, v in p["floor_ms"].items():
        assert close_to_printed(floors[k], v, 1)
    for k in ("fp16", "w8a8"):
        assert abs(1e3 / floors[k] - p["tokens_per_s_batch1"][k]) < 1e-9
    assert abs(1e3 / floors["w4a16"] - p["tokens_per_s_batch1"]["w4a16"]) / 480 < 0.02
    assert abs(roofline.step_compute(P, 1, peak) * 1e3 - p["compute_ms_per_batch"]["w4a16"]) < 1e-12
    assert abs(roofline.step_compute(P, 1, peak8) * 1e3 - p["compute_ms_per_batch"]["w8a8"]) < 1e-12
    b4 = roofline.crossover_batch(bpw4, bw, peak)
    b8 = roofline.crossover_batch(1.0, bw, peak8)
    assert int(b4) == p["compute_bound_near_batch"]["w4a16"]            # 51.56
    assert abs(b8 - p["compute_bound_near_batch"]["w8a8"]) < 1e-9
    # W4A16 compute time meets W8A8's flat memory floor
    cross = floors["w8a8"] / (roofline.step_compute(P, 1, peak) * 1e3)
    assert abs(cross - p["lines_cross_near_batch"]) < 1e-9
    for k, pk in (("w4a16", peak), ("w8a8", peak8)):
        t = roofline.t_roof(0, 2 * P * 256, bw, pk) * 1e3
        assert close_to_printed(t, p["batch256_ms"][k], 1)
    assert roofline.algo_bytes(1, 4096, 4096, 128) == 4096 * 2048 + 32 * 4096 * 2 + 32 * 2048 + 8192 + 8192
