"""GPU parity: the HIP path through the C ABI against the CPU oracle.

* dequantized weights: bit-exact (uint16 patterns) on ragged shapes, every format;
* GEMM: max|y - y_ref| <= 1e-3 max|y_ref| (fp64 oracle), element by element on sizes
  the oracle finishes in seconds (several strips, ragged M and K), and on sampled
  16-column strips at the full sizes of the benchmarked workloads;
* exact special cases: one-hot rows reproduce W_hat bit for bit, power-of-two scales with
  small-integer activations give exact sums; bf16 output equals RNE of fp32 output;
  repeated runs are bit-identical.
"""
import numpy as np
import pytest

import oracle
from weight_only_int4_w4a16_amd import synth

from gpu_common import (assert_close, device_inputs, from_dev, oracle_columns, out_values, run_swiglu,
                        require_gpu, rtn_case, run_gemm, sample_strips, to_dev, torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _announce(msg):
    print(f"[case] {msg}", flush=True)


# ------------------------------------------------------------------ bit-exact dequant

@pytest.mark.parametrize("K,N,g,act,fmt", [
    (256, 32, 128, "f16", "asym"),
    (352, 48, 32, "f16", "asym"),      # ragged K: last 128-block has 3 of 4 steps
    (320, 64, 64, "f16", "asym"),
    (384, 16, 128, "f16", "sym"),
    (4096, 4096, 128, "f16", "asym"),  # the single-GEMV workload, whole matrix
    (288, 32, 32, "bf16", "asym"),
    (512, 48, 128, "bf16", "sym"),
    (448, 32, 64, "f16", "nf4"),
    (256, 32, 64, "bf16", "nf4"),
])
def test_dequant_bit_exact(K, N, g, act, fmt):
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    _announce(f"dequant K={K} N={N} g={g} {act} {fmt}")
    c = rtn_case(1, K, N, g, act, sym=(fmt == "sym"), seed=K + N, nf4=(fmt == "nf4"))
    d = device_inputs(c)
    if fmt == "nf4":
        wt = w4.dequant_nf4(d["packed"], d["scales"], d["codebook"], K, g,
                            torch.float16 if act == "f16" else torch.bfloat16)
    else:
        wt = w4.dequant(d["packed"], d["scales"], d["qzeros"], K, g)
    torch.cuda.synchronize()
    got = from_dev(wt)
    exp = c["w_hat"]
    got_bits = got.view(np.uint16) if got.dtype == np.float16 else got
    exp_bits = exp.view(np.uint16) if exp.dtype == np.float16 else exp
    bad = np.argwhere(got_bits != exp_bits)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"


# ------------------------------------------------------------------ small GEMMs, all outputs

SMALL = [
    # M, K, N, g, act, fmt
    (1, 512, 256, 128, "f16", "asym"),
    (3, 352, 48, 32, "f16", "asym"),
    (16, 1024, 128, 64, "f16", "asym"),
    (17, 512, 64, 128, "f16", "asym"),
    (33, 256, 96, 32, "f16", "asym"),
    (64, 512, 64, 128, "f16", "asym"),
    (100, 384, 80, 128, "f16", "asym"),
    (1, 1024, 64, 128, "f16", "sym"),
    (8, 640, 32, 128, "f16", "sym"),
    (1, 512, 64, 128, "bf16", "asym"),
    (5, 288, 48, 32, "bf16", "asym"),
    (40, 512, 32, 64, "bf16", "sym"),
    (1, 512, 64, 64, "f16", "nf4"),
    (12, 448, 48, 64, "f16", "nf4"),
    (2, 256, 32, 64, "bf16", "nf4"),
    (70, 256, 32, 64, "f16", "nf4"),
    # decode launches with activations too large for LDS (16 rows of 8192 k: 256 KiB)
    (16, 8192, 32, 128, "f16", "asym"),
    (16, 8192, 64, 64, "f16", "nf4"),       # fp16 NF4 levels gathered per word (no nibble-order x)
    (9, 4224, 48, 64, "bf16", "sym"),
    (16, 8320, 32, 32, "f16", "asym"),
    (16, 1024, 48, 64, "bf16", "asym"),
    # 17..32 rows on small weights (K N <= 2^24): the decode kernel, one launch per 16 rows
    (17, 512, 64, 128, "bf16", "asym"),
    (32, 1024, 48, 64, "bf16", "asym"),
    (20, 8320, 32, 32, "f16", "asym"),
    # just past 16 rows on larger weights: one ragged 64-row tile of the batched kernel
    (17, 4096, 4112, 128, "f16", "asym"),
    (24, 2048, 8208, 64, "bf16", "sym"),
    (50, 8192, 32, 128, "f16", "asym"),
    # persistent decode workgroups (more tiles than resident slots, x staged once): one and
    # two strips per tile, waves with one group and with several, a ragged K, g32
    (16, 4096, 16416, 128, "f16", "asym"),
    (13, 3968, 16432, 128, "bf16", "asym"),
    (12, 4224, 32784, 64, "bf16", "sym"),
    (15, 2080, 32784, 32, "f16", "asym"),
    (12, 4096, 16416, 128, "f16", "sym"),
    (8, 4096, 32784, 32, "f16", "asym"),
    # 4..16 rows on the skinny kernel (one round of workgroups filling more than half the chip)
    (4, 2048, 8704, 32, "f16", "asym"),
    (5, 1024, 9216, 64, "f16", "nf4"),
    (8, 4096, 10240, 128, "bf16", "sym"),
    (4, 2048, 12288, 64, "bf16", "nf4"),
    (4, 2048, 20480, 32, "f16", "asym"),     # groups of 32 over one to two rounds of tiles
    (12, 4096, 6144, 64, "bf16", "nf4"),     # a quarter to a half of the chip's column tiles
    # groups of 32 and 64 with four-block pipeline groups (one scale and zero word per block
    # and strip, shared between the lanes of a column): waves with several groups, a ragged
    # last group, two-strip SwiGLU-free tiles at g128 beside them
    (1, 4096, 64, 32, "f16", "asym"),
    (1, 6016, 48, 32, "bf16", "asym"),
    (4, 8192, 48, 32, "f16", "sym"),
    (2, 4096, 32, 64, "f16", "asym"),
    (1, 2944, 64, 32, "f16", "nf4"),
    (6, 4096, 80, 64, "bf16", "nf4"),
    # the smallest shapes: one 32-k step, one 16-column strip
    (1, 32, 16, 32, "f16", "asym"),
    (7, 64, 16, 64, "bf16", "sym"),
    (33, 32, 16, 32, "f16", "asym"),
    (17, 32, 16, 32, "f16", "sym"),
    (40, 96, 16, 32, "bf16", "nf4"),
    # batched kernel (M > 16): ragged M, N not a multiple of the 512-column tile, ragged K,
    # and K long enough to be split across workgroups (K >= 2048)
    (65, 256, 48, 128, "f16", "asym"),
    (128, 384, 272, 32, "f16", "asym"),
    (200, 2048, 64, 128, "f16", "asym"),
    (130, 2144, 96, 32, "bf16", "asym"),
    (97, 2080, 48, 32, "f16", "sym"),
    (256, 512, 256, 64, "f16", "nf4"),
    (300, 1024, 128, 128, "bf16", "sym"),
    (129, 2048, 32, 64, "bf16", "nf4"),
    # skinny kernel (17..64 rows; K split across eight waves, reduced in LDS): uneven wave
    # slices with idle waves (33 and 9 k-blocks), ragged K, a ragged last column tile (17 and
    # 9 strips), one and two 32-row tiles, every format
    (24, 4224, 4112, 32, "f16", "asym"),
    (48, 1152, 272, 64, "f16", "nf4"),
    (64, 2080, 144, 32, "bf16", "asym"),
    (37, 640, 80, 64, "bf16", "sym"),
    (61, 4096, 48, 128, "f16", "sym"),
    (18, 2048, 8208, 128, "bf16", "nf4"),
    # skinny kernel over several launch rounds: one k-block per wave (a slice shorter than a
    # pass of the two-set pipeline), and waves without blocks beside a ragged column tile
    (30, 1024, 20480, 64, "f16", "asym"),
    (25, 1152, 16400, 32, "bf16", "sym"),
    # skinny kernel with 128-row tiles (four waves, where 64-row tiles would need a second
    # launch round): ragged M, a ragged K split 3/3/3/0 over the waves, every format
    (96, 512, 8256, 128, "f16", "asym"),
    (80, 1152, 8704, 32, "bf16", "sym"),
    (128, 640, 8256, 64, "f16", "nf4"),
    # skinny kernel on 4608-deep weights with 128-row tiles, from 224 rows on 128-row tiles
    # (two of them, the second ragged), 16 rows on a fifth of the chip's worth of column tiles
    (100, 4608, 8320, 128, "f16", "asym"),
    (240, 3584, 6144, 64, "f16", "nf4"),
    (168, 4096, 6208, 32, "bf16", "asym"),
    (176, 5120, 4096, 128, "bf16", "asym"),
    (16, 3072, 5120, 32, "f16", "sym"),
    # skinny kernel past 128 rows (one round of 64-row tiles): a ragged last row tile
    (160, 768, 3072, 128, "f16", "asym"),
    (256, 1024, 4096, 64, "bf16", "nf4"),
    # medium tile (128 x 128, two k-groups, one strip pair per wave): groups of 32 or 64 and
    # NF4 from 192 rows on; a ragged last row tile, an odd block count split over the two
    # k-groups, a ragged K
    (200, 1024, 8192, 32, "f16", "asym"),
    (256, 1152, 8192, 64, "f16", "nf4"),
    (224, 640, 8192, 32, "bf16", "sym"),
    (208, 1184, 8192, 32, "f16", "asym"),
]


@pytest.mark.parametrize("M,K,N,g,act,fmt", SMALL)
def test_gemm_small_all_outputs(M, K, N, g, act, fmt):
    torch = torch_mod()
    _announce(f"gemm M={M} K={K} N={N} g={g} {act} {fmt}")
    c = rtn_case(M, K, N, g, act, sym=(fmt == "sym"), seed=7 * M + K, nf4=(fmt == "nf4"))
    d = device_inputs(c)
    y_ref = oracle.gemm_ref(c["x"], c["w_hat"], act)
    y32 = run_gemm(c, d, out_dtype=torch.float32)
    assert_close(from_dev(y32).astype(np.float64), y_ref, "fp32 out")
    y16 = run_gemm(c, d)
    if act == "f16":
        assert_close(out_values(from_dev(y16), torch.float16), y_ref, "fp16 out")
    else:
        # bf16 output is the nearest-even rounding of the same fp32 accumulation
        exp = oracle.round_nearest_bf16_bits(from_dev(y32).astype(np.float64))
        assert np.array_equal(from_dev(y16), exp)


# SwiGLU epilogue on a fused gate+up weight [K, N2]: decode (x in LDS and not, persistent
# workgroups, one and several groups per wave) and batched (both tiles, with and without a
# K split), every format
SWIGLU = [
    (1, 512, 64, 128, "f16", "asym"),
    (3, 352, 96, 32, "bf16", "asym"),
    (16, 1024, 128, 64, "f16", "sym"),
    (5, 14336, 64, 64, "f16", "asym"),       # x from global (too large for LDS at 5 rows)
    (12, 4096, 16416, 128, "f16", "asym"),   # persistent, one group per wave
    (9, 4224, 32832, 64, "bf16", "nf4"),     # persistent, several groups per wave
    (2, 1024, 96, 64, "bf16", "nf4"),
    (4, 1024, 96, 64, "f16", "nf4"),         # fp16 NF4, x in LDS in nibble order, SwiGLU tile
    (17, 512, 64, 128, "bf16", "asym"),      # decode, two launches (16 + 1 rows)
    (20, 4096, 4128, 128, "bf16", "asym"),   # batched 64x256, K split
    (130, 2144, 96, 32, "f16", "sym"),
    (300, 1024, 544, 128, "f16", "asym"),    # batched 64x256, ragged tile
    (257, 2080, 2080, 32, "f16", "nf4"),
    (513, 2080, 16416, 32, "bf16", "asym"),  # batched 128x512
    (48, 1024, 96, 64, "f16", "nf4"),        # skinny, two row tiles, ragged gate half
    (33, 2176, 160, 128, "bf16", "sym"),     # skinny, ragged K
    (8, 2048, 10240, 128, "bf16", "sym"),    # skinny at 8 rows (its workgroups fill the chip)
    (96, 1024, 8320, 128, "f16", "asym"),    # skinny, 128-row tile
    (150, 1024, 4096, 64, "f16", "nf4"),     # skinny past 128 rows, ragged last row tile
]


@pytest.mark.parametrize("M,K,N2,g,act,fmt", SWIGLU)
def test_swiglu_all_outputs(M, K, N2, g, act, fmt):
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    _announce(f"swiglu M={M} K={K} N2={N2} g={g} {act} {fmt} kernel={w4.kernel_name(M, K, N2, g)}")
    c = rtn_case(M, K, N2, g, act, sym=(fmt == "sym"), seed=11 * M + K, nf4=(fmt == "nf4"))
    d = device_inputs(c)
    y_ref = oracle.gemm_ref(c["x"], c["w_hat"], act)
    h_ref = oracle.swiglu_ref(c["x"], c["w_hat"], act)
    bound = oracle.swiglu_bound(y_ref)
    h32 = from_dev(run_swiglu(c, d, out_dtype=torch.float32)).astype(np.float64)
    assert h32.shape == (M, N2 // 2)
    assert np.all(np.isfinite(h32))
    err = np.max(np.abs(h32 - h_ref))
    assert err <= bound, f"fp32 out: max|h - h_ref| = {err:.3e} > {bound:.3e}"
    # 16-bit output: the same fp32 value rounded once to the activation type
    h16 = from_dev(run_swiglu(c, d))
    if act == "f16":
        assert np.array_equal(h16.view(np.uint16), h32.astype(np.float32).astype(np.float16).view(np.uint16))
    else:
        assert np.array_equal(h16, oracle.round_nearest_bf16_bits(h32))


def test_swiglu_gate_and_up_halves():
    """One-hot rows: h is SiLU of the gate half's dequantized row times the up half's."""
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    for M in (4, 40):   # decode and batched
        c = rtn_case(M, 256, 64, 64, "f16", seed=21 + M)
        x = np.zeros((M, 256), np.float16)
        for m in range(M):
            x[m, (37 * m) % 256] = 1
        c["x"] = x
        d = device_inputs(c)
        h = from_dev(run_swiglu(c, d, out_dtype=torch.float32)).astype(np.float64)
        rows = c["w_hat"].astype(np.float64)[[(37 * m) % 256 for m in range(M)]]
        h_ref = oracle.silu(rows[:, :32]) * rows[:, 32:]
        assert np.max(np.abs(h - h_ref)) <= 1e-6 * max(1.0, np.max(np.abs(h_ref)))


def test_swiglu_rejects_odd_strip_halves():
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    c = rtn_case(2, 256, 48, 64, "f16", seed=5)   # N2 = 48: halves of 24 columns
    d = device_inputs(c)
    with pytest.raises(w4.W4A16Error):
        run_swiglu(c, d)


@pytest.mark.parametrize("M,K,N,g,sym", [(1, 512, 256, 128, False), (8, 1024, 128, 32, True),
                                         (96, 512, 192, 64, False)])
def test_gptq_codes_end_to_end(M, K, N, g, sym):
    """Weights quantized by the oracle's GPTQ on correlated calibration inputs run through the
    same kernels: parity with the oracle GEMM, and on the calibration rows the GPU output is
    closer to x W than the RTN weights' GPU output ("4.3 Weight-only INT4", section 2.1)."""
    torch = torch_mod()
    _announce(f"gptq M={M} K={K} N={N} g={g} sym={sym}")
    rng = np.random.default_rng(M + K)
    W = synth.gaussian_weight(K, N, 90 + M)
    C = 0.9 ** np.abs(np.subtract.outer(np.arange(K), np.arange(K)))
    X = rng.normal(0, 1, (max(4 * K, 256), K)) @ np.linalg.cholesky(C).T
    x = X[:M].astype(np.float16)
    errs = []
    for quant in ("gptq", "rtn"):
        if sym:
            q, s = (oracle.gptq_quantize(W, X, g, symmetric=True) if quant == "gptq"
                    else oracle.quantize_rtn_sym(W, g))
            qw, qz = oracle.pack_codes(oracle.to_offset_binary(q)), None
            w_hat = oracle.dequant_sym(qw, s, g)
        else:
            q, s, z = oracle.gptq_quantize(W, X, g) if quant == "gptq" else oracle.quantize_rtn_asym(W, g)
            qw, qz = oracle.pack_codes(q), oracle.pack_zeros(z)
            w_hat = oracle.dequant_affine(qw, s, qz, g)
        c = {"M": M, "K": K, "N": N, "g": g, "act": "f16", "x": x, "nf4": False,
             "qweight": qw, "scales": s, "qzeros": qz}
        y = from_dev(run_gemm(c, device_inputs(c), out_dtype=torch.float32)).astype(np.float64)
        assert_close(y, oracle.gemm_ref(x, w_hat), f"{quant} codes")
        errs.append(np.linalg.norm(y - x.astype(np.float64) @ W))
    assert errs[0] < errs[1], f"GPTQ output error {errs[0]:.4g} not below RTN {errs[1]:.4g}"


def test_gemm_m0_is_noop():
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    c = rtn_case(1, 256, 32, 128)
    d = device_inputs(c)
    x0 = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    y = w4.gemm(x0, d["packed"], d["scales"], d["qzeros"], 128)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)


# ------------------------------------------------------------------ exact special cases

@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_one_hot_rows_reproduce_w_hat_exactly(act):
    torch = torch_mod()
    _announce(f"one-hot {act}")
    K, N = 384, 64
    c = rtn_case(1, K, N, 128, act, seed=99)
    ks = np.array([0, 1, 7, 8, 127, 128, 200, 383])
    x = np.zeros((len(ks), K), np.float32)
    x[np.arange(len(ks)), ks] = 1.0
    c["x"] = x.astype(np.float16) if act == "f16" else synth.f32_to_bf16_bits(x)
    c["M"] = len(ks)
    d = device_inputs(c)
    y = from_dev(run_gemm(c, d))
    exp = c["w_hat"][ks]
    assert np.array_equal(y.view(np.uint16) if act == "f16" else y,
                          exp.view(np.uint16) if act == "f16" else exp)


def test_power_of_two_scales_integer_activations_exact():
    torch = torch_mod()
    _announce("pow2 exact")
    rng = np.random.default_rng(5)
    M, K, N, g = 7, 1024, 64, 32
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    e = rng.integers(3, 7, size=(K // g, N))
    s = (2.0 ** -e).astype(np.float16)
    xi = rng.integers(-3, 4, size=(M, K))
    c = {"M": M, "K": K, "N": N, "g": g, "act": "f16", "nf4": False,
         "x": xi.astype(np.float16), "qweight": oracle.pack_codes(q), "scales": s,
         "qzeros": oracle.pack_zeros(z)}
    d = device_inputs(c)
    y = from_dev(run_gemm(c, d, out_dtype=torch.float32)).astype(np.float64)
    w_hat = oracle.dequant_affine(c["qweight"], s, c["qzeros"], g)
    y_ref = oracle.gemm_ref(c["x"], w_hat)
    # every partial sum is a multiple of 2**-6 below 2**24 * 2**-6: exact in fp32
    assert np.array_equal(y, y_ref)


def test_repeat_runs_are_bit_identical():
    torch = torch_mod()
    c = rtn_case(16, 2048, 256, 128, seed=3)
    d = device_inputs(c)
    a = from_dev(run_gemm(c, d, out_dtype=torch.float32))
    b = from_dev(run_gemm(c, d, out_dtype=torch.float32))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("M,K,N,g", [(1, 28672, 512, 128), (4, 28672, 256, 128), (16, 14336, 256, 32)])
def test_large_activation_channels(M, K, N, g):
    """"4.3 Weight-only INT4", section 3.1: a few input channels carry activations far above the
    rest. One channel in 32 is scaled by 10..100 (so |x| reaches several hundred) on the fp16
    decode path, which multiplies the exact integers 1024 + q and -(1024 + z) and cancels them
    in fp32 sums before each group's scale (about ten bits of the 24 cancel): every output stays
    within the 1e-3 max|y_ref| bound of the fp64 oracle."""
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    _announce(f"large channels M={M} K={K} N={N} g={g} kernel={w4.kernel_name(M, K, N, g)}")
    c = rtn_case(M, K, N, g, "f16", seed=K + N + M)
    x = c["x"].astype(np.float64)
    ch = np.arange(7, K, 32)
    x[:, ch] *= np.linspace(10.0, 100.0, len(ch))[None, :]
    c["x"] = x.astype(np.float16)
    assert np.max(np.abs(c["x"].astype(np.float64))) > 200
    d = device_inputs(c)
    y_ref = oracle.gemm_ref(c["x"], c["w_hat"])
    y = from_dev(run_gemm(c, d, out_dtype=torch.float32)).astype(np.float64)
    assert_close(y, y_ref, "fp32 out, outlier channels")


# ------------------------------------------------------------------ the single-GEMV workload

def test_single_gemv_4096x4096_all_outputs():
    """x fp16 [1,4096], W [4096,4096] ~ N(0, 0.02) asymmetric g128: every output."""
    torch = torch_mod()
    _announce("single GEMV 4096x4096")
    c = rtn_case(1, 4096, 4096, 128, "f16", seed=synth.seed_for(1, 0, 0))
    d = device_inputs(c)
    y_ref = oracle.gemm_ref(c["x"], c["w_hat"])
    assert_close(out_values(from_dev(run_gemm(c, d)), torch.float16), y_ref, "fp16 out")
    assert_close(from_dev(run_gemm(c, d, torch.float32)).astype(np.float64), y_ref, "fp32 out")


# ------------------------------------------------------------------ full sizes, sampled strips

FULL = []
for (K, N) in ((4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096)):   # 8B-shaped, g128
    for M in (1, 4, 16):
        FULL.append((M, K, N, 128, "f16", "asym"))
for (K, N) in ((8192, 10240), (8192, 8192), (8192, 57344), (28672, 8192)):  # 70B-shaped, sym
    for M in (1, 8, 32):
        FULL.append((M, K, N, 128, "f16", "sym"))
for M in (1, 2, 4, 8, 16, 32, 64, 128, 256):                                # crossover sweep
    FULL.append((M, 4096, 14336, 128, "f16", "asym"))
    FULL.append((M, 4096, 14336, 32, "f16", "asym"))
    FULL.append((M, 4096, 14336, 64, "f16", "nf4"))
FULL.append((2048, 8192, 28672, 128, "bf16", "asym"))                       # prefill-shaped


# ragged M, K and N on each batched geometry (test_abi_cpu pins which one a shape gets):
# 64x256 tiles, 128x512 tiles, and 128x512 tiles with K split in two
FULL.append((257, 2080, 44048, 32, "f16", "asym"))
FULL.append((513, 2080, 44048, 32, "f16", "asym"))
FULL.append((129, 4224, 28688, 64, "bf16", "asym"))
# 12..16 rows on large weights whose x exceeds the decode kernel's LDS: the batched kernel
FULL.append((16, 8192, 57344, 128, "f16", "sym"))
FULL.append((12, 28672, 8192, 128, "bf16", "asym"))
# the skinny kernel's wider bands at full size: groups of 32 over two rounds of column tiles at
# 8 rows, 128-row tiles on 8192-deep K, 128-row tiles from 160 rows (NF4)
FULL.append((8, 8192, 28672, 32, "f16", "asym"))
FULL.append((96, 8192, 10240, 128, "bf16", "asym"))
FULL.append((192, 4096, 6144, 64, "f16", "nf4"))


@pytest.mark.parametrize("M,K,N,g,act,fmt", FULL)
def test_full_size_sampled_strips(M, K, N, g, act, fmt):
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    _announce(f"full M={M} K={K} N={N} g={g} {act} {fmt} kernel={w4.kernel_name(M, K, N, g)}")
    seed = synth.seed_for(9, K // 128 + N // 1024, 0)
    qweight, scales, qzeros = synth.timing_weights(K, N, g, seed, symmetric=(fmt != "asym"),
                                                   scale_dtype=act)
    x = synth.activations(M, K, seed + synth.ROLE_X, act)
    case = {"M": M, "K": K, "N": N, "g": g, "act": act, "nf4": fmt == "nf4", "x": x,
            "qweight": qweight, "scales": scales, "qzeros": qzeros}
    if fmt == "nf4":
        case["codebook"] = oracle.nf4_codebook()
        case["scales"] = synth.random_scales(K // g, N, seed + 7, "f16", 0.02, 0.09)
    d = device_inputs(case)
    cols = sample_strips(N, 6, seed)
    y_ref = oracle_columns(x, qweight, case["scales"], qzeros, g, act, cols,
                           nf4=case["nf4"], codebook=case.get("codebook"))
    y = from_dev(run_gemm(case, d, out_dtype=torch.float32)).astype(np.float64)
    assert_close(y[:, cols], y_ref, "fp32 out, sampled strips")
    del d
    torch.cuda.empty_cache()


def test_graph_replays_match_eager():
    """The benchmark replays a captured HIP graph of GEMM launches: every replay, with eager
    work and synchronisation between replays, must equal the eager result bit for bit."""
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    cases = [rtn_case(1, 1024, 256, 128, seed=11), rtn_case(4, 512, 128, 32, seed=12),
             rtn_case(130, 2048, 64, 128, seed=13),     # batched kernel, K split in two
             rtn_case(40, 2048, 8208, 128, seed=14)]    # skinny kernel
    devs = [device_inputs(c) for c in cases]
    outs = [torch.empty((c["M"], c["N"]), dtype=torch.float16, device="cuda") for c in cases]

    def step():
        for c, d, o in zip(cases, devs, outs):
            w4.gemm(d["x"], d["packed"], d["scales"], d["qzeros"], c["g"], out=o)

    step()
    torch.cuda.synchronize()
    eager = [from_dev(o).copy() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for o in outs:
            o.fill_(0)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert np.array_equal(from_dev(o).view(np.uint16), e.view(np.uint16)), f"replay {r}"


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 1 << 20, (3 << 20) + 16 * 7])
def test_read_probe_reads_every_chunk_once(nbytes):
    """The streaming-read probe (the bandwidth ceiling reported by the benchmark): the XOR of
    its sink words is the XOR of every 32-bit word of the buffer, so a chunk read twice
    (cancelled) or skipped changes it."""
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    words = np.random.default_rng(nbytes).integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    w4.read_probe(buf, sink)
    torch.cuda.synchronize()
    folded = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(folded) == int(np.bitwise_xor.reduce(words))
