"""GPU parity of the AWQ-scaled GEMM (``w4a16_gemm_awq``) against the CPU oracle.

"4.3 Weight-only INT4", section 3.2: the deployed weight is the INT4 format of S W and the
GEMM multiplies the scaled activations, Y_hat = (X S^-1) D(Q(S W)). The library forms
x' = RN(x * s_inv) as it stages x (decode kernel LDS, batched kernel's 64x256 LDS tile;
decode shapes whose x does not fit in LDS, and the 128x512 tile, scale into the workspace
first). Checked here:

* x' itself, bit for bit, on every path: sparse x and one-hot weight columns make the fp32
  output the scaled activations exactly;
* the GEMM within max|y - y_ref| <= 1e-3 max|y_ref| against ``oracle.gemm_ref`` of
  ``oracle.awq.scale_activations``: whole outputs on small shapes, sampled strips at full
  size, every format and path (ragged K, persistent decode, split K);
* weights from the oracle's AWQ search on inputs with salient channels: parity, and the GPU
  output closer to x W than the GPU output of plain RTN weights.
"""
import numpy as np
import pytest

import oracle
from weight_only_int4_w4a16_amd import synth

from gpu_common import (assert_close, assert_graph_replays_match_eager, from_dev, oracle_columns,
                        require_gpu, sample_strips, to_dev, torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _run_awq(x, s_inv, qweight, scales, qzeros, g, act, out_dtype=None):
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    xd = to_dev(x, act)
    sd = to_dev(s_inv, act)
    packed = w4.pack(to_dev(qweight, "i32"))
    sc = to_dev(scales, act)
    qz = None if qzeros is None else to_dev(qzeros, "i32")
    y = w4.gemm_awq(xd, sd, packed, sc, qz, g, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


def _path(M, K, N, g):
    import weight_only_int4_w4a16_amd as w4
    return f"{w4.kernel_name(M, K, N, g)} ws={w4.awq_workspace_bytes(M, K, N, g)}"


# (M, K, N, g, act, fmt): decode with x in LDS (one and two strips per tile, every group
# size, ragged K), persistent decode, decode with x scaled into the workspace, batched tiles
# (64x256, 128x512, K split)
SMALL = [
    (1, 1024, 512, 128, "f16", "asym"),
    (1, 1056, 256, 32, "bf16", "sym"),      # ragged K: the last 128-block has one 32-k step
    (3, 2112, 384, 64, "f16", "sym"),
    (7, 4096, 640, 128, "bf16", "asym"),
    (16, 2048, 1024, 32, "f16", "asym"),
    (9, 9216, 256, 128, "f16", "asym"),     # x does not fit in LDS: scaled into the workspace
    (16, 8320, 512, 64, "bf16", "asym"),
    (17, 1024, 768, 128, "f16", "asym"),    # decode, two launches (16 + 1 rows)
    (20, 4096, 4128, 128, "bf16", "asym"),  # batched 64x256 tile, just past 16 rows
    (40, 2080, 512, 32, "bf16", "sym"),
    (130, 2048, 64, 128, "f16", "asym"),    # batched, K split in two
    (8, 4096, 10240, 128, "f16", "asym"),   # skinny at 8 rows: x scaled into the workspace
    (24, 2048, 16400, 64, "bf16", "sym"),   # skinny, 32-row tile, ragged column tile
    (96, 1024, 8320, 128, "f16", "asym"),   # skinny, 128-row tile
]


@pytest.mark.parametrize("M,K,N,g,act,fmt", SMALL)
def test_awq_gemm_matches_oracle(M, K, N, g, act, fmt):
    torch = torch_mod()
    _announce(f"awq M={M} K={K} N={N} g={g} {act} {fmt} {_path(M, K, N, g)}")
    seed = synth.seed_for(11, K // 32 + N // 16 + M, 0)
    W = synth.gaussian_weight(K, N, seed)
    x = synth.activations(M, K, seed + synth.ROLE_X, act)
    s_inv = synth.channel_scales(K, seed + synth.ROLE_XSCALE, act)
    Ws = oracle.awq.scale_weight(W, s_inv, act)
    if fmt == "sym":
        q, s = oracle.quantize_rtn_sym(Ws, g, act)
        qw, qz = oracle.pack_codes(oracle.to_offset_binary(q)), None
    else:
        q, s, z = oracle.quantize_rtn_asym(Ws, g, act)
        qw, qz = oracle.pack_codes(q), oracle.pack_zeros(z)
    w_hat = oracle.dequant_affine(qw, s, qz, g, act)
    y_ref = oracle.gemm_ref(oracle.awq.scale_activations(x, s_inv, act), w_hat, act)
    y = from_dev(_run_awq(x, s_inv, qw, s, qz, g, act, torch.float32)).astype(np.float64)
    assert_close(y, y_ref, "fp32 out")
    # 16-bit output is the round-to-nearest-even of the fp32 result
    y16 = from_dev(_run_awq(x, s_inv, qw, s, qz, g, act))
    if act == "f16":
        assert np.array_equal(y16.view(np.uint16), y.astype(np.float32).astype(np.float16).view(np.uint16))
    else:
        assert np.array_equal(y16, synth.f32_to_bf16_bits(y.astype(np.float32)))


FULL = [
    (1, 4096, 28672, 128, "f16", "asym"),   # 8B gate+up, two strips per tile
    (1, 14336, 4096, 128, "f16", "asym"),
    (4, 8192, 10240, 128, "f16", "sym"),
    (16, 4096, 28672, 128, "f16", "asym"),  # persistent workgroups
    (8, 8192, 57344, 128, "bf16", "sym"),   # persistent workgroups
    (16, 14336, 4096, 128, "f16", "asym"),  # x scaled into the workspace
    (256, 4096, 14336, 128, "f16", "asym"),
    (512, 2080, 44048, 32, "f16", "asym"),  # 128x512 tile: x scaled into the workspace
    (129, 4224, 28688, 64, "bf16", "asym"), # and K split: x' after the partials
    (2048, 8192, 28672, 128, "bf16", "asym"),
]


@pytest.mark.parametrize("M,K,N,g,act,fmt", FULL)
def test_awq_full_size_sampled_strips(M, K, N, g, act, fmt):
    torch = torch_mod()
    _announce(f"awq full M={M} K={K} N={N} g={g} {act} {fmt} {_path(M, K, N, g)}")
    seed = synth.seed_for(12, K // 128 + N // 1024, 0)
    qweight, scales, qzeros = synth.timing_weights(K, N, g, seed, symmetric=(fmt != "asym"),
                                                   scale_dtype=act)
    x = synth.activations(M, K, seed + synth.ROLE_X, act)
    s_inv = synth.channel_scales(K, seed + synth.ROLE_XSCALE, act)
    cols = sample_strips(N, 6, seed)
    y_ref = oracle_columns(oracle.awq.scale_activations(x, s_inv, act), qweight, scales, qzeros,
                           g, act, cols)
    y = from_dev(_run_awq(x, s_inv, qweight, scales, qzeros, g, act, torch.float32))
    assert_close(y[:, cols].astype(np.float64), y_ref, "fp32 out, sampled strips")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,K,N,act", [
    (1, 4096, 512, "f16"),       # decode, x in LDS
    (1, 2048, 256, "bf16"),
    (16, 2048, 28672, "f16"),    # persistent decode
    (12, 14336, 256, "bf16"),    # x scaled into the workspace
    (16, 14336, 512, "f16"),
    (64, 2048, 512, "f16"),      # batched
    (300, 1024, 1024, "bf16"),
    (1024, 2048, 16384, "bf16"), # batched 128x512 tile: x scaled into the workspace
])
def test_awq_scaled_activations_bit_exact(M, K, N, act):
    """Each row of x holds one nonzero per 128-k block and column n of W_hat is the unit
    vector of one channel k_n, so every product and partial sum is exact and the fp32 output
    is x'[:, k_n] = RN(x[:, k_n] * s_inv[k_n]) bit for bit."""
    torch = torch_mod()
    _announce(f"awq exact M={M} K={K} N={N} {act} {_path(M, K, N, 128)}")
    KC = K // 128
    rng = np.random.default_rng(M * 7 + K)
    pos = (37 * np.arange(M)[:, None] + 11 * np.arange(KC)[None, :]) % 128     # (M, KC)
    vals = rng.standard_normal((M, KC)) * 4
    x64 = np.zeros((M, K))
    x64[np.arange(M)[:, None], 128 * np.arange(KC)[None, :] + pos] = vals
    x = x64.astype(np.float16) if act == "f16" else synth.f32_to_bf16_bits(x64.astype(np.float32))
    s_inv = synth.channel_scales(K, M + K, act, spread=8.0)
    n = np.arange(N)
    m_of, b_of = n % M, (n // M) % KC
    k_n = 128 * b_of + pos[m_of, b_of]
    q = np.full((K, N), 8, np.uint8)
    q[k_n, n] = 9
    z = np.full((K // 128, N), 8, np.uint8)
    one = np.ones((K // 128, N))
    scales = one.astype(np.float16) if act == "f16" else synth.f32_to_bf16_bits(one.astype(np.float32))
    y = from_dev(_run_awq(x, s_inv, oracle.pack_codes(q), scales, oracle.pack_zeros(z), 128, act,
                          torch.float32))
    xs = oracle.awq.scale_activations(x, s_inv, act)
    exp = xs.astype(np.float32) if act == "f16" else oracle.bf16_bits_to_f64(xs).astype(np.float32)
    assert y.dtype == np.float32 and np.count_nonzero(exp[:, k_n]) >= N
    assert np.array_equal(y, exp[:, k_n])   # float32 values: equal values are equal bits (+-0 aside)


@pytest.mark.parametrize("M,act,sym", [(1, "f16", False), (16, "bf16", True), (64, "f16", False)])
def test_awq_search_end_to_end(M, act, sym):
    """Weights from the oracle's AWQ search on inputs with 1/32 salient channels (10x): the
    GPU output matches the oracle and is closer to x W than the GPU output of plain RTN
    weights on the same rows ("4.3 Weight-only INT4", section 3.1)."""
    torch = torch_mod()
    K, N, g = 1024, 256, 128
    _announce(f"awq search M={M} K={K} N={N} {act} sym={sym}")
    rng = np.random.default_rng(31 + M)
    X = rng.standard_normal((512, K))
    X[:, rng.choice(K, K // 32, replace=False)] *= 10.0
    W = synth.gaussian_weight(K, N, 77)
    quant, s_inv, alpha, errs = oracle.awq.awq_quantize(W, X, g, act, sym)
    assert alpha > 0
    xq = X[:M].astype(np.float16) if act == "f16" else synth.f32_to_bf16_bits(X[:M].astype(np.float32))
    xv = xq.astype(np.float64) if act == "f16" else oracle.bf16_bits_to_f64(xq)
    errs_gpu = []
    for use_awq in (True, False):
        if use_awq:
            qq = quant
            si = s_inv
        else:
            qq = oracle.quantize_rtn_sym(W, g, act) if sym else oracle.quantize_rtn_asym(W, g, act)
            si = oracle.awq.candidate_scales(X, 0.0, act)      # S = I
        if sym:
            qw, qz = oracle.pack_codes(oracle.to_offset_binary(qq[0])), None
        else:
            qw, qz = oracle.pack_codes(qq[0]), oracle.pack_zeros(qq[2])
        w_hat = oracle.dequant_affine(qw, qq[1], qz, g, act)
        y = from_dev(_run_awq(xq, si, qw, qq[1], qz, g, act, torch.float32)).astype(np.float64)
        assert_close(y, oracle.gemm_ref(oracle.awq.scale_activations(xq, si, act), w_hat, act),
                     f"awq={use_awq}")
        errs_gpu.append(np.linalg.norm(y - xv @ W))
    assert errs_gpu[0] < errs_gpu[1], f"AWQ {errs_gpu[0]:.4g} not below RTN {errs_gpu[1]:.4g}"



def test_awq_graph_replays_match_eager():
    """Every AWQ path captured in one HIP graph (LDS prologue, persistent, workspace pre-pass
    for decode, for the skinny kernel and for the 128x512 tile, split K): replays equal the
    eager run bit for bit."""
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    shapes = [(1, 1024, 512), (16, 2048, 28672), (12, 14336, 256), (130, 2048, 64), (1024, 2048, 16384),
              (40, 2048, 4096)]
    calls, outs = [], []
    for i, (M, K, N) in enumerate(shapes):
        _announce(f"awq graph M={M} K={K} N={N} {_path(M, K, N, 128)}")
        qw, sc, qz = synth.timing_weights(K, N, 128, 70 + i, scale_dtype="f16")
        x = to_dev(synth.activations(M, K, 80 + i, "f16"), "f16")
        s_inv = to_dev(synth.channel_scales(K, 90 + i, "f16"), "f16")
        args = (x, s_inv, w4.pack(to_dev(qw, "i32")), to_dev(sc, "f16"), to_dev(qz, "i32"), 128)
        ws = torch.empty(max(w4.awq_workspace_bytes(M, K, N, 128), 256), dtype=torch.uint8, device="cuda")
        out = torch.empty((M, N), dtype=torch.float16, device="cuda")
        calls.append((args, ws, out))
        outs.append(out)

    def step():
        for args, ws, out in calls:
            w4.gemm_awq(*args, out=out, workspace=ws)

    assert_graph_replays_match_eager(step, outs)
