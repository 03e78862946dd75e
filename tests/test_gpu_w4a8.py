"""GPU parity of the W4A8 path (``w4a16_gemm_w4a8``, ``w4a16_quantize_act_int8``) against the
CPU oracle (``oracle.w4a8``).

* per-token INT8 activations and their fp32 scales: bit for bit (the codes are decisions the
  kernel and the oracle take in the same fp32 arithmetic), including ties and zero rows;
* the GEMM: the integer sum is exact on both sides and the kernel applies the two scales in
  fp32, so every element is within 3 fp32 roundings of the fp64 oracle,
  |y - y_ref| <= 3 * 2^-24 |y_ref| (plus the 16-bit output rounding, checked as RNE of the fp32
  result); whole outputs on small shapes (ragged K, both tiles, ragged last tile), sampled
  strips at the prefill and crossover sizes;
* against the W4A16 GEMM on the same codes: the difference stays within the activation
  quantization bound sx/2 * sum_k |W_hat[k, n]|.
"""
import numpy as np
import pytest

import oracle
from weight_only_int4_w4a16_amd import synth

from gpu_common import (assert_graph_replays_match_eager, from_dev, require_gpu, sample_strips,
                        to_dev, torch_mod)

pytestmark = pytest.mark.gpu

REL = 3.0 * 2.0 ** -24 * (1 + 1e-6)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _x(M, K, act, seed):
    return synth.activations(M, K, seed, act)


def _run(x, qweight, wscale, act, out_dtype=None):
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    packed = w4.pack(to_dev(qweight, "i32"))
    y = w4.gemm_w4a8(to_dev(x, act), packed, to_dev(np.ascontiguousarray(wscale.reshape(-1)), act),
                     out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,K,act", [(1, 4096, "f16"), (7, 14336, "bf16"), (64, 1056, "f16"),
                                     (300, 8192, "bf16"), (5, 32, "f16")])
def test_quantize_act_bit_exact(M, K, act):
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    _announce(f"w4a8 quantize M={M} K={K} {act}")
    x = _x(M, K, act, 51 + M)
    if M >= 5:   # a zero row, and a row of ties (max 127 gives sx = 1: codes are rint(x))
        x[1] = 0
        ties = np.resize(np.array([127.0, 63.5, -0.5, 2.5, -3.5, 0.25], np.float32), K)
        x[2] = ties.astype(np.float16) if act == "f16" else synth.f32_to_bf16_bits(ties)
    xq, sx = w4.quantize_act_int8(to_dev(x, act))
    torch.cuda.synchronize()
    xq_ref, sx_ref = oracle.w4a8.quantize_act_int8(x, act)
    assert np.array_equal(from_dev(sx).view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(from_dev(xq), xq_ref)


SMALL = [
    (1, 1024, 256, "f16"),
    (17, 2080, 512, "bf16"),      # ragged K (the last 128-block has one 32-k step), K split in 2
    (64, 4096, 1024, "f16"),      # K split in 4
    (130, 2048, 768, "bf16"),     # K split in 2
    (600, 1024, 16384, "f16"),    # 128x512 tiles, last row tile ragged
    (257, 512, 44048, "bf16"),    # N not a multiple of the tile width
]


@pytest.mark.parametrize("M,K,N,act", SMALL)
def test_w4a8_gemm_matches_oracle(M, K, N, act):
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    _announce(f"w4a8 M={M} K={K} N={N} {act} {w4.w4a8_kernel_name(M, K, N)}")
    seed = synth.seed_for(13, K // 32 + N // 16 + M, 0)
    W = synth.gaussian_weight(K, N, seed)
    q, s = oracle.quantize_rtn_sym(W, K, act)                 # one scale per output channel
    qw = oracle.pack_codes(oracle.to_offset_binary(q))
    x = _x(M, K, act, seed + synth.ROLE_X)
    y_ref = oracle.w4a8.gemm_w4a8_ref(x, qw, s, act)
    y = from_dev(_run(x, qw, s, act, torch.float32)).astype(np.float64)
    assert np.all(np.isfinite(y))
    assert np.all(np.abs(y - y_ref) <= REL * np.abs(y_ref)), np.max(np.abs(y - y_ref) / np.abs(y_ref).max())
    y16 = from_dev(_run(x, qw, s, act))
    if act == "f16":
        assert np.array_equal(y16.view(np.uint16), y.astype(np.float32).astype(np.float16).view(np.uint16))
    else:
        assert np.array_equal(y16, synth.f32_to_bf16_bits(y.astype(np.float32)))


@pytest.mark.parametrize("M,K,N,act", [(64, 4096, 14336, "f16"), (256, 4096, 14336, "f16"),
                                       (2048, 8192, 28672, "bf16"), (4096, 4096, 14336, "bf16")])
def test_w4a8_full_size_sampled_strips(M, K, N, act):
    torch = torch_mod()
    _announce(f"w4a8 full M={M} K={K} N={N} {act}")
    seed = synth.seed_for(14, K // 128 + N // 1024, 0)
    qweight, _, _ = synth.timing_weights(K, N, 128, seed, symmetric=True, scale_dtype=act)
    wscale = synth.random_scales(1, N, seed + synth.ROLE_SCALES, act)
    x = _x(M, K, act, seed + synth.ROLE_X)
    cols = sample_strips(N, 6, seed)
    y_ref = oracle.w4a8.gemm_w4a8_ref(x, qweight[:, cols], wscale[:, cols], act)
    y = from_dev(_run(x, qweight, wscale, act, torch.float32))[:, cols].astype(np.float64)
    assert np.all(np.abs(y - y_ref) <= REL * np.abs(y_ref))
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,act", [(48, "f16"), (512, "bf16")])
def test_w4a8_against_w4a16_within_activation_bound(M, act):
    """The same per-channel codes through the W4A16 GEMM (the scale repeated in every group of
    128): |y_w4a8 - y_w4a16| <= sx/2 * sum_k |W_hat[k, n]| plus the 16-bit rounding slack of
    W_hat's entries."""
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    K, N = 4096, 2048
    _announce(f"w4a8 vs w4a16 M={M} {act}")
    W = synth.gaussian_weight(K, N, 61)
    q, s = oracle.quantize_rtn_sym(W, K, act)
    qw = oracle.pack_codes(oracle.to_offset_binary(q))
    x = _x(M, K, act, 62)
    y8 = from_dev(_run(x, qw, s, act, torch.float32)).astype(np.float64)
    s_g = np.ascontiguousarray(np.repeat(s, K // 128, axis=0))
    packed = w4.pack(to_dev(qw, "i32"))
    y16 = from_dev(w4.gemm(to_dev(x, act), packed, to_dev(s_g, act), None, 128,
                           out_dtype=torch.float32)).astype(np.float64)
    w_hat = oracle.dequant_sym(qw, s, K, act)
    wv = w_hat.astype(np.float64) if act == "f16" else oracle.bf16_bits_to_f64(w_hat)
    xv = x.astype(np.float64) if act == "f16" else oracle.bf16_bits_to_f64(x)
    _, sx = oracle.w4a8.quantize_act_int8(x, act)
    bound = 0.5 * sx.astype(np.float64)[:, None] * np.abs(wv).sum(axis=0)[None, :]
    slack = 2.0 ** -7 * np.abs(xv) @ np.abs(wv) + 1e-3 * np.abs(y16).max()
    assert np.all(np.abs(y8 - y16) <= bound + slack)


def test_w4a8_graph_replays_match_eager():
    """The quantizer, both GEMM tiles and the split-K reduction captured in one HIP graph:
    replays equal the eager run bit for bit."""
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    calls, outs = [], []
    for i, (M, K, N, act) in enumerate([(64, 2048, 1024, "f16"), (600, 1024, 16384, "bf16"),
                                        (130, 4096, 2048, "f16")]):   # the last with K split
        _announce(f"w4a8 graph M={M} K={K} N={N} {act}")
        qw, _, _ = synth.timing_weights(K, N, 128, 100 + i, symmetric=True, scale_dtype=act)
        sw = synth.random_scales(1, N, 110 + i, act).reshape(-1)
        x = to_dev(_x(M, K, act, 120 + i), act)
        ws = torch.empty(w4.w4a8_workspace_bytes(M, K, N), dtype=torch.uint8, device="cuda")
        out = torch.empty((M, N), dtype=x.dtype, device="cuda")
        calls.append(((x, w4.pack(to_dev(qw, "i32")), to_dev(sw, act)), ws, out))
        outs.append(out)

    def step():
        for args, ws, out in calls:
            w4.gemm_w4a8(*args, out=out, workspace=ws)

    assert_graph_replays_match_eager(step, outs)
