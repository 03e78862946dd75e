"""Helpers shared by the GPU parity tests: build oracle-side inputs, move them to the
device, run the library through its C ABI, and compare with the oracle."""
from __future__ import annotations

import numpy as np

import oracle
from weight_only_int4_w4a16_amd import synth

RTOL = 1e-3   # max|y - y_ref| <= 1e-3 * max|y_ref|


def torch_mod():
    import torch
    return torch


def require_gpu():
    import pytest
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_dev(a: np.ndarray, kind: str):
    """numpy -> cuda tensor. kind: 'f16' (np.float16), 'bf16' (uint16 bits), 'i32'."""
    torch = torch_mod()
    if kind == "f16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).cuda()
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda().view(torch.bfloat16)
    if kind == "i32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    raise ValueError(kind)


def from_dev(t) -> np.ndarray:
    """cuda tensor -> numpy: fp16 -> np.float16, bf16 -> uint16 bits, fp32 -> float32."""
    torch = torch_mod()
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_values(a: np.ndarray, dtype) -> np.ndarray:
    torch = torch_mod()
    if dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def rtn_case(M, K, N, g, act="f16", sym=False, seed=0, nf4=False):
    """Gaussian weights quantized by the oracle; returns a dict of canonical host tensors."""
    W = synth.gaussian_weight(K, N, seed)
    x = synth.activations(M, K, seed + 1, act)
    case = {"M": M, "K": K, "N": N, "g": g, "act": act, "x": x, "nf4": nf4}
    if nf4:
        cb = oracle.nf4_codebook()
        codes, a = oracle.quantize_nf4(W, cb, g)
        case.update(qweight=oracle.pack_codes(codes), scales=a, qzeros=None, codebook=cb)
        case["w_hat"] = oracle.dequant_nf4(case["qweight"], a, cb, g, act)
    elif sym:
        q, s = oracle.quantize_rtn_sym(W, g, act)
        case.update(qweight=oracle.pack_codes(oracle.to_offset_binary(q)), scales=s, qzeros=None)
        case["w_hat"] = oracle.dequant_sym(case["qweight"], s, g, act)
    else:
        q, s, z = oracle.quantize_rtn_asym(W, g, act)
        case.update(qweight=oracle.pack_codes(q), scales=s, qzeros=oracle.pack_zeros(z))
        case["w_hat"] = oracle.dequant_affine(case["qweight"], s, case["qzeros"], g, act)
    return case


def device_inputs(case):
    torch = torch_mod()
    import weight_only_int4_w4a16_amd as w4
    act = case["act"]
    d = {"x": to_dev(case["x"], act), "qweight": to_dev(case["qweight"], "i32")}
    d["packed"] = w4.pack(d["qweight"])
    if case["nf4"]:
        d["scales"] = to_dev(case["scales"], "f16")
        d["codebook"] = to_dev(case["codebook"], "f16")
    else:
        d["scales"] = to_dev(case["scales"], act)
    d["qzeros"] = None if case.get("qzeros") is None else to_dev(case["qzeros"], "i32")
    torch.cuda.synchronize()
    return d


def run_gemm(case, d, out_dtype=None):
    import weight_only_int4_w4a16_amd as w4
    if case["nf4"]:
        y = w4.gemm_nf4(d["x"], d["packed"], d["scales"], d["codebook"], case["g"], out_dtype=out_dtype)
    else:
        y = w4.gemm(d["x"], d["packed"], d["scales"], d["qzeros"], case["g"], out_dtype=out_dtype)
    torch_mod().cuda.synchronize()
    return y


def run_swiglu(case, d, out_dtype=None):
    import weight_only_int4_w4a16_amd as w4
    if case["nf4"]:
        h = w4.gemm_nf4_swiglu(d["x"], d["packed"], d["scales"], d["codebook"], case["g"],
                               out_dtype=out_dtype)
    else:
        h = w4.gemm_swiglu(d["x"], d["packed"], d["scales"], d["qzeros"], case["g"],
                           out_dtype=out_dtype)
    torch_mod().cuda.synchronize()
    return h


def assert_close(y: np.ndarray, y_ref: np.ndarray, what: str = ""):
    err = np.max(np.abs(y - y_ref)) if y.size else 0.0
    bound = RTOL * np.max(np.abs(y_ref)) if y.size else 0.0
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert err <= bound, f"{what}: max|y - y_ref| = {err:.3e} > {bound:.3e}"


def sample_strips(N: int, count: int, seed: int) -> np.ndarray:
    """Column indices of ``count`` 16-column strips: first, last and random ones."""
    nst = N // 16
    rng = np.random.default_rng(seed)
    picks = {0, nst - 1}
    picks.update(rng.choice(nst, size=min(count, nst), replace=False).tolist())
    strips = np.array(sorted(picks))
    return (strips[:, None] * 16 + np.arange(16)[None, :]).ravel()


def oracle_columns(x, qweight, scales, qzeros, g, act, cols, nf4=False, codebook=None):
    """Oracle output for the given columns (multiples of whole 8-column zero words)."""
    qw = qweight[:, cols]
    s = scales[:, cols]
    if nf4:
        w_hat = oracle.dequant_nf4(qw, s, codebook, g, act)
    else:
        qz = None
        if qzeros is not None:
            words = np.unique(cols // 8)
            zfull = oracle.unpack_zeros(qzeros[:, words])               # (G, 8*len(words))
            colpos = {w: i for i, w in enumerate(words)}
            idx = np.array([colpos[c // 8] * 8 + c % 8 for c in cols])
            qz = oracle.pack_zeros(zfull[:, idx])
        w_hat = oracle.dequant_affine(qw, s, qz, g, act)
    return oracle.gemm_ref(x, w_hat, act)


def assert_graph_replays_match_eager(step, outs, replays: int = 4):
    """Run ``step`` (launches writing ``outs``) eagerly, capture it in a HIP graph, and check
    that every replay, with eager work and synchronisation between replays, reproduces the
    eager outputs bit for bit."""
    torch = torch_mod()
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(replays):
        for o in outs:
            o.fill_(0)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o.view(torch.int16) if o.element_size() == 2 else o.view(torch.int32),
                               e.view(torch.int16) if e.element_size() == 2 else e.view(torch.int32)), \
                f"replay {r}, output {i}"
