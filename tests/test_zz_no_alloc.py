"""w4a16_gemm_static, the GEMM entry point that allocates nothing: its split-K scratch is the
library's static device array. Through the C ABI it must give w4a16_gemm's result bit for
bit (the same kernels and summation order), on consecutive calls that share the array, the
second call smaller than the first."""
import ctypes

import numpy as np
import pytest

from gpu_common import device_inputs, from_dev, require_gpu, rtn_case, torch_mod

pytestmark = pytest.mark.gpu

LIMIT = 64 << 20   # W4A16_STATIC_SCRATCH_BYTES


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _both(case, d, out_dtype):
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    ref = w4.gemm(d["x"], d["packed"], d["scales"], d["qzeros"], case["g"], out_dtype=out_dtype)
    got = w4.gemm_static(d["x"], d["packed"], d["scales"], d["qzeros"], case["g"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return from_dev(ref), from_dev(got)


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def test_static_scratch_matches_workspace_path_twice_shrinking():
    require_gpu()
    import weight_only_int4_w4a16_amd as w4
    torch = torch_mod()
    # first a shape whose batched launch splits K (scratch in use), then a smaller one that
    # splits K too, then a decode shape that needs no scratch
    shapes = [(130, 8192, 4096, 128, "f16"), (136, 2048, 512, 64, "bf16"), (3, 1024, 512, 32, "f16")]
    needs = [w4.workspace_bytes(M, K, N, g) for (M, K, N, g, _) in shapes]
    assert needs[0] > needs[1] > 0 and needs[2] == 0 and needs[0] <= LIMIT
    for (M, K, N, g, act), need in zip(shapes, needs):
        _announce(f"static M={M} K={K} N={N} g={g} {act} need={need} kernel={w4.kernel_name(M, K, N, g)}")
        c = rtn_case(M, K, N, g, act, seed=M + K + N)
        d = device_inputs(c)
        for odt in (torch.float32, None):
            ref, got = _both(c, d, odt)
            assert np.array_equal(_bits(got), _bits(ref)), (M, K, N, odt)


def test_static_rejects_shapes_beyond_its_scratch():
    """A shape whose split-K partials exceed the static array returns W4A16_ERR_WORKSPACE
    before anything is launched (no pointers are dereferenced)."""
    import weight_only_int4_w4a16_amd as w4
    L = w4.lib()
    vp = ctypes.c_void_p
    big = None
    for (M, K, N) in ((1152, 32768, 10752), (1024, 32768, 10240), (640, 32768, 16384)):
        if w4.workspace_bytes(M, K, N, 128) > LIMIT:   # K split into fp32 partial tiles
            big = (M, K, N)
            break
    assert big is not None
    M, K, N = big
    assert L.w4a16_gemm_static(vp(16), M, K, N, 0, vp(16), vp(16), vp(16), 128, vp(16), 0, None) == 4
    assert L.w4a16_gemm_static(vp(16), 4, 100, N, 0, vp(16), vp(16), vp(16), 128, vp(16), 0, None) == 1
    assert L.w4a16_gemm_static(None, 0, K, N, 0, None, None, None, 128, None, 0, None) == 0
