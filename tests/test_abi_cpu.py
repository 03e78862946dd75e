"""CPU-only checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments on the host before any HIP call. No kernel is launched here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    from weight_only_int4_w4a16_amd import binding
    return binding.lib()


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for n in ("w4a16_pack", "w4a16_gemm", "w4a16_gemm_nf4", "w4a16_dequant",
              "w4a16_dequant_nf4", "w4a16_packed_bytes", "w4a16_workspace_bytes", "w4a16_kernel_name",
              "w4a16_gemm_awq", "w4a16_awq_workspace_bytes", "w4a16_gemm_swiglu",
              "w4a16_status_string", "w4a16_version"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in include/w4a16.h but not exported"


def test_packed_bytes(L):
    from weight_only_int4_w4a16_amd import packed_bytes
    assert packed_bytes(4096, 4096) == 4096 * 4096 // 2
    assert packed_bytes(352, 48) == 384 * 48 // 2          # K padded to a multiple of 128
    assert packed_bytes(4096, 24) == 0                      # N % 16 != 0
    assert packed_bytes(0, 16) == 0
    assert packed_bytes(8192, 57344) == 8192 * 57344 // 2


def _gemm(L, x=16, M=1, K=4096, N=4096, act=0, packed=16, scales=16, qzeros=16, g=128,
          out=16, odt=0, ws=256, wsb=1 << 30):
    vp = ctypes.c_void_p
    return L.w4a16_gemm(vp(x) if x else None, M, K, N, act, vp(packed) if packed else None,
                        vp(scales) if scales else None, vp(qzeros) if qzeros else None, g,
                        vp(out) if out else None, odt, vp(ws) if ws else None, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=100), 1),              # K % 8
    (dict(K=4096 + 32, g=128), 1), # K % g
    (dict(g=48), 1),               # group size not in {32, 64, 128}
    (dict(N=4100), 1),             # N % 8
    (dict(N=4104), 2),             # N % 16: well-formed, not implemented
    (dict(M=-1), 1),
    (dict(act=2), 1),              # fp32 activations
    (dict(act=0, odt=1), 1),       # bf16 out for fp16 activations
    (dict(x=0), 1),                # null x
    (dict(packed=0), 1),
    (dict(scales=0), 1),
    (dict(out=0), 1),
    (dict(x=8), 1),                # misaligned x (needs 16 bytes)
    (dict(scales=3), 1),           # misaligned scales
    (dict(qzeros=2), 1),           # misaligned zeros
])
def test_gemm_rejects_bad_arguments_before_launch(L, kw, status):
    assert _gemm(L, **kw) == status


def test_gemm_m0_is_a_noop(L):
    assert _gemm(L, M=0, x=0, packed=0, scales=0, out=0, ws=0, wsb=0) == 0


def test_workspace_bytes(L):
    from weight_only_int4_w4a16_amd import workspace_bytes
    assert workspace_bytes(0, 4096, 4096, 128) == 0
    assert workspace_bytes(1, 4096, 4096, 100) == 0
    for M, K, N in ((1, 4096, 4096), (16, 14336, 4096), (16, 4096, 28672), (1, 352, 48)):
        assert workspace_bytes(M, K, N, 32) == 0    # the decode kernels reduce in LDS
    # batched kernel: no workspace when the output tiles fill the chip, otherwise K is split
    # and the workspace holds the S fp32 partial tiles (rows padded to the tile's height:
    # 64 rows for the small tile, chosen when large tiles would not cover the chip)
    assert workspace_bytes(2048, 8192, 28672, 128) == 0
    assert workspace_bytes(200, 2048, 64, 128) == 8 * 256 * 64 * 4    # 8 slices of 2 k-blocks
    assert workspace_bytes(48, 4096, 28672, 128) == 2 * 64 * 28672 * 4   # 2 slices
    assert workspace_bytes(32, 4096, 28672, 128) == 0     # the skinny kernel reduces in LDS


def test_awq_rejects_bad_s_inv_and_sizes_its_workspace(L):
    from weight_only_int4_w4a16_amd import awq_workspace_bytes, workspace_bytes
    vp = ctypes.c_void_p
    for s_inv in (None, vp(18)):                       # missing, or not 16-byte aligned
        st = L.w4a16_gemm_awq(vp(16), s_inv, 1, 4096, 4096, 0, vp(16), vp(16), vp(16), 128,
                              vp(16), 0, vp(256), 1 << 30, None)
        assert st == 1
    assert L.w4a16_gemm_awq(None, None, 0, 4096, 4096, 0, None, None, None, 128, None, 0,
                            None, 0, None) == 0        # M = 0 is a no-op
    # decode shapes whose x fits in LDS (rows * K * 2 <= 128 KiB) need nothing; the others
    # get rows * K * 2 bytes for the scaled activations; batched shapes as the plain GEMM
    assert awq_workspace_bytes(1, 14336, 4096, 128) == 0
    assert awq_workspace_bytes(16, 4096, 28672, 128) == 0
    assert awq_workspace_bytes(8, 14336, 4096, 128) == 8 * 14336 * 2
    assert awq_workspace_bytes(16, 14336, 4096, 128) == 16 * 14336 * 2
    assert awq_workspace_bytes(9, 9216, 256, 128) == 9 * 9216 * 2
    # batched shapes: the activation tiles go to LDS untouched, so x' comes from a pre-pass
    assert awq_workspace_bytes(200, 2048, 64, 128) == workspace_bytes(200, 2048, 64, 128) + 200 * 2048 * 2
    assert awq_workspace_bytes(24, 4096, 14336, 128) == 24 * 4096 * 2   # skinny kernel: x' only
    assert awq_workspace_bytes(2048, 8192, 28672, 128) == 2048 * 8192 * 2   # 128x512 tile
    assert awq_workspace_bytes(129, 4224, 28688, 64) == \
        workspace_bytes(129, 4224, 28688, 64) + 129 * 4224 * 2                 # and K split
    assert awq_workspace_bytes(513, 2080, 44048, 32) == (513 * 2080 * 2 + 255) // 256 * 256
    assert awq_workspace_bytes(16, 4096, 4104, 128) == 0   # N % 16: no shape


def test_w4a8_workspace_and_geometry(L):
    from weight_only_int4_w4a16_amd import w4a8_workspace_bytes, w4a8_kernel_name

    def a256(b):
        return (b + 255) // 256 * 256
    # xq (M K bytes), sx and xsum (M * 4 each), and with K split the S int32 partial sums
    assert w4a8_workspace_bytes(2048, 8192, 28672) == a256(2048 * 8192) + 2 * a256(2048 * 4)
    assert w4a8_kernel_name(2048, 8192, 28672) == "w4a8_128x512"
    # 64 x 256 tiles: 1 x 56 = 56 of them, K (32 blocks) cut in 4 slices of 8
    assert w4a8_kernel_name(64, 4096, 14336) == "w4a8_64x256_splitk"
    assert w4a8_workspace_bytes(64, 4096, 14336) == a256(64 * 4096) + 2 * a256(64 * 4) + 4 * 64 * 14336 * 4
    assert w4a8_kernel_name(256, 4096, 14336) == "w4a8_64x256_splitk"          # 224 tiles, S = 2
    assert w4a8_workspace_bytes(256, 4096, 14336) == a256(256 * 4096) + 2 * a256(256 * 4) + 2 * 256 * 14336 * 4
    assert w4a8_kernel_name(1, 1024, 256) == "w4a8_64x256"                      # 8 blocks: no split
    assert w4a8_workspace_bytes(0, 4096, 4096) == 0
    assert w4a8_workspace_bytes(16, 4100, 4096) == 0 and w4a8_kernel_name(16, 4100, 4096) == "none"
    vp = ctypes.c_void_p
    assert L.w4a16_gemm_w4a8(vp(16), 16, 4096, 4096, 0, vp(16), vp(16), vp(16), 0, None, 0, None) == 4
    assert L.w4a16_gemm_w4a8(vp(16), 16, 4072, 4096, 0, vp(16), vp(16), vp(16), 0, vp(256), 1 << 30, None) == 2
    assert L.w4a16_gemm_w4a8(vp(16), 16, 4096, 4096, 0, vp(16), None, vp(16), 0, vp(256), 1 << 30, None) == 1


def test_dispatch_between_decode_and_batched_kernels(L):
    from weight_only_int4_w4a16_amd import kernel_name
    assert kernel_name(16, 4096, 28672, 128).startswith("w4a16_decode")    # x fits in LDS
    assert kernel_name(16, 14336, 4096, 128).startswith("w4a16_decode")    # K N < 2^27
    # 4..16 rows where one round of skinny workgroups fills more than half the chip (K <= 8192):
    # skinny from 8 rows (g128), 4 (groups of 32 or 64, NF4 blocks of 64)
    assert kernel_name(16, 8192, 10240, 128).startswith("w4a16_skinny")   # 160 column tiles
    assert kernel_name(8, 4096, 14336, 128).startswith("w4a16_skinny")
    assert kernel_name(7, 4096, 14336, 128).startswith("w4a16_decode")
    assert kernel_name(4, 4096, 14336, 32).startswith("w4a16_skinny")
    assert kernel_name(3, 4096, 14336, 32).startswith("w4a16_decode")
    assert kernel_name(4, 4096, 14336, 64).startswith("w4a16_skinny")
    assert kernel_name(16, 8192, 8192, 128).startswith("w4a16_decode")    # 128 column tiles
    assert kernel_name(8, 16384, 14336, 128).startswith("w4a16_decode")   # deeper than 8192
    assert kernel_name(11, 8192, 57344, 128).startswith("w4a16_decode")    # fewer than 12 rows
    # x beyond the decode kernel's LDS: skinny up to 8192 deep, batched beyond
    assert kernel_name(12, 8192, 57344, 128).startswith("w4a16_skinny")
    assert kernel_name(16, 28672, 8192, 128).startswith("w4a16_tiled")
    assert kernel_name(17, 2048, 4096, 128).startswith("w4a16_decode")     # K N < 2^24
    # 17..128 rows: skinny up to 8192-deep K; at 17..32 rows for up to 1024 column tiles, at
    # 33..128 rows within one launch round and (8192-deep) from 160 column tiles
    assert kernel_name(17, 4096, 4096, 128).startswith("w4a16_skinny")
    assert kernel_name(32, 4096, 4096, 128).startswith("w4a16_skinny")
    assert kernel_name(128, 4096, 4096, 128).startswith("w4a16_skinny")
    assert kernel_name(17, 4096, 6144, 128).startswith("w4a16_skinny")
    assert kernel_name(32, 4096, 28672, 128).startswith("w4a16_skinny")
    assert kernel_name(24, 8192, 10240, 128).startswith("w4a16_skinny")
    assert kernel_name(64, 8192, 10240, 128).startswith("w4a16_skinny")
    assert kernel_name(32, 8192, 8192, 128).startswith("w4a16_skinny")
    assert kernel_name(64, 8192, 8192, 128).startswith("w4a16_tiled")      # 128 tiles < 160
    assert kernel_name(32, 8192, 57344, 128).startswith("w4a16_skinny")    # 896 tiles <= 1024
    assert kernel_name(32, 8192, 73728, 128).startswith("w4a16_tiled")     # 1152 tiles > 1024
    assert kernel_name(17, 14336, 4096, 128).startswith("w4a16_tiled")     # deeper than 8192
    assert kernel_name(64, 4096, 14336, 128).startswith("w4a16_skinny")
    # 65..128 rows where 64-row tiles would take two rounds: 128-row tiles (K <= 4096)
    assert kernel_name(96, 4096, 14336, 128) == "w4a16_skinny_128x64"     # 224 workgroups
    assert kernel_name(128, 4096, 14336, 128) == "w4a16_skinny_128x64"
    assert kernel_name(128, 8192, 14336, 128) == "w4a16_skinny_128x64"    # 8192 deep, one round
    assert kernel_name(128, 8192, 28672, 128).startswith("w4a16_tiled")   # 448 workgroups
    assert kernel_name(128, 4096, 4096, 128) == "w4a16_skinny_64x64"      # one round of 64 rows
    # 129..256 rows: one round of 64-row tiles filling at least half the chip, K <= 4096
    assert kernel_name(129, 4096, 4096, 128) == "w4a16_skinny_64x64"      # 192 workgroups
    assert kernel_name(256, 4096, 4096, 128) == "w4a16_skinny_64x64"      # 256 workgroups
    assert kernel_name(257, 4096, 4096, 128).startswith("w4a16_tiled")
    assert kernel_name(200, 2048, 64, 128).startswith("w4a16_tiled")      # 4 workgroups
    assert kernel_name(192, 4096, 14336, 128).startswith("w4a16_tiled")
    # up to 6144-deep K the skinny kernel keeps one launch round at 33..256 rows, and from 224
    # rows takes one round of 128-row tiles on 3072..6144-deep weights
    assert kernel_name(96, 5120, 5120, 128) == "w4a16_skinny_64x64"
    assert kernel_name(128, 5120, 13824, 128) == "w4a16_skinny_128x64"
    assert kernel_name(160, 5120, 5120, 128) == "w4a16_skinny_64x64"
    assert kernel_name(256, 4096, 6144, 128) == "w4a16_skinny_128x64"
    assert kernel_name(256, 2048, 8192, 128).startswith("w4a16_tiled")     # K < 3072
    assert kernel_name(160, 4096, 6144, 128) == "w4a16_skinny_128x64"     # from 160 rows, K 4096
    assert kernel_name(192, 3072, 8192, 128).startswith("w4a16_tiled")     # K < 4096 below 224 rows
    assert kernel_name(144, 4096, 6144, 128).startswith("w4a16_tiled")
    assert kernel_name(96, 8192, 10240, 128) == "w4a16_skinny_128x64"     # 128-row tiles to K 8192
    assert kernel_name(64, 8192, 8192, 128).startswith("w4a16_tiled")      # 64-row tiles: K > 6144
    # 16 rows with a quarter to a half of the chip's worth of column tiles, K 3072..6144
    assert kernel_name(16, 5120, 5120, 128).startswith("w4a16_skinny")
    assert kernel_name(12, 5120, 5120, 128).startswith("w4a16_decode")
    assert kernel_name(16, 2048, 8192, 128).startswith("w4a16_decode")
    # groups of 32/64: the quarter-to-half band from 12 rows, one to two rounds from 4 rows
    assert kernel_name(12, 4096, 6144, 32).startswith("w4a16_skinny")
    assert kernel_name(8, 4096, 6144, 32).startswith("w4a16_decode")
    assert kernel_name(12, 2048, 8192, 32).startswith("w4a16_decode")    # K < 3072
    assert kernel_name(4, 8192, 28672, 32).startswith("w4a16_skinny")    # 448 column tiles
    assert kernel_name(4, 8192, 28672, 128).startswith("w4a16_decode")
    assert kernel_name(4, 8192, 36864, 32).startswith("w4a16_decode")    # 576 column tiles


def test_nf4_requires_codebook(L):
    vp = ctypes.c_void_p
    st = L.w4a16_gemm_nf4(vp(16), 1, 4096, 4096, 0, vp(16), vp(16), None, 64, vp(16), 0,
                          vp(256), 1 << 30, None)
    assert st == 1


def test_pack_and_dequant_reject_bad_arguments(L):
    vp = ctypes.c_void_p
    assert L.w4a16_pack(vp(16), 100, 4096, vp(32), None) == 1
    assert L.w4a16_pack(vp(16), 4096, 24, vp(32), None) == 2
    assert L.w4a16_pack(vp(16), 4096, 4096, vp(16), None) == 1      # aliasing
    assert L.w4a16_pack(None, 4096, 4096, vp(16), None) == 1
    assert L.w4a16_dequant(vp(16), vp(16), None, 4096, 4096, 128, 2, vp(16), None) == 1
    assert L.w4a16_dequant_nf4(vp(16), vp(16), None, 4096, 4096, 64, 0, vp(16), None) == 1


def test_kernel_name_and_strings(L):
    from weight_only_int4_w4a16_amd import kernel_name, version
    assert kernel_name(1, 4096, 4096, 128).startswith("w4a16_decode")
    assert kernel_name(0, 4096, 4096, 128) == "none"
    assert kernel_name(16, 4096, 4096, 128).startswith("w4a16_decode")
    # decode parity shapes that run persistent workgroups (256 compute units)
    for M, K, N, g in ((16, 4096, 16416, 128), (13, 3968, 16432, 128), (12, 4224, 32784, 64),
                       (15, 2080, 32784, 32), (12, 4096, 16416, 128), (8, 4096, 32784, 32),
                       (16, 4096, 28672, 128)):
        assert kernel_name(M, K, N, g).endswith("_persist"), (M, K, N, g)
    assert not kernel_name(1, 4096, 28672, 128).endswith("_persist")
    assert kernel_name(17, 4096, 4096, 128).startswith("w4a16_skinny")
    assert kernel_name(17, 4096, 6144, 128).startswith("w4a16_skinny")
    assert kernel_name(65, 4096, 4096, 128).startswith("w4a16_skinny")
    assert kernel_name(65, 14336, 4096, 128).startswith("w4a16_tiled")
    # the ragged full-size parity shapes land on each batched geometry (256 compute units)
    assert kernel_name(257, 2080, 44048, 32) == "w4a16_tiled_64x256"
    assert kernel_name(513, 2080, 44048, 32) == "w4a16_tiled_128x512"
    assert kernel_name(129, 4224, 28688, 64) == "w4a16_tiled_128x512_splitk"
    assert kernel_name(2048, 8192, 28672, 128) == "w4a16_tiled_128x512"
    # the medium tile replaces the unsplit two-k-group small tile for groups of 32 or 64
    # (NF4 blocks of 64 too) from 192 rows on, and only there
    assert kernel_name(256, 4096, 14336, 128) == "w4a16_tiled_64x256_kg2"
    assert kernel_name(256, 4096, 14336, 32) == "w4a16_tiled_128x128_kg2"
    assert kernel_name(256, 4096, 14336, 64) == "w4a16_tiled_128x128_kg2"
    assert kernel_name(192, 4096, 14336, 32) == "w4a16_tiled_128x128_kg2"
    assert kernel_name(128, 4096, 14336, 32) == "w4a16_skinny_128x64"
    assert kernel_name(512, 4096, 14336, 32) == "w4a16_tiled_64x256"
    for s in range(5):
        assert L.w4a16_status_string(s)
    assert version()


def test_oracle_and_product_share_no_code():
    """The oracle imports nothing from the product package and vice versa (the seeded
    input module ``synth`` is the one shared piece and holds none of the method)."""
    prod = os.path.join(ROOT, "weight_only_int4_w4a16_amd")
    orc = os.path.join(ROOT, "oracle")
    for d, banned in ((orc, r"weight_only_int4_w4a16_amd|synth"), (prod, r"\boracle\b")):
        for dirpath, _, files in os.walk(d):
            for f in files:
                if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h", ".c")):
                    text = open(os.path.join(dirpath, f)).read()
                    code = re.sub(r'""".*?"""', "", text, flags=re.S)
                    imports = [ln for ln in code.splitlines()
                               if re.match(r"\s*(import|from|#include)\b", ln)]
                    for ln in imports:
                        assert not re.search(banned, ln), f"{f}: {ln}"


def test_synth_module_holds_no_method_arithmetic():
    src = open(os.path.join(ROOT, "weight_only_int4_w4a16_amd", "synth.py")).read()
    for banned in ("rint", "clip(", "matmul", "@", "dequant", "<< np.uint32(4"):
        assert banned not in src.split('"""', 2)[-1], banned


# ---------------------------------------------------------------- binding tensor checks
# The C ABI receives no buffer sizes, so the binding checks every tensor against the shape
# the call implies before a pointer is taken. These run on CPU tensors: a well-shaped call
# gets as far as the device check ("device tensors"); a mis-shaped one must stop earlier,
# at the shape check.

def _cpu_affine(M=4, K=256, N=64, g=128, dt=None, zeros=True):
    import torch
    from weight_only_int4_w4a16_amd import packed_bytes
    dt = torch.float16 if dt is None else dt
    return dict(x=torch.zeros((M, K), dtype=dt), packed=torch.zeros(packed_bytes(K, N) // 4, dtype=torch.int32),
                scales=torch.zeros((K // g, N), dtype=dt),
                qzeros=torch.zeros((K // g, N // 8), dtype=torch.int32) if zeros else None, g=g)


def _raises_arg(fn, match):
    from weight_only_int4_w4a16_amd import W4A16Error
    with pytest.raises(W4A16Error, match=match) as e:
        fn()
    assert e.value.status == 1


def test_binding_well_shaped_call_reaches_the_device_check():
    import weight_only_int4_w4a16_amd as w4
    a = _cpu_affine()
    _raises_arg(lambda: w4.gemm(a["x"], a["packed"], a["scales"], a["qzeros"], a["g"]), "device tensors")


@pytest.mark.parametrize("what", ["out_rows", "out_cols", "out_dtype", "scales_rows", "scales_dtype",
                                  "qzeros_cols", "packed_short", "x_1d", "workspace_short"])
def test_binding_gemm_rejects_wrong_shapes(what):
    import torch
    import weight_only_int4_w4a16_amd as w4
    # (the short-workspace case needs a shape whose kernel takes a workspace: K split)
    a = _cpu_affine(M=200, K=2048, N=64) if what == "workspace_short" else _cpu_affine(M=40, K=4096, N=4096)
    kw = {}
    if what == "out_rows":
        kw["out"] = torch.zeros((39, 4096), dtype=torch.float16)
    elif what == "out_cols":
        kw["out"] = torch.zeros((40, 4080), dtype=torch.float16)
    elif what == "out_dtype":
        kw["out"] = torch.zeros((40, 4096), dtype=torch.bfloat16)
    elif what == "scales_rows":
        a["scales"] = torch.zeros((31, 4096), dtype=torch.float16)
    elif what == "scales_dtype":
        a["scales"] = torch.zeros((32, 4096), dtype=torch.float32)
    elif what == "qzeros_cols":
        a["qzeros"] = torch.zeros((32, 256), dtype=torch.int32)
    elif what == "packed_short":
        a["packed"] = a["packed"][:-1]
    elif what == "x_1d":
        a["x"] = torch.zeros(4096, dtype=torch.float16)
    elif what == "workspace_short":
        need = w4.workspace_bytes(200, 2048, 64, 128)
        assert need > 0
        kw["workspace"] = torch.zeros(need - 1, dtype=torch.uint8)
    _raises_arg(lambda: w4.gemm(a["x"], a["packed"], a["scales"], a["qzeros"], a["g"], **kw),
                "shape|dtype|bytes|2-D")


def test_binding_other_entry_points_reject_wrong_shapes():
    import torch
    import weight_only_int4_w4a16_amd as w4
    from weight_only_int4_w4a16_amd import packed_bytes
    a = _cpu_affine(M=2, K=512, N=64, g=64)
    x, pk, sc, qz = a["x"], a["packed"], a["scales"], a["qzeros"]
    absmax = torch.zeros((8, 64), dtype=torch.float16)
    cb = torch.zeros(16, dtype=torch.float16)
    m = "shape|dtype|bytes|2-D|even"
    _raises_arg(lambda: w4.gemm_nf4(x, pk, absmax, torch.zeros(15, dtype=torch.float16), 64), m)
    _raises_arg(lambda: w4.gemm_nf4(x, pk, absmax[:7], cb, 64), m)
    _raises_arg(lambda: w4.gemm_nf4(x, pk, absmax, cb, 64, out=torch.zeros((2, 32), dtype=torch.float16)), m)
    _raises_arg(lambda: w4.gemm_awq(x, torch.zeros(511, dtype=torch.float16), pk, sc, qz, 64), m)
    _raises_arg(lambda: w4.gemm_awq(x, torch.zeros(512, dtype=torch.bfloat16), pk, sc, qz, 64), m)
    _raises_arg(lambda: w4.gemm_swiglu(x, pk, sc, qz, 64, out=torch.zeros((2, 64), dtype=torch.float16)), m)
    _raises_arg(lambda: w4.gemm_nf4_swiglu(x, pk, absmax, cb, 64, out=torch.zeros((2, 64), dtype=torch.float16)), m)
    _raises_arg(lambda: w4.gemm_w4a8(x, pk, torch.zeros((64,), dtype=torch.float16),
                                     out=torch.zeros((2, 63), dtype=torch.float16)), m)
    _raises_arg(lambda: w4.gemm_w4a8(x, pk[:10], torch.zeros((64,), dtype=torch.float16)), m)
    _raises_arg(lambda: w4.dequant(pk, sc[:3], qz, 512, 64), m)
    _raises_arg(lambda: w4.dequant(pk[: packed_bytes(512, 64) // 8], sc, qz, 512, 64), m)
    _raises_arg(lambda: w4.dequant_nf4(pk, absmax, cb[:8], 512, 64), m)
    _raises_arg(lambda: w4.dequant_nf4(pk, absmax, cb, 512, 128), m)
