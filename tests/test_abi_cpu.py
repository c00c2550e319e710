"""Host-side checks of the C ABI: the library loads, exports every entry
point the header declares, and rejects bad arguments before launching."""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    from mixture_experts_layer_wave_amd import binding as B

    decl = _declared()
    assert len(decl) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (moe_\w+)", out))
    for name in decl:
        assert name in exported, name
        assert name in B.EXPORTS, name
        getattr(B.lib, name)


def test_abi_version_and_status_strings():
    from mixture_experts_layer_wave_amd import binding as B

    ver = int(re.search(r"#define MOE_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert B.moe_abi_version() == ver
    for st in range(0, -7, -1):
        assert B.moe_status_string(st) != "unknown status"
    assert B.moe_status_string(-99) == "unknown status"


def test_workspace_bytes():
    from mixture_experts_layer_wave_amd import binding as B

    n, d, E, k, f = 4096, 1024, 8, 1, 4096
    ws = B.moe_workspace_bytes((n, d, E, k, f), "bf16")
    R = n * k
    # hidden [R][d_ff] bf16 and pile outputs [R][d] f32 dominate
    assert ws >= R * f * 2 + R * d * 4 + n * E * 4
    assert ws % 256 == 0
    assert B.moe_workspace_bytes((n, d, E, 9, f), "bf16") == 0  # k > E
    assert B.moe_workspace_bytes((n, d, E, k, f), 7) == 0


def test_workspace_holds_the_down_pass_planes_the_tile_plan_needs():
    """The bf16 down pass's block tile and K split are chosen on the host from
    the shape, and the workspace sizes the f32 planes they need.  With about
    512 rows per expert (Switch-shaped, one expert per token) 320 x 256 tiles
    in four K splits make one round of 256 blocks: four planes of the pile
    outputs.  With about 2048 rows per expert (Mixtral-shaped, top-2) the
    pass runs unsplit over 3.5 rounds of 320 x 256 tiles, and the piles' last
    row tiles take the two-way tail split: two planes of E x 320 rows."""
    from mixture_experts_layer_wave_amd import binding as B

    def extra(n, d, E, k, f):
        R = n * k
        splits = -(-d // 256)  # router K splits (256-deep, d a multiple of 32 here)
        small = R * f * 2 + R * d * 4 + splits * n * E * 4  # hidden, pile outputs, logits
        return B.moe_workspace_bytes((n, d, E, k, f), "bf16") - small, R

    got, R = extra(4096, 1024, 8, 1, 4096)
    planes = 4 * R * 1024 * 4
    assert planes <= got < planes + (1 << 20)
    got, R = extra(8192, 4096, 8, 2, 14336)
    tail = 2 * 8 * 320 * 4096 * 4
    assert tail <= got < tail + (1 << 20)


@pytest.mark.parametrize("shape,status", [
    (None, -1),
    ((0, 8, 4, 1, 8), -2),
    ((4, 8, 4, 5, 8), -2),
    ((4, 8, 1025, 1, 8), -2),
    ((4, 8, 64, 33, 8), -2),
    ((4, 8, 4, 1, 8, 2), -2),
])
def test_forward_rejects_bad_shapes_before_launch(shape, status):
    import ctypes

    from mixture_experts_layer_wave_amd import binding as B

    sp = None if shape is None else ctypes.byref(B._shape(shape))
    w = B.ExpertWeights(1, None, None, None, None, None, None)
    assert B.lib.moe_forward(sp, None, 1, None, None, ctypes.byref(w), None, 1, None, None, None, 0, None) == status


def test_dtype_and_null_errors_before_launch():
    import ctypes

    from mixture_experts_layer_wave_amd import binding as B

    sp = ctypes.byref(B._shape((4, 64, 4, 2, 64)))
    w = B.ExpertWeights(1, None, None, None, None, None, None)
    # bf16 weights with f32 activations: dtype error, checked first
    assert B.lib.moe_forward(sp, None, 0, None, None, ctypes.byref(w), None, 1, None, None, None, 0, None) == -3
    # MXFP4 needs d % 32 == 0
    sp2 = ctypes.byref(B._shape((4, 40, 4, 2, 64)))
    w4 = B.ExpertWeights(2, None, None, None, None, None, None)
    assert B.lib.moe_forward(sp2, None, 1, None, None, ctypes.byref(w4), None, 1, None, None, None, 0, None) == -2
    # missing weight pointers
    assert B.lib.moe_forward(sp, None, 1, None, None, ctypes.byref(w), None, 1, None, None, None, 0, None) == -1
    assert B.lib.moe_router_topk(sp, None, 1, None, None, None, None, None, None) == -1
    assert B.lib.moe_combine(sp, None, 1, None, None, None, 1, None) == -1
    assert B.lib.moe_dispatch(sp, None, None, None, None, None, None, 1, None, None, 0, None) == -1


def test_product_path_fails_loudly_without_library(tmp_path):
    """Importing the binding from a copy of the package without the built
    library raises instead of falling back to anything."""
    import shutil
    import sys

    pkg = os.path.join(ROOT, "mixture_experts_layer_wave_amd")
    dst = tmp_path / "mixture_experts_layer_wave_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    code = "import mixture_experts_layer_wave_amd.binding"
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0 and "not built" in r.stderr


def test_router_stats_errors_before_launch():
    import ctypes

    from mixture_experts_layer_wave_amd import binding as B

    shape = (100, 64, 8, 2, 64)
    sp = ctypes.byref(B._shape(shape))
    need = B.moe_router_stats_workspace_bytes(shape)
    assert need >= 100 * 8 and need % 256 == 0
    assert B.moe_router_stats_workspace_bytes((0, 64, 8, 2, 64)) == 0
    fake = 1 << 20  # never dereferenced: every check below fails before a launch
    assert B.lib.moe_router_stats(None, fake, fake, 1.0, fake, fake, fake, fake, need, None) == -1
    assert B.lib.moe_router_stats(sp, None, fake, 1.0, fake, fake, fake, fake, need, None) == -1
    assert B.lib.moe_router_stats(sp, fake, fake, 1.0, fake, fake, None, fake, need, None) == -1
    assert B.lib.moe_router_stats(sp, fake, fake, 1.0, fake, fake, fake, None, need, None) == -5
    assert B.lib.moe_router_stats(sp, fake, fake, 1.0, fake, fake, fake, fake, need - 1, None) == -5
    assert B.lib.moe_router_stats(sp, fake, fake, 1.0, fake, fake, fake, fake + 4, need, None) == -4


def test_slots_and_active_experts_errors_before_launch():
    import ctypes

    from mixture_experts_layer_wave_amd import binding as B

    shape = (16, 64, 8, 2, 64)
    sp = ctypes.byref(B._shape(shape))
    fake = 1 << 20  # never dereferenced: every check below fails before a launch
    assert B.lib.moe_active_experts(None, fake, fake, fake, None) == -1
    assert B.lib.moe_active_experts(sp, None, fake, fake, None) == -1
    assert B.lib.moe_active_experts(sp, fake, fake, None, None) == -1
    assert B.lib.moe_active_experts(ctypes.byref(B._shape((0, 64, 8, 2, 64))), fake, fake, fake, None) == -2
    # a slot table needs at least one physical slot
    w = B.ExpertWeights(1, fake, fake, fake, None, None, None, fake, 0)
    y = fake
    assert B.lib.moe_expert_down(sp, fake, fake, ctypes.byref(w), y, None) == -2


def test_w4a8_sizes_and_errors_before_launch():
    import ctypes

    from mixture_experts_layer_wave_amd import binding as B

    # MXFP8 matrix: codes, then scales from a 256-B boundary, pitch rounded to 4
    assert B.moe_mxfp8_bytes(3, 96) == 512 + 3 * 4
    assert B.moe_mxfp8_bytes(4096, 2880) == 4096 * 2880 + 4096 * 92
    assert B.moe_mxfp8_bytes(0, 64) == 0
    assert B.moe_mxfp8_bytes(4, 40) == 0 and B.moe_mxfp8_bytes(-1, 64) == 0
    fake = 1 << 20  # never dereferenced: every check below fails before a launch
    assert B.lib.moe_quantize_mxfp8(4, 40, fake, 1, fake, None) == -2
    assert B.lib.moe_quantize_mxfp8(4, 64, fake, 2, fake, None) == -3
    assert B.lib.moe_quantize_mxfp8(4, 64, None, 1, fake, None) == -1
    assert B.lib.moe_quantize_mxfp8(4, 64, fake + 8, 1, fake, None) == -4
    assert B.lib.moe_quantize_mxfp8(0, 64, None, 1, None, None) == 0

    mx8 = B.MOE_MXFP8
    big_ws = 1 << 30
    sp = ctypes.byref(B._shape((16, 64, 8, 2, 64)))
    fwd = lambda shape, w: B.lib.moe_forward(shape, fake, 1, fake, None, ctypes.byref(w), fake, 1,
                                             None, None, fake, big_ws, None)
    # the W4A8 mode needs MXFP4 weights, and a known mode
    assert fwd(sp, B.ExpertWeights(1, fake, fake, fake, None, None, None, None, 0, mx8)) == -3
    assert fwd(sp, B.ExpertWeights(2, fake, fake, fake, fake, fake, fake, None, 0, 7)) == -3
    w4 = B.ExpertWeights(2, fake, fake, fake, fake, fake, fake, None, 0, mx8)
    # K past what the GEMM keeps of a tile's weight scales
    assert fwd(ctypes.byref(B._shape((16, 7200, 8, 2, 64))), w4) == -2
    assert fwd(ctypes.byref(B._shape((16, 64, 8, 2, 7200))), w4) == -2
    # moe_expert_up in the mode takes MXFP8 rows (act = MOE_MXFP8), aligned
    assert B.lib.moe_expert_up(sp, fake, 1, None, fake, ctypes.byref(w4), fake, None) == -3
    assert B.lib.moe_expert_up(sp, None, mx8, None, fake, ctypes.byref(w4), fake, None) == -1
    assert B.lib.moe_expert_up(sp, fake + 8, mx8, None, fake, ctypes.byref(w4), fake, None) == -4
    # MXFP8 rows without the mode
    w0 = B.ExpertWeights(2, fake, fake, fake, fake, fake, fake, None, 0, 0)
    assert B.lib.moe_expert_up(sp, fake, mx8, None, fake, ctypes.byref(w0), fake, None) == -3
    assert B.lib.moe_grouped_ffn(sp, fake, mx8, fake, ctypes.byref(w0), fake, 0, fake, big_ws, None) == -3
    # the workspace of MXFP4 covers the mode's encoded input and hidden
    n, d, E, k, f = 4096, 2880, 128, 4, 2880
    R = n * k
    ws = B.moe_workspace_bytes((n, d, E, k, f), "mxfp4")
    assert ws >= B.moe_mxfp8_bytes(R, d) + B.moe_mxfp8_bytes(R, f)


def test_boundary_choices_before_launch():
    """The boundary's documented choices, checked before anything launches:
    moe_router_topk needs a logits buffer (the library holds no device
    memory of its own); moe_grouped_ffn writes f32 or bf16 pile outputs and
    moe_combine reads either; the
    workspace size is a function of the shape and the weight dtype; the
    expert GEMMs' 32-bit operand offsets bound the batch."""
    import ctypes

    from mixture_experts_layer_wave_amd import binding as B

    fake = 1 << 20  # never dereferenced: every call below fails before a launch
    sp = ctypes.byref(B._shape((16, 64, 8, 2, 64)))
    # logits = NULL is rejected
    assert B.lib.moe_router_topk(sp, fake, 1, fake, None, None, fake, fake, None) == -1
    # grouped FFN: F32 and BF16 outputs pass the dtype check (and then stop at
    # the misaligned output); other output dtypes do not
    w = B.ExpertWeights(1, fake, fake, fake, None, None, None)
    big = 1 << 30
    ffn = lambda out, y: B.lib.moe_grouped_ffn(sp, fake, 1, fake, ctypes.byref(w), y, out, fake, big, None)
    assert ffn(B.MOE_BF16, fake + 8) == -4
    assert ffn(B.MOE_F32, fake + 8) == -4
    assert ffn(B.MOE_MXFP4, fake) == -3
    assert ffn(B.MOE_MXFP8, fake) == -3
    # workspace: (shape, weight dtype); MXFP8 is not a weight dtype
    assert B.moe_workspace_bytes((16, 64, 8, 2, 64), "bf16") > 0
    assert B.moe_workspace_bytes((16, 64, 8, 2, 64), "mxfp4") > 0
    assert B.moe_workspace_bytes((16, 64, 8, 2, 64), "mxfp8") == 0
    # n k max(d, d_ff) must stay below 2^30 with bf16 / MXFP4 weights
    fwd = lambda shape, wd: B.lib.moe_forward(ctypes.byref(B._shape(shape)), fake, 1, fake, None,
                                              ctypes.byref(B.ExpertWeights(wd, fake, fake, fake, fake, fake, fake)),
                                              fake, 1, None, None, fake, 1 << 40, None)
    # combine: f32 or bf16 pile outputs in; bf16 in needs d % 8 == 0
    comb = lambda shape, din: B.lib.moe_combine(ctypes.byref(B._shape(shape)), fake, din, fake,
                                                fake, fake, 1, None)
    assert comb((16, 60, 8, 2, 64), B.MOE_BF16) == -2
    assert comb((16, 60, 8, 2, 64), B.MOE_MXFP4) == -3
    assert comb((16, 64, 8, 2, 64), B.MOE_MXFP8) == -3
    assert fwd((65536, 4096, 8, 2, 14336), 1) == -2   # 131072 x 14336 rows of bf16 hidden
    assert fwd((16, 32768, 8, 2, 32768), 2) == -2     # one expert matrix past 2^30 elements
