"""The C-ABI library loads and exports what include/mk.h declares, and its
host-side checks reject bad arguments before touching the GPU (CPU only)."""
import json
import os

import pytest

from mixture_experts_layer_device_amd import binding as B  # noqa: E402  (fails loudly if not built)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_every_declared_function_is_exported():
    names = B.declared_functions()
    assert len(names) >= 14
    missing = [n for n in names if not hasattr(B.lib, n)]
    assert not missing, missing


def test_header_constants_parsed():
    assert B.MK_OK == 0 and B.MK_ERR_SHAPE == -2 and B.MK_DEVERR_SCHED_OVERFLOW == 2
    assert B.MK_FULL_LAYER == 0 and B.MK_EXPERT_SHARE == 1 and B.MK_MXFP8 == 1


def test_two_wave_rule_host_side():
    g = json.load(open(os.path.join(GOLDEN, "two_wave_floor.json")))
    assert B.mk_two_wave_rows(g["H"], g["I"], g["n_cu"], g["tile_m"], g["tile_n"]) == g["rows"]
    assert B.mk_two_wave_rows(7168, 2048, 256, 256, 256) == 8192


def test_config_defaults():
    c = B.mk_config_default()
    assert c.minibatch_rows == 0 and c.precision == B.MK_BF16 and c.ring_bytes == 256 << 20
    assert c.sched_capacity_mult == 1.0 and c.renorm == 1 and c.enable_backward == 0


@pytest.mark.parametrize("kw,code", [
    (dict(H=100), B.MK_ERR_SHAPE), (dict(I=96), B.MK_ERR_SHAPE), (dict(max_rows=0), B.MK_ERR_SHAPE),
    (dict(E=0), B.MK_ERR_LIMIT), (dict(E=2000), B.MK_ERR_LIMIT), (dict(k=33), B.MK_ERR_LIMIT),
])
def test_workspace_rejects_bad_shapes(kw, code):
    args = dict(max_rows=1024, H=256, I=128, E=8, k=2)
    args.update(kw)
    with pytest.raises(B.MkError) as ei:
        B.mk_workspace_create(B.mk_config_default(), **args)
    assert ei.value.status == code


def test_workspace_rejects_bad_config():
    c = B.mk_config_default()
    c.minibatch_rows = 4096
    c.ring_bytes = 4096 * 512 - 1            # smaller than one minibatch of H=256 bf16 rows
    with pytest.raises(B.MkError) as ei:
        B.mk_workspace_create(c, 8192, 256, 128, 8, 2)
    assert ei.value.status == B.MK_ERR_RING
    c = B.mk_config_default(); c.precision = 7
    with pytest.raises(B.MkError) as ei:
        B.mk_workspace_create(c, 8192, 256, 128, 8, 2)
    assert ei.value.status == B.MK_ERR_CONFIG
    c = B.mk_config_default(); c.sched_capacity_mult = 0.0
    with pytest.raises(B.MkError) as ei:
        B.mk_workspace_create(c, 8192, 256, 128, 8, 2)
    assert ei.value.status == B.MK_ERR_CONFIG
    # a workspace with the backward (bf16 or MXFP8) tiles I by 256
    c = B.mk_config_default(); c.precision = B.MK_MXFP8; c.enable_backward = 1
    with pytest.raises(B.MkError) as ei:
        B.mk_workspace_create(c, 8192, 256, 128, 8, 2)
    assert ei.value.status == B.MK_ERR_SHAPE
    c = B.mk_config_default(); c.enable_backward = 1
    with pytest.raises(B.MkError) as ei:
        B.mk_workspace_create(c, 8192, 256, 384, 8, 2)
    assert ei.value.status == B.MK_ERR_SHAPE


def test_quantize_rejects_bad_k_without_gpu():
    with pytest.raises(B.MkError) as ei:
        B.mk_mxfp8_quantize(1, 4, 48, 1, 1)
    assert ei.value.status == B.MK_ERR_SHAPE


def test_status_strings():
    assert B.mk_status_string(0) == "ok"
    assert "ring" in B.mk_status_string(B.MK_ERR_RING)


def test_wgrad_mxfp8_needs_mxfp8_and_the_backward():
    for prec, bwd in ((B.MK_BF16, 1), (B.MK_MXFP8, 0)):
        c = B.mk_config_default(); c.precision = prec; c.enable_backward = bwd; c.wgrad_mxfp8 = 1
        with pytest.raises(B.MkError) as ei:
            B.mk_workspace_create(c, 8192, 256, 256, 8, 2)
        assert ei.value.status == B.MK_ERR_CONFIG, (prec, bwd)


def test_config_struct_layout_matches_the_header(tmp_path):
    """sizeof and every field offset of mk_config as a C compiler lays it out
    from include/mk.h, against the binding's ctypes structure."""
    import ctypes
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    fields = [f[0] for f in B.MkConfig._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "mk.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(mk_config));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(mk_config, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(B.MkConfig)
    assert got[1:] == [getattr(B.MkConfig, f).offset for f in fields]


def test_wgrad_mxfp8_row_space_limit():
    """Many experts over tiny minibatches: the weight gradients' padded row
    space (every segment rounded up to 32 rows) would pass the quantisers'
    grid limit, so the workspace is refused before any allocation."""
    c = B.mk_config_default(); c.precision = B.MK_MXFP8; c.enable_backward = 1; c.wgrad_mxfp8 = 1
    c.minibatch_rows = 32
    with pytest.raises(B.MkError) as ei:
        B.mk_workspace_create(c, 1 << 20, 256, 256, 1024, 8)
    assert ei.value.status == B.MK_ERR_LIMIT


def test_minibatch_count_limit():
    c = B.mk_config_default()
    c.minibatch_rows = 8
    with pytest.raises(B.MkError) as ei:
        B.mk_workspace_create(c, 8 * 65536, 256, 128, 8, 2)
    assert ei.value.status == B.MK_ERR_LIMIT


def test_fused_forward_needs_bf16():
    c = B.mk_config_default()
    c.precision = B.MK_MXFP8
    c.fused_forward = 1
    with pytest.raises(B.MkError) as ei:
        B.mk_workspace_create(c, 4096, 256, 256, 8, 2)
    assert ei.value.status == B.MK_ERR_CONFIG


def test_debug_fused_waits_rejects_a_null_workspace():
    assert B.lib.mk_debug_fused_waits(None, 0, 0) == B.MK_ERR_NULL
