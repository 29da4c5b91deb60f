"""The C ABI library: it loads without a GPU, exports every declared symbol and
validates arguments on the host (no device work is started here)."""

import ctypes
import os
import re

import pytest

from free_block_sparse_amd import SparseprConfig, make_config, sparsepr_config_default, sparsepr_validate
from free_block_sparse_amd import _lib
from free_block_sparse_amd._lib import SparseprHeadStats, SparseprTensors, lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sparsepr.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparsepr_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "sparsepr_attention" in names and len(names) >= 12
    handle = lib()
    for n in names:
        assert hasattr(handle, n), n
    # and the binding declares a signature for each of them
    assert set(names) <= set(_lib._SIGS), set(names) - set(_lib._SIGS)


def test_struct_sizes_match_header_layout(tmp_path):
    """Sizes and field offsets of the ctypes structures equal what a C
    compiler makes of include/sparsepr.h."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"sparsepr_config": SparseprConfig, "sparsepr_tensors": SparseprTensors,
               "sparsepr_head_stats": SparseprHeadStats}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "sparsepr.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-std=c11", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                          check=True).stdout.splitlines())
    for cname, cls in structs.items():
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(cls, f).offset, (cname, f)


def test_config_defaults():
    cfg = sparsepr_config_default(32760, 128)
    assert cfg.density == pytest.approx(0.25) and cfg.probe_rows == 64
    assert cfg.n_kv_groups == 255 and cfg.n_q_groups == 255
    assert cfg.residual_rank == 32 and cfg.kmeans_iters == 10
    assert cfg.n_sample_q == 256 and cfg.key_coord_rank == 32
    assert cfg.ridge_lambda == pytest.approx(1.0) and cfg.ridge_mode == 0
    assert cfg.router == 0 and cfg.alpha == pytest.approx(0.9)
    assert sparsepr_config_default(100000, 64).n_kv_groups == 256


@pytest.mark.parametrize("field,value", [
    ("density", 0.0), ("density", -1.0), ("probe_rows", -1), ("probe_rows", 300),
    ("n_kv_groups", 0), ("n_q_groups", 2000), ("residual_rank", 65), ("ridge_lambda", -1.0),
    ("kmeans_iters", 0), ("n_sample_q", 0), ("n_sample_q", 257), ("key_coord_rank", 0),
    ("rank_cut", 1.0), ("partition_mode", 7), ("ridge_mode", 2), ("router", 2),
])
def test_validation_rejects_bad_settings(field, value):
    cfg = make_config(4096, 64, n_kv_groups=32, n_q_groups=32)
    assert sparsepr_validate(cfg, 1, 2, 4096, 64, 0) == 0
    setattr(cfg, field, value)
    assert sparsepr_validate(cfg, 1, 2, 4096, 64, 0) != 0


def test_validation_rejects_bad_shapes():
    cfg = make_config(4096, 64)
    assert sparsepr_validate(cfg, 1, 2, 4096, 96, 0) == -2     # head dim
    assert sparsepr_validate(cfg, 1, 2, 4096, 64, 5) == -2     # dtype
    assert sparsepr_validate(cfg, 0, 2, 4096, 64, 0) == -1     # batch
    assert sparsepr_validate(cfg, 1, 2, 1, 64, 0) == -1        # N
    small = make_config(4096, 64, n_kv_groups=64)
    assert sparsepr_validate(small, 1, 1, 50, 64, 0) == -1     # more groups than tokens


def test_workspace_grows_with_the_problem():
    cfg = make_config(8192, 64, n_kv_groups=64, n_q_groups=64)
    n = ctypes.c_size_t(0)
    sizes = []
    for N in (1024, 4096, 8192):
        assert lib().sparsepr_workspace_size(ctypes.byref(cfg), 1, 2, N, 64, 0, ctypes.byref(n)) == 0
        sizes.append(n.value)
    assert sizes[0] < sizes[1] < sizes[2] and sizes[0] % 256 == 0


def test_entry_points_reject_null_arguments_before_any_device_work():
    cfg = make_config(1024, 64, n_kv_groups=16, n_q_groups=16)
    io = SparseprTensors()
    io.B, io.H, io.N, io.d, io.dtype = 1, 1, 1024, 64, 0
    for arr in (io.q_strides, io.k_strides, io.v_strides, io.o_strides):
        arr[0], arr[1], arr[2], arr[3] = 65536, 65536, 64, 1
    # null tensor pointers
    assert lib().sparsepr_attention(ctypes.byref(cfg), ctypes.byref(io), None, 0, None, None) == -1
    assert lib().sparsepr_dense_attention(None, 0.0, None) == -1
    assert lib().sparsepr_workspace_size(None, 1, 1, 1024, 64, 0, None) == -1
    # misaligned pointer / non-unit d stride are reported as unsupported layouts
    io.q = io.k = io.v = 0x1000
    io.o = 0x2008
    assert lib().sparsepr_attention(ctypes.byref(cfg), ctypes.byref(io), None, 0, None, None) == -2
    io.o = 0x2000
    io.q_strides[3] = 2
    assert lib().sparsepr_attention(ctypes.byref(cfg), ctypes.byref(io), None, 0, None, None) == -2
    io.q_strides[3] = 1
    # missing / too small workspace
    assert lib().sparsepr_attention(ctypes.byref(cfg), ctypes.byref(io), None, 0, None, None) == -1
    assert lib().sparsepr_attention(ctypes.byref(cfg), ctypes.byref(io), 0x10000, 1024, None, None) == -3


def test_status_strings():
    assert lib().sparsepr_status_string(0) == b"ok"
    assert b"workspace" in lib().sparsepr_status_string(-3)


@pytest.mark.parametrize("alpha,ok", [(0.9, True), (1.0, True), (0.0, False), (-0.1, False), (1.5, False)])
def test_alpha_router_target_must_lie_in_0_1(alpha, ok):
    cfg = make_config(4096, 64, n_kv_groups=32, n_q_groups=32, router="alpha", alpha=alpha)
    assert (sparsepr_validate(cfg, 1, 2, 4096, 64, 0) == 0) == ok


def test_noalloc_rejects_requests_beyond_its_scratch_before_any_device_call():
    """A call whose workspace exceeds the fixed scratch returns the workspace
    error from the host-side checks, before the library touches a device
    (the pointers below are never dereferenced)."""
    import free_block_sparse_amd as sp
    from free_block_sparse_amd import _lib

    L = _lib.lib()
    H, N, d = 40, 32760, 128
    cfg = sp.make_config(N, d, n_kv_groups=256, n_q_groups=256)
    nb = ctypes.c_size_t(0)
    assert L.sparsepr_workspace_size(ctypes.byref(cfg), 1, H, N, d, 0, ctypes.byref(nb)) == 0
    assert nb.value > L.sparsepr_noalloc_scratch_bytes()
    io = _lib.SparseprTensors()
    fake = [4096, 8192, 12288, 16384]
    io.q, io.k, io.v, io.o = fake
    st = [H * N * d, N * d, d, 1]
    for f in ("q_strides", "k_strides", "v_strides", "o_strides"):
        getattr(io, f)[:] = st
    io.B, io.H, io.N, io.d, io.dtype = 1, H, N, d, 0
    assert L.sparsepr_attention_noalloc(ctypes.byref(cfg), ctypes.byref(io), None, None) == -3
