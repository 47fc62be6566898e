"""The C ABI library: it builds, loads, and exports every entry point that
include/fg.h declares; host-only calls behave as documented (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

from sync_protocols_amd import fg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "fg.h")).read()
    return sorted(set(re.findall(r"^(?:fg_status|const char\*)\s+(fg_\w+)\(", src, re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("fg_init", "fg_gather_gemm", "fg_barrier", "fg_stats", "fg_destroy", "fg_strerror"):
        assert n in names
    assert set(names) == set(fg.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = fg.load_library()
    for n in _declared():
        assert hasattr(lib, n), n


def test_strerror_and_capacity_host_only():
    assert fg.strerror(fg.ETIMEOUT) == "device wait timed out"
    cfg = fg.make_config(4, 2048, 4096, 4096)
    assert fg.capacity(cfg) == 8192
    cfg = fg.make_config(8, 8192, 7168, 2048, n_groups=8)
    assert fg.capacity(cfg) == ((8 * 8192 + 8 * 127 + 127) // 128) * 128


@pytest.mark.parametrize("bad", [dict(K=100), dict(K=64), dict(N=100), dict(n_shards=0), dict(n_shards=65),
                                 dict(n_groups=0), dict(tile_n=64)])
def test_capacity_rejects_bad_configs(bad):
    args = dict(n_shards=4, max_rows_per_shard=256, K=256, N=512)
    args.update(bad)
    cfg = fg.make_config(**args)
    out = C.c_int32(0)
    assert fg.load_library().fg_capacity(C.byref(cfg), C.byref(out)) == fg.EINVAL


def test_null_arguments_rejected_without_gpu():
    lib = fg.load_library()
    assert lib.fg_init(None, 0, None) == fg.EINVAL
    assert lib.fg_destroy(None) == fg.EINVAL
    assert lib.fg_stats(None, None, 0) == fg.EINVAL
    assert lib.fg_litmus(None, 10, 0, None) == fg.EINVAL
    assert lib.fg_combine(None, None, None, None, None, 0, None) == fg.EINVAL


def _c_layout(tmp_path):
    """sizeof / offsetof of every ABI struct field, from the C header compiled with gcc."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are not available")
    structs = {"fg_config": fg.FgConfig, "fg_stats_t": fg.FgStats, "fg_route": fg.FgRoute, "fg_views_t": fg.FgViews}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "fg.h"', 'int main(void) {']
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    return structs, dict((" ".join(l.split()[:2]), int(l.split()[2])) for l in out.splitlines())


def test_binding_structs_match_the_header(tmp_path):
    structs, c = _c_layout(tmp_path)
    for cname, py in structs.items():
        assert C.sizeof(py) == c[f"{cname} size"], cname
        for fname, _ in py._fields_:
            assert getattr(py, fname).offset == c[f"{cname} {fname}"], (cname, fname)


def test_binding_constants_match_the_header():
    src = open(os.path.join(ROOT, "include", "fg.h")).read()
    defs = dict(re.findall(r"^#define (FG_\w+) (\d+)", src, re.M))
    assert int(defs["FG_COUNTER_STRIDE"]) == fg.COUNTER_STRIDE
    for name, val in re.findall(r"^\s+(FG_(?:CALL|FAULT)_\w+) = 1u << (\d+)", src, re.M):
        assert getattr(fg, name[3:]) == 1 << int(val), name
