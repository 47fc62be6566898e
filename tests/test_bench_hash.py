"""The traffic record is keyed to the kernel code: bench.kernel_source_hash
ignores comments and white space, and changes with any code token."""
import os
import shutil

import bench


def _copy_tree(tmp_path):
    root = tmp_path / "r"
    shutil.copytree(os.path.join(bench.ROOT, "sync_protocols_amd", "csrc"), root / "sync_protocols_amd" / "csrc")
    shutil.copytree(os.path.join(bench.ROOT, "include"), root / "include")
    return root


def _hash(root):
    saved = bench.ROOT
    bench.ROOT = str(root)
    try:
        return bench.kernel_source_hash()
    finally:
        bench.ROOT = saved


def test_hash_ignores_comments_and_spacing_but_not_code(tmp_path):
    root = _copy_tree(tmp_path)
    h0 = _hash(root)
    assert h0 == bench.kernel_source_hash()
    f = root / "sync_protocols_amd" / "csrc" / "fg_gemm.hpp"
    src = f.read_text()
    f.write_text("// an added line comment\n/* and a block\n   comment */\n" + src.replace("\n", "\n\n", 3))
    assert _hash(root) == h0
    f.write_text(src.replace("constexpr int kPolA = kPolSC1;", "constexpr int kPolA = 0;"))
    assert _hash(root) != h0
