"""The library carries the digest of the kernel sources it was built from, and
the binding refuses a library whose digest is not the tree's (CPU only)."""
import os
import shutil

import pytest

from sparse_mixture_experts_argmax_amd import _lib as L
from sparse_mixture_experts_argmax_amd.source_digest import CSRC, source_digest


def test_library_matches_the_tree():
    assert L.LIB.moe_source_digest().decode() == source_digest()


def _copy(tmp_path):
    d = tmp_path / "csrc"
    shutil.copytree(CSRC, d)
    return str(d)


def test_comments_and_blank_space_do_not_count(tmp_path):
    d = _copy(tmp_path)
    p = os.path.join(d, "combine.hip")
    with open(p) as fh:
        text = fh.read()
    with open(p, "w") as fh:
        fh.write("// a new comment line\n\n" + text.replace("\n", "\n\n", 3) + "/* trailing */\n")
    assert source_digest(d) == source_digest()


def test_a_code_change_counts(tmp_path):
    d = _copy(tmp_path)
    p = os.path.join(d, "combine.hip")
    with open(p) as fh:
        text = fh.read()
    assert "CMB_MAXK = 8" in text
    with open(p, "w") as fh:
        fh.write(text.replace("CMB_MAXK = 8", "CMB_MAXK = 4"))
    assert source_digest(d) != source_digest()


def test_a_stale_library_is_refused(monkeypatch):
    monkeypatch.setattr(L, "source_digest", lambda: "0000000000000000")
    with pytest.raises(RuntimeError, match="built from other sources"):
        L.load()
