"""Digest of the HIP sources that libmoe.so is built from.

build.py compiles it into the library (moe_source_digest() in include/moe.h);
the loader compares it with the sources in the tree and refuses a library
built from other code.  Comments and blank space are removed first, so a
reworded comment does not make a library stale.  The profile summaries record
the same digest next to their counters.
"""
from __future__ import annotations

import glob
import hashlib
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
_COMMENT = re.compile(r"/\*.*?\*/|//[^\n]*", re.S)


def source_digest(csrc: str = CSRC) -> str:
    """sha256 (first 16 hex digits) over csrc/*.hip and csrc/*.h, by file name
    order, each file's name then its code without comments or blank space."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(csrc, "*"))):
        if path.endswith((".hip", ".h")):
            h.update(os.path.basename(path).encode())
            with open(path, encoding="utf-8") as fh:
                code = _COMMENT.sub(" ", fh.read())
            h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]
