"""Test helper: the built native library (building it if it is missing)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import range_masked_attention_amd as ffa  # noqa: E402


def ensure_built():
    if not os.path.exists(ffa.lib_path()):
        from range_masked_attention_amd import _build
        _build.build()
    return ffa.load_library()
