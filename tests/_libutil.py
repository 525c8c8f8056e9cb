"""Locate (and build only if missing) the HIP library for the tests."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")


def ensure_built() -> str:
    from bit_block_quantized_nvfp4_amd import _lib, build

    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    return _lib.LIB_PATH


def declared_functions():
    """Names of the functions declared in include/*.h (C prototypes)."""
    names = []
    for fn in sorted(os.listdir(HEADER_DIR)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(HEADER_DIR, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, re.M):
            names.append(m.group(1))
    return sorted(set(names))
