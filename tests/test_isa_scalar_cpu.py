"""The library's device code writes memory through vector instructions
only: no scalar stores, scalar atomics, or scalar-cache write-back or
discard anywhere in the gfx950 assembly of our own sources (built here).
The folded combine relies on device-scope fences, which must compile to
vector L2 write-back / invalidate, not to scalar-cache operations."""

import os
import re

import pytest

from tests.test_isa_cpu import CSRC, _device_asm

SCALAR_WRITES = re.compile(
    r"^\s*s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)\w*\b")


@pytest.mark.parametrize("src", sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))
def test_no_scalar_memory_writes(src):
    asm = _device_asm(os.path.join(CSRC, src))
    bad = [l.strip() for l in asm.splitlines() if SCALAR_WRITES.match(l.split(";", 1)[0])]
    assert not bad, bad[:5]
