"""The C ABI library loads, exports every function include/attn_bwd.h
declares, and rejects bad arguments before touching the GPU (CPU only)."""
import ctypes
import os
import re

import pytest

import tile_scheduling_attn_amd as tsa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "attn_bwd.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 14
    lib = ctypes.CDLL(tsa.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(tsa.EXPORTS) == names


def test_tile_sizes():
    assert tsa.attn_bwd_tile_size("bf16") == 128
    assert tsa.attn_bwd_tile_size("fp32") == 64
    assert tsa.attn_bwd_tile_size(7) == -1


def test_workspace_bytes():
    # fp32 accumulator b*h*s_pad*d*4 dominates; s padded to 128
    ws = tsa.attn_bwd_workspace_bytes(2, 16, 8192, 128, 0, "shift")
    assert ws >= 2 * 16 * 8192 * 128 * 4 + 2 * 16 * 8192 * 4
    assert ws % 256 == 0
    assert tsa.attn_bwd_workspace_bytes(1, 1, 100, 64, 0, 0) >= 128 * 64 * 4
    assert tsa.attn_bwd_workspace_bytes(1, 1, 128, 96, 0, 0) == 0
    assert tsa.attn_bwd_workspace_bytes(-1, 1, 128, 64, 0, 0) == 0


def _call(**kw):
    args = dict(q=0, k=0, v=0, o=0, dO=0, lse=0, dq=0, dk=0, dv=0, b=1, h=1, s=128, d=64,
                causal=0, schedule=0, dtype=0, scale=0.125, workspace=0, workspace_bytes=0, stream=0)
    args.update(kw)
    return tsa.attn_bwd_deterministic_ex(**args)


def test_argument_errors_need_no_gpu():
    assert _call() == -1                       # null pointers
    assert "null" in tsa.last_error()
    assert _call(b=-1) == -1
    assert _call(s=-5) == -1
    assert _call(causal=2) == -1
    assert _call(schedule=5) == -1
    assert _call(dtype=3) == -1
    assert _call(scale=float("nan")) == -1
    assert _call(d=96) == -2
    assert "64 or 128" in tsa.last_error()
    # misaligned (but non-null) pointers are rejected before any device call
    assert _call(q=8, k=16, v=16, o=16, dO=16, lse=16, dq=16, dk=16, dv=16) == -1
    assert "aligned" in tsa.last_error()


def test_empty_problem_is_a_no_op():
    assert _call(b=0) == 0
    assert _call(h=0) == 0
    assert _call(s=0) == 0
    assert tsa.attn_bwd_deterministic(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 4, 128, 64, 0, 0) == 0


def _fwd(**kw):
    args = dict(q=0, k=0, v=0, o=0, lse=0, b=1, h=1, s=128, d=64, causal=0, dtype=0, scale=0.125, stream=0)
    args.update(kw)
    return tsa.attn_fwd(**args)


def test_forward_argument_errors_need_no_gpu():
    assert _fwd() == -1                        # null pointers
    assert "null" in tsa.last_error()
    assert _fwd(b=-1) == -1
    assert _fwd(causal=2) == -1
    assert _fwd(dtype=3) == -1
    assert _fwd(scale=float("inf")) == -1
    assert _fwd(d=32) == -2
    assert _fwd(q=8, k=16, v=16, o=16, lse=16) == -1
    assert "aligned" in tsa.last_error()
    assert _fwd(q=16, k=16, v=16, o=16, lse=2) == -1
    assert _fwd(b=0) == 0 and _fwd(s=0) == 0
