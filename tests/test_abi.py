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
    assert _call(schedule=6) == -1
    assert "schedule" in tsa.last_error()
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


def test_scale_must_be_positive():
    """Masked logits start at -inf before the scale multiplies them: a zero
    scale would turn them into NaN and a negative one into +inf, so both
    entry points reject scale <= 0 before touching the GPU."""
    ptrs = dict(q=16, k=16, v=16, o=16, dO=16, lse=16, dq=16, dk=16, dv=16)
    for bad in (0.0, -0.0, -0.125, float("-inf")):
        assert _call(scale=bad, **ptrs) == -1, bad
        assert "positive" in tsa.last_error()
        assert _fwd(scale=bad, q=16, k=16, v=16, o=16, lse=16) == -1, bad
        assert "positive" in tsa.last_error()


def test_size_limits_return_status_codes():
    """Sizes past the library's limits come back as status codes instead of
    overflowing 32-bit offsets or exhausting host memory."""
    ptrs = dict(q=16, k=16, v=16, o=16, dO=16, lse=16, dq=16, dk=16, dv=16)
    assert _call(s=262145, **ptrs) == -2
    assert "262144" in tsa.last_error()
    assert _fwd(s=262145, q=16, k=16, v=16, o=16, lse=16) == -2
    assert _call(b=65536, h=65536, **ptrs) == -1            # b*h beyond an int
    assert _call(b=1 << 14, h=1 << 10, s=262144, d=128, **ptrs) == -1  # b*h*s*d >= 2^40
    assert tsa.attn_bwd_workspace_bytes(1, 1, 262145, 128, 0, 0) == 0
    assert tsa.attn_bwd_workspace_bytes(65536, 65536, 128, 64, 0, 0) == 0
    # the host-side schedule tools bound n and the simulated problem
    for fn in (lambda: tsa.attn_sched_size(2049, 0, "shift"),
               lambda: tsa.attn_sched_min_workers(2049, 1, "naive"),
               lambda: tsa.attn_dagsim(2049, 0, "shift", 1, 8, 1, 1.0, 1.0),
               lambda: tsa.attn_dagsim(2048, 0, "naive", 64, 8, 1, 1.0, 1.0),      # 2^28 tasks
               lambda: tsa.attn_dagsim(8, 0, "naive", 1, (1 << 20) + 1, 1, 1.0, 1.0)):
        with pytest.raises(tsa.AttnError) as e:
            fn()
        assert e.value.code == -2
    assert tsa.attn_sched_size(2048, 1, "symmetric_shift")[0] == 1024


def test_status_codes_are_named():
    for code in (-1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert code in tsa.STATUS
    header = open(HEADER).read()
    for code, name in tsa.STATUS.items():
        assert re.search(rf"\b{name}\s*=\s*{code}\b", header), name


# ------------------------------------------------------------ binding checks
torch = pytest.importorskip("torch")


@pytest.fixture
def host_as_device(monkeypatch):
    """Let host tensors stand in for device tensors so that the binding's
    shape, type, layout and placement checks can be exercised without a GPU;
    every case below must be rejected before the C ABI is called."""
    monkeypatch.setattr(tsa, "_on_device", lambda t: True)


def _inputs(dtype=None, b=1, h=2, s=16, d=64):
    dtype = dtype or torch.bfloat16
    q, k, v, o, do = (torch.zeros(b, h, s, d, dtype=dtype) for _ in range(5))
    lse = torch.zeros(b, h, s, dtype=torch.float32)
    return q, k, v, o, do, lse


def test_backward_rejects_host_tensors():
    q, k, v, o, do, lse = _inputs()
    with pytest.raises(ValueError, match="device tensor"):
        tsa.backward(q, k, v, o, do, lse, False)


@pytest.mark.parametrize("case", ["lse_dtype", "lse_shape", "lse_layout", "k_shape", "v_dtype",
                                  "dq_dtype", "dk_shape", "dv_layout", "out_device", "ws_layout",
                                  "ws_device", "q_rank", "q_dtype"])
def test_backward_rejects_bad_tensors(host_as_device, case):
    q, k, v, o, do, lse = _inputs()
    out = [torch.zeros_like(q) for _ in range(3)]
    ws = None
    if case == "lse_dtype":
        lse = lse.double()
    elif case == "lse_shape":
        lse = torch.zeros(1, 2, 15)
    elif case == "lse_layout":
        lse = torch.zeros(1, 2, 32)[:, :, ::2]
    elif case == "k_shape":
        k = torch.zeros(1, 2, 16, 128, dtype=torch.bfloat16)
    elif case == "v_dtype":
        v = v.float()
    elif case == "dq_dtype":
        out[0] = out[0].float()
    elif case == "dk_shape":
        out[1] = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    elif case == "dv_layout":
        out[2] = torch.zeros(1, 2, 64, 16, dtype=torch.bfloat16).transpose(2, 3)
    elif case == "out_device":
        out[0] = torch.empty_like(q, device="meta")
    elif case == "ws_layout":
        ws = torch.zeros(64, 64, dtype=torch.uint8)[:, ::2]
    elif case == "ws_device":
        ws = torch.empty(4096, dtype=torch.uint8, device="meta")
    elif case == "q_rank":
        q = q[0]
    elif case == "q_dtype":
        q, k, v, o, do = (t.half() for t in (q, k, v, o, do))
    with pytest.raises(ValueError):
        tsa.backward(q, k, v, o, do, lse, False, out=out, workspace=ws, stream=0)


@pytest.mark.parametrize("case", ["o_dtype", "lse_shape", "lse_dtype", "o_device"])
def test_forward_rejects_bad_outputs(host_as_device, case):
    q, k, v, o, _, lse = _inputs()
    if case == "o_dtype":
        o = o.float()
    elif case == "lse_shape":
        lse = torch.zeros(1, 2, 16, 1)
    elif case == "lse_dtype":
        lse = lse.half()
    elif case == "o_device":
        o = torch.empty_like(q, device="meta")
    with pytest.raises(ValueError):
        tsa.forward(q, k, v, False, out=(o, lse), stream=0)


def test_debug_hooks_validate_arguments():
    assert tsa.lib.attn_bwd_set_debug(0, -1, 0) == -1
    assert tsa.lib.attn_bwd_set_debug(0, 70000, 0) == -1
    assert tsa.lib.attn_bwd_set_debug(64, 0, 7) == 0
    assert tsa.lib.attn_bwd_set_debug(0, 0, 0) == 0


def test_auto_schedule_is_accepted_and_resolve_checks_arguments():
    assert tsa.SCHEDULES["auto"] == 5
    ptrs = dict(q=16, k=16, v=16, o=16, dO=16, lse=16, dq=16, dk=16, dv=16)
    assert _call(schedule=5, d=96, **ptrs) == -2      # AUTO passes the schedule check
    assert tsa.lib.attn_bwd_resolve_schedule(0, 1, 128, 64, 0, 0) == -1
    assert tsa.lib.attn_bwd_resolve_schedule(1, 1, 128, 96, 0, 0) == -2
    assert tsa.lib.attn_bwd_resolve_schedule(1, 1, 128, 64, 2, 0) == -1
    assert tsa.attn_bwd_workspace_bytes(2, 16, 8192, 128, 0, "auto") >= \
        tsa.attn_bwd_workspace_bytes(2, 16, 8192, 128, 0, "shift")


def test_set_tile_validates_and_restores_the_default():
    assert tsa.lib.attn_bwd_set_tile(1, 64) == -2
    assert tsa.lib.attn_bwd_set_tile(0, 96) == -1
    assert tsa.lib.attn_bwd_set_tile(0, 64) == 0
    assert tsa.attn_bwd_tile_size("bf16") == 64
    assert tsa.lib.attn_bwd_set_tile(0, 0) == 0
    assert tsa.attn_bwd_tile_size("bf16") == 128
    assert tsa.attn_bwd_tile_size("fp32") == 64


def test_atomic_rate_validates_arguments_before_any_gpu_call():
    import ctypes
    ms, adds = ctypes.c_float(1.0), ctypes.c_double(1.0)
    r = tsa.lib.attn_bwd_atomic_rate
    assert r(None, 1 << 20, 4, None, ctypes.byref(ms), ctypes.byref(adds)) == -1   # null buffer
    assert ms.value == 0 and adds.value == 0                                      # outputs cleared
    assert r(ctypes.c_void_p(256 + 16), 1 << 20, 4, None, None, None) == -1        # misaligned
    assert r(ctypes.c_void_p(256), 65535, 4, None, None, None) == -1               # below one tile
    assert r(ctypes.c_void_p(256), 1 << 20, 0, None, None, None) == -1             # no tasks
    assert r(ctypes.c_void_p(256), 1 << 20, 65537, None, None, None) == -1         # too many tasks
    with pytest.raises(tsa.AttnError):
        tsa.attn_bwd_atomic_rate(__import__("torch").zeros(1 << 14), 4)            # host tensor


def test_wait_histogram_validates_arguments_before_any_gpu_call():
    assert tsa.lib.attn_bwd_get_wait_hist(None) == -1


def test_handoff_latency_validates_arguments_before_any_gpu_call():
    import ctypes
    r = tsa.lib.attn_bwd_handoff_latency
    n = tsa.lib.attn_bwd_handoff_bytes()
    assert n >= 2 * 65536
    ns = ctypes.c_double(1.0)
    assert r(None, n, 8, 100, 0, None, ctypes.byref(ns), None, None) == -1 and ns.value == 0
    assert r(ctypes.c_void_p(256 + 8), n, 8, 100, 0, None, None, None, None) == -1     # misaligned
    assert r(ctypes.c_void_p(256), n - 1, 8, 100, 0, None, None, None, None) == -1     # too small
    assert r(ctypes.c_void_p(256), n, 0, 100, 0, None, None, None, None) == -1         # pong 0 is ping
    assert r(ctypes.c_void_p(256), n, 64, 100, 0, None, None, None, None) == -1
    assert r(ctypes.c_void_p(256), n, 8, 1, 0, None, None, None, None) == -1           # one turn
    assert r(ctypes.c_void_p(256), n, 8, 100, 3, None, None, None, None) == -1         # unknown mode


def test_set_tile_shape_validates_and_restores_the_default():
    assert tsa.lib.attn_bwd_set_tile_shape(1, 64, 128) == -2      # fp32 has no choice
    for br, bc in ((128, 64), (32, 128), (64, 256), (96, 96)):
        assert tsa.lib.attn_bwd_set_tile_shape(0, br, bc) == -1
    assert tsa.lib.attn_bwd_set_tile_shape(0, 64, 128) == 0
    assert tsa.attn_bwd_tile_shape("bf16") == (64, 128)
    assert tsa.attn_bwd_tile_size("bf16") == 128                   # the KV tile
    assert tsa.lib.attn_bwd_set_tile(0, 64) == 0                   # square 64 x 64
    assert tsa.attn_bwd_tile_shape("bf16") == (64, 64)
    assert tsa.lib.attn_bwd_set_tile_shape(0, 0, 0) == 0
    assert tsa.attn_bwd_tile_shape("bf16") == (128, 128)
    assert tsa.attn_bwd_tile_shape("fp32") == (64, 64)


def test_set_main_kernel_validates_and_round_trips():
    assert tsa.attn_bwd_main_kernel() == "auto"                    # the default
    for bad in (-1, 3, 7):
        assert tsa.lib.attn_bwd_set_main_kernel(bad) == -1
    assert tsa.attn_bwd_main_kernel() == "auto"
    assert tsa.lib.attn_bwd_set_main_kernel(1) == 0
    assert tsa.attn_bwd_main_kernel() == "pair"
    tsa.attn_bwd_set_main_kernel("four_wave")
    assert tsa.lib.attn_bwd_main_kernel() == 0
    tsa.attn_bwd_set_main_kernel("auto")
    assert tsa.lib.attn_bwd_main_kernel() == 2


def test_resolve_main_kernel_follows_the_settings():
    r = tsa.attn_bwd_resolve_main_kernel
    assert tsa.attn_bwd_main_kernel() == "auto"
    assert r(128, True, "bf16", "symmetric_shift") == "pair"       # default: pair under the causal mask at d = 128
    assert r(128, True, "bf16", "auto") == "pair"
    assert r(128, False, "bf16", "shift") == "four_wave"
    assert r(64, True, "bf16", "symmetric_shift") == "four_wave"
    assert r(128, True, "bf16", "atomic") == "four_wave"           # no pair form of ATOMIC
    assert r(128, True, "fp32", "descending") == "four_wave"
    tsa.attn_bwd_set_main_kernel("pair")
    try:
        assert r(128, False, "bf16", "shift") == "pair"
        assert r(64, False, "bf16", "naive") == "pair"
        tsa.attn_bwd_set_tile_shape("bf16", 64, 128)
        try:
            assert r(128, True, "bf16", "shift") == "four_wave"    # 128 x 128 tiles only
        finally:
            tsa.attn_bwd_set_tile_shape("bf16", 0, 0)
        tsa.attn_bwd_set_main_kernel("four_wave")
        assert r(128, True, "bf16", "symmetric_shift") == "four_wave"
    finally:
        tsa.attn_bwd_set_main_kernel("auto")
    assert tsa.lib.attn_bwd_resolve_main_kernel(96, 1, 0, 1) == -2
    assert tsa.lib.attn_bwd_resolve_main_kernel(128, 2, 0, 1) == -1
    assert tsa.lib.attn_bwd_resolve_main_kernel(128, 1, 0, 9) == -1
