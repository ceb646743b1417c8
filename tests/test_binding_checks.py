"""The binding's checks of caller-supplied output buffers and workspaces (CPU).

The C ABI receives bare device addresses, so the binding is the only place
that can see a buffer's size and type: a too-small, mistyped, strided or
misplaced output must raise before any call reaches the library."""
import pytest
import torch

from long_context_kv_ts_amd import ops


def test_out_accepts_none_and_exact_buffers():
    assert ops._out(None, "x", (3, 4), torch.float32, "cpu") is None
    t = torch.empty((3, 4), dtype=torch.float32)
    assert ops._out(t, "x", (3, 4), torch.float32, "cpu") is t


@pytest.mark.parametrize("t,exc,needle", [
    (torch.empty((3, 5), dtype=torch.float32), ValueError, "shape"),          # too large
    (torch.empty((2, 4), dtype=torch.float32), ValueError, "shape"),          # too small
    (torch.empty((12,), dtype=torch.float32), ValueError, "shape"),           # same size, other shape
    (torch.empty((3, 4), dtype=torch.float16), TypeError, "dtype"),
    (torch.empty((3, 4), dtype=torch.bfloat16), TypeError, "dtype"),
    (torch.empty((4, 3), dtype=torch.float32).t(), ValueError, "contiguous"),
])
def test_out_rejects(t, exc, needle):
    with pytest.raises(exc, match=needle):
        ops._out(t, "x", (3, 4), torch.float32, "cpu")


def test_out_rejects_other_device():
    t = torch.empty((3, 4), dtype=torch.float32, device="meta")
    with pytest.raises(ValueError, match="expected"):
        ops._out(t, "x", (3, 4), torch.float32, "cpu")


def test_workspace_checks_bytes_not_elements():
    ops._workspace(None, "ws", 1 << 20, "cpu")
    ok = torch.empty(256, dtype=torch.float32)                  # 1024 bytes
    assert ops._workspace(ok, "ws", 1024, "cpu") is ok
    with pytest.raises(ValueError, match="1025 required"):
        ops._workspace(ok, "ws", 1025, "cpu")
    with pytest.raises(ValueError, match="contiguous"):
        ops._workspace(torch.empty((64, 64), dtype=torch.uint8)[:, ::2], "ws", 16, "cpu")


def test_partials_must_be_fp32_on_the_gpu():
    with pytest.raises(ValueError, match="o_part"):
        ops._parts(None, None)
    with pytest.raises(ValueError, match="GPU"):
        ops._parts(torch.empty((2, 3, 128)), torch.empty((2, 3)))


def test_partials_take_fp32_or_bf16_only():
    with pytest.raises(TypeError, match="float32 or bfloat16"):
        ops._parts(torch.empty((2, 3, 128), dtype=torch.float16), torch.empty((2, 3)))
    with pytest.raises(TypeError, match="float32 or bfloat16"):
        ops._part_dtype(None, torch.float16)
    # a given o_part decides the form; the keyword only sizes a new one
    assert ops._part_dtype(torch.empty(1, dtype=torch.bfloat16), torch.float32) == torch.bfloat16
    assert ops._part_dtype(None, torch.bfloat16) == torch.bfloat16
    assert ops._part_code(torch.empty(1, dtype=torch.bfloat16)) == ops.TS_BF16
    assert ops._part_code(torch.empty(1, dtype=torch.float32)) == ops.TS_F32
