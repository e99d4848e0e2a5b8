"""The Python binding's own checks (CPU only): it refuses host memory and
mis-shaped, mis-typed or non-contiguous tensors before anything reaches the
C ABI, and it raises when the library is missing (there is no CPU fallback)."""

import os
import subprocess
import sys

import pytest
import torch

from tests.conftest import ROOT


def test_cache_refuses_host_memory():
    import sliding_window_attention_ring_amd as swa
    with pytest.raises(ValueError, match="GPU"):
        swa.KVCache("bf16", 1, 1, 64, 16, device="cpu")
    with pytest.raises(ValueError, match="kind"):
        swa.KVCache("int4", 1, 1, 64, 16)
    with pytest.raises(ValueError, match="layout"):
        swa.KVCache("bf16", 1, 1, 64, 16, layout="tree")


def test_paged_cache_checks_its_block_table_shape(monkeypatch):
    """The kernels read the table as [B][W/16]; a table of another shape is
    refused before any device memory is allocated (allocation is stubbed
    out here, so a table of the right shape stops there)."""
    import sliding_window_attention_ring_amd as swa
    from sliding_window_attention_ring_amd import cache as cmod

    class Stop(Exception):
        pass

    def no_gpu(*a, **k):
        raise Stop()

    monkeypatch.setattr(cmod.torch, "empty", no_gpu)
    for shape in [(2, 3), (2, 5), (8,), (1, 4)]:
        with pytest.raises((ValueError, Stop)) as e:
            swa.KVCache("bf16", 2, 1, 64, 64, layout="paged", num_pages=16,
                        block_table=torch.zeros(shape, dtype=torch.int32))
        assert e.type is ValueError or shape == (2, 4)


def test_tensor_checks():
    from sliding_window_attention_ring_amd.cache import _need
    t = torch.zeros((2, 3), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        _need(t, (2, 3), torch.float32, "x")
    with pytest.raises(TypeError):
        _need([1, 2], (2,), torch.float32, "x")


class _FakeCuda:
    """Stands in for a GPU tensor to reach the shape, dtype and layout checks."""
    is_cuda = True

    def __init__(self, shape, dtype, contiguous=True):
        self.shape, self.dtype, self._c = shape, dtype, contiguous

    def is_contiguous(self):
        return self._c


def test_shape_dtype_and_layout_checks(monkeypatch):
    from sliding_window_attention_ring_amd import cache
    monkeypatch.setattr(cache.torch, "Tensor", _FakeCuda)
    cache._need(_FakeCuda((2, 3), torch.bfloat16), (2, 3), torch.bfloat16, "x")  # passes
    with pytest.raises(ValueError, match="expected"):
        cache._need(_FakeCuda((2, 4), torch.bfloat16), (2, 3), torch.bfloat16, "x")
    with pytest.raises(ValueError, match="expected"):
        cache._need(_FakeCuda((2, 3), torch.float32), (2, 3), torch.bfloat16, "x")
    with pytest.raises(ValueError, match="contiguous"):
        cache._need(_FakeCuda((2, 3), torch.bfloat16, contiguous=False), (2, 3), torch.bfloat16, "x")


def test_missing_library_raises():
    code = ("import sliding_window_attention_ring_amd._capi as c\n"
            "try:\n    c.lib()\nexcept RuntimeError as e:\n    print('raised:', e)\n")
    env = dict(os.environ, SWA_LIB=os.path.join(ROOT, "no_such_dir", "libswa.so"))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, env=env,
                         timeout=120)
    assert res.returncode == 0, res.stderr
    assert "raised:" in res.stdout and "missing" in res.stdout


def test_workspace_must_be_gpu_memory():
    from sliding_window_attention_ring_amd import cache
    with pytest.raises(ValueError, match="GPU tensor"):
        cache.workspace_init(torch.zeros(64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU tensor"):
        cache._workspace(None, torch.zeros(64, dtype=torch.uint8))


class _FakeArg(_FakeCuda):
    def dim(self):
        return len(self.shape)


def test_every_entry_point_checks_its_tensor_shapes(monkeypatch):
    """A tensor of the wrong shape never reaches the C ABI, which sees only
    pointers: each entry point of the binding rejects one (the shapes follow
    the cache: B, H, D, W; one new token per fused step)."""
    import types
    import sliding_window_attention_ring_amd as swa
    from sliding_window_attention_ring_amd import cache as cmod
    monkeypatch.setattr(cmod.torch, "Tensor", _FakeCuda)
    bf = torch.bfloat16
    rows = types.SimpleNamespace(B=2, H=3, D=64, W=32, kind="bf16", input_dtype=bf)
    i8 = types.SimpleNamespace(B=2, H=3, D=128, W=32, kind="int8", input_dtype=bf)
    cases = [
        lambda: swa.kv_append(rows, _FakeArg((2, 3, 5, 64), bf), _FakeArg((2, 3, 4, 64), bf)),
        lambda: swa.kv_append(rows, _FakeArg((2, 3, 5, 32), bf), _FakeArg((2, 3, 5, 32), bf)),
        lambda: swa.decode_attn(rows, _FakeArg((2, 3, 32), bf)),
        lambda: swa.decode_attn(rows, _FakeArg((2, 3, 64), torch.float32)),
        lambda: swa.decode_attn_int8_witness(i8, _FakeArg((2, 3, 64), bf)),
        lambda: swa.decode_attn_int8_witness_tv(i8, _FakeArg((3, 2, 128), bf)),
        lambda: swa.decode_attn_int8_dither(i8, _FakeArg((2, 3, 127), bf), 1e-3),
        lambda: swa.decode_step(rows, _FakeArg((2, 3, 2, 64), bf), _FakeArg((2, 3, 2, 64), bf),
                                _FakeArg((2, 3, 64), bf)),
        lambda: swa.decode_step(rows, _FakeArg((2, 3, 1, 64), bf), _FakeArg((2, 3, 1, 64), bf),
                                _FakeArg((2, 3, 63), bf)),
        lambda: swa.decode_step_int8(i8, _FakeArg((2, 3, 1, 128), bf), _FakeArg((2, 2, 1, 128), bf),
                                     _FakeArg((2, 3, 128), bf)),
        lambda: swa.decode_step_int8_static(i8, _FakeArg((2, 3, 1, 128), bf), _FakeArg((2, 3, 1, 128), bf),
                                            _FakeArg((2, 3, 128), torch.float32)),
        lambda: swa.kv_truncate(rows, _FakeArg((3,), torch.int32)),
    ]
    for i, call in enumerate(cases):
        with pytest.raises(ValueError, match="expected"):
            call()
