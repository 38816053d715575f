"""The product path has no CPU fallback: host tensors are refused, and without the HIP
library every entry point raises."""
import pytest
import torch

import blockwise_fp8_gemm_amd as pf


@pytest.fixture
def no_library(monkeypatch, tmp_path):
    monkeypatch.setattr(pf, "LIB_PATH", str(tmp_path / "libpuro_fp8.so"))
    monkeypatch.setattr(pf, "_lib", None)


def test_missing_library_raises(no_library):
    with pytest.raises(ImportError, match="not built"):
        pf.lib()


@pytest.mark.parametrize("call", [
    lambda x: pf.puro_fp8_quant_act(x),
    lambda x: pf.puro_fp8_quant_weight(x),
    lambda x: pf.puro_fp8_quant_transpose(x),
    lambda x: pf.puro_fp8_quant_dual(x),
    lambda x: pf.puro_fp8_quant_weight_grouped([x]),
    lambda x: pf.puro_fp8_swiglu_quant_dual(x, x),
    lambda x: pf.puro_fp8_gemm_workspace_size("NT", 128, 128, 128, "128x128"),
])
def test_entry_points_raise_without_library(no_library, call):
    """Host tensors are refused before the library is touched; with no library the first
    call that reaches it raises ImportError.  Nothing computes on the CPU."""
    x = torch.zeros((128, 128), dtype=torch.bfloat16)
    with pytest.raises((ImportError, ValueError), match="not built|on the GPU"):
        call(x)


def test_gemm_raises_without_library(no_library):
    q = torch.zeros((128, 128), dtype=torch.uint8)
    s = torch.ones((128, 1), dtype=torch.float32)
    sw = torch.ones((1, 1), dtype=torch.float32)
    with pytest.raises((ImportError, ValueError), match="not built|on the GPU"):
        pf.puro_fp8_gemm("NT", q, s, q, sw, bgran="128x128", out_dtype=torch.float32)
    with pytest.raises((ImportError, ValueError), match="not built|on the GPU"):
        pf.puro_fp8_gemm_grouped("NT", [(q, s, q, sw)], bgran="128x128", out_dtype=torch.float32)


def test_host_tensors_are_refused():
    """With the library present, host tensors are still refused (no CPU path)."""
    x = torch.zeros((128, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on the GPU"):
        pf.puro_fp8_quant_dual(x)
