"""The Python binding's argument checks (host only): every buffer a kernel
reads or writes in full must have the exact shape and dtype the call implies,
since most sizes never reach the library."""

import pytest
import torch

import gated_mlp_transformer_amd as g


def test_need_accepts_exact_and_none():
    g._need("f", "t", torch.empty((3, 4), dtype=torch.int32), (3, 4), torch.int32)
    g._need("f", "t", None, (3, 4), torch.int32)


@pytest.mark.parametrize("t", [torch.empty((3, 5), dtype=torch.int32),
                               torch.empty((12,), dtype=torch.int32),
                               torch.empty((3, 4), dtype=torch.int64)])
def test_need_rejects_other_shapes_and_dtypes(t):
    with pytest.raises(ValueError, match="f: t must be"):
        g._need("f", "t", t, (3, 4), torch.int32)


def test_block_scales_required_for_fp8_only():
    ok = torch.empty((2, 16, 32), dtype=torch.float32)
    g._block_scales("f", g.MF_FP8_E4M3, 2, 2048, 4096, s_gate=ok)
    g._block_scales("f", g.MF_BF16, 2, 2048, 4096, s_gate=None)   # bf16 takes no scales
    with pytest.raises(ValueError, match="need s_gate"):
        g._block_scales("f", g.MF_FP8_E4M3, 2, 2048, 4096, s_gate=None)
    with pytest.raises(ValueError, match="s_gate must be"):
        g._block_scales("f", g.MF_FP8_E4M3, 2, 2048, 4096,
                        s_gate=torch.empty((2, 32, 16), dtype=torch.float32))
