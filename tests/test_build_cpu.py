"""CPU tests of the build's code placement: for each block kernel it places,
the pads it chooses put every listed form's main loop at its target offset
within a 32-byte instruction block (read back from the assembled device
code), and without the assembler tools the build still succeeds, with the
loops where the compiler puts them.  No GPU is used; needs hipcc."""
import os
import shutil
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from context_ring_attention_cp_amd import build as B  # noqa: E402

needs_hipcc = pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None,
                                 reason="hipcc not available")


@needs_hipcc
@pytest.mark.parametrize("src", sorted(B.PLACEMENT))
def test_main_loops_land_on_their_targets(src):
    os.makedirs(B.BUILD, exist_ok=True)
    pads = B._placement_pads(src, verbose=False)
    offs = B._loop_offsets(src, pads)
    forms = B.PLACEMENT[src]["forms"]
    assert set(forms) <= set(offs), f"main loop not found for {set(forms) - set(offs)}"
    for form, target in forms.items():
        assert offs[form] % 32 == target, (src, form, offs[form] % 32, target)
        assert 0 <= pads[form] < 8


@needs_hipcc
def test_placement_without_the_tools_keeps_the_kernels(monkeypatch, capsys):
    monkeypatch.setattr(B, "LLVM", "/nonexistent-llvm-bin")
    pads = B._placement_pads("attn_fp8.hip", verbose=False)
    assert pads == {f: 0 for f in B.PLACEMENT["attn_fp8.hip"]["forms"]}
    assert "placement skipped" in capsys.readouterr().err
