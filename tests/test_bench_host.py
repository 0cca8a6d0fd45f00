"""Host-side checks of bench.py (CPU): the one-GPU rule and the algorithmic bytes its
roofline lines divide by, the latter against closed forms written from the Llama-7B
architecture (vocabulary 32000, hidden 4096, MLP 11008, 32 layers), not from
bench.py's own accounting."""
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Llama-7B: embedding and output head [32000, 4096]; per layer q, k, v, o [4096, 4096],
# gate and up [11008, 4096], down [4096, 11008], two norms [4096]; a final norm [4096].
V, HID, MLP, LAYERS = 32000, 4096, 11008, 32
P2 = 2 * V * HID + LAYERS * (4 * HID * HID + 3 * HID * MLP)       # 2-D parameters
P1 = LAYERS * 2 * HID + HID                                        # 1-D parameters
RC = 2 * (V + HID) + LAYERS * (4 * (HID + HID) + 3 * (HID + MLP))  # rows + columns of the 2-D ones


def test_llama7b_counts():
    wl = workloads.WORKLOADS["adafactor_llama7b"]
    assert len(wl.specs) == 2 + LAYERS * 9 + 1
    assert sum(s.numel for s in wl.specs) == P2 + P1 == 6_738_415_616


def test_adafactor_apply_bytes():
    """Per parameter of a factored tensor: G (bf16) read, X and M (fp32) read and
    written, 2 + 8 + 8 = 18 bytes; a 1-D tensor also reads its full second moment
    (22); each row and column statistic is read once (4 bytes)."""
    b = bench.algorithmic_bytes(workloads.WORKLOADS["adafactor_llama7b"])
    assert b["adafactor_apply"] == 18 * P2 + 22 * P1 + 4 * RC == 121_302_829_056


def test_came_apply_and_lamb_moments_bytes():
    """CAME's apply of a factored tensor: M read, X read and written (12 bytes), plus
    the residual row and column statistics. LAMB's moment pass: G (2), X read (4),
    M and V read and written (16)."""
    came = bench.algorithmic_bytes(workloads.WORKLOADS["came_llama7b"])
    assert came["came_apply"] == 12 * P2 + 4 * RC
    lamb = bench.algorithmic_bytes(workloads.WORKLOADS["lamb_llama7b"])
    assert lamb["lamb_moments"] == 22 * (P2 + P1)


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})],
                         ids=["gpus-2", "world-size-2"])
def test_more_than_one_gpu_is_refused(argv, env):
    """The step exchanges nothing between GPUs, so bench.py takes no multi-GPU figure:
    it exits with status 2 and says why, before it imports torch."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                       timeout=120, env={**os.environ, **env}, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_galore_bytes():
    """GaLore at rank 256 projects all 226 two-dimensional tensors, each with d = 4096
    (the shorter side). Projection: G (bf16, 2 bytes per element), both moments read
    and written and N's two bf16 planes written (20 bytes per element of [D][r]), U^T
    read (2 per element of [r][d]). Back-projection: W read and written, N's planes
    and U read once."""
    specs = workloads.WORKLOADS["adafactor_llama7b"].specs
    shapes = [s.shape for s in specs]
    r, d = 256, HID
    two_d = [s for s in shapes if len(s) == 2]
    assert len(two_d) == 2 + 7 * LAYERS == 226
    sum_big = sum(max(s) for s in two_d)
    assert sum_big == 2 * V + LAYERS * (4 * HID + 3 * MLP)
    for xb, back in ((4, 56_063_688_704), (2, 29_111_091_200)):
        b = bench.galore_bytes_flops(shapes, r, xb)
        assert b["galore_project"] == 2 * P2 + 20 * r * sum_big + 2 * r * d * 226
        assert b["galore_back"] == 2 * xb * P2 + 4 * r * sum_big + 2 * r * d * 226 == back
        assert b["flops_back"] == 2 * b["flops_project"] == 4 * r * P2
        assert b["galore_adamw"] == (2 + 2 * xb + 16) * P1
