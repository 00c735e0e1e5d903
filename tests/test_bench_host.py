"""Host-side helpers of bench.py (no GPU): the kernel each launch runs, as the
line and the traffic record name it, and the algorithmic bytes a launch is
charged with."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("s_q,S,pool,kernel", [
    (1, 10, "bf16", "decode_kernel4t<bf16 pool, partial, 16 parts"),     # up to 16 jobs: head tiles x column quarters
    (6, 5, "bf16", "decode_kernel4t<bf16 pool, partial, 8 parts"),
    (16, 4, "bf16", "decode_kernel4t<bf16 pool, partial, 4 parts"),
    (96, 1, "bf16", "decode_kernel8h<bf16 pool, direct, 2 head halves"),
    (160, 1, "bf16", "decode_kernel8p<bf16 pool, direct, 1 column part"),
    (384, 1, "bf16", "decode_kernel8m<bf16 pool, direct: decode_kernel8p's body over 256 jobs"),
    (1, 8, "fp8", "decode_kernel4t<fp8 pool, partial, 16 parts"),
    (16, 8, "fp8", "decode_kernel8h<fp8 pool, partial, 2 head halves"),
    (300, 1, "fp8", "decode_kernel8m<fp8 pool, direct: decode_kernel8p's body over 256 jobs"),
])
def test_kernel_label_follows_the_launch_plan(s_q, S, pool, kernel):
    assert bench.kernel_label(s_q, S, pool).startswith(kernel)


def test_kernel_bytes():
    # gathered rows + Q + indices per token; the direct path also writes the bf16 output
    assert bench.kernel_bytes("single", 10) == 640 * 1152 + 64 * 576 * 2 + 640 * 4 == 813568
    assert bench.kernel_bytes("large384", 1) == 813568 + 64 * 512 * 2
