"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
algorithmic byte counts that the roofline fractions are priced on, each
written out tensor by tensor for the named workloads."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("batch, dim, L, esz", [(8, 1536, 2048, 4),      # 130m-like layer, fp32
                                                (4, 5120, 4096, 2),      # 2.8b-like layer, bf16
                                                (1, 1536, 1 << 20, 2)])  # long context, bf16
def test_scan_bytes_tensor_by_tensor(batch, dim, L, esz):
    N = 16
    u = delta = z = out = batch * dim * L * esz
    B = C = batch * N * L * esz
    A = dim * N * 4
    D = bias = dim * 4
    last = batch * dim * N * 4
    assert bench.scan_bytes(batch, dim, L, N, esz) == u + delta + z + out + B + C + A + D + bias + last


def test_headline_and_layer_byte_counts():
    """The figures quoted with the committed profiles."""
    assert bench.scan_bytes(8, 1536, 2048, 16, 4) == 405_647_360
    assert bench.scan_bytes(4, 5120, 4096, 16, 2) == 673_816_576
    assert bench.scan_bytes(1, 1536, 1 << 20, 16, 2) == 12_952_219_648
    assert bench.scan_bwd_bytes(8, 1536, 2048, 16, 4) == 809_721_856
    assert bench.scan_bwd_bytes(4, 5120, 4096, 16, 2) == 1_513_832_448


def test_decode_bytes_tensor_by_tensor():
    batch, dim, N, esz = 256, 5120, 16, 2
    state = 2 * batch * dim * N * 4            # fp32 state read and written
    x = dt = z = out = batch * dim * esz
    B = C = batch * N * esz
    params = dim * N * 4 + 2 * dim * 4         # A, D, bias
    assert bench.decode_bytes(batch, dim, N, esz) == state + x + dt + z + out + B + C + params
    assert bench.decode_bytes(batch, dim, N, esz) == 178_642_944
