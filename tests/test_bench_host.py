"""Host logic of bench.py: the algorithmic byte counts its roofline divides
by (no GPU)."""
import numpy as np

import bench
from mixture_experts_layer_layout_amd import synth


def test_backward_bytes_count_weights_once_each_way():
    w = synth.WORKLOADS["dsv3-fwdbwd-zipf"]
    counts = np.full(w.E, w.R // w.E)
    act = w.T * w.d * 2
    saved = 3 * w.R * w.I * 2
    small = w.R * 4 * 4 + (w.E + 1) * 8
    weights = w.E * 3 * w.I * w.d * 2
    # bf16: the weights read, their gradients written, both bf16
    assert bench.algorithmic_bytes(w, counts, "backward") == 2 * weights + 3 * act + saved + w.R * 4 + small
    # MXFP8: codes and scales read (1 + 1/32 bytes an element), bf16 gradients written
    wq = synth.WORKLOADS["dsv3-fwdbwd-zipf-mxfp8"]
    codes = int(w.E * 3 * w.I * w.d * (1 + 1 / 32))
    assert bench.algorithmic_bytes(wq, counts, "backward") == codes + weights + 3 * act + saved + w.R * 4 + small
    # experts without rows move no weight bytes
    counts[:16] = 0
    assert bench.algorithmic_bytes(w, counts, "backward") == \
        2 * (w.E - 16) * 3 * w.I * w.d * 2 + 3 * act + saved + w.R * 4 + small


def test_forward_bytes():
    w = synth.WORKLOADS["dsv3-bf16"]
    counts = np.full(w.E, w.R // w.E)
    small = w.R * 4 * 4 + (w.E + 1) * 8
    want = w.E * 3 * w.I * w.d * 2 + 2 * w.T * w.d * 2 + w.E * w.d * 2 + w.T * w.E * 4 + small
    assert bench.algorithmic_bytes(w, counts, "forward") == want
