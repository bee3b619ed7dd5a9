"""The persistent kernels' claim / wait / abort protocol, run on the CPU.

tests/protocol_model.cpp compiles the device's own claiming and bounded-wait
code (mixture_experts_layer_layout_amd/csrc/protocol.h) with host atomics
and drives it from std::threads standing in for workgroups, over the phases
of the persistent forward and backward (MoK flash §02: GPU-local counters
tell the expert side that a batch is complete).  It is built with
ThreadSanitizer: any consumer read that no counter orders after its
producer's write is reported, and every consumed value is checked.

Cases: one launch holding every phase and the default launch split, for the
forward and the backward, with 1 to 16 workers starting on random
sub-queues; a forward whose gather of row tile 0 never raises its counter,
which must end with MOE_ERR_TIMEOUT, every worker exited and no task of
that tile run; and every wait with a tiny spin limit (whichever expires
first aborts the call), which must drain without a race.  Two planted
mistakes (an up projection that does not wait, a task that runs after its
wait failed) must make the model fail.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "protocol_model.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _build(tmp_path_factory, defines=()):
    out = tmp_path_factory.mktemp("model") / "protocol_model"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread", "-o", str(out), SRC]
    cmd += [f"-D{d}" for d in defines]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return str(out)


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    return _build(tmp_path_factory)


def _run(binary, scenario, workers, seed):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    return subprocess.run([binary, scenario, str(workers), str(seed)], capture_output=True, text=True, env=env,
                          timeout=120)


@pytest.mark.parametrize("scenario", ["fwd-single", "fwd-default", "bwd-single", "bwd-default"])
def test_protocol_completes_without_races(model, scenario):
    for workers in (1, 2, 5, 16):
        for seed in range(3):
            r = _run(model, scenario, workers, seed)
            assert r.returncode == 0, (scenario, workers, seed, r.stdout, r.stderr[-3000:])
            assert r.stdout.startswith("ok status=0"), r.stdout


def test_tiny_spin_limit_drains_without_races(model):
    for workers in (1, 4, 16):
        for seed in range(3):
            r = _run(model, "fwd-tiny", workers, seed)
            assert r.returncode == 0, (workers, seed, r.stdout, r.stderr[-3000:])
            assert r.stdout.startswith(("ok status=0", "ok status=-5")), r.stdout


def test_dropped_counter_times_out_and_drains(model):
    for workers in (1, 3, 16):
        for seed in range(3):
            r = _run(model, "fwd-drop", workers, seed)
            assert r.returncode == 0, (workers, seed, r.stdout, r.stderr[-3000:])
            assert r.stdout.startswith("ok status=-5"), r.stdout   # MOE_ERR_TIMEOUT


@pytest.mark.parametrize("plant,scenario", [("PLANT_NO_READY_WAIT", "fwd-single"),
                                            ("PLANT_RUN_AFTER_FAILED_WAIT", "fwd-drop")])
def test_planted_protocol_mistake_is_caught(tmp_path_factory, plant, scenario):
    binary = _build(tmp_path_factory, [plant])
    failed = False
    for seed in range(6):
        r = _run(binary, scenario, 8, seed)
        if r.returncode != 0:
            failed = True
            break
    assert failed, f"the model did not catch {plant}"


def test_exchanged_buffers_keep_producers_on_separate_lines(tmp_path):
    """tests/exchange_lines.cpp: over random expert loads, no 128-byte line
    of a buffer exchanged inside one launch (tile-slotted source index and
    MXFP8 H scales, router slices, gathered rows, H, H codes) holds bytes of
    two producers that consumers wait for separately; the row-indexed source
    index of the earlier layout must share lines for some loads (so the check
    can fail)."""
    binary = tmp_path / "exchange_lines"
    subprocess.run(["g++", "-std=c++17", "-O2", "-o", str(binary), os.path.join(HERE, "exchange_lines.cpp")],
                   check=True, capture_output=True, text=True)
    for seed in (1, 2, 3):
        r = subprocess.run([str(binary), "400", str(seed)], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
