"""The host-side diagnostics and tuning switches, read from the environment
once per process, so each case runs in a child process:
  OMM_LOG=1         every launch prints its kernel choice to stderr;
  OMM_TILE=MxNxK    forces the 256x256x64 or 128x128x64 bf16 / fp16 tile path
                    (bench sweeps): the forced path must still match the oracle."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from onnx_matmul_family_amd import synth
from tests.gpu_util import check_close

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, {root!r})
from onnx_matmul_family_amd import _omm as om, synth
from onnx_matmul_family_amd.hostdev import dev, host_f64
M, N, K, seed = {M}, {N}, {K}, {seed}
rng = np.random.default_rng(seed)
A = synth.store(synth.normal(rng, (M, K), 0.05), "bf16")
B = synth.store(synth.normal(rng, (N, K), 0.05), "bf16")
Y = om.gemm(dev(A, "bf16"), dev(B, "bf16"), None, 1.0, 0.0, 0, 1)
q = om.qlinear_matmul(*(dev(x) for x in (np.ones((256, 256), np.int8), np.array(0.5, np.float32),
                                          np.array(0, np.int8), np.ones((256, 256), np.int8),
                                          np.array(0.5, np.float32), np.array(0, np.int8),
                                          np.array(1.0, np.float32), np.array(0, np.int8))))
torch.cuda.synchronize()
np.save({out!r}, host_f64(Y))
"""


def run_child(tmp_path, env_extra, M, N, K, seed):
    out = str(tmp_path / "y.npy")
    code = CHILD.format(root=ROOT, M=M, N=N, K=K, seed=seed, out=out)
    env = dict(os.environ)
    env.pop("OMM_LOG", None)
    env.pop("OMM_TILE", None)
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    return np.load(out), r.stderr


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check(got, M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = synth.store(synth.normal(rng, (M, K), 0.05), "bf16")
    B = synth.store(synth.normal(rng, (N, K), 0.05), "bf16")
    y, t = oracle.gemm(A, B, None, 1.0, 0.0, 0, 1, dt="bf16")
    check_close(got, y, t, "bf16", "gemm %dx%dx%d" % (M, N, K))


def test_log_reports_kernel_choices(tmp_path):
    got, err = run_child(tmp_path, {"OMM_LOG": "1"}, 1024, 1024, 512, 1)
    lines = [l for l in err.splitlines() if l.startswith("omm: ")]
    assert any("bf16 M=1024 N=1024 K=512" in l and "128x128x64 tiles" in l for l in lines), err
    assert any("qlinear i8 x i8 -> i8 M=256 N=256 K=256" in l and "16x16x64" in l for l in lines), err
    check(got, 1024, 1024, 512, 1)
    # silent without the switch
    _, err = run_child(tmp_path, {}, 64, 64, 64, 2)
    assert not any(l.startswith("omm: ") for l in err.splitlines())


@pytest.mark.parametrize("tile,M,N,K", [("128x128x64", 4096, 4096, 128), ("256x256x64", 1024, 1280, 320)])
def test_tile_override_forces_the_path_and_matches(tmp_path, tile, M, N, K):
    got, err = run_child(tmp_path, {"OMM_TILE": tile, "OMM_LOG": "1"}, M, N, K, 3)
    want = tile.split("x")[0] + "x" + tile.split("x")[1] + "x64 tiles"
    assert any(("bf16 M=%d" % M) in l and want in l and "(OMM_TILE)" in l for l in err.splitlines()), err
    check(got, M, N, K, 3)
