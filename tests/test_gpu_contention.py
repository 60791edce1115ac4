"""Contention check ("GLM on an A100, in Vx", section "What the GPU found":
many processes share one GPU, each checking every op against an independent
answer).  Eight fresh worker processes (contention_worker.py) run their own
seeded decode workloads on the one GPU at the same time; each checks its
repeated steps bit for bit and its result against the oracle, and the parent
compares every worker's result bit for bit with the same workload run alone in
this process beforehand."""
import os
import subprocess
import sys
import time

import numpy as np
import pytest
import torch

from sparse_attention_14_amd import device, inputs

import contention_worker
from gpu_util import gpu_decode_step

pytestmark = pytest.mark.gpu

WORKERS = 8
HERE = os.path.dirname(os.path.abspath(__file__))


def test_eight_processes_share_the_gpu(tmp_path):
    refs = {}
    for w in range(WORKERS):
        p = inputs.make_problem(contention_worker.workload(w))
        out, lse, scores, idx, _ = gpu_decode_step(device.upload(p))
        refs[w] = {"out": out.cpu().numpy(), "lse": lse.cpu().numpy(), "scores": scores.cpu().numpy(),
                   "idx": idx.cpu().numpy()}
    torch.cuda.synchronize()
    print(f"single-process references for {WORKERS} workloads done; starting {WORKERS} workers", flush=True)
    env = dict(os.environ)
    procs = []
    try:
        for w in range(WORKERS):
            cmd = [sys.executable, "-u", os.path.join(HERE, "contention_worker.py"), "--worker", str(w), "--steps",
                   "20", "--out", str(tmp_path / f"w{w}.npz")]
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, env=env))
        deadline = time.time() + 300
        logs = {}
        for w, pr in enumerate(procs):
            try:
                text, _ = pr.communicate(timeout=max(deadline - time.time(), 1))
            except subprocess.TimeoutExpired:
                raise AssertionError(f"worker {w} did not finish in time")
            logs[w] = text.decode(errors="replace")
            print(f"worker {w} exited with {pr.returncode}: {logs[w].strip().splitlines()[-1:]}", flush=True)
        bad = [w for w, pr in enumerate(procs) if pr.returncode != 0]
        assert not bad, "workers failed:\n" + "\n".join(f"--- worker {w}\n{logs[w][-2000:]}" for w in bad)
    finally:
        for pr in procs:
            if pr.poll() is None:
                pr.kill()
                pr.wait()
    for w in range(WORKERS):
        got = np.load(tmp_path / f"w{w}.npz")
        for key, ref in refs[w].items():
            assert np.array_equal(got[key].view(np.uint8), ref.view(np.uint8)), \
                f"worker {w}: {key} differs from the single-process run"
