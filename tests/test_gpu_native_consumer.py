"""GPU: the library used from a native program through its C header alone.

tests/native/abi_consumer (built by __graft_entry__.build() from
abi_consumer.cpp) allocates device memory with hipMalloc, lays a ragged list out
in one buffer per stream with a 3-element gap after each tensor (so tensors
start at every 16-byte phase), runs 3 mixed steps with adamw_multi_tensor_step
on a stream of its own and then adamw_check_finite on the gradients, and writes
back the counter, the flag and every state stream.  The test writes its
seeded inputs, runs it as a child process, and holds its output to the CPU
oracle bit for bit: no torch or Python sits between the program and the
library.
"""
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import to_np

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_consumer")
NUMELS = [1000, 7, 4099, 1, 20000, 0, 65536 + 5, 9]
STEPS = 3


def test_native_consumer_matches_the_oracle(tmp_path):
    if not os.path.exists(EXE):
        raise FileNotFoundError(f"{EXE} is missing: build it with __graft_entry__.build()")
    arena = workloads.make_state("mixed", NUMELS, "cpu", seed=7700, align_elems=1, random_moments=True)
    host = {k: to_np(arena.bufs[k]).copy() for k in ("p", "g", "m", "v", "master")}
    hp = oracle.HParams()
    with open(tmp_path / "in.bin", "wb") as f:
        f.write(struct.pack("<q", len(NUMELS)) + struct.pack(f"<{len(NUMELS)}q", *NUMELS))
        f.write(struct.pack("<i", STEPS))
        f.write(struct.pack("<6f", hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.inv_scale))
        for k in ("p", "g", "m", "v", "master"):        # the ABI's stream order
            f.write(host[k].tobytes())
    torch.cuda.synchronize()
    r = subprocess.run([EXE, str(tmp_path / "in.bin"), str(tmp_path / "out.bin")], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    raw = open(tmp_path / "out.bin", "rb").read()
    step, flag = struct.unpack("<ii", raw[:8])
    n = sum(NUMELS)
    got, pos = {}, 8
    for k, dt in (("p", np.uint16), ("m", np.float32), ("v", np.float32), ("master", np.float32)):
        size = n * np.dtype(dt).itemsize
        got[k] = np.frombuffer(raw[pos:pos + size], dtype=dt)
        pos += size
    assert pos == len(raw)
    tensors = [{k: host[k][o:o + c] for k in host} for o, c in zip(np.cumsum([0] + NUMELS[:-1]), NUMELS)]
    t = 0
    for _ in range(STEPS):
        t = oracle.step_list("mixed", tensors, hp, t)
    assert step == t == STEPS and flag == 0
    for k in got:
        assert np.array_equal(got[k].view(np.uint8), host[k].view(np.uint8)), f"stream {k} differs from the oracle"
