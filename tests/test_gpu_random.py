"""GPU parity on seeded random configurations through the C ABI: sequence count
and lengths (empty, single-token, partial and several chunks), key-head
grouping, head sizes, input type, gate form, output epilogue, slot caches and
segment length (so that the map pass, the prefix and the output pass of the
first segments on the second stream all take part), each against the fp64
oracle with the same options."""

import numpy as np
import pytest

from tests.test_gpu_options import _prefill_case

pytestmark = pytest.mark.gpu

CASES = 24


def _config(i):
    r = np.random.default_rng(1000 + i)
    N = int(r.integers(1, 5))
    lens = [int(r.choice([0, 1, 63, 64, 65, int(r.integers(1, 400))])) for _ in range(N)]
    if sum(lens) == 0:
        lens[0] = 130
    Hk = int(r.choice([1, 2]))
    H = Hk * int(r.choice([1, 2]))
    K, V = int(r.choice([64, 128])), int(r.choice([64, 128]))
    dt = str(r.choice(["bf16", "f32"]))
    gates = str(r.choice(["pre", "plain"]))
    norm = bool(r.integers(0, 2))
    z_act = [None, "none", "sigmoid"][int(r.integers(0, 3))]
    slots = None
    if r.integers(0, 2):
        slots = [int(x) for x in r.permutation(N + 2)[:N]]
        if N > 1 and r.integers(0, 2):
            slots[int(r.integers(0, N))] = -1
    seg = [None, "1", "2", "3"][int(r.integers(0, 4))]
    return dict(lens=lens, Hk=Hk, H=H, K=K, V=V, dt=dt, gates=gates, norm=norm, z_act=z_act, slots=slots, seg=seg)


@pytest.mark.parametrize("i", range(CASES))
def test_random_configuration(i, monkeypatch):
    c = _config(i)
    print(f"  case {i}: {c}", flush=True)
    if c["seg"] is not None:
        monkeypatch.setenv("KDA_SEG_CHUNKS", c["seg"])
    _prefill_case(2000 + i, c["lens"], c["Hk"], c["H"], c["K"], c["V"], c["dt"], gates=c["gates"], norm=c["norm"],
                  z_act=c["z_act"], slots=c["slots"])
