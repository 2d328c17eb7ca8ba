"""Hand-worked fixtures under tests/golden/ (each file states its derivation and source)."""
import os

import numpy as np

import oracle
import synth

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read(name):
    out = {}
    with open(os.path.join(GOLD, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = np.array([float(v) for v in val.split()])
    return out


def test_int4_group_ties():
    g = _read("int4_group_ties.txt")
    K = 64
    x = np.zeros(K, np.float32)
    x[:len(g["x"])] = g["x"]
    xb = synth.f32_to_bf16_bits(x[None, :])
    codes, scales, _ = oracle.quant_act_int4(xb, np.ones(K, np.float32))
    assert scales[0, 0] == np.float32(g["scale"][0])
    q = oracle.unpack_int4(codes)[0]
    assert np.array_equal(q[:len(g["codes"])], g["codes"].astype(np.int8))
    assert np.all(q[len(g["codes"]):] == 0)
