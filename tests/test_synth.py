"""The seeded input generator: determinism, independence from thread count,
distributions, and exact bf16 rounding.  CPU only."""
import os
import subprocess
import sys

import numpy as np
import torch

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_deterministic_and_stream_separated():
    a = synth.normal_f32(1001, 0, synth.T_X, 0, 1.0)
    b = synth.normal_f32(1001, 0, synth.T_X, 0, 1.0)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, synth.normal_f32(1001, 1, synth.T_X, 0, 1.0))
    assert not np.array_equal(a, synth.normal_f32(1001, 0, synth.T_WG, 0, 1.0))
    assert not np.array_equal(a, synth.normal_f32(1001, 0, synth.T_X, 1, 1.0))
    # a prefix of a longer stream is the shorter stream
    assert np.array_equal(synth.normal_f32(4000, 0, synth.T_X, 0, 1.0)[:1001], a)


def test_independent_of_thread_count():
    code = ("import synth,sys;import numpy as np;"
            "a=synth.normal_bf16(300001,5,3,7,0.1);sys.stdout.write(str(int(a.astype(np.int64).sum())))")
    outs = set()
    for n in ("1", "3", "8"):
        env = dict(os.environ, OMP_NUM_THREADS=n, PYTHONPATH=ROOT)
        outs.add(subprocess.check_output([sys.executable, "-c", code], env=env, cwd=ROOT))
    assert len(outs) == 1


def test_moments():
    z = synth.normal_f32(1_000_000, 0, synth.T_TEST, 0, 1.0).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert abs(((z - z.mean()) ** 4).mean() / z.var() ** 2 - 3) < 0.05      # normal kurtosis
    u = synth.uniform_f32(1_000_000, 0, synth.T_TEST, 1, -0.05, 0.05).astype(np.float64)
    assert u.min() >= -0.05 and u.max() < 0.05 and abs(u.mean()) < 2e-4


def test_bf16_is_round_to_nearest_even_of_f32():
    f = synth.normal_f32(200_001, 2, synth.T_TEST, 3, 0.7)
    b = synth.normal_bf16(200_001, 2, synth.T_TEST, 3, 0.7)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)


def test_config_shapes():
    c = synth.C1
    inp = synth.gen_inputs(c)
    assert inp["x"].shape == (64, 128) and inp["x"].dtype == np.float32
    assert inp["w13"].shape == (16, 128, 128) and inp["w2"].shape == (16, 128, 64)
    assert inp["ws13"].shape == (128, 128) and inp["ws2"].shape == (128, 64)
    assert inp["gate_w"].shape == (16, 128) and inp["bias"].shape == (16,)
    assert np.all(np.abs(inp["bias"]) <= 0.1)
    np.testing.assert_allclose(inp["w13"].std(), 1 / np.sqrt(128), rtol=0.05)
    np.testing.assert_allclose(inp["w2"].std(), 1 / np.sqrt(64), rtol=0.05)
