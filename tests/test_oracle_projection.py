"""Pins of the down-projection oracle (`project_latent`) and of its fp64 ->
bf16 rounding (`f64_to_bf16_bits`).

* brute force: each output written out as an exactly summed dot product
  (math.fsum over the products, which are exact in float64 for bf16 inputs)
  over output row n of the weight, on non-square shapes, so a transposed
  operand or a swapped c_kv / k_pe split fails;
* a closed form: with w_down = [I | 0] the projection returns the first
  d_c + d_rope features of h bit for bit;
* rounding: equal to torch's bf16 conversion wherever no double rounding is
  involved (inputs exactly representable in binary32), ties to even at exact
  midpoints, and rounded up just above a midpoint.
"""
import math

import numpy as np
import torch

from oracle import bf16_bits_to_f64, f64_to_bf16_bits, project_latent
from workload import make_projection_inputs


def test_project_latent_brute_force():
    T, d_model, d_c, d_rope = 3, 40, 6, 4
    inp = make_projection_inputs(T, d_model, d_c + d_rope, seed=3)
    c, k = project_latent(inp.h, inp.w_down, d_c)
    assert c.shape == (T, d_c) and k.shape == (T, d_rope)
    h = bf16_bits_to_f64(inp.h)
    w = bf16_bits_to_f64(inp.w_down)
    for t in range(T):
        for n in range(d_c + d_rope):
            exact = math.fsum(h[t, j] * w[n, j] for j in range(d_model))
            want = f64_to_bf16_bits(np.array([exact]))[0]
            got = c[t, n] if n < d_c else k[t, n - d_c]
            assert got == want, (t, n)


def test_identity_weight_returns_the_features():
    T, d_model, d_c, d_rope = 5, 24, 8, 4
    inp = make_projection_inputs(T, d_model, d_c + d_rope, seed=1)
    eye = np.zeros((d_c + d_rope, d_model), dtype=np.float32)
    eye[np.arange(d_c + d_rope), np.arange(d_c + d_rope)] = 1.0
    w_bits = (eye.view(np.uint32) >> 16).astype(np.uint16)
    c, k = project_latent(inp.h, w_bits, d_c)
    assert np.array_equal(c, inp.h[:, :d_c]) and np.array_equal(k, inp.h[:, d_c:d_c + d_rope])


def test_bf16_rounding_matches_torch_without_double_rounding():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(100000) * rng.choice([1e-4, 1.0, 1e4], 100000)).astype(np.float32)
    got = f64_to_bf16_bits(x.astype(np.float64))
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_bf16_rounding_midpoints():
    step = 2.0 ** -7                                   # bf16 spacing in [1, 2)
    x = np.array([1 + step / 2, 1 + 1.5 * step, -(1 + step / 2), 1 + step / 2 + 2.0 ** -40, 0.0, -0.0])
    got = bf16_bits_to_f64(f64_to_bf16_bits(x))
    assert list(got[:4]) == [1.0, 1 + 2 * step, -1.0, 1 + step]
    assert got[4] == 0.0 and np.signbit(got[5])
