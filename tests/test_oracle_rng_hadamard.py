"""Pins of the oracle's sign generator and Hadamard transform.

Philox4x32-10 is compared with an independent implementation: the header-only
Philox engine shipped in torch's C++ headers, compiled here with g++.  The
Hadamard matrix is compared with scipy's, and the float32 fast transform with
an exact matrix product on integer inputs.
"""

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import hadamard, philox

_PHILOX_CPP = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  unsigned long long seed = strtoull(argv[1], 0, 0);
  unsigned long long offset = strtoull(argv[2], 0, 0);
  at::Philox4_32 e(seed, 0, offset);
  for (int i = 0; i < 4; ++i) printf("%u\n", (unsigned)e());
  return 0;
}
"""


def _torch_philox_block(tmpdir, seed, offset):
    exe = os.path.join(tmpdir, "philox_ref")
    if not os.path.exists(exe):
        src = os.path.join(tmpdir, "philox_ref.cpp")
        with open(src, "w") as f:
            f.write(_PHILOX_CPP)
        inc = os.path.join(os.path.dirname(torch.__file__), "include")
        subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc, src, "-o", exe],
                       check=True, capture_output=True)
    out = subprocess.run([exe, str(seed), str(offset)], check=True, capture_output=True, text=True)
    return [int(x) for x in out.stdout.split()]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_philox_matches_torch_header_engine():
    # torch's engine: key = (seed lo, seed hi), counter = (offset lo, offset hi, subseq lo, subseq hi)
    with tempfile.TemporaryDirectory() as td:
        try:
            _torch_philox_block(td, 1, 0)
        except (subprocess.CalledProcessError, FileNotFoundError) as e:  # pragma: no cover
            pytest.skip(f"cannot build the torch Philox reference: {e}")
        for seed in (0, 1, 0x5EED, 0xDEADBEEFCAFEF00D, 2**64 - 1):
            for off in (0, 1, 7, 2**33 + 5):
                ref = _torch_philox_block(td, seed, off)
                ours = philox.philox4x32_10((off & 0xFFFFFFFF, off >> 32, 0, 0),
                                            (seed & 0xFFFFFFFF, seed >> 32))
                assert ours == ref, (seed, off)


def test_sign_vector_values_and_seed_dependence():
    s = philox.sign_vector(0x5EED, 128)
    assert s.dtype == np.float32 and s.shape == (128,)
    assert set(np.unique(s).tolist()) <= {-1.0, 1.0}
    assert np.array_equal(philox.sign_vector(0x5EED, 64), s[:64])
    assert not np.array_equal(philox.sign_vector(1, 128), s)
    # over many seeds each channel is close to balanced
    mean = np.mean([philox.sign_vector(sd, 128) for sd in range(400)], axis=0)
    assert np.all(np.abs(mean) < 0.3)


def test_sign_vector_bit_order():
    words = philox.philox4x32_10((0, 0, 0, 0), (0x5EED, 0))
    s = philox.sign_vector(0x5EED, 128)
    for c in (0, 1, 31, 32, 63, 64, 127):
        bit = (words[c // 32] >> (c % 32)) & 1
        assert s[c] == (-1.0 if bit else 1.0)


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_sylvester_matches_scipy_and_is_orthogonal(d):
    h = hadamard.sylvester(d)
    assert np.array_equal(h, scipy.linalg.hadamard(d))
    assert np.array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))


@pytest.mark.parametrize("d", [4, 64, 128])
def test_fwht_exact_on_integers(d):
    rng = np.random.default_rng(d)
    x = rng.integers(-1000, 1000, size=(50, d)).astype(np.float32)
    got = hadamard.fwht_f32(x)
    ref = (x.astype(np.int64) @ scipy.linalg.hadamard(d)).astype(np.float32)
    assert np.array_equal(got, ref)


def test_fwht_float32_error_bound():
    rng = np.random.default_rng(11)
    d = 128
    x = rng.standard_normal((1000, d)).astype(np.float32)
    got = hadamard.fwht_f32(x).astype(np.float64)
    ref = x.astype(np.float64) @ scipy.linalg.hadamard(d)
    # 7 stages, each adds at most half an ulp of a partial sum bounded by sum |x|
    bound = 7 * 2.0 ** -24 * np.abs(x).astype(np.float64).sum(axis=1, keepdims=True)
    assert np.all(np.abs(got - ref) <= bound)
    assert np.array_equal(hadamard.fwht_f64(x), ref)


def test_fwht_stage_order_is_observable():
    # the float32 result depends on the stage order: this is why the order is fixed
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2000, 8)).astype(np.float32) * np.float32(1e3)
    fwd = hadamard.fwht_f32(x)
    y = x.copy()
    for h in (4, 2, 1):                        # reversed order
        z = y.reshape(-1, 8 // (2 * h), 2, h)
        a, b = z[..., 0, :], z[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(-1, 8)
    assert not np.array_equal(fwd, y)
