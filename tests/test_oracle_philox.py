"""Pins for the oracle's Philox, uniform mapping and Gumbel transform (CPU only).

* Philox4x64-10 instantiation of the generic code == numpy.random.Philox
  (an independent library implementation), which validates the round
  structure, the high/low product split, the word permutation and key bumps.
* Philox4x32-10 instantiation == rocRAND's host-compiled Philox4x32-10
  engine (a second independent library implementation), validating the
  32-bit multipliers and Weyl constants.
* The uniform mapping's end points and the Gumbel(0,1) moments (mean is the
  Euler-Mascheroni constant, variance pi^2/6) from the textbook distribution.
"""

import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import philox


def _numpy_block(key, counter, advance):
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                          counter=np.array(counter, dtype=np.uint64))
    raw = bg.random_raw(4 * (advance + 1))
    return [int(x) for x in raw[4 * advance:4 * advance + 4]]


def _ours64(key, counter):
    out = philox.philox4(tuple([c] for c in counter), key, width=64)
    return [int(w[0]) for w in out]


@pytest.mark.parametrize("key,counter", [
    ((0, 0), (0, 0, 0, 0)),
    ((0x0123456789ABCDEF, 0xFEDCBA9876543210), (5, 7, 11, 13)),
    ((2**64 - 1, 2**64 - 1), (2**64 - 3, 2**64 - 1, 0, 1)),
    ((12345, 678), (2**63, 3, 2**62 + 9, 17)),
])
def test_philox4x64_matches_numpy(key, counter):
    # numpy bumps its counter before producing each block, so its first block
    # is the bijection applied to counter + 1 (little-endian 256-bit add).
    c = list(counter)
    i = 0
    while True:
        c[i] = (c[i] + 1) % 2**64
        if c[i] != 0 or i == 3:
            break
        i += 1
    assert _ours64(key, c) == _numpy_block(key, counter, 0)


def test_philox4x64_second_block_matches_numpy():
    key, counter = (99, 1), (41, 0, 0, 0)
    assert _ours64(key, (43, 0, 0, 0)) == _numpy_block(key, counter, 1)


_ROCRAND_PROBE = r"""
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  // args: seed subsequence offset4  -> counter = (offset4 lo, offset4 hi, subseq lo, subseq hi)
  unsigned long long seed = strtoull(argv[1], 0, 0), sub = strtoull(argv[2], 0, 0),
                     off = strtoull(argv[3], 0, 0);
  rocrand_state_philox4x32_10 st;
  rocrand_init(seed, sub, off * 4ULL, &st);
  uint4 r = rocrand4(&st);
  printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_probe():
    hdr = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    gxx = shutil.which("g++")
    if not (gxx and os.path.exists(hdr)):
        pytest.skip("rocRAND header or g++ not available")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "probe.cpp")
    exe = os.path.join(d, "probe")
    with open(src, "w") as f:
        f.write(_ROCRAND_PROBE)
    r = subprocess.run([gxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        src, "-o", exe], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("could not build rocRAND host probe: " + r.stderr[:300])
    yield exe
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("seed,c0,c1,c2,c3", [
    (0, 0, 0, 0, 0),
    (0, 1, 0, 0, 0),
    (2**64 - 1, 2**32 - 1, 2**30 - 1, 2**32 - 1, 2**32 - 1),  # offset*4 must fit 64 bits
    (0x243F6A8885A308D3, 0x13198A2E, 0x03707344, 0xA4093822, 0x299F31D0),
    (42, 1000, 8191, 31, 0),
    (7, 32767, 131071, 7, 0),
])
def test_philox4x32_matches_rocrand(rocrand_probe, seed, c0, c1, c2, c3):
    off4 = c0 + (c1 << 32)
    sub = c2 + (c3 << 32)
    out = subprocess.run([rocrand_probe, str(seed), str(sub), str(off4)], capture_output=True,
                         text=True, check=True).stdout.split()
    ref = [int(x) for x in out]
    ours = philox.philox4(([c0], [c1], [c2], [c3]), (seed & 0xFFFFFFFF, seed >> 32), width=32)
    assert [int(w[0]) for w in ours] == ref


def test_keyformer_words_counter_layout(rocrand_probe):
    # word (j mod 4) of the block at counter (j//4, pos, head, 0)
    seed, head, pos = 123456789, 5, 8000
    j = np.arange(40)
    words = philox.keyformer_words(seed, head, pos, j)
    for jj in (0, 3, 4, 17, 39):
        out = subprocess.run([rocrand_probe, str(seed), str(head), str((jj // 4) + (pos << 32))],
                             capture_output=True, text=True, check=True).stdout.split()
        assert int(words[jj]) == int(out[jj % 4])


def test_uniform_open_endpoints():
    u = philox.uniform_open(np.array([0, 511, 512, 2**32 - 1], dtype=np.uint64))
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24
    assert u[2] == 3 * 2.0 ** -24
    assert u[3] == 1.0 - 2.0 ** -24
    assert np.all((u > 0) & (u < 1))
    # every value is exactly representable in float32
    assert np.all(u.astype(np.float32).astype(np.float64) == u)


def test_uniformity_chi_square():
    words = philox.keyformer_words(0, 0, np.arange(64)[:, None], np.arange(4096)[None, :])
    u = philox.uniform_open(words).ravel()
    hist, _ = np.histogram(u, bins=64, range=(0, 1))
    exp = u.size / 64
    chi2 = ((hist - exp) ** 2 / exp).sum()
    # 63 degrees of freedom: mean 63, sd ~11.2; 6 sd bound
    assert chi2 < 63 + 6 * math.sqrt(2 * 63)


def test_gumbel_moments():
    words = philox.keyformer_words(2024, 3, np.arange(256)[:, None], np.arange(4096)[None, :])
    z = philox.gumbel(philox.uniform_open(words)).ravel()
    n = z.size
    euler_gamma = 0.5772156649015329
    var = math.pi ** 2 / 6
    assert abs(z.mean() - euler_gamma) < 5 * math.sqrt(var / n)
    # variance of the sample variance for Gumbel: (mu4 - sigma^4)/n, mu4 = 27/5 sigma^4
    assert abs(z.var() - var) < 5 * math.sqrt((27 / 5 - 1) * var ** 2 / n)


def test_gumbel_cdf_at_points():
    # F(z) = exp(-exp(-z)); the mapping is monotone, so u -> zeta inverts the cdf.
    u = np.array([0.1, 0.5, 0.9])
    z = philox.gumbel(u)
    assert np.allclose(np.exp(-np.exp(-z)), u, rtol=0, atol=1e-15)
