"""Pins for the oracle's Philox4x32-10 and its uniform streams.

The generator is Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3"
(SC'11).  Independent pins: rocRAND's own Philox4x32-10 engine (open-source
header code, compiled here for the host), and the closed forms of the Weyl key
increments.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND host reference")
    exe = str(tmp_path_factory.mktemp("rr") / "philox_ref")
    subprocess.run([hipcc, "-O1", "-o", exe, os.path.join(HERE, "philox_rocrand_ref.cpp")],
                   check=True, capture_output=True, timeout=300)

    def run(queries):
        """queries: list of (seed, subsequence, offset, n) -> list of uint32 lists."""
        text = "".join(f"{s} {ss} {o} {n}\n" for s, ss, o, n in queries)
        out = subprocess.run([exe], input=text, capture_output=True, text=True,
                             check=True, timeout=60).stdout
        return [[int(w, 16) for w in line.split()] for line in out.strip().splitlines()]
    return run


def _ctr_query(seed, ctr):
    """rocRAND's engine: key = seed, counter words (0,1) advance with offset/4,
    counter words (2,3) are the subsequence.  The 64-bit offset holds 4x the
    counter, so word 1 must stay below 2**30."""
    assert int(ctr[1]) < 2**30
    c0, c1, c2, c3 = (int(v) for v in ctr)
    return (seed, c2 | (c3 << 32), 4 * (c0 | (c1 << 32)), 4)


def test_weyl_constants_closed_form():
    # floor(2**32 * frac(golden ratio)) and floor(2**32 * (sqrt(3) - 1))
    w0 = ((math.isqrt(5 << 128) - (1 << 64)) >> 1) >> 32
    w1 = (math.isqrt(3 << 128) - (1 << 64)) >> 32
    assert philox.PHILOX_W0 == w0
    assert philox.PHILOX_W1 == w1


def test_philox_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(7)
    cases = [(0, (0, 0, 0, 0)),
             (0xFFFFFFFFFFFFFFFF, (0xFFFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF)),
             (1, (1, 0, 0, 0)), (123456789, (5, 7, 11, 13))]
    for _ in range(60):
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        ctr = tuple(int(v) for v in rng.integers(0, 2**32, size=4))
        ctr = (ctr[0], ctr[1] >> 2, ctr[2], ctr[3])
        cases.append((seed, ctr))
    ref = rocrand_ref([_ctr_query(s, c) for s, c in cases])
    for (seed, ctr), want in zip(cases, ref):
        got = philox.philox4x32_10(np.array(ctr), philox.key_of_seed(seed))
        assert [int(v) for v in got] == want, (seed, ctr)


def test_stream_layout_matches_rocrand(rocrand_ref):
    """Each stream's counter layout, checked through the independent engine."""
    seed = 0x0123456789ABCDEF
    b, a = 77, 3
    js = [0, 1, 2, 3, 4, 2047, 2048, 151935]
    q_tok = [(seed, b | (2 << 32), 4 * ((j >> 2) | (a << 32)) + (j & 3), 1) for j in js]
    w_tok = [r[0] for r in rocrand_ref(q_tok)]
    assert np.array_equal(philox.u_token(seed, b, a, js), philox.uniform_open(w_tok))

    cs = [0, 1, 2, 3, 4, 74]
    q_blk = [(seed, b | (1 << 32), 4 * ((c >> 2) | (a << 32)) + (c & 3), 1) for c in cs]
    w_blk = [r[0] for r in rocrand_ref(q_blk)]
    assert np.array_equal(philox.u_block(seed, b, a, cs), philox.uniform_open(w_blk))

    ii = [0, 1, 11]
    q_acc = [(seed, b, 4 * (i << 32), 1) for i in ii]
    w_acc = [r[0] for r in rocrand_ref(q_acc)]
    assert np.array_equal(philox.u_accept(seed, b, ii), philox.uniform_accept(w_acc))


def test_uniform_maps_exact_and_in_range():
    w = np.array([0, 1, 255, 256, 511, 512, 0x7FFFFFFF, 0xFFFFFFFF], dtype=np.uint64)
    ua = philox.uniform_accept(w)
    uo = philox.uniform_open(w)
    assert ua[0] == 0.0 and ua[-1] == 1.0 - 2.0**-24
    assert uo[0] == 2.0**-24 and uo[-1] == 1.0 - 2.0**-24
    assert np.all(ua < 1.0) and np.all(uo > 0.0) and np.all(uo < 1.0)
    # exactly representable in float32
    assert np.array_equal(ua.astype(np.float32).astype(np.float64), ua)
    assert np.array_equal(uo.astype(np.float32).astype(np.float64), uo)


def test_uniforms_are_uniform():
    from scipy import stats
    u = philox.u_token(42, 3, 1, np.arange(200000))
    counts, _ = np.histogram(u, bins=50, range=(0.0, 1.0))
    assert stats.chisquare(counts).pvalue > 1e-3
    u2 = np.concatenate([philox.u_accept(9, b, np.arange(16)) for b in range(2000)])
    counts, _ = np.histogram(u2, bins=32, range=(0.0, 1.0))
    assert stats.chisquare(counts).pvalue > 1e-3


def test_gumbel_closed_form():
    u = np.array([np.exp(-1.0), 0.5, 2.0**-24])
    g = philox.gumbel(u)
    assert abs(g[0]) < 1e-15                       # -ln(-ln e^-1) = 0
    assert abs(g[1] + math.log(math.log(2.0))) < 1e-15
    assert g[2] < -2.8
