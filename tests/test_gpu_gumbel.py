"""The device Gumbel variates against -ln(-ln u) over every uniform the
Philox words can give (u = (2n + 1) 2^-24, n < 2^23): tests/gumbel_probe
evaluates the fp32 form (level 2) and the double form (level-1 keys) of
csrc/philox.h on the GPU; NumPy's float64 logs are the reference.  The
bounds are the ones the sampling error budget uses."""
import os
import subprocess

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gumbel_probe")


def test_gumbel_variates_within_their_bounds(tmp_path):
    if not os.path.exists(BIN):
        pytest.fail("tests/gumbel_probe is missing: build the package first")
    out = tmp_path / "g.f64"
    print("[gpu-case] gumbel probe, 2^23 uniforms", flush=True)
    r = subprocess.run([BIN, str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    g = np.fromfile(out, dtype="<f8")
    n = 1 << 23
    assert g.size == 2 * n
    u = (2.0 * np.arange(n, dtype=np.float64) + 1.0) * 2.0 ** -24
    exact = -np.log(-np.log(u))
    err32 = np.abs(g[:n] - exact)
    errw = np.abs(g[n:] - exact)
    print(f"max error: fp32 form {err32.max():.3e}, double form {errw.max():.3e}", flush=True)
    assert err32.max() < 2.0e-6
    assert errw.max() < 2.0e-7
