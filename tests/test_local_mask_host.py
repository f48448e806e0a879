"""Host check of the kernels' local-visibility logic (csrc/local_mask.h).

CPU only.  The header's LocalVis (the 64-bit key masks, the tile key ranges
and the transposed relation of the dK/dV pass) is compiled with g++ behind a
few shims for the device qualifiers, run over random windows and grids, and
compared with the oracle's visibility rule (oracle.local_visible): the masks
must be exactly the visible keys, and the key ranges must contain every
visible key of their rows.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import local_visible

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_25_amd", "csrc")

PROG = r"""
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
using std::max;
using std::min;
#define __device__
#define __forceinline__ inline
static inline float __int_as_float(int x) { float f; std::memcpy(&f, &x, 4); return f; }
static inline int __float_as_int(float f) { int x; std::memcpy(&x, &f, 4); return x; }
#define __builtin_amdgcn_rcpf(x) (1.0f / (x))
#define __builtin_amdgcn_exp2f(x) exp2f(x)
#include "local_mask.h"
// stdin: wl wr cols nr nc N lim transposed; stdout per position p: the mask
// words of keys 0.., then the key range of rows 0..p
int main() {
  int wl, wr, cols, nr, nc, n, lim, tr;
  while (std::scanf("%d %d %d %d %d %d %d %d", &wl, &wr, &cols, &nr, &nc, &n, &lim, &tr) == 8) {
    attn::LocalVis v{wl, wr, cols, nr, nc};
    if (tr) v = v.transposed();
    for (int p = 0; p < n; ++p) {
      const attn::LocalVis::Row w = v.row(p);
      for (int j0 = 0; j0 < n; j0 += 64)
        std::printf("%llu ", (unsigned long long)v.bits(w, j0, lim));
      int lo, hi;
      v.key_range(0, p, lim, lo, hi);
      std::printf("| %d %d\n", lo, hi);
    }
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("lm")
    (d / "t.cpp").write_text(PROG)
    subprocess.run([cxx, "-O1", "-std=c++17", f"-I{CSRC}", str(d / "t.cpp"), "-o",
                    str(d / "t")], check=True)
    return str(d / "t")


def _run(prog, wl, wr, cols, nr, nc, n, lim, tr=0):
    out = subprocess.run([prog], input=f"{wl} {wr} {cols} {nr} {nc} {n} {lim} {tr}\n",
                         capture_output=True, text=True, check=True).stdout.splitlines()
    vis, rng = [], []
    for line in out:
        words, r = line.split("|")
        bits = []
        for wd in words.split():
            x = int(wd)
            bits += [(x >> i) & 1 for i in range(64)]
        vis.append(bits[:n])
        rng.append(tuple(int(t) for t in r.split()))
    return np.array(vis, dtype=bool), rng


def _cases():
    rng = np.random.default_rng(11)
    cases = [(3, 0, 0, 0, 0, 130, 130), (0, 0, 0, 0, 0, 200, 200), (400, 400, 0, 0, 0, 200, 150),
             (400, 400, 56, 5, 5, 300, 300), (400, 0, 7, 2, 3, 200, 200), (400, 400, 1, 70, 1, 260, 260),
             (50, 20, 13, 3, 4, 333, 300)]
    for _ in range(12):
        n = int(rng.integers(1, 400))
        open_ = 2 * n
        wl = int(rng.choice([open_, int(rng.integers(0, n + 1))]))
        wr = int(rng.choice([open_, 0, int(rng.integers(0, n + 1))]))
        cols = int(rng.choice([0, int(rng.integers(1, 60))]))
        nr = int(rng.integers(1, 8)) if cols else 0
        nc = min(int(rng.integers(1, 8)), cols) if cols else 0
        cases.append((wl, wr, cols, nr, nc, n, int(rng.integers(0, n + 1))))
    return cases


@pytest.mark.parametrize("case", _cases())
def test_masks_and_ranges_match_the_oracle(prog, case):
    wl, wr, cols, nr, nc, n, lim = case
    grid = (cols, nr, nc) if cols else None
    want = local_visible(np.arange(n), n, window=(wl, wr), grid=grid)
    want[:, lim:] = False
    got, ranges = _run(prog, wl, wr, cols, nr, nc, n, lim)
    np.testing.assert_array_equal(got, want)
    for p, (lo, hi) in enumerate(ranges):
        keys = np.nonzero(want[:p + 1].any(axis=0))[0]
        if keys.size:
            assert lo <= keys.min() and keys.max() <= hi, (p, lo, hi, keys.min(), keys.max())
        if grid is None and keys.size:
            assert (lo, hi) == (keys.min(), keys.max())   # exact for a window


@pytest.mark.parametrize("case", _cases()[:8])
def test_transposed_masks_are_the_columns(prog, case):
    """transposed(): bit p of key j's mask iff the query at p sees key j."""
    wl, wr, cols, nr, nc, n, _ = case
    grid = (cols, nr, nc) if cols else None
    want = local_visible(np.arange(n), n, window=(wl, wr), grid=grid).T
    got, _ = _run(prog, wl, wr, cols, nr, nc, n, n, tr=1)
    np.testing.assert_array_equal(got, want)
