"""The kernels' relative-distance bucket, built for the host from the same header, against the
oracle's bucket over every distance |d| < 70,000 (both signs), and its inverse on the bucket starts.

The kernels' bias indexing must be bit-exact; this compiles device_common.h's rel_bucket /
rel_bucket_start (declared __host__ __device__) into a small host program with hipcc.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.bucket import bucket

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

SRC = r"""
#include <cstdio>
#include "device_common.h"
int main() {
  for (int d = -70000; d < 70000; ++d) std::printf("%d\n", jfa::rel_bucket(d));
  for (int u = 16; u < 64; ++u) std::printf("%d\n", jfa::rel_bucket_start(u));
  return 0;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_device_bucket_equals_reference_on_every_distance(tmp_path):
    src = tmp_path / "bucket_check.hip"
    src.write_text(SRC)
    exe = tmp_path / "bucket_check"
    r = subprocess.run([HIPCC, "-O1", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"), "-I",
                        os.path.join(ROOT, "jagged_sequence_amd", "csrc"), str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    vals = np.array(out, dtype=np.int64)
    d = np.arange(-70000, 70000)
    np.testing.assert_array_equal(vals[: len(d)], bucket(d))
    starts = vals[len(d):]
    for u, s in zip(range(16, 64), starts):
        assert bucket(s) == u and bucket(s - 1) == u - 1, (u, s)
