"""The checked build against the product library, bit for bit.

libcsa2_checked.so is the same source compiled with -DCSA2_CHECKED: every
kernel takes its work in a scrambled workgroup order (a bijection of the
workgroup index chosen by the CSA2_WG_ORDER salt), so each cross-workgroup
hand-off (the last-arriving workgroup of the pool select, the digit
histograms, the tie lists, the dynamic scan schedule, the split partials)
sees another arrival order, and index bounds that the kernels rely on raise
CSA2_FLAG_CHECK when they fail.  The same seeded cases (tests/_checked_cases.py)
run in this process on libcsa2.so and in two child processes on the checked
library with two salts; every output must be identical and no flag raised."""
import os
import subprocess
import sys

import numpy as np
import pytest

import fp4_compressed_sparse_amd as csa2
from tests._gpu import log, require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_checked_build_matches_product_in_scrambled_orders(tmp_path):
    require_gpu()
    assert os.path.exists(csa2.CHECKED_LIB_PATH), "libcsa2_checked.so is not built (build.py builds both)"
    from tests._checked_cases import run_cases
    ref = run_cases()
    assert ref.pop("flags")[0] == 0
    log(f"product library: {len(ref)} outputs")
    for salt in (1, 2):
        out = tmp_path / f"checked_{salt}.npz"
        env = dict(os.environ, CSA2_LIB_PATH=csa2.CHECKED_LIB_PATH, CSA2_WG_ORDER=str(salt))
        log(f"checked library, workgroup-order salt {salt}")
        r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "_checked_cases.py"), str(out)],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
        got = dict(np.load(out))
        assert got.pop("loaded_checked")[0] == 1, "the child did not load libcsa2_checked.so"
        assert got.pop("flags")[0] == 0, "the checked build raised device flags"
        assert sorted(got) == sorted(ref)
        bad = [k for k in ref if got[k].shape != ref[k].shape or got[k].tobytes() != ref[k].tobytes()]
        assert not bad, f"salt {salt}: outputs differ from the product library: {bad[:10]}"
        log(f"salt {salt}: {len(ref)} outputs bit-identical, no flags")
