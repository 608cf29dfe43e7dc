"""Write tests/golden/input_fingerprints.json: SHA-256 of the first 48 rows and
the last row of every seeded input tensor of every workload (the GEMM
workloads' operands included).  Calls only the input generator module (no
GPU code, no oracle arithmetic)."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from row_wise_normalization_rmsnorm_amd.workloads import GEMM_WORKLOADS, WORKLOADS  # noqa: E402
from tests.test_oracle_workloads import _fingerprint, _gemm_fingerprint  # noqa: E402

if __name__ == "__main__":
    fp = {name: _fingerprint(w) for name, w in WORKLOADS.items()}
    gfp = {name: _gemm_fingerprint(w) for name, w in GEMM_WORKLOADS.items()}
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_fingerprints.json")
    with open(out, "w") as f:
        json.dump({"what": "sha256 of rows 0..47 and the last row of each input tensor, then gamma",
                   "fingerprints": fp, "gemm_fingerprints": gfp}, f, indent=1, sort_keys=True)
    print(out)
