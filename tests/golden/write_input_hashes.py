"""Write tests/golden/input_hashes.json: SHA-256 of the generator's output for
the two small workloads (calls only the input generator)."""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from gemm_inputs import make_workload, sha256  # noqa: E402

out = {}
for name in ("square_256", "square_1024_int"):
    _, a, b = make_workload(name)
    out[name] = {"A": sha256(a), "B": sha256(b)}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_hashes.json")
with open(path, "w") as f:
    json.dump(out, f, indent=1)
    f.write("\n")
print(path)
