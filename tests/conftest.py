import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Worst relative L2 error of every attention parity case (and the
    near-tie counts of the other checks), so that the figures survive
    pytest's output capture."""
    mod = sys.modules.get("gpu_util")
    results = getattr(mod, "RESULTS", None) if mod else None
    if not results:
        return
    terminalreporter.write_sep("-", "parity summary (attention: worst per-sequence relative L2 error)")
    for label, r in results.items():
        extra = " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                         for k, v in r.items())
        terminalreporter.write_line(f"{label}: {extra}")
    path = os.environ.get("TV_PARITY_SUMMARY")
    if path:
        import json
        with open(path, "w") as f:
            json.dump(results, f, indent=1)
