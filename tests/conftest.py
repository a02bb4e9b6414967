import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    import margins
    t = margins.table()
    if not t:
        return
    terminalreporter.section("worst max|GPU - oracle| / RMS(oracle) per test (bound 2e-3)")
    for test, (what, err) in t.items():
        terminalreporter.write_line(f"{err:.3e}  {test}  [{what}]")
    worst = max(err for _, err in t.values())
    terminalreporter.write_line(f"overall worst: {worst:.3e} over {len(t)} tests")
    try:
        out = os.path.join(ROOT, "gpurun_out")
        os.makedirs(out, exist_ok=True)
        with open(os.path.join(out, "gpu_margins.json"), "w") as f:
            json.dump({k: {"what": w, "max_abs_over_rms": e} for k, (w, e) in t.items()}, f, indent=1)
    except OSError:
        pass
