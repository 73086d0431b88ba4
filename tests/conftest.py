import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


def pytest_terminal_summary(terminalreporter):
    """The worst |err| / tolerance the fp16-path parity checks saw, per check
    (written to $TQ2_PARITY_REPORT as JSON when that is set)."""
    worst = {}
    for name, mod in list(sys.modules.items()):
        if name.endswith("test_gpu_parity"):
            worst.update(getattr(mod, "WORST", {}) or {})
    if not worst:
        return
    terminalreporter.section("fp16 parity: worst |err| / tolerance per check")
    for key, ratio in sorted(worst.items()):
        terminalreporter.write_line(f"{ratio:.6f}  {key}")
    path = os.environ.get("TQ2_PARITY_REPORT")
    if path:
        with open(path, "w") as f:
            json.dump(dict(sorted(worst.items())), f, indent=1)
