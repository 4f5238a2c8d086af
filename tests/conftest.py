import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    from long_context_decode_kv_amd.build import ensure_built
    ensure_built()


def pytest_terminal_summary(terminalreporter):
    """Parity summary of the GPU comparisons against the oracle: count, the
    worst max |err| and RMSE of out, the worst lse error, and the cases."""
    mod = sys.modules.get("gpu_cases")
    rep = getattr(mod, "REPORT", None)
    if not rep:
        return
    tr = terminalreporter
    tr.write_sep("-", f"oracle parity: {len(rep)} comparisons")
    lse = [r[3] for r in rep if r[3] is not None]
    tr.write_line(f"worst max|out err| {max(r[1] for r in rep):.3e}, worst out RMSE {max(r[2] for r in rep):.3e}, "
                  f"worst max|lse err| {max(lse) if lse else 0.0:.3e} (bound 2e-3)")
    for r in sorted(rep, key=lambda r: -r[1])[:5]:
        tr.write_line(f"  {r[0]}: max|out err| {r[1]:.3e}, RMSE {r[2]:.3e}")
