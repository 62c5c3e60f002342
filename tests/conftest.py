import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: long CPU statistical test")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Parity counts of the GPU decode tests, per workload (see
    gpu_util.compare_frames), after the run."""
    gu = sys.modules.get("gpu_util")
    table = getattr(gu, "PARITY", None)
    if not table:
        return
    tr = terminalreporter
    tr.write_line("parity vs oracle (frames: exact / reproduced by one near-tie flip "
                  "/ unexplained; frames carrying a near-tie flag; exact frames whose "
                  "flag bits differ)")
    tot = {"frames": 0, "exact": 0, "flip": 0, "unexplained": 0}
    for tag in sorted(table):
        a = table[tag]
        for k in tot:
            tot[k] += a[k]
        tr.write_line(f"  {tag}: {a['frames']}: {a['exact']} / {a['flip']} / "
                      f"{a['unexplained']}; flagged {a['flagged']}; flag bits differ "
                      f"{a['flag_diff']}")
    tr.write_line(f"  total: {tot['frames']} frames: {tot['exact']} exact, "
                  f"{tot['flip']} flip, {tot['unexplained']} unexplained")
