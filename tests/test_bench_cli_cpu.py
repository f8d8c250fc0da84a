"""bench.py's command line on a machine without a GPU: asking for several GPUs
is refused with a JSON error line and exit status 2, before any GPU work."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_several_gpus_are_refused():
    for n in ("2", "8"):
        r = subprocess.run([sys.executable, "bench.py", "--gpus", n], cwd=ROOT, capture_output=True, text=True,
                           timeout=120)
        assert r.returncode == 2
        line = json.loads(r.stdout.strip().splitlines()[-1])
        assert "one GPU" in line["error"]
