"""The library shares the HIP runtime torch loaded (one runtime per process),
whatever is imported first (no GPU needed)."""
import subprocess
import sys


def test_single_hip_runtime_in_process():
    code = ("import recurrent_state_cache_amd, torch\n"
            "m = open('/proc/self/maps').read()\n"
            "libs = {l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}\n"
            "print(len(libs))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         check=True, cwd=__import__("os").path.dirname(__import__("os").path.dirname(__file__)))
    assert out.stdout.strip() == "1", out.stdout
