"""bench.py on the CPU: a run on more than one GPU is refused with a message
(the path is built for one GPU), and the byte counts and timing summaries it
reports follow from their definitions."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_update_bytes_per_element():
    """Fused update: grad read, master read and written, both moments read and
    written, all at their widths, and the 16-bit param written."""
    import bench

    class W:
        state_dtype, param_dtype = "fp32", "bf16"
    assert bench.update_bytes(W) == 30
    W.state_dtype = "bf16"
    assert bench.update_bytes(W) == 22
    W.state_dtype, W.param_dtype = "fp32", "fp32"
    assert bench.update_bytes(W) == 28
    assert bench.gradpass_bytes(W) == 4
    # bf16 main grads (2 B read) and an fp16 master (2 B read, 2 B written)
    W.param_dtype, W.grad_dtype = "bf16", "bf16"
    assert bench.update_bytes(W) == 28 and bench.gradpass_bytes(W) == 2
    W.master_dtype = "fp16"
    assert bench.update_bytes(W) == 24
    W.state_dtype = "bf16"
    assert bench.update_bytes(W) == 16


def test_spread_of_kernel_times():
    import bench
    assert bench.spread([3.0, 1.0, 2.0, 10.0]) == {"ms_median": 2.5, "ms_min": 1.0, "ms_max": 10.0}
