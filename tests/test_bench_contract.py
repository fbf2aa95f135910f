"""bench.py's command-line contract on a host without a GPU: more than one GPU
is refused with a message and a non-zero status before any device is touched
(this path measures one GPU's share; its output rows shard without
communication)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for argv, env in ((["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "4"})):
        e = dict(os.environ, **env)
        res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                             capture_output=True, text=True, env=e, timeout=300)
        assert res.returncode == 2, (argv, env, res.stderr)
        assert "runs on one GPU" in res.stderr
        assert res.stdout == ""
