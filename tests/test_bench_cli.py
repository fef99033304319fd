"""bench.py command line, on the host: more than one GPU is refused with a
message before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout


def test_bench_fixes_host_threads_before_numpy():
    # the oracle baseline's BLAS pool is sized when numpy loads: bench.py sets
    # the thread count from the CPU affinity before that import
    code = ("import bench, json; from threadpoolctl import threadpool_info; "
            "print(json.dumps([bench.HOST_CORES, max(i['num_threads'] for i in threadpool_info())]))")
    env = dict(os.environ)
    env.pop("OMP_NUM_THREADS", None)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stderr
    cores, blas = __import__("json").loads(r.stdout.strip().splitlines()[-1])
    assert cores == len(os.sched_getaffinity(0))
    assert blas == cores
