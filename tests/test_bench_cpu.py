"""Host-side checks of bench.py: the one-GPU refusal, the algorithmic bytes
behind the decode roofline, and the recorded HBM traffic it reports."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                           env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, (argv, env, r.stderr)
        assert "one GPU" in r.stderr
        assert r.stdout == ""  # no JSON line


def test_decode_algorithmic_bytes():
    """Per (request, state head) unit: the d_k x d_v BF16 state read and
    written, v read and o written (d_v each), g and beta (4 bytes each); q and
    k (d_k each) once per q/k head, shared by H_v / H_qk state heads."""
    bench = load_bench()
    B, Hqk, Hv, d = 512, 16, 32, 128
    unit = 2 * d * d * 2 + 2 * d * 2 + 2 * 4
    qk = 2 * d * 2 * B * Hqk
    state, rest = bench.decode_bytes_per_launch(B, Hqk, Hv, d, d)
    assert state + rest == unit * B * Hv + qk == 1086455808


def test_recorded_traffic_is_plausible_when_current():
    """The committed counter summary is used only while the decode sources
    hash to the profiled ones; when used, it lies just above the algorithmic
    bytes (every state byte read and written once)."""
    bench = load_bench()
    t = bench.recorded_traffic()
    if t is None:
        return  # decode sources changed since the counters were taken: bench reports null
    algo = sum(bench.decode_bytes_per_launch(512, 16, 32, 128, 128))
    assert algo <= t <= 1.05 * algo
