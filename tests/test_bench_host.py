"""bench.py's host-side contract, on the CPU: it measures one GPU and says so
when asked for more (before it imports torch or touches a device); its
kernel-source hash ignores comments, so that the stored HBM-traffic summary
stays valid across comment edits and is dropped for any code change; and it
checks every timed output against the digest of the oracle's output, stored
by tests/golden/make_bench_hashes.py, which must be what that script
computes from the oracle now."""
import hashlib
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(args, env_extra=None):
    env = {**os.environ, **(env_extra or {})}
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench(["--gpus", "2"])
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr and r.stdout == ""
    r = _bench(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_kernel_source_hash_ignores_comments(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    csrc = tmp_path / "moe_swiglu_epilogue_amd" / "csrc"
    csrc.mkdir(parents=True)
    code = "int f(int x) {\n    return x + 1;   // one more\n}\n"
    (csrc / "moe_nvfp4.hip").write_text("/* header */\n" + code)
    (csrc / "nvfp4_device.hpp").write_text("#pragma once\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (csrc / "moe_nvfp4.hip").write_text("// another header\n\n" + code.replace("one more", "plus one"))
    assert bench.kernel_source_hash() == h0
    (csrc / "moe_nvfp4.hip").write_text(code.replace("x + 1", "x + 2"))
    assert bench.kernel_source_hash() != h0


def test_output_check_compares_digests(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import torch
    import bench
    a = torch.arange(16, dtype=torch.uint8)
    b = torch.zeros(4, dtype=torch.float32)
    f = tmp_path / "h.json"
    f.write_text(json.dumps({"a": hashlib.sha256(a.numpy().tobytes()).hexdigest(),
                             "b": "0" * 64}))
    monkeypatch.setattr(bench, "EXPECTED_HASHES", str(f))
    oc = bench.OutputCheck()
    assert oc.check("a", a, a.clone()) is True
    assert oc.check("b", b) is False
    assert oc.check("c", b) is None
    r = oc.report()
    assert (r["checked"], r["matched"], r["mismatched"], r["unchecked"]) == (2, 1, ["b"], ["c"])
    bf = torch.tensor([1.0, -2.0], dtype=torch.bfloat16)
    assert oc.digest(bf) == hashlib.sha256(bf.view(torch.int16).numpy().tobytes()).hexdigest()


def _stored():
    with open(os.path.join(ROOT, "tests", "golden", "bench_output_sha256.json")) as f:
        return json.load(f)


def test_stored_digests_cover_every_checked_output():
    with open(os.path.join(ROOT, "bench.py")) as f:
        keys = set(re.findall(r'oc\.check\("([^"]+)"', f.read()))
    assert keys == set(_stored())


def test_stored_digests_are_the_oracles():
    """About 25 s of oracle work over every bench workload but the GEMM."""
    sys.path.insert(0, os.path.join(ROOT, "tests", "golden"))
    import make_bench_hashes
    assert make_bench_hashes.compute() == _stored()
