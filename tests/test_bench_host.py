"""Host-side contract of bench.py (no GPU): the multi-GPU refusal and where `traffic` comes from."""
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_only_from_counters_taken_on_this_kernel_source(tmp_path, monkeypatch):
    text = open(os.path.join(ROOT, "profiles", "rs_kernel_llama3_1_70b_layer_pmc.md")).read()
    recorded = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text).group(1)
    kernel = re.search(r"rs_kernel_name:\s*(.+)", text).group(1).strip()
    hbm = float(re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text).group(1))
    # the committed summary is read when its hash matches the kernel source and its kernel the launch's...
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: recorded)
    assert bench.read_traffic("llama3_1_70b_layer", kernel) == hbm
    # ...and ignored (null) for another kernel or any other source
    assert bench.read_traffic("llama3_1_70b_layer", "some_other_kernel<8>") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.read_traffic("llama3_1_70b_layer", kernel) is None
    assert bench.read_traffic("no_such_workload", kernel) is None
    # the counters moved every algorithmic byte about once (reads + writes within 1% of 20 B per output)
    algorithmic = int(re.search(r"algorithmic_bytes_per_launch:\s*([0-9]+)", text).group(1))
    assert abs(hbm / algorithmic - 1.0) < 0.01


def _oracle_imports(path):
    """(enclosing function or None, line) of every import of the oracle package in a source file."""
    import ast

    tree = ast.parse(open(path).read())
    found = []

    def visit(node, fn):
        for child in ast.iter_child_nodes(node):
            if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)):
                visit(child, child.name)
                continue
            if isinstance(child, ast.Import) and any(a.name.split(".")[0] == "oracle" for a in child.names):
                found.append((fn, child.lineno))
            if isinstance(child, ast.ImportFrom) and (child.module or "").split(".")[0] == "oracle":
                found.append((fn, child.lineno))
            visit(child, fn)

    visit(tree, None)
    return found


def test_oracle_only_in_the_cpu_baseline_leg_and_never_in_the_package():
    """The oracle is test infrastructure: bench.py touches it only in cpu_baseline, and nothing in the
    package or the input generators imports it."""
    uses = _oracle_imports(os.path.join(ROOT, "bench.py"))
    assert uses and all(fn == "cpu_baseline" for fn, _ in uses), uses
    for d in ("all_gather_placement_amd", "workloads"):
        for f in sorted(os.listdir(os.path.join(ROOT, d))):
            if f.endswith(".py"):
                assert _oracle_imports(os.path.join(ROOT, d, f)) == [], (d, f)


def test_profile_commands_use_flags_bench_py_knows():
    """Every bench.py command a committed profile summary gives uses only options bench.py accepts,
    so each summary can be re-made from the committed files."""
    known = set(bench.parser()._option_string_actions)
    seen = 0
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        for block in re.findall(r"```\n(.*?)```", text, flags=re.S):
            for line in block.splitlines():
                if "bench.py" not in line:
                    continue
                cmd = line.split("bench.py", 1)[1].split("#", 1)[0]
                flags = re.findall(r"(?<!\S)(--[a-z0-9][a-z0-9-]*)", cmd)
                unknown = [f for f in flags if f not in known]
                assert not unknown, (name, line, unknown)
                seen += 1
    assert seen >= 15
