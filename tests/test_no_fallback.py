"""The product path has no CPU fallback and does not reach the oracle (CPU).

  - every entry point of the Python binding refuses CPU tensors with a status
    instead of computing anything on the host;
  - without libgdn_hip.so the package raises ImportError naming the build
    step (checked in a fresh interpreter whose library path points nowhere);
  - no module of the package imports the oracle, and the oracle imports
    nothing from the package: the two share only the seeded input generator,
    which the tests pass to both.
"""
import ast
import os
import subprocess
import sys

import pytest
import torch

import linear_attention_recurrence_recurrent_amd as gdn
from linear_attention_recurrence_recurrent_amd import GdnError, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_attention_recurrence_recurrent_amd")


def _cpu_ops():
    return synth.random_operands(1, 5, 1, 2, 16, 16, dtype="f32", seed=3)


@pytest.mark.parametrize("call", ["scan", "scan_noalloc", "recurrent_step", "three_pass"])
def test_recurrence_refuses_host_tensors(call):
    o = _cpu_ops()
    if call != "scan" and call != "scan_noalloc":
        o = {n: (t[:, :1].contiguous() if t.dim() >= 3 and n != "s0" else t) for n, t in o.items()}
    fn = {"scan": gdn.scan, "scan_noalloc": gdn.scan_noalloc, "recurrent_step": gdn.recurrent_step,
          "three_pass": gdn.recurrent_step_three_pass}[call]
    with pytest.raises(GdnError) as e:
        fn(o["q"], o["k"], o["v"], o["log_decay"], o["beta"], o["s0"], o["z"], o["w"])
    assert "GPU" in str(e.value)


def test_producers_refuse_host_tensors():
    a = torch.randn(64)
    with pytest.raises(GdnError, match="GPU"):
        gdn.gates(a, a.clone())
    with pytest.raises(GdnError, match="GPU"):
        gdn.conv_silu(torch.randn(1, 8, 16), torch.randn(16, 4))


def test_missing_library_raises_import_error():
    code = ("from linear_attention_recurrence_recurrent_amd import _native\n"
            "_native.LIB_PATH = '/nonexistent/libgdn_hip.so'\n"
            "import linear_attention_recurrence_recurrent_amd as gdn\n"
            "try:\n"
            "    gdn.abi_version()\n"
            "except ImportError as e:\n"
            "    print('ImportError:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("ImportError:") and "not built" in r.stdout


def _imports(path):
    names = set()
    for node in ast.walk(ast.parse(open(path).read())):
        if isinstance(node, ast.Import):
            names.update(a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            names.add(node.module or "")
    return names


def test_package_and_oracle_import_nothing_of_each_other():
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            assert not any(n.split(".")[0] == "oracle" for n in _imports(os.path.join(PKG, f))), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            names = _imports(os.path.join(ROOT, "oracle", f))
            assert not any(n.startswith("linear_attention_recurrence_recurrent_amd") for n in names), f
