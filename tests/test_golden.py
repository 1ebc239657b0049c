"""The stored golden fixture is what its committed generator writes from the
seeded workload and the oracle (so a change to either shows up here)."""
import importlib.util
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_golden_is_current(tmp_path):
    spec = importlib.util.spec_from_file_location(
        "make_tiny_golden", os.path.join(HERE, "golden", "make_tiny_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    out = tmp_path / "tiny_decode.txt"
    mod.main(str(out))
    with open(os.path.join(HERE, "golden", "tiny_decode.txt")) as f:
        assert out.read_text() == f.read()
