"""The seeded generator draws the same tensors everywhere: every tensor's
SHA-256 (dtype, shape and bytes) against tests/golden/synth_manifest.txt,
written by tests/golden/make_synth_manifest.py.  The oracle and the GPU path
both read these inputs, so a platform where numpy's streams drew differently
would fail here before any parity test."""
import importlib.util
from pathlib import Path

GOLDEN = Path(__file__).parent / "golden"


def _maker():
    spec = importlib.util.spec_from_file_location("make_synth_manifest", GOLDEN / "make_synth_manifest.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_generator_matches_manifest():
    want = dict(line.split() for line in (GOLDEN / "synth_manifest.txt").read_text().splitlines())
    mk = _maker()
    got = {name: mk.digest(a) for name, a in mk.tensors()}
    assert set(got) == set(want)
    bad = [n for n in got if got[n] != want[n]]
    assert not bad, bad
