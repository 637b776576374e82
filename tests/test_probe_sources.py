"""The measurement probes under paged_kv_cache_469_amd/probes are generated
(gen_*_probe.py beside them writes the .hip that build() compiles).  These
CPU tests run each generator into a scratch folder and check that the
committed source is exactly what it writes, so the summaries under
profiles/ that quote a probe come from the generator as committed."""

import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBES = os.path.join(ROOT, "paged_kv_cache_469_amd", "probes")


@pytest.mark.parametrize("gen, out", [("gen_lds_probe.py", "lds_probe.hip"),
                                      ("gen_phase_probe.py", "phase_probe.hip")])
def test_committed_probe_is_the_generators_output(gen, out, tmp_path):
    spec = importlib.util.spec_from_file_location(gen[:-3], os.path.join(PROBES, gen))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.HERE = str(tmp_path)      # the generator writes beside itself; here into the scratch folder
    mod.main()
    with open(tmp_path / out) as f:
        written = f.read()
    with open(os.path.join(PROBES, out)) as f:
        committed = f.read()
    assert written == committed
