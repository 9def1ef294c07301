"""bench.py against the library's kernel list (host only): every kernel the
library can time with a probe has a byte/flop model and a rule naming its HIP
kernels, the forward probe range matches the launches of ssd_fwd, and the
names the rules match are the ones the library's kernel trace reports."""
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from state_space_model_mamba2_amd import _lib, inputs  # noqa: E402


def test_every_probe_has_a_model():
    for name in inputs.WORKLOADS:
        shape = inputs.workload(name)
        esz = 4 if shape.dtype == "f32" else 2
        assert set(bench.kernel_model(shape, esz)) == set(_lib.KERNELS), name


def test_forward_probe_range():
    # ssd_fwd launches the kernels before the chunk-state backward, in probe-id order
    assert _lib.KERNELS[:_lib.N_FWD_KERNELS] == ["cumsum_bmm", "chunk_state", "state_passing", "chunk_scan"]


def test_models_are_positive_where_work_is():
    shape = inputs.workload("mamba2_2p7b")
    m = bench.kernel_model(shape, 2)
    for k, (nbytes, nflops) in m.items():
        assert nbytes > 0, k
        assert nflops >= 0, k
    # the chunk GEMM kernels do matrix-core work
    for k in ["cumsum_bmm", "chunk_state", "chunk_scan", "chunk_state_bwd", "chunk_scan_bwd", "dw_heads", "bc_final"]:
        assert m[k][1] > 0, k


def test_trace_names_match_rules():
    # every library kernel in the committed 2.7B-shape kernel trace is claimed by exactly one
    # bench probe rule, and every probe finds at least one kernel there
    path = os.path.join(ROOT, "profiles", "kernels_mamba2_2p7b.md")
    names = re.findall(r"\| `(_ZN3ssd[^`]*|void ssd::[^`]*|ssd::[^`]*)` \|", open(path).read())
    assert names, "no library kernels in the committed trace"
    claimed = {k: 0 for k in _lib.KERNELS}
    for n in names:
        owners = [k for k in _lib.KERNELS if bench.kernel_matches(k, n)]
        assert len(owners) == 1, (n, owners)
        claimed[owners[0]] += 1
    assert all(v > 0 for v in claimed.values()), claimed
