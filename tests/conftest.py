import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload")


from structured_decision_head_amd import synth  # noqa: E402


def tiny_spec(seed=7, B=2, lengths=(14, 22), fields="random", **over):
    """Tiny dimensions for brute-force pins: H=64, D=32, 4 heads, F=64."""
    head = synth.HeadConfig(hidden_size=64, width=32, heads=4, routing_layers=2, layers=2,
                            feedforward=64, vocab_size=97, num_types=3)
    kw = dict(name="tiny", seed=seed, head=head, B=B, L=None,
              lengths=("uniform", lengths[0], lengths[1]), fields=fields,
              field_range=(1, 3), choice_opts=(2, 3), score_levels=3,
              instr_len=(1, 3), opt_len=(1, 3), prefix=2, suffix=2, filler=(1, 1, 0, 0, 0))
    kw.update(over)
    return synth.CaseSpec(**kw)


def table_reader(case):
    return lambda ids: case.table[np.asarray(ids, dtype=np.int64)]


@pytest.fixture(scope="session")
def tiny_case():
    return synth.make_case(tiny_spec())
