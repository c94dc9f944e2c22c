"""The tile table's recorded occupancies (workgroups per compute unit, which
the selection's fill model uses) against the HIP runtime's answer for the
kernels this library was built with: a kernel change that alters register
or LDS use without a re-measured table fails here."""
from __future__ import annotations

import pytest

import dense_fp32_matrix_02_amd as sg
from tests import _gpu as G
from tests._table import read_table

pytestmark = pytest.mark.gpu


def test_table_occupancy_matches_the_runtime():
    G.require_gpu()
    ids = {n: i for i, n in enumerate(sg.config_names())}
    stale = []
    for pair, (cands, _, _) in read_table().items():
        for name, occ in cands:
            got = sg.sgemm_mi355_config_occupancy(ids[name])
            print(f"[gpu] {name}: table {occ}, runtime {got}", flush=True)
            if got != occ:
                stale.append((name, occ, got))
    assert not stale, f"re-measure the tile table: {stale}"
