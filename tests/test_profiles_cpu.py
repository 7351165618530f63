"""The committed rocprofv3 summaries against the algorithmic byte model: for
every mover role the calibrated HBM bytes per launch (FETCH_SIZE and
WRITE_SIZE, scaled by a plain copy's readings) must lie within 5% of the
bytes the method has to move, so no kernel moves a byte twice; and the
windowed refresh's traffic must match its line-floor writes plus the sector
reads its partial writes cost, within 5%."""
import json
import os
import sys

import pytest

import workloads as W

R = pytest.importorskip("recurrent_state_cache_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _recorded(workload):
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("traffic_bytes:"):
                return json.loads(line[len("traffic_bytes:"):])
    raise AssertionError(f"no traffic_bytes line in {path}")


@pytest.mark.parametrize("workload", ["mixed", "gdn", "kda"])
def test_recorded_traffic_matches_the_byte_model(workload):
    cfg, _ = bench._workload(workload)
    P = R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    pack, unpack, pack_q, unpack_q = bench._algorithmic_bytes(P)
    n = cfg.n_ckpt
    # a launch's bytes: the call's bytes over its launches (dasc_plan_launches)
    model = {role: b * n / P.launches(role, n)[0]
             for role, b in (("pack", pack), ("unpack", unpack), ("pack_int8", pack_q),
                             ("unpack_int8", unpack_q))}
    Wn = W.windows(cfg)
    model["refresh_windowed"] = (bench._windowed_bytes(P, Wn, decay_bytes=4)
                                 + bench._windowed_sector_reads(P, Wn))
    rec = _recorded(workload)
    for role, b in model.items():
        ratio = rec[role] / b
        assert 0.95 <= ratio <= 1.05, f"{workload} {role}: {rec[role]} B measured, {b} B model"
