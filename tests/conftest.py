import json
import os
import sys
from dataclasses import replace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI)")


# Parity records: every GPU lockstep appends its measured errors, noise floors
# and compared / excluded token counts here; the session writes them to
# parity_records.json in the run's results folder (RECORDS_DIR) so that the
# numbers behind each tolerance decision survive the run (pytest itself
# swallows the test's prints).
RECORDS_DIR = "gpurun_out"
PARITY_RECORDS = []
CURRENT_TEST = {"id": None}


@pytest.fixture(autouse=True)
def _current_test(request):
    CURRENT_TEST["id"] = request.node.nodeid
    yield
    CURRENT_TEST["id"] = None


def record_parity(rec):
    """Append one record and rewrite the file (a crash mid-session keeps
    every record written so far)."""
    rec = dict(rec)
    rec["test"] = CURRENT_TEST["id"]
    PARITY_RECORDS.append(rec)
    out = os.path.join(ROOT, RECORDS_DIR)
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, "parity_records.json"), "w") as f:
        json.dump(PARITY_RECORDS, f, indent=1)


@pytest.fixture(scope="session")
def hand_cases():
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        return json.load(f)


def tiny_hybrid_config():
    """A tiny pair whose target mixes GatedDeltaNet and attention layers
    (3 GDN + 1 attention, the hybrid layout at toy width) for CPU checks."""
    from dflash_block_diffusion_amd import configs as C
    base = C.tiny()
    kinds = (C.LAYER_GDN, C.LAYER_GDN, C.LAYER_GDN, C.LAYER_ATTN)
    t = replace(base.target, n_layers=4, layer_kinds=kinds, gdn_heads=8, gdn_dk=32,
                gdn_dv=32, fmt=C.FMT_F32)
    return replace(base, name="tiny-hybrid", target=t, sel_layers=(1, 3))
