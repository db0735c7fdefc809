"""PA_DEBUG_CHECK=1: with the variable set, every entry point copies its device-resident
index data to the host and rejects contract violations (include/pagedkv.h) with
PA_ERR_INVALID and a message, before launching anything; valid inputs give the same bits
as without the checks.

The variable is read once per process, so the checked calls run in a fresh child
process (tests/_debug_check_child.py) started with it set; this process, which has no
such variable, runs the same valid inputs for the bit comparison."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from _gpu import log, pk

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))

# every case the child runs, with a phrase its message must contain
EXPECTED = {
    "decode table id = num_blocks": "outside",
    "decode table id = -1": "outside",
    "decode_no_alloc table id = num_blocks": "outside",
    "decode_no_alloc table id = -1": "outside",
    "decode seq_len above max_seq_len": "seq_lens[3]",
    "decode_append two sequences append into one slot": "both append into slot",
    "decode_append newest slot read by another sequence": "is also read by sequence 3",
    "write slot outside the pool": "beyond the pool",
    "write slot named twice": "named twice",
    "copy src == dst": "onto itself",
    "copy dst repeated": "repeated",
    "copy dst is also a src": "both a src and a dst",
    "copy pair outside the pool": "outside",
    "swap dst repeated": "repeated",
    "swap pair outside the pools": "outside the pools",
    "multi_query q_start[0] != 0": "q_start must run from 0",
    "multi_query q_start[-1] != total_q": "q_start must run from 0",
    "multi_query more queries than max_q_len": "max_q_len",
    "multi_query more queries than tokens": "with 16 queries",
    "multi_query table id outside the pool": "outside",
    "shared_prefix group_start[-1] != num_seqs": "group_start",
    "shared_prefix prefix longer than a member": "prefix_lens[1]",
    "shared_prefix member not sharing the prefix": "does not share",
}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pk()


def test_debug_checks_reject_bad_index_data_and_keep_valid_bits(tmp_path):
    env = dict(os.environ, PA_DEBUG_CHECK="1")
    log("debug checks: child process with PA_DEBUG_CHECK=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "_debug_check_child.py"), str(tmp_path)],
                       env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    cases = {c["case"]: c for c in json.loads(r.stdout.strip().splitlines()[-1])["cases"]}
    assert set(cases) == set(EXPECTED), sorted(set(cases) ^ set(EXPECTED))
    for name, phrase in EXPECTED.items():
        c = cases[name]
        assert c["status"] == 1, (name, c)                       # PA_ERR_INVALID
        assert phrase in c["message"], (name, c["message"])
        assert c["untouched"], f"{name}: the call changed its output or pool"
        log(f"debug checks: {name}: {c['message']}")

    # the same valid calls here, without the checks
    sys.path.insert(0, HERE)
    import _debug_check_child as child
    assert os.environ.get("PA_DEBUG_CHECK", "") != "1"
    mine = child.run_valid(*child.inputs())
    theirs = np.load(os.path.join(tmp_path, "debug_valid.npz"))
    assert set(theirs.files) == set(mine)
    for k in mine:
        assert np.array_equal(mine[k], theirs[k]), f"{k}: bits differ with PA_DEBUG_CHECK=1"
    log(f"debug checks: valid outputs bit-identical ({', '.join(sorted(mine))})")
