"""GPU: peers publish while the FFN side is already waiting on the device.

"[RFC]: Async GPU Connector", "Window and slot layout" (payload and flag are
ordered on the sender's stream, so a receiver that sees the flag sees the
whole payload) and "Risks and alternatives" (a device-side wait on the
flags instead of a host poll); "[RFC]: Async AFD for Prefill on Ascend NPU",
"Asynchronous work-item contract" (write before ready; a work item is ready
once its participants published; the FFN side may take any ready replica).

In every scenario the FFN-side call (a run, an any-ready run, two runs on a
ring of depth 2, a serve loop) is enqueued first, its wait kernel is seen
still pending after a host delay, and only then do the peers pack (and
enqueue their unpacks, which wait on the device for the replies).  Each
publish thus lands while a wait kernel on another stream spins on its flag,
and each reply while an unpack spins.  Every wait is bounded
(poll_timeout_us), so a publish that never arrives ends as AFD_ERR_TIMEOUT
with every kernel exiting.  Outputs are checked against the oracle and a
synchronous run's bits.  The scenarios (tests/concurrent_scenarios.py) run
in one child process with a fresh runtime: the spinning wait and the packs
must sit on distinct hardware queues, which a process that has already used
many streams cannot promise.
"""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
NAMES = [
    "run_waits_then_peers_publish[none_early]",
    "run_waits_then_peers_publish[peer0_early]",
    "ready_run_gathers_a_peer_that_arrives_during_the_window",
    "ready_run_waits_for_the_first_peer",
    "ring_depth_two_next_stage_published_while_the_first_runs",
    "serve_loop_with_peers_publishing_during_the_loop",
]


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("concurrent") / "res.json")
    env = dict(os.environ, GPU_MAX_HW_QUEUES="8")
    say("[concurrent] running the scenarios in a child process")
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "concurrent_scenarios.py"), out], env=env,
                       timeout=600, capture_output=True, text=True)
    say(r.stdout[-4000:])
    if r.returncode != 0:
        say(r.stderr[-4000:])
    res = json.load(open(out)) if os.path.exists(out) else {}
    res["_rc"] = r.returncode
    return res


@pytest.mark.timeout(700)
@pytest.mark.parametrize("name", NAMES)
def test_publish_while_waiting(results, name):
    assert results["_rc"] == 0, "the scenario process failed"
    assert results.get(name) == "ok", results.get(name)
