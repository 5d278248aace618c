"""The checking build (libbase_layer_checks.so, compiled with BASE_CHECKS):
the auction's kernels verify its invariants on the device -- every expert
holds at most T/E tokens, sorted best first during the bulk rounds (bulk
resolve and the late-round launch), the phase end never overfills an
expert, and after the solve every expert holds exactly T/E distinct tokens
-- and report a failure as BASE_ERR_INVARIANT. Runs in a child process so
that this process keeps the product library; covers every path of the solve
(the late-round launch of small solves, the two-launch rounds, the crowded
expert's filtered re-scan, the phase ends) and one layer forward.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import json, sys
import numpy as np
import torch
sys.path.insert(0, ROOT)
from balanced_token_expert_amd import api, build
from balanced_token_expert_amd import workloads as W
from tests.gpu_util import to_dev
api.load(build.LIB_CHECKS)
out = []
cases = [W.workload(1), W.custom(8192, 128, 256, None, kind="mixture", wid=971),
         W.workload(2), W.custom(32768, 128, 256, None, kind="skew", wid=972)]
for wl in cases:
    w = W.gen_centroids(wl)
    h = W.gen_tokens(wl, centroids=w)
    s = api.base_affinity(to_dev(h, wl.dtype), to_dev(w, wl.dtype))
    c = api.cfg(wl.eps_start, wl.eps_end, wl.eps_factor, max_bids=2000 * wl.T)
    r = api.base_assign_auction(s, c)
    torch.cuda.synchronize()
    st = api.read_stats(r["stats"])
    cnt = np.bincount(r["assign"].cpu().numpy(), minlength=wl.E)
    out.append(dict(case=wl.name, status=int(st.status), balanced=bool((cnt == wl.T // wl.E).all()),
                    phases=int(st.phases)))
# one balanced layer forward (the auction inside the layer call)
wl = W.custom(2048, 16, 128, 256, dtype="bf16", act="gelu", kind="iid", wid=973)
host = W.gen_all(wl)
dev = {k: to_dev(v, wl.dtype) for k, v in host.items()}
r = api.base_layer_forward(dev["h"], dev["w"], dev["W1"], dev["W2"], api.BASE_ACT_GELU,
                           api.BASE_ROUTE_BALANCED, api.cfg(1.0, 1e-4, 10.0))
torch.cuda.synchronize()
cnt = np.bincount(r["assign"].cpu().numpy(), minlength=wl.E)
out.append(dict(case="layer_t2048_e16", status=int(api.read_stats(r["stats"]).status),
                balanced=bool((cnt == wl.T // wl.E).all()), phases=0))
print("RESULT " + json.dumps(out), flush=True)
"""


def test_checking_build_auction_invariants():
    from balanced_token_expert_amd import build
    assert os.path.exists(build.LIB_CHECKS), "libbase_layer_checks.so not built"
    p = subprocess.run([sys.executable, "-c", "ROOT = %r\n" % ROOT + CHILD], cwd=ROOT,
                       capture_output=True, text=True, timeout=240)
    line = [l for l in p.stdout.splitlines() if l.startswith("RESULT ")]
    assert p.returncode == 0 and line, (p.returncode, p.stdout[-2000:], p.stderr[-2000:])
    res = json.loads(line[0][len("RESULT "):])
    print(res)
    assert len(res) == 5
    for r in res:
        assert r["status"] == 0, r
        assert r["balanced"], r
