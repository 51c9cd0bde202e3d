"""The README's usage example, run as written on a small group and checked
against the oracle (so the documented call sequence stays correct)."""
import math
import os
import re

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, check, dev, host
from workloads.gen import random_small_group

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs_and_matches_the_oracle():
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    hq, hkv, d, p, lens = 32, 8, 128, 96, [40, 0, 70, 33]
    g = random_small_group(51, hq, hkv, d, p, lens, "bf16")
    cu = g["cu_seqlens"]
    t = {k: dev(g[k], "bf16") for k in g if k != "cu_seqlens"}
    # two microbatches of the four suffixes, each with its own cu_seqlens
    mbs, refs = [], []
    for idx in ([0, 1], [2, 3]):
        r0, r1 = int(cu[idx[0]]), int(cu[idx[-1] + 1])
        sub = np.concatenate([[0], np.cumsum([cu[i + 1] - cu[i] for i in idx])]).astype(np.int32)
        mbs.append((sub, t["q_s"][r0:r1], t["k_s"][r0:r1], t["v_s"][r0:r1], t["do_s"][r0:r1]))
    env = {"q_p": t["q_p"], "k_p": t["k_p"], "v_p": t["v_p"], "do_p": t["do_p"],
           "microbatches": mbs}
    exec(compile(code, "README.md", "exec"), env)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    hmap = oracle.head_map(hq, hkv)
    ref = oracle.suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"], cu,
                                  scale, hmap)
    tol = TOL["bf16"]
    check("gK after both microbatches", host(env["gk"]), ref["gk"], tol)
    check("gV after both microbatches", host(env["gv"]), ref["gv"], tol)
    rdq, rdk, rdv = oracle.prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"], g["do_p"],
                                                  ref["gk"], ref["gv"], scale, hmap)
    check("dQ_P", host(env["dq_p"]), rdq, tol)
    check("dK_P", host(env["dk_p"]), rdk, tol)
    check("dV_P", host(env["dv_p"]), rdv, tol)
