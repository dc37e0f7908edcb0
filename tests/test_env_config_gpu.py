"""SKINNY_CONFIG on the GPU: a child process with the override set computes Y = X W^T + R
through skinny_addmm_bf16, the entry point that names no configuration; its output must equal, bit for bit, the
explicit-configuration call on the same seeded inputs in this process (the override routes the
compute, not only the selection)."""
import json
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest
import torch

from decode_skinny_addmm_amd import synth

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import decode_skinny_addmm_amd as sk
from decode_skinny_addmm_amd import synth
M, N, K = (int(v) for v in sys.argv[2].split(","))
X, ws, rs = synth.make_inputs(M, N, K, seed=11)
R = rs[0].cuda()
Y = sk.addmm_default(X.cuda(), ws[0].cuda(), R, torch.empty_like(R))
torch.cuda.synchronize()
np.save(sys.argv[3], synth.bits(Y.cpu()))
print(json.dumps(sk.select_config(M, N, K)))
"""


@pytest.fixture(scope="module")
def sk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_skinny_addmm_amd as d
    d.ops.lib()
    return d


@pytest.mark.parametrize("M,N,K", [(4, 1024, 3584), (40, 512, 1024)])
def test_env_config_routes_the_compute(sk, M, N, K):
    # a built configuration the table does not pick for this M: the direct MFMA path
    cfg = next(c for c in sk.configs() if c["path"] == 1 and c["m_tile"] == 16)
    assert cfg != sk.select_config(M, N, K)
    value = ",".join(str(cfg[k]) for k in ("path", "block_size", "outputs_per_block", "k_unroll", "vector_width",
                                           "m_tile", "k_split", "k_stage"))
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "y.npy")
        print("env config", value, (M, N, K), flush=True)
        out = subprocess.run([sys.executable, "-c", CHILD, ROOT, "%d,%d,%d" % (M, N, K), path],
                             env=dict(os.environ, SKINNY_CONFIG=value), capture_output=True, text=True,
                             timeout=300)
        assert out.returncode == 0, out.stderr[-2000:]
        assert json.loads(out.stdout.strip().splitlines()[-1]) == cfg
        y_env = np.load(path)
    X, ws, rs = synth.make_inputs(M, N, K, seed=11)
    y_cfg = synth.bits(sk.addmm(X.cuda(), ws[0].cuda(), rs[0].cuda(), config=cfg).cpu())
    torch.cuda.synchronize()
    assert np.array_equal(y_env, y_cfg)
