"""The usage example of the README runs as written, and its decode and
prefill outputs match the float64 oracle."""

import re
import os

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import ROOT
from tests.helpers import assert_lse_close, assert_out_close, bits

pytestmark = pytest.mark.gpu


def test_readme_example():
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    torch.manual_seed(0)
    ns = {}
    exec(compile(code, "README.md", "exec"), ns)
    torch.cuda.synchronize()
    kv, seq, bt = ns["kv"], ns["seq"], ns["bt"]
    assert seq.cpu().tolist() == [37]
    assert ns["pos"].cpu().tolist() == [34, 35, 36]
    k = bits(kv[:, 0])
    v = bits(kv[:, 1])
    # the appended rows are in place (page 2, slots 2..4, every head)
    assert np.array_equal(k[2, :, 2:5].transpose(1, 0, 2), bits(ns["k_new"]))
    btn = bt.cpu().numpy()
    ref = oracle.batch_prefill(bits(ns["q"]), "bf16", k, v, "bf16", btn, np.array([37]),
                               np.array([37]), 128 ** -0.5, True, "HND")
    assert_out_close(ns["out"], ref[0], torch.bfloat16)
    assert_lse_close(ns["lse"], ref[1])
