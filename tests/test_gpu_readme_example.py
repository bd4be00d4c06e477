"""The README's decode-step example runs as written, and its output matches the oracle."""
import os
import re

import numpy as np
import pytest
import torch

from oracle import oracle_attn_decode_cache

from gpu_util import assert_parity

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_decode_step_example():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    ns = {}
    exec(compile(code, "README.md", "exec"), ns)
    torch.cuda.synchronize()
    out = ns["out"].cpu().numpy()
    assert np.all(np.isfinite(out))
    S, KV, D, CAP, NQ = ns["S"], ns["KV"], ns["D"], ns["CAP"], ns["NQ"]
    ref = oracle_attn_decode_cache(ns["q"].cpu().numpy(), ns["k_cache"].cpu().numpy(), ns["v_cache"].cpu().numpy(),
                                   ns["v_scales"].cpu().numpy(), ns["slot_ids"], ns["positions"], S, CAP, 0, 0,
                                   NQ, KV, D, D ** -0.5)
    assert ref.shape == out.shape == (S, NQ, D)
    assert_parity(out, ref, "README example")
