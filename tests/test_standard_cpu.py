"""CPU check of the standard-attention baseline that bench.py times beside the
tiled kernels: its forward and its written-out backward (float32 on the host)
agree with the fp64 oracle, with causal and key-padding masks."""

import importlib.util
import os

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_52_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("causal,klr", [(False, None), (True, None), (False, (9, 40)),
                                        (True, (20, 40))])
def test_standard_baseline_cpu(causal, klr):
    bench = load_bench()
    prob = inputs.make_problem(2, 2, 40, 16, "fp32", seed=5 + 7 * causal, causal=causal,
                               key_len_range=klr, scale=0.3)
    q, k, v, do = (torch.from_numpy(x.copy()) for x in (prob.q, prob.k, prob.v, prob.do))
    mask = bench.standard_attention_mask(prob, torch.device("cpu"))
    o, p = bench.standard_forward(q, k, v, float(prob.scale), mask)
    dq, dk, dv = bench.standard_backward(q, k, v, do, p, float(prob.scale))
    args = [x.astype(np.float64) for x in (prob.q, prob.k, prob.v)]
    kw = dict(causal=causal, key_lens=prob.key_lens)
    ro, _ = oracle.forward(*args, float(prob.scale), **kw)
    rdq, rdk, rdv = oracle.backward(*args, prob.do.astype(np.float64), float(prob.scale), **kw)
    for name, got, ref in (("o", o, ro), ("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        assert np.abs(got.double().numpy() - ref).max() <= 1e-5, name
