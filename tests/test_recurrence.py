"""The tiled online-softmax recurrence that the HIP kernel runs, modelled
here in fp64 on the CPU, reaches the oracle's plain definition.

The recurrence: the pages' attention pipeline runs QK^T per key tile (stage
T), then softmax with rescale (stage C), then PV (stage U). Tawa,
section III-D, describes the coarse-grained pipeline. PipeThreader's
"core method" lists the softmax and rescale tasks. Per key tile the row keeps
a running max m, a running sum l and an unnormalised output acc:
    m'  = max(m, max_j s_j)
    a   = exp(m - m')
    l   = a*l + sum_j exp(s_j - m')
    acc = a*acc + sum_j exp(s_j - m') v_j
and at the end o = acc / l, lse = m + ln l. This model lives in the tests
only. The oracle does not use it.
"""
import math

import numpy as np
import pytest

import oracle


def online_rows(q, k, v, scale, causal, bn):
    N, d = k.shape
    o = np.zeros((N, d))
    lse = np.zeros(N)
    for i in range(N):
        m, l, acc = -math.inf, 0.0, np.zeros(d)
        for j0 in range(0, N, bn):
            js = np.arange(j0, min(j0 + bn, N))
            if causal:
                js = js[js <= i]
            if js.size == 0:
                continue
            s = scale * (k[js] @ q[i])
            m2 = max(m, s.max())
            a = math.exp(m - m2) if m != -math.inf else 0.0
            p = np.exp(s - m2)
            l = a * l + p.sum()
            acc = a * acc + p @ v[js]
            m = m2
        o[i] = acc / l
        lse[i] = m + math.log(l)
    return o, lse


@pytest.mark.parametrize("bn", [1, 7, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_equals_definition(bn, causal):
    N, d = 150, 16
    r = np.random.default_rng(bn * 10 + causal)
    q, k, v = (r.standard_normal((1, 1, N, d)).astype(np.float16) for _ in range(3))
    k = (k.astype(np.float32) * 3).astype(np.float16)
    scale = np.float32(1 / math.sqrt(d))
    o_ref, l_ref = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
    o, l = online_rows(q[0, 0].astype(np.float64), k[0, 0].astype(np.float64),
                       v[0, 0].astype(np.float64), float(scale), causal, bn)
    np.testing.assert_allclose(o, o_ref[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, l_ref[0, 0], rtol=0, atol=1e-12)
