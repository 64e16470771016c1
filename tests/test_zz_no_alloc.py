"""fmha_bwd_noalloc (through the C ABI) against fmha_bwd with a caller
workspace: the same kernels on the same inputs, so the gradients must agree
bit for bit. Two calls in a row, the second on a smaller problem, show that
what the fixed workspace keeps from one call does not leak into the next; a
call at the workspace's limit covers its full extent."""
import numpy as np
import pytest

from software_pipelining_fmha_amd import fmha, inputs

pytestmark = pytest.mark.gpu


def _problem(B, H, N, d, causal, seed):
    import torch
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=seed)
    do = inputs.draw_dout(B, H, N, d, seed=seed + 1)
    tq, tk, tv, tdo = (torch.from_numpy(x).to("cuda:0") for x in (q, k, v, do))
    o, lse = fmha.forward(tq, tk, tv, causal=causal)
    return tq, tk, tv, o, lse, tdo


def _same(a, b):
    for x, y in zip(a, b):
        assert np.array_equal(x.cpu().numpy().view(np.uint16), y.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_workspace_entry_point_twice(causal, device):
    import torch
    for B, H, N, d in ((2, 4, 1000, 128), (1, 3, 333, 64)):
        print("noalloc B=%d H=%d N=%d d=%d causal=%d" % (B, H, N, d, causal), flush=True)
        tq, tk, tv, o, lse, tdo = _problem(B, H, N, d, causal, 900 + N + causal)
        ref = fmha.backward(tq, tk, tv, o, lse, tdo, causal=causal)
        got = [torch.full_like(tq, float("nan")) for _ in range(3)]
        fmha.backward_noalloc(tq, tk, tv, o, lse, tdo, causal=causal, dq=got[0], dk=got[1],
                              dv=got[2])
        torch.cuda.synchronize()
        _same(ref, got)


def test_noalloc_at_its_row_limit(device):
    """B*H*N = FMHA_BWD_NOALLOC_MAX_ROWS (B1 H128 N16384 d64): the workspace's
    whole extent is in use. Inputs are seeded device-side normal draws."""
    import torch
    B, H, N, d = 1, 128, 16384, 64
    assert B * H * N == fmha.FMHA_BWD_NOALLOC_MAX_ROWS
    print("noalloc at the limit B=%d H=%d N=%d d=%d" % (B, H, N, d), flush=True)
    g = torch.Generator(device="cuda:0").manual_seed(1234)
    tq, tk, tv, tdo = (torch.randn((B, H, N, d), generator=g, device="cuda:0",
                                   dtype=torch.float32).half() for _ in range(4))
    o, lse = fmha.forward(tq, tk, tv, causal=True)
    ref = fmha.backward(tq, tk, tv, o, lse, tdo, causal=True)
    got = fmha.backward_noalloc(tq, tk, tv, o, lse, tdo, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(ref, got):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    # one row more is refused before anything is enqueued
    big = torch.empty((B, H, N + 1, d), dtype=torch.float16, device="cuda:0")
    big_lse = torch.empty((B, H, N + 1), dtype=torch.float32, device="cuda:0")
    with pytest.raises(fmha.FmhaError) as e:
        fmha.backward_noalloc(big, big, big, big, big_lse, big)
    assert e.value.status == fmha.FMHA_ERR_TOO_LARGE
