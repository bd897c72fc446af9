"""gdn_rollback_static (the rollback for callers that cannot allocate) against
gdn_rollback, through the C ABI: the same marked state, draft rows, history
and accepted lengths give the same state and history, bit for bit, on two
calls in a row, the second with fewer units than the first (the library's
count area then still holds the first call's longer count list).  A call
with more units than the area holds is refused before anything runs."""
import ctypes as C

import numpy as np
import pytest
import torch

import gated_deltanet_recurrent_amd as gdn
import synth

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "beta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    gdn.lib()
    yield
    torch.cuda.synchronize()


def host(t):
    return np.ascontiguousarray(t.detach().cpu().numpy())


def cycle(dims, N, M, seed, acc, static_counts):
    """mark(S, hist) -> step_m -> rollback(accepted) with one entry point."""
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(seed, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    hist = torch.randn((N, 3, cd), generator=gen, device="cuda")
    xc = torch.randn((M, N, cd), generator=gen, device="cuda")
    slab = gdn.Slab(N, dims, hist_floats_per_unit=3 * cd)
    slab.mark(S, hist)
    gdn.step_m(S, *(inp[n] for n in NAMES))
    hist.add_(1.0)                              # the history moved on meanwhile
    slab.rollback(S, acc, *(inp[n] for n in NAMES), hist=hist, xc_raw=xc,
                  static_counts=static_counts)
    torch.cuda.synchronize()
    return host(S), host(hist)


@pytest.mark.parametrize("dims", [synth.DIMS128, synth.DIMS64])
def test_rollback_static_equals_rollback_on_two_calls(dims):
    for N, M, seed in ((9, 6, 201), (4, 3, 202)):          # second call: fewer units
        acc = [(5 * u + 1) % (M + 1) for u in range(N)]
        acc[0], acc[-1] = M, 0
        want_S, want_h = cycle(dims, N, M, seed, acc, static_counts=False)
        got_S, got_h = cycle(dims, N, M, seed, acc, static_counts=True)
        assert got_S.tobytes() == want_S.tobytes(), (N, "state")
        assert got_h.tobytes() == want_h.tobytes(), (N, "history")


def test_rollback_static_refuses_more_units_than_its_area():
    L = gdn.lib()
    vh, kh, kd, vd = 1, 1, 64, 64
    N = (1 << 16) + 1
    nb = gdn.slab_bytes(N, (vh, kh, kd, vd))
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    s = gdn.gdn_slab()
    assert L.gdn_slab_init(C.byref(s), C.c_void_p(buf.data_ptr()), nb, N, vh, kh, kd, vd, 0) == 0
    S = torch.zeros((N, vh, kd, vd), device="cuda")
    assert L.gdn_mark(C.byref(s), C.c_void_p(S.data_ptr()), None, None) == 0
    acc = np.zeros(N, np.int32)
    rc = L.gdn_rollback_static(C.byref(s), C.c_void_p(S.data_ptr()), None, None, None, None,
                               None, None, None, 0, 4, 1, acc.ctypes.data_as(C.c_void_p), None)
    assert rc == gdn.GDN_EUNSUPPORTED
    assert s.armed == 1                          # refused: nothing changed
    torch.cuda.synchronize()
