"""Workspace handling on the GPU, through the C ABI.

* The per-stream workspace cache gives the same bits as a stream-ordered
  allocation per call, while the buffer grows and is reused at smaller sizes.
* Two streams working at once keep their own buffers: interleaved calls give
  the results each problem gives alone.
* A failing workspace allocation (forced from the host with
  KEOPS_OPT_FAIL_ALLOC) makes every entry point that needs workspace return
  KEOPS_ERR_ALLOC and leave its outputs untouched: nothing was enqueued.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from parity import check_sum, dev, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import geometric_map_reduce_amd as gm

OPTS = ("KEOPS_OPT_SPLIT_J", "KEOPS_OPT_ROWS", "KEOPS_OPT_WS_CACHE", "KEOPS_OPT_FAIL_ALLOC")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _options():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    for o in OPTS:
        gm.keops_set_option(getattr(gm, o), 0)
    yield
    for o in OPTS:
        gm.keops_set_option(getattr(gm, o), 0)


def _case(seed, M, N, D=3, E=1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = rng.standard_normal((N, D)).astype(np.float32)
    b = rng.standard_normal((N, E)).astype(np.float32)
    g = rng.standard_normal((M, E)).astype(np.float32)
    return x, y, b, g


def _all_ops(X, Y, B, G, sigma):
    """Every reduction that takes split-j workspace, as host arrays."""
    d, i = gm.keops_kmin(X, Y, 5)
    r = [gm.keops_gauss_sum(X, Y, B, sigma), gm.keops_gauss_lse(X, Y, B, sigma),
         gm.keops_gauss_grad_x(X, Y, B, G, sigma), d, i]
    torch.cuda.synchronize()
    return [host(t) for t in r]


def _bits(a):
    return a.view(np.int64) if a.dtype == np.int64 else a.view(np.int32)


def test_cache_equals_per_call_allocation():
    # growing, shrinking and growing again; four j-splits force the workspace
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, 4)
    for k, (M, N) in enumerate([(300, 2000), (2000, 5000), (100, 800), (5000, 9000)]):
        say(f"workspace cache vs per-call allocation: M={M} N={N}")
        x, y, b, g = _case(k, M, N)
        X, Y, B, G = dev(x), dev(y), dev(b), dev(g)
        gm.keops_set_option(gm.KEOPS_OPT_WS_CACHE, 0)
        cached = _all_ops(X, Y, B, G, 0.7)
        gm.keops_set_option(gm.KEOPS_OPT_WS_CACHE, 2)
        fresh = _all_ops(X, Y, B, G, 0.7)
        gm.keops_set_option(gm.KEOPS_OPT_WS_CACHE, 0)
        again = _all_ops(X, Y, B, G, 0.7)
        for c, f, a in zip(cached, fresh, again):
            assert np.array_equal(_bits(c), _bits(f)) and np.array_equal(_bits(c), _bits(a))
        if k == 0:
            a_ref, n_ref = oracle.gauss_sum(x, y, b, 0.7)
            check_sum(cached[0], a_ref, n_ref)


def test_two_streams_keep_their_own_buffers():
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, 3)
    probs = []
    for k, (M, N) in enumerate([(1500, 6000), (2500, 4000)]):
        x, y, b, _ = _case(10 + k, M, N)
        X, Y, B = dev(x), dev(y), dev(b)
        alone = gm.keops_gauss_sum(X, Y, B, 0.5)
        torch.cuda.synchronize()
        probs.append((X, Y, B, host(alone)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    outs = [[], []]
    for rep in range(6):
        for k in (0, 1):
            X, Y, B, _ = probs[k]
            with torch.cuda.stream(streams[k]):
                outs[k].append(gm.keops_gauss_sum(X, Y, B, 0.5, stream=streams[k]))
    torch.cuda.synchronize()
    for k in (0, 1):
        for o in outs[k]:
            assert np.array_equal(host(o).view(np.int32), probs[k][3].view(np.int32))


def _expect_alloc_failure(fn, outs):
    sentinel = 12345.0
    for o in outs:
        o.fill_(sentinel if o.dtype == torch.float32 else 777)
    torch.cuda.synchronize()
    with pytest.raises(gm.KeopsError) as ei:
        fn()
    assert ei.value.status == -3
    torch.cuda.synchronize()
    for o in outs:
        want = sentinel if o.dtype == torch.float32 else 777
        assert bool((o == want).all())


def test_alloc_failure_enqueues_nothing():
    x, y, b, g = _case(3, 700, 3000)
    X, Y, B, G = dev(x), dev(y), dev(b), dev(g)
    M, N = x.shape[0], y.shape[0]
    out = torch.empty((M, 1), device="cuda")
    outg = torch.empty((M, 3), device="cuda")
    outy = torch.empty((N, 3), device="cuda")
    idx = torch.empty((M, 1), device="cuda", dtype=torch.int64)
    kd = torch.empty((M, 4), device="cuda")
    ki = torch.empty((M, 4), device="cuda", dtype=torch.int64)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, 4)        # every dense call takes workspace
    gm.keops_set_option(gm.KEOPS_OPT_FAIL_ALLOC, 1)
    cases = [
        ("sum", lambda: gm.keops_gauss_sum(X, Y, B, 0.6, out=out), [out]),
        ("lse", lambda: gm.keops_gauss_lse(X, Y, B, 0.6, out=out), [out]),
        ("grad_x", lambda: gm.keops_gauss_grad_x(X, Y, B, G, 0.6, out=outg), [outg]),
        ("grad_y", lambda: gm.keops_gauss_grad_y(X, Y, B, G, 0.6, out=outy), [outy]),
        ("max", lambda: gm.keops_gauss_max(X, Y, B, 0.6, out=out, out_idx=idx), [out, idx]),
        ("laplace", lambda: gm.keops_laplace_sum(X, Y, B, 0.6, out=out), [out]),
        ("kmin", lambda: gm.keops_kmin(X, Y, 4, out_d=kd, out_idx=ki), [kd, ki]),
        ("few rows", lambda: gm.keops_gauss_sum(X[:16], Y, B, 0.6, out=out[:16]), [out]),
        ("ranges", lambda: gm.keops_gauss_sum_ranges(
            X, Y, B, 0.6, np.array([[0, M]], np.int64), np.array([1], np.int64), np.array([[0, N]], np.int64),
            out=out), [out]),
        ("cg", lambda: gm.keops_gauss_cg(Y, B, 0.6, 1.0, out=outy[:, :1].contiguous()), []),
    ]
    for name, fn, outs in cases:
        say(f"forced allocation failure: {name}")
        _expect_alloc_failure(fn, outs)
    # the switch off again: the same calls run
    gm.keops_set_option(gm.KEOPS_OPT_FAIL_ALLOC, 0)
    a = host(gm.keops_gauss_sum(X, Y, B, 0.6, out=out))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, 0.6)
    check_sum(a, a_ref, n_ref)
