"""swe_step_noalloc, the entry point that allocates nothing, against swe_step.

Both calls run the same kernels; the no-allocation call keeps the batch's
bookkeeping in a static device array that every call on the GPU shares.  Its
results must equal swe_step's bit for bit (states, dt history, elapsed time),
on two calls in a row where the second runs a smaller input (whatever the
first left in the shared array must not leak into it), on consecutive calls
of one context, alternating contexts, every kernel path, and at the step
limit.
"""
import numpy as np
import pytest

import inputs
from helpers import say

pytestmark = pytest.mark.gpu


def _ctx(w, path=0, precision=None):
    import finite_volume_shallow_amd as swe
    desc, keep = swe.desc_from_workload(w, path=path, precision=precision)
    ctx = swe.swe_create_mesh(desc)
    del keep
    swe.swe_set_state(ctx, w.z, w.state)
    return ctx


def _step(ctx, n, cfl, noalloc):
    import finite_volume_shallow_amd as swe
    t, last = (swe.swe_step_noalloc if noalloc else swe.swe_step)(ctx, n, cfl)
    return t, last, swe.swe_get_dt_history(ctx), swe.swe_get_state(ctx)


def _same(a, b, what):
    ta, la, ha, sa = a
    tb, lb, hb, sb = b
    assert ta == tb and la == lb, (what, ta, tb, la, lb)
    assert np.array_equal(ha, hb), what
    for x, y in zip(sa, sb):
        assert np.array_equal(x, y), what


# name: (workload factory, precision, path, steps of the two calls)
PAIRS = {
    "grid-64x64-then-24x16": ((lambda: inputs.dam_break(), lambda: inputs.dam_break(nx=24, ny=16)), "f64", 0, (30, 12)),
    "flow-f32-160x96-then-40x24": ((lambda: inputs.smooth_flow(nx=160, ny=96), lambda: inputs.smooth_flow(nx=40, ny=24)),
                                   "f32", 0, (40, 20)),
    "tri-36-then-12": ((lambda: inputs.circular_dam_break(nq=36), lambda: inputs.circular_dam_break(nq=12)), "f64", 0,
                       (25, 10)),
    "two-layer-20-then-8": ((lambda: inputs.two_layer_dam_break(nq=20), lambda: inputs.two_layer_dam_break(nq=8)),
                            "f64", 0, (20, 8)),
    "edge-grid-48x32-then-16x8": ((lambda: inputs.dam_break(nx=48, ny=32), lambda: inputs.dam_break(nx=16, ny=8)),
                                  "f64", 1, (15, 6)),
    "recompute-tri-30-then-10": ((lambda: inputs.circular_dam_break(nq=30), lambda: inputs.circular_dam_break(nq=10)),
                                 "f64", 3, (12, 5)),
}


@pytest.mark.parametrize("name", list(PAIRS))
def test_noalloc_matches_step_on_two_calls(name):
    import finite_volume_shallow_amd as swe
    (big, small), prec, path, (n1, n2) = PAIRS[name]
    for make, n in ((big, n1), (small, n2)):
        w = make()
        say(f"[noalloc] {name} cells={w.ncells} steps={n} path={path} prec={prec}")
        ref_ctx, na_ctx = _ctx(w, path, prec), _ctx(w, path, prec)
        try:
            _same(_step(ref_ctx, n, w.cfl, False), _step(na_ctx, n, w.cfl, True), f"{name} first call")
            # the context continues: a second batch of each kind
            _same(_step(ref_ctx, n // 2 + 1, w.cfl, False), _step(na_ctx, n // 2 + 1, w.cfl, True),
                  f"{name} continued")
        finally:
            swe.swe_destroy(ref_ctx)
            swe.swe_destroy(na_ctx)


def test_noalloc_alternating_contexts_and_mixed_calls():
    """Two contexts take turns on the shared array; a context mixes both
    calls.  Each must give what swe_step alone gives."""
    import finite_volume_shallow_amd as swe
    wa, wb = inputs.circular_dam_break(nq=24), inputs.dam_break(nx=40, ny=24)
    ra, rb, na, nb = _ctx(wa), _ctx(wb), _ctx(wa), _ctx(wb)
    try:
        for k, (n, mixed) in enumerate(((7, False), (5, True), (9, False))):
            ref_a, ref_b = _step(ra, n, wa.cfl, False), _step(rb, n, wb.cfl, False)
            got_a = _step(na, n, wa.cfl, not mixed)
            got_b = _step(nb, n, wb.cfl, True)
            _same(ref_a, got_a, f"context a, batch {k}")
            _same(ref_b, got_b, f"context b, batch {k}")
    finally:
        for c in (ra, rb, na, nb):
            swe.swe_destroy(c)


def test_noalloc_step_limit():
    import finite_volume_shallow_amd as swe
    w = inputs.dam_break(nx=16, ny=8)
    ref, na = _ctx(w), _ctx(w)
    try:
        with pytest.raises(swe.SweError) as e:
            swe.swe_step_noalloc(na, swe.SWE_NOALLOC_MAX_STEPS + 1, w.cfl)
        assert e.value.status == swe.SWE_E_INVAL
        _same(_step(ref, swe.SWE_NOALLOC_MAX_STEPS, w.cfl, False),
              _step(na, swe.SWE_NOALLOC_MAX_STEPS, w.cfl, True), "at the limit")
    finally:
        swe.swe_destroy(ref)
        swe.swe_destroy(na)
