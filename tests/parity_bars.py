"""Parity bars shared by the GPU tests.

Attention outputs O are convex combinations of V rows, so their bar is
absolute: max-abs 2e-2 and mean-abs 2e-3 for bf16 inputs, 1e-4 for fp32.
Gradients are unbounded and stored in the input dtype; their bar is the same
absolute one plus the storage rounding of each element, element by element.
"""
import numpy as np
import torch

TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}
# Relative storage rounding of a stored gradient element: half an ulp of a
# bf16 value x is at most 2^-8 |x| (7 stored mantissa bits), of an fp32 value
# at most 2^-24 |x|; fp32 takes one ulp (2^-23) to leave room for the order
# of its float32 sums.
REL = {"bf16": 2.0 ** -8, "f32": 2.0 ** -23}


# Unit roundoff of the format in which the MFMA kernels take P and dS as
# operands: a product's factor rounded to bf16 moves the product by at most
# 2^-8 of itself (8 significant bits).
OPERAND_U = {"bf16": 2.0 ** -8, "f32": 2.0 ** -24}


def grad_bar(want, dtype, terms=None):
    """Per-element bar of a gradient: the absolute bar of O plus the storage
    rounding of the element (gradients are unbounded and stored in the input
    dtype, so an element of magnitude m carries up to REL * m of rounding on its
    own, beyond the arithmetic error that the absolute part covers).

    terms (optional): for each element, the sum of the squares of the products
    it sums (the oracle's with_terms).  The MFMA kernels round one factor of
    every product (dS for dQ and dK, P for dV) to bf16, which moves product t
    by at most u |t| (u = 2^-8), to nearest, so with a sign that varies from
    product to product; taken as independent and uniform, the sum moves by a
    standard deviation of at most u sqrt(sum t^2 / 3).  The bar adds six of
    them.  Without terms the bar is the strict one (paths whose arithmetic is
    fp32 throughout)."""
    bar = TOL[dtype][0] + REL[dtype] * np.abs(want)
    if terms is not None:
        bar = bar + 6.0 * OPERAND_U[dtype] * np.sqrt(np.asarray(terms, dtype=np.float64) / 3.0)
    return bar


def assert_close(got, want, dtype, what, grad=False, terms=None, log=print):
    """O is a convex combination of V rows, so its bar is absolute.  Gradients
    take grad_bar() element by element, and a mean-abs bar scaled by
    max(1, mean |reference|), plus (with terms) twice the mean standard
    deviation of the operand rounding.  Prints the worst error-to-bar ratio, where it
    falls, how many elements exceed the literal absolute bar, and (with terms)
    the worst ratio under the strict bar as well."""
    mx, mean = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bar = grad_bar(want, dtype, terms) if grad else np.full_like(want, mx)
    mean_bar = mean * max(1.0, float(np.abs(want).mean())) if grad else mean
    if grad and terms is not None:
        # the mean |error| of a zero-mean sum of roundings with standard
        # deviation s is about 0.8 s; the bar adds two of the mean s
        mean_bar += 2.0 * float(np.mean(OPERAND_U[dtype] * np.sqrt(np.asarray(terms, dtype=np.float64) / 3.0)))
    ratio = err / bar
    w = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    strict = ""
    if grad and terms is not None:
        strict = f" strict-bar worst {float((err / grad_bar(want, dtype)).max()):.3f}"
    log(f"{what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e} (bar {mean_bar:.2e}) "
          f"worst err/bar {ratio[w]:.3f} (err {err[w]:.3e}, |ref| {abs(want[w]):.3e}, bar {bar[w]:.3e}){strict} "
          f"max|ref| {np.abs(want).max():.3e} over-{mx:g} {int((err > mx).sum())} of {err.size}")
    assert ratio[w] <= 1.0, f"{what}: error {err[w]} > bar {bar[w]} at {w} (ref {want[w]})"
    assert err.mean() <= mean_bar, f"{what}: mean-abs {err.mean()} > {mean_bar}"


def check_gradient_sums(dk, dv, do, dtype, what, log=None):
    """Whole-tensor identities of the masked-softmax gradient, one head at a
    time: every row of dS sums to zero, so the sum of dK over all keys is 0
    for each channel; every row of P sums to one, so the sum of dV over all
    keys equals the sum of dO over all query rows.  Sums in float64 of the
    stored outputs.  Bar: the per-element gradient bar b_t of each summed
    element (grad_bar at the element's own magnitude), with the element errors
    taken as independent and at most b_t (variance at most b_t^2 / 3 each), at
    six standard deviations: 6 sqrt(sum_t b_t^2 / 3) per channel.  log, if
    given, receives one line with the worst ratio over all heads."""
    worst = {}
    for h in range(dk.shape[1]):
        k = dk[:, h, :].double()
        v = dv[:, h, :].double()
        o = do[:, h, :].double()
        sums = {"sum dK": k.sum(0), "sum dV - sum dO": v.sum(0) - o.sum(0)}
        for name, x, t in (("sum dK", sums["sum dK"], k), ("sum dV - sum dO", sums["sum dV - sum dO"], v)):
            b = TOL[dtype][0] + REL[dtype] * t.abs()
            bar = 6.0 * torch.sqrt((b * b).sum(0) / 3.0)
            ratio = float((x.abs() / bar).max())
            print(f"{what} head {h} {name}: max |sum| {float(x.abs().max()):.3e}, worst sum/bar {ratio:.3f}",
                  flush=True)
            assert ratio <= 1.0, f"{what} head {h}: {name} {float(x.abs().max())} exceeds its bar"
            worst[name] = max(worst.get(name, 0.0), ratio)
    if log is not None:
        log(f"{what}: gradient sums over {dk.shape[1]} heads, worst sum/bar " +
            ", ".join(f"{n} {r:.3f}" for n, r in worst.items()))
