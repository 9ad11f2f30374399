"""Cost and accuracy of exact Local Linear Attention against Parallax (CPU).

LLA gets each row's probe from a linear solve; done by conjugate gradients,
every iteration reads all of the row's visible keys again, on top of the
three passes both estimators share in this form (scores, key mean, weighted
values).  Parallax reads the probe as an input, so it keeps one pass over
the keys per row (the fused kernel's) however the probe was made (review
page "Parallax: Parameterized Local Linear Attention for Language Modeling",
sec. 1-2: LLA's per-token solve is what makes it I/O-heavy).  This test
records, for a fixed budget of CG iterations, how far the LLA output still
is from the converged solve, and how many key passes that budget costs."""
import time

import numpy as np

from bruteforce import visible_mask


def test_lla_cg_budget_accuracy_and_passes(orc):
    L, d = 256, 32
    rng = np.random.default_rng(11)
    q, k, v = (0.3 * rng.standard_normal((L, d)) for _ in range(3))
    scale = d ** -0.5
    rows = np.arange(2 * d, L)          # rows whose local covariance is well conditioned
    mask = visible_mask(L)
    assert mask[rows].sum(axis=1).min() >= 2 * d
    exact, _, it_exact = orc.lla_rows(q[rows], rows, k, v, scale, max_iters=8 * d, tol=0.0)
    print("\n[lla] budget | rel. error of the intercept | key passes per row (LLA / Parallax)")
    errs = []
    for budget in (0, 1, 2, 4, 8, 16, d, 2 * d):
        o, _, it = orc.lla_rows(q[rows], rows, k, v, scale, max_iters=budget, tol=0.0)
        err = float(np.linalg.norm(o - exact) / np.linalg.norm(exact))
        errs.append(err)
        print("[lla] %5d | %.3e | %d / 1" % (budget, err, int(it.max()) + 3))
        assert np.all(it <= budget)
    # no probe at all (budget 0) is plain softmax attention: far from LLA
    assert errs[0] > 1e-2
    # the error falls with the budget and the solve converges within 2d iterations
    assert errs[3] < errs[1] < errs[0]
    assert errs[-1] < 1e-9
    # timing of the two oracles on the same rows (fp64, one thread): LLA's solve
    # dominates its cost
    t0 = time.perf_counter()
    orc.lla_rows(q[rows], rows, k, v, scale, max_iters=2 * d, tol=0.0, nthreads=1)
    t_lla = time.perf_counter() - t0
    t0 = time.perf_counter()
    orc.rows(q[rows], np.zeros((len(rows), d)), rows, k, v, scale, nthreads=1)
    t_plx = time.perf_counter() - t0
    print("[lla] CPU time for %d rows: LLA (2d CG iterations) %.4f s, Parallax form %.4f s"
          % (len(rows), t_lla, t_plx))
    assert t_lla > t_plx
