"""Planted mistakes for the oracle's self-test.

Each entry rewrites a few lines of a copy of ``oracle/parallax_oracle.c``
(never the file itself) to plant one plausible mistake: a dropped term, a
wrong sign or index, a transposed operand.  ``test_oracle.py`` builds every
such copy and requires it to fail at least one pin, which shows the pins
would catch that mistake in the oracle.  Every ``old`` text occurs exactly
once in the oracle source.
"""
from __future__ import annotations

import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SOURCE = os.path.join(ROOT, "oracle", "parallax_oracle.c")

# number: (what the mistake is, [(old text, new text), ...])
MUTANTS = {
    1: ('correction with the wrong sign', [
        ((
            "            continue;\n"
            "        double w = z[j] * (1.0 + c[j]);\n"
            "        const double *vj = v + j * (long)d;"),
         (
            "            continue;\n"
            "        /* planted mistake: correction with the wrong sign */\n"
            "        double w = z[j] * (1.0 - c[j]);\n"
            "        const double *vj = v + j * (long)d;")),
    ]),
    2: ('correction not centred on kbar', [
        ((
            "        for (int t = 0; t < d; ++t) {\n"
            "            s += r_i[t] * (kj[t] - kbar[t]);\n"
            "        }"),
         (
            "        for (int t = 0; t < d; ++t) {\n"
            "            /* planted mistake: correction not centred on kbar */\n"
            "            s += r_i[t] * kj[t];\n"
            "        }")),
    ]),
    3: ('softmax scale also applied to the correction', [
        ((
            "        }\n"
            "        c[j] = s;"),
         (
            "        }\n"
            "        /* planted mistake: softmax scale also applied to the correction */\n"
            "        s *= scale;\n"
            "        c[j] = s;")),
    ]),
    4: ('sink keys visible ahead of the query', [
        ((
            "{\n"
            "    if (j < 0 || j > i)"),
         (
            "{\n"
            "    /* planted mistake: sink keys visible even ahead of the query */\n"
            "    if (j >= 0 && j < n_sink)\n"
            "        return 1;\n"
            "    if (j < 0 || j > i)")),
    ]),
    5: ('window boundary off by one (W + 1 keys)', [
        ((
            "        return 0;\n"
            "    if (window <= 0 || i - j < window || j < n_sink)\n"
            "        return 1;"),
         (
            "        return 0;\n"
            "    /* planted mistake: window boundary off by one (W+1 keys) */\n"
            "    if (window <= 0 || i - j <= window || j < n_sink)\n"
            "        return 1;")),
    ]),
    6: ('log-sum-exp without the max', [
        ((
            "    }\n"
            "    *lse_i = m + log(ell);\n"
            "    for (long j = 0; j <= last; ++j)"),
         (
            "    }\n"
            "    /* planted mistake: log-sum-exp without the max */\n"
            "    *lse_i = log(ell);\n"
            "    for (long j = 0; j <= last; ++j)")),
    ]),
    7: ('key mean with unnormalised weights', [
        ((
            "            continue;\n"
            "        double w = z[j];\n"
            "        for (int t = 0; t < d; ++t)"),
         (
            "            continue;\n"
            "        /* planted mistake: key mean with unnormalised weights */\n"
            "        double w = z[j] * ell;\n"
            "        for (int t = 0; t < d; ++t)")),
    ]),
    8: ('probe read against the values, not the keys', [
        ((
            "        for (int t = 0; t < d; ++t) {\n"
            "            s += r_i[t] * (kj[t] - kbar[t]);\n"
            "        }"),
         (
            "        for (int t = 0; t < d; ++t) {\n"
            "            /* planted mistake: probe read against the values, not the keys */\n"
            "            s += r_i[t] * (v[j * (long)d + t] - kbar[t]);\n"
            "        }")),
    ]),
    9: ('plain softmax term dropped', [
        ((
            "            continue;\n"
            "        double w = z[j] * (1.0 + c[j]);\n"
            "        const double *vj = v + j * (long)d;"),
         (
            "            continue;\n"
            "        /* planted mistake: plain softmax term dropped */\n"
            "        double w = z[j] * c[j];\n"
            "        const double *vj = v + j * (long)d;")),
    ]),
    10: ('weights taken from the previous key', [
        ((
            "            continue;\n"
            "        double w = z[j] * (1.0 + c[j]);\n"
            "        const double *vj = v + j * (long)d;"),
         (
            "            continue;\n"
            "        /* planted mistake: weights taken from the previous key */\n"
            "        double w = (j > 0 ? z[j - 1] : z[j]) * (1.0 + c[j]);\n"
            "        const double *vj = v + j * (long)d;")),
    ]),
    11: ('backward: softmax adjoint without its mean term', [
        ((
            "            mean_dp += p[j] * dp[j];\n"
            ""),
         (
            "            mean_dp += p[j] * dp[j];\n"
            "    /* planted mistake: softmax adjoint without its mean term */\n"
            "    mean_dp = 0.0;\n"
            "")),
    ]),
    12: ('backward: adjoint of the key mean with the wrong sign', [
        ((
            "    for (int t = 0; t < d; ++t)\n"
            "        dkbar[t] = -sum_dc * r_i[t];\n"
            ""),
         (
            "    for (int t = 0; t < d; ++t)\n"
            "        /* planted mistake: adjoint of the key mean with the wrong sign */\n"
            "        dkbar[t] = sum_dc * r_i[t];\n"
            "")),
    ]),
    13: ('backward: query gradient without the softmax scale', [
        ((
            "        for (int t = 0; t < d; ++t) {\n"
            "            dq_i[t] += scale * dz * kj[t];\n"
            "            dk[j * (long)d + t] += scale * dz * q_i[t];"),
         (
            "        for (int t = 0; t < d; ++t) {\n"
            "            /* planted mistake: query gradient without the softmax scale */\n"
            "            dq_i[t] += dz * kj[t];\n"
            "            dk[j * (long)d + t] += scale * dz * q_i[t];")),
    ]),
    14: ('backward: value gradient without the probe correction', [
        ((
            "            continue;\n"
            "        double u = p[j] * (1.0 + c[j]);\n"
            "        for (int t = 0; t < d; ++t)"),
         (
            "            continue;\n"
            "        /* planted mistake: value gradient without the probe correction */\n"
            "        double u = p[j];\n"
            "        for (int t = 0; t < d; ++t)")),
    ]),
    15: ('backward: probe gradient not centred on kbar', [
        ((
            "        for (int t = 0; t < d; ++t) {\n"
            "            dr_i[t] += dc[j] * (kj[t] - kbar[t]);\n"
            "            dk[j * (long)d + t] += dc[j] * r_i[t];"),
         (
            "        for (int t = 0; t < d; ++t) {\n"
            "            /* planted mistake: probe gradient not centred on kbar */\n"
            "            dr_i[t] += dc[j] * kj[t];\n"
            "            dk[j * (long)d + t] += dc[j] * r_i[t];")),
    ]),
    16: ('backward: key gradient missing its p * dkbar term', [
        ((
            "        dp[j] += dot(dkbar, k + j * (long)d, d);\n"
            "        for (int t = 0; t < d; ++t)\n"
            "            dk[j * (long)d + t] += p[j] * dkbar[t];\n"
            "    }"),
         (
            "        dp[j] += dot(dkbar, k + j * (long)d, d);\n"
            "    }")),
    ]),
    17: ('general decode: query heads mapped to kv heads round-robin', [
        ((
            "        for (long h = 0; h < Hq && rc == 0; ++h) {\n"
            "            long hk = h / g;\n"
            "            long bh = b * Hq + h;"),
         (
            "        for (long h = 0; h < Hq && rc == 0; ++h) {\n"
            "            /* planted mistake: query heads mapped to kv heads round-robin */\n"
            "            long hk = h % Hkv;\n"
            "            long bh = b * Hq + h;")),
    ]),
    18: ('exact LLA: covariance product not centred on kbar', [
        ((
            "            double c = 0.0;\n"
            "            for (int t = 0; t < d; ++t)"),
         (
            "            double c = 0.0;\n"
            "            /* planted mistake: covariance product not centred on kbar */\n"
            "            for (int t = 0; t < d; ++t)")),
        ((
            "            for (int t = 0; t < d; ++t)\n"
            "                c += (kj[t] - kbar[t]) * dir[t];\n"
            "            c *= p[j];"),
         (
            "            for (int t = 0; t < d; ++t)\n"
            "                c += kj[t] * dir[t];\n"
            "            c *= p[j];")),
        ((
            "            for (int t = 0; t < d; ++t)\n"
            "                Ad[t] += c * (kj[t] - kbar[t]);\n"
            "        }"),
         (
            "            for (int t = 0; t < d; ++t)\n"
            "                Ad[t] += c * kj[t];\n"
            "        }")),
    ]),
    19: ('projection: the weight read transposed', [
        ((
            "            for (long t = 0; t < K; ++t)\n"
            "                s += x[i * K + t] * w[n * K + t];\n"
            "            y[i * N + n] = s;"),
         (
            "            for (long t = 0; t < K; ++t)\n"
            "                /* planted mistake: the weight read transposed */\n"
            "                s += x[i * K + t] * w[(t % N) * K + (n % K)];\n"
            "            y[i * N + n] = s;")),
    ]),
    20: ('Hadamard: normalisation dropped', [
        ((
            "            }\n"
            "    const double norm = 1.0 / sqrt((double)n);\n"
            "#pragma omp parallel for num_threads(nthreads) schedule(static)"),
         (
            "            }\n"
            "    /* planted mistake: the normalisation dropped */\n"
            "    const double norm = 1.0;\n"
            "#pragma omp parallel for num_threads(nthreads) schedule(static)")),
    ]),
    21: ('Hadamard: lower-left block sign flipped', [
        ((
            "                h[i * n + j + m] = e;\n"
            "                h[(i + m) * n + j] = e;\n"
            "                h[(i + m) * n + j + m] = -e;\n"
            "            }"),
         (
            "                h[i * n + j + m] = e;\n"
            "                /* planted mistake: the sign of the lower-left block flipped */\n"
            "                h[(i + m) * n + j] = -e;\n"
            "                h[(i + m) * n + j + m] = e;\n"
            "            }")),
    ]),
    22: ('Hadamard: alpha applied to the input features', [
        ((
            "            for (long t = 0; t < n; ++t)\n"
            "                s += y[i * n + t] * h[t * n + c];\n"
            "            s *= norm;"),
         (
            "            for (long t = 0; t < n; ++t)\n"
            "                /* planted mistake: alpha applied to the input features */\n"
            "                s += y[i * n + t] * (alpha ? alpha[t] : 1.0) * h[t * n + c];\n"
            "            s *= norm;")),
        ((
            "            s *= norm;\n"
            "            if (alpha)\n"
            "                s *= alpha[c];\n"
            "            if (beta)"),
         (
            "            s *= norm;\n"
            "            if (beta)")),
    ]),
    23: ('Hadamard: beta added before alpha', [
        ((
            "            s *= norm;\n"
            "            if (alpha)"),
         (
            "            s *= norm;\n"
            "            /* planted mistake: beta added before the scaling by alpha */\n"
            "            if (beta)\n"
            "                s += beta[c];\n"
            "            if (alpha)")),
        ((
            "                s *= alpha[c];\n"
            "            if (beta)\n"
            "                s += beta[c];\n"
            "            out[i * n + c] = s;"),
         (
            "                s *= alpha[c];\n"
            "            out[i * n + c] = s;")),
    ]),
    24: ('Based: square term dropped', [
        ((
            "            const double x = scale * dot;\n"
            "            const double w = 1.0 + x + 0.5 * x * x;\n"
            "            den += w;"),
         (
            "            const double x = scale * dot;\n"
            "            /* planted mistake: the second-order term dropped */\n"
            "            const double w = 1.0 + x;\n"
            "            den += w;")),
    ]),
    25: ("Based: the query's own key left out", [
        ((
            "        double den = 0.0;\n"
            "        for (long j = 0; j <= i; ++j) {\n"
            "            double dot = 0.0;"),
         (
            "        double den = 0.0;\n"
            "        /* planted mistake: the query's own key left out */\n"
            "        for (long j = 0; j < i; ++j) {\n"
            "            double dot = 0.0;")),
    ]),
    26: ('Based: normalised by the key count', [
        ((
            "            const double w = 1.0 + x + 0.5 * x * x;\n"
            "            den += w;\n"
            "            for (long e = 0; e < dv; ++e)"),
         (
            "            const double w = 1.0 + x + 0.5 * x * x;\n"
            "            /* planted mistake: normalised by the number of keys */\n"
            "            den += 1.0;\n"
            "            for (long e = 0; e < dv; ++e)")),
    ]),
    27: ('Based: square of the unscaled product', [
        ((
            "            const double x = scale * dot;\n"
            "            const double w = 1.0 + x + 0.5 * x * x;\n"
            "            den += w;"),
         (
            "            const double x = scale * dot;\n"
            "            /* planted mistake: the square taken of the unscaled product */\n"
            "            const double w = 1.0 + x + 0.5 * dot * dot;\n"
            "            den += w;")),
    ]),
}

def mutant_source(n: int, source: str = ORACLE_SOURCE) -> str:
    """The oracle source with planted mistake ``n`` applied."""
    with open(source) as f:
        text = f.read()
    for old, new in MUTANTS[n][1]:
        if text.count(old) != 1:
            raise ValueError("mutant %d: its target text is not unique in the oracle" % n)
        text = text.replace(old, new)
    return text
