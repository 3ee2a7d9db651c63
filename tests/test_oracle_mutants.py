"""Plant a plausible mistake in a copy of the oracle's C source (on the CPU), build it, and check
that the pin suite catches it. The real oracle source is never modified."""
import inspect

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

# (name, text in oracle.c, replacement): each is a mistake a careful reader could make.
MUTANTS = [
    ("decay sign flipped", "exp(dt * a_row[n])", "exp(-dt * a_row[n])"),
    ("skip term dropped", "if (j->D) y += skip * x;", ""),
    ("gate uses sigmoid, not SiLU", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    ("B read as [nb, N, L]", "b_tok[n], j->zoh_flag", "j->B[(b * N + n) * L + t], j->zoh_flag"),
    ("C read with B's pointer", "const double *c_tok = j->C +", "const double *c_tok = j->B +"),
    ("A indexed by batch", "const double *a_row = j->A + d * N;", "const double *a_row = j->A + b * N;"),
    ("bias added after softplus", "const double dt = j->softplus_flag ? oracle_softplus(r) : r;",
     "const double dt = j->softplus_flag ? oracle_softplus(dr_row[t]) + bias : r;"),
    ("softplus loses small-value accuracy", "return pos + log1p(exp(-fabs(r)));",
     "return pos + log(1.0 + exp(-fabs(r)));"),
    ("Euler gain without the step", "if (!zoh || a == 0.0) return dt * b;", "if (!zoh || a == 0.0) return b;"),
    ("ZOH gain without 1/a", "return expm1(dt * a) / a * b;", "return expm1(dt * a) * b;"),
    ("input enters squared", "h[n] = abar * h[n] + bbar * x;", "h[n] = abar * h[n] + bbar * x * x;"),
    ("gate read one token late", "y *= oracle_silu(z_row[t]);", "y *= oracle_silu(z_row[t > 0 ? t - 1 : 0]);"),
    ("readout skips the last state", "for (int64_t n = 0; n < N; ++n) y += c_tok[n] * h[n];",
     "for (int64_t n = 0; n + 1 < N; ++n) y += c_tok[n] * h[n];"),
    ("decode step without softplus", "const double dt = oracle_softplus(delta[row]);", "const double dt = delta[row];"),
    ("decode reads B by channel", "input_gain(dt, a, B[b * N + n], zoh_flag)", "input_gain(dt, a, B[(d % nb) * N + n], zoh_flag)"),
    ("state not zeroed per row", "for (int64_t n = 0; n < N; ++n) h[n] = 0.0;",
     "if (row == j->row_begin) for (int64_t n = 0; n < N; ++n) h[n] = 0.0;"),
    ("conv taps paired in reverse", "const int64_t s = t - (K - 1) + k;", "const int64_t s = t - k;"),
    ("conv window one token late", "                    const int64_t s = t - (K - 1) + k;\n", "                    const int64_t s = t - K + k;\n"),
    ("conv taps shared by all channels", "if (s >= 0) pre += w[d * K + k] * xr[s];", "if (s >= 0) pre += w[k] * xr[s];"),
    ("conv bias dropped", "                double pre = bias ? bias[d] : 0.0;\n                for (int64_t k = 0; k < K; ++k) {",
     "                double pre = 0.0;\n                for (int64_t k = 0; k < K; ++k) {"),
    ("conv window shifts the wrong way",
     "for (int64_t k = 0; k + 1 < K; ++k) win[k] = win[k + 1];\n            win[K - 1] = x[b * nd + d];",
     "for (int64_t k = K - 1; k > 0; --k) win[k] = win[k - 1];\n            win[0] = x[b * nd + d];"),
    ("bwd adjoint carried without the decay", "lam[n] = a * l;", "lam[n] = l;"),
    ("bwd dA without the step", "dA[d * N + n] += l * hp * a * dt;", "dA[d * N + n] += l * hp * a;"),
    ("bwd dC from the previous state", "dC[(b * L + t) * N + n] += dy * h[t * N + n];", "dC[(b * L + t) * N + n] += dy * hp;"),
    ("bwd softplus derivative dropped", "const double dr = softplus_flag ? ddt / (1.0 + exp(-r)) : ddt;", "const double dr = ddt;"),
    ("bwd gate derivative of the sigmoid alone", "dz[row + t] = dout[row + t] * y * sg * (1.0 + zt * (1.0 - sg));",
     "dz[row + t] = dout[row + t] * y * sg;"),
    ("bwd decay term dropped from dDelta", "ddt += l * (hp * a * a_row[n] + bt[n] * ut);", "ddt += l * bt[n] * ut;"),
    ("ssd decay sign flipped", "const double decay = exp(j->a[(b * L + t) * H + h]);",
     "const double decay = exp(-j->a[(b * L + t) * H + h]);"),
    ("ssd decay applied to the new write too", "st[p * N + n] = decay * st[p * N + n] + xt[p] * bt[n];",
     "st[p * N + n] = decay * (st[p * N + n] + xt[p] * bt[n]);"),
    ("ssd readout with b instead of c", "acc += st[p * N + n] * ct[n];", "acc += st[p * N + n] * bt[n];"),
    ("ssd heads mapped to groups cyclically", "g = h / (H / G);", "g = h % G;"),
    ("ssd state not reset per row", "memset(st, 0, (size_t)(P * N) * sizeof(double));",
     "if (row == j->row_begin) memset(st, 0, (size_t)(P * N) * sizeof(double));"),
    ("ssd stream read from the next head", "const double *xt = j->x + ((b * L + t) * H + h) * P;",
     "const double *xt = j->x + ((b * L + t) * H + (h + 1) % H) * P;"),
    ("ssd readout before the update",
     "st[p * N + n] = decay * st[p * N + n] + xt[p] * bt[n];\n                    acc += st[p * N + n] * ct[n];",
     "acc += st[p * N + n] * ct[n];\n                    st[p * N + n] = decay * st[p * N + n] + xt[p] * bt[n];"),
]


def _pin_calls():
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = list(inspect.signature(fn).parameters)
        if params == ["oracle_mod"]:
            calls.append((name, fn, ()))
        elif params == ["oracle_mod", "field"]:
            for f in ("u", "delta", "z", "B", "C"):
                calls.append(("%s[%s]" % (name, f), fn, (f,)))
        elif params == ["oracle_mod", "softplus"]:
            for sp in (True, False):
                calls.append(("%s[%s]" % (name, sp), fn, (sp,)))
    return calls


def _failing_pins(mod):
    failed = []
    for name, fn, extra in _pin_calls():
        try:
            with np.errstate(all="ignore"):
                fn(mod, *extra)
        except Exception:  # an assertion, or a mutant that misbehaves outright
            failed.append(name)
    return failed


def test_mutant_table_applies_to_current_source():
    src = oracle.source_text()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, "mutation %r no longer matches oracle.c" % name


def test_unmodified_copy_passes_every_pin(tmp_path):
    so = oracle.build_variant(oracle.source_text(), str(tmp_path), "oracle_copy")
    assert _failing_pins(oracle.Variant(so)) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = oracle.source_text()
    assert src.count(old) == 1
    so = oracle.build_variant(src.replace(old, new), str(tmp_path), "oracle_mutant")
    failed = _failing_pins(oracle.Variant(so))
    assert failed, "no pin caught the planted mistake %r" % name
