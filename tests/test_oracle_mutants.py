"""Planted mistakes in a copy of the oracle (CPU only) must each fail a pin.

Each C mutant is the oracle's C source with one plausible slip (a wrong
rounding tie, a leaked future row, a flipped tie-break, an off-by-one window, a
dropped scale, a wrong sign ...).  The copy is compiled to a temporary library
and the pin suite is run against it; at least one pin must fail.  Each Python
mutant is a copy of the oracle package's layer-mode rules (``run_layers``) with
one slip (a Reindex layer that keeps the earlier indices, a window-only layer
that also attends to the main set, every layer on the first cache ...), loaded
as a module in place of the oracle for the pin suite.  This shows the pins are
strong enough to notice such a slip in the real oracle.
"""
import inspect
import os
import subprocess
import types

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "csa2_oracle.c")
PY_SRC = oracle.__file__

MUTANTS = {
    "rounding ties away from zero": ("return (q % 2 == 0) ? q : q + 1;", "return q + 1;"),
    "rounding truncates": ("if (2 * r > n) return q + 1;", "if (2 * r > 2 * n) return q + 1;"),
    "partial block reads future rows": ("if (last > t) last = t;", ""),
    "tie goes to the higher id": ("return (a->id < b->id) ? -1 : (a->id > b->id);",
                                  "return (a->id > b->id) ? -1 : (a->id < b->id);"),
    "own block not eligible": ("? (t + 1) / B : t / B + 1;", "? (t + 1) / B : (t + 1) / B;"),
    "excluded tail block kept": ("? (t + 1) / B : t / B + 1;", "? t / B + 1 : t / B + 1;"),
    "whole-block tail reads visible rows only": ("int key_limit = (tail == ORC_TAIL_WHOLE) ? T - 1 : t;",
                                                 "int key_limit = t;"),
    "query's own position excluded": ("if (p > t) break;", "if (p >= t) break;"),
    "score sign flipped": ("s += (int64_t)a[c] * (int64_t)b[c];", "s -= (int64_t)a[c] * (int64_t)b[c];"),
    "pool one short": ("n_pool = P;", "n_pool = P - 1;"),
    "window one short": ("int nw = (W > 0) ? t - w0 + 1 : 0;", "int nw = (W > 0) ? t - w0 : 0;"),
    "scale dropped on main logits": ("logit[i] = scale * acc;", "logit[i] = acc;"),
    "window logits use main keys": ("load_elem(k_swa, elem, (size_t)r * D + c);",
                                    "load_elem(k_main, elem, (size_t)(r + swa_first) * D + c);"),
    "value index transposed": ("load_elem(v_main, elem, (size_t)topk[i] * D + c);",
                               "load_elem(v_main, elem, (size_t)c * D + topk[i] % D);"),
    "normaliser ignores the window": ("for (int i = 0; i < cnt + nw; i++) {\n            logit[i] = exp(logit[i] - m);    /* now the unnormalised weight */\n            z += logit[i];",
                                      "for (int i = 0; i < cnt + nw; i++) {\n            logit[i] = exp(logit[i] - m);    /* now the unnormalised weight */\n            if (i < cnt) z += logit[i];"),
    "lse drops the max": ("lse[h] = m + log(z);", "lse[h] = log(z);"),
    "compressed entry visible before it completes": ("return (int)(((int64_t)t + 1) / r);",
                                                     "return (int)((int64_t)t / r + 1);"),
    "compressed entries one late": ("return (int)(((int64_t)t + 1) / r);", "return (int)((int64_t)t / r);"),
}


def _pin_calls():
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argnames, values = params[0].args
            argnames = [a.strip() for a in argnames.split(",")]
            for v in values:
                v = v if len(argnames) > 1 else (v,)
                yield name, (lambda fn=fn, v=v, a=argnames: fn(**dict(zip(a, v))))
        else:
            yield name, fn


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, tmp_path):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique/found: {old!r}"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-shared", "-fPIC", "-o", str(so), str(path), "-lm"])
    caught = []
    with oracle.using(str(so)):
        for name, call in _pin_calls():
            try:
                call()
            except (AssertionError, ValueError):   # a failed check or a rejected input: the pin noticed
                caught.append(name)
                break
    assert caught, f"no pin noticed the planted mistake: {mutant}"


# Slips in the layer-mode rules of oracle/__init__.py (run_layers).
PY_MUTANTS = {
    "a Reindex layer keeps the earlier indices": (
        "            current = sel\n        elif mode == \"reindex_tokens\":",
        "            current = sel if mode == \"full\" else current\n        elif mode == \"reindex_tokens\":"),
    "window-only layers after a Full layer attend to the main set too": (
        'if mode == "swa":', 'if mode == "swa" and current is None:'),
    "every layer reads the first cache": (
        "k_idx, k_main, v_main = wl.cache(max(n_full - 1, 0))", "k_idx, k_main, v_main = wl.cache(0)"),
    "a Full layer after the first reads the previous cache": (
        "k_idx, k_main, v_main = wl.cache(max(n_full - 1, 0))", "k_idx, k_main, v_main = wl.cache(max(n_full - 2, 0))"),
    "Reuse layers attend to the window alone": (
        "            topk, cnt = current[2], current[3]", "            topk, cnt = None, None"),
    "a token-only Reindex layer does not pass its selection on": (
        "            sel = (current[0], current[1], topk, cnt)\n            res[\"index\"][layer] = dict(zip((\"blk_ids\", \"blk_cnt\", \"topk\", \"topk_cnt\"), sel))\n            current = sel",
        "            sel = (current[0], current[1], topk, cnt)\n            res[\"index\"][layer] = dict(zip((\"blk_ids\", \"blk_cnt\", \"topk\", \"topk_cnt\"), sel))"),
}


@pytest.mark.parametrize("mutant", sorted(PY_MUTANTS))
def test_pins_catch_planted_mode_rule_mistake(mutant, monkeypatch):
    old, new = PY_MUTANTS[mutant]
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation site not unique/found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = PY_SRC          # the mutant loads the same compiled C oracle
    exec(compile(src.replace(old, new), PY_SRC, "exec"), mod.__dict__)
    monkeypatch.setattr(pins, "oracle", mod)
    caught = []
    for name, call in _pin_calls():
        try:
            call()
        except (AssertionError, ValueError):   # a failed check or a rejected input: the pin noticed
            caught.append(name)
            break
    assert caught, f"no pin noticed the planted mistake: {mutant}"
