"""Mutation check of the oracle's pins (test infrastructure, CPU only).

Each mutant plants one plausible mistake in a copy of the fp64 oracle -- a
dropped scale, an off-by-one visibility or window bound, a swapped gate, a
missing softmax-Jacobian term, a wrong tie order, a shifted decode output --
builds that copy and runs the oracle pins (tests/test_oracle_pins.py) against
it.  A mutant that leaves every pin passing is reported as SURVIVED: some
output of the oracle is then not pinned by anything but itself.

The repository's own oracle is never modified: everything happens in a
temporary directory holding copies of oracle/, the pin tests and their
fixtures.  Usage: python tests/oracle_mutants.py [substring ...]
(substrings select mutants by name).  Exit status 1 if any mutant survives.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C = "oracle/nsa_oracle.c"
PY = "oracle/__init__.py"

# (file, name, original text, mutated text); each original occurs exactly once
MUTANTS = [
    (C, "pool divisor", "= s / p->blk;", "= s / (p->blk - 1);"),
    (C, "pool token shift", "s += x[kidx(p, b, j * p->blk + i, g, d)];",
     "s += x[kidx(p, b, j * p->blk + (i + 1) % p->blk, g, d)] * (i == 0 ? 2.0 : (i == p->blk - 1 ? 0.0 : 1.0));"),
    (C, "attend drops the scale", "logit[i] = p->scale * s;", "logit[i] = s;"),
    (C, "attend lse without the maximum", "return m + log(l);", "return log(l);"),
    (C, "attend lse + 1", "return m + log(l);", "return m + log(l) + 1.0;"),
    (C, "attend output not normalised", "for (int d = 0; d < D; ++d) o[d] /= l;",
     "for (int d = 0; d < D; ++d) o[d] /= (l + 1e-3);"),
    (C, "compressed visibility one short", "int ncv = (t + 1) / blk; /* complete blocks visible to t (reading) */",
     "int ncv = t / blk;"),
    (C, "compressed visibility one long", "int ncv = (t + 1) / blk; /* complete blocks visible to t (reading) */",
     "int ncv = (t + 1) / blk + ((t + 1) / blk < nc_all ? 1 : 0);"),
    (C, "importance not summed over heads", "S[j] += prh[j];", "S[j] = prh[j];"),
    (C, "importance drops a head", "              if (ncv > 0) {\n                double m = -INFINITY;",
     "              if (ncv > 0 && hh < G - 1 + (G == 1)) {\n                double m = -INFINITY;"),
    (C, "compressed probabilities unnormalised", "prh[j] /= l;\n", "prh[j] /= 1.0;\n"),
    (C, "lse_cmp + 1", "lse_cmp[((size_t)b * Hq + h) * T + t] = m + log(l);",
     "lse_cmp[((size_t)b * Hq + h) * T + t] = m + log(l) + 1.0;"),
    (C, "lse_cmp without the maximum", "lse_cmp[((size_t)b * Hq + h) * T + t] = m + log(l);",
     "lse_cmp[((size_t)b * Hq + h) * T + t] = log(l);"),
    (C, "own block not forced", "if (own != 0) out[n++] = own;", ""),
    (C, "block 0 not forced", "  out[n++] = 0;\n  if (own != 0)", "  if (own != 0)"),
    (C, "ties to the higher index", "return (x->j < y->j) ? -1 : (x->j > y->j);",
     "return (x->j > y->j) ? -1 : (x->j < y->j);"),
    (C, "ascending importance", "if (x->s > y->s) return -1;\n  if (x->s < y->s) return 1;",
     "if (x->s < y->s) return -1;\n  if (x->s > y->s) return 1;"),
    (C, "own block also a candidate",
     "int ncand = own > 1 ? own - 1 : 0;\n  if (ncand <= m) {\n    for (int j = 1; j < own; ++j) out[n++] = j;\n"
     "    *gap = INFINITY;\n  } else {\n    for (int j = 1; j < own; ++j) { buf[j - 1].s = S[j]; buf[j - 1].j = j; }",
     "int ncand = own > 1 ? own : 0;\n  if (ncand <= m) {\n    for (int j = 1; j < own; ++j) out[n++] = j;\n"
     "    *gap = INFINITY;\n  } else {\n    for (int j = 1; j <= own; ++j) { buf[j - 1].s = S[j]; buf[j - 1].j = j; }"),
    (C, "sorting when every candidate fits", "if (ncand <= m) {", "if (ncand <= m - 1) {"),
    (C, "gap sign", "*gap = (m > 0 ? buf[m - 1].s : INFINITY) - buf[m].s;",
     "*gap = buf[m].s - (m > 0 ? buf[m - 1].s : INFINITY);"),
    (C, "selection not causal",
     "for (int s = sel[i] * blk; s < (sel[i] + 1) * blk && s <= t && s < T; ++s)\n                keys[nk++] = s;",
     "for (int s = sel[i] * blk; s < (sel[i] + 1) * blk && s < T; ++s)\n                keys[nk++] = s;"),
    (C, "selection strictly causal",
     "for (int s = sel[i] * blk; s < (sel[i] + 1) * blk && s <= t && s < T; ++s)\n                keys[nk++] = s;",
     "for (int s = sel[i] * blk; s < (sel[i] + 1) * blk && s < t && s < T; ++s)\n                keys[nk++] = s;"),
    (C, "window one longer", "int w0 = t - window + 1 > 0 ? t - window + 1 : 0;",
     "int w0 = t - window > 0 ? t - window : 0;"),
    (C, "window one shorter", "int w0 = t - window + 1 > 0 ? t - window + 1 : 0;",
     "int w0 = t - window + 2 > 0 ? t - window + 2 : 0;"),
    (C, "lse_win + 1", "lse_win[((size_t)b * Hq + h) * T + t] = lsw;",
     "lse_win[((size_t)b * Hq + h) * T + t] = lsw + 1.0;"),
    (C, "lse_sel + 1", "lse_sel[((size_t)b * Hq + h) * T + t] = lse;",
     "lse_sel[((size_t)b * Hq + h) * T + t] = lse + 1.0;"),
    (C, "selection and window gates swapped", "+= gt[1] * os[d] + gt[2] * ow[d];",
     "+= gt[2] * os[d] + gt[1] * ow[d];"),
    (C, "compression gate index", "* Hq + h) * 3 + 0] * oc[d];", "* Hq + h) * 3 + 1] * oc[d];"),
    (C, "wrong KV group",
     "double lse = attend(&p, qv, k, v, b, g, keys, nk, os, logit);\n              if (lse_sel)",
     "double lse = attend(&p, qv, k, v, b, (g + 1) % Hkv, keys, nk, os, logit);\n              if (lse_sel)"),
    (C, "selection dq drops the scale", "dqv[d] += scale * dS * kv[d];", "dqv[d] += dS * kv[d];"),
    (C, "selection dk drops the scale", "dkv[d] += scale * dS * qv[d];", "dkv[d] += dS * qv[d];"),
    (C, "selection gradient without Delta",
     "double dS = P * (dP - delta);\n              double* dkv",
     "double dS = P * dP;\n              double* dkv"),
    (C, "selection Delta from the ungated dO", "delta += dos[d] * os[d];",
     "delta += dout[qidx(&p, b, t, h, d)] * os[d];"),
    (C, "selection gradient without its gate", "dos[d] = gs * dout[qidx(&p, b, t, h, d)];",
     "dos[d] = dout[qidx(&p, b, t, h, d)];"),
    (C, "selection gradient with the window gate",
     "double gs = gates[(((size_t)b * T + t) * Hq + h) * 3 + 1];",
     "double gs = gates[(((size_t)b * T + t) * Hq + h) * 3 + 2];"),
    (C, "selection dv from the ungated dO", "dvv[d] += P * dos[d];\n              }",
     "dvv[d] += P * dout[qidx(&p, b, t, h, d)];\n              }"),
    (C, "full gradient dk drops the scale", "dkv[d] += p->scale * dS * qv[d];", "dkv[d] += dS * qv[d];"),
    (C, "full gradient dq drops the scale", "dqv[d] += p->scale * dS * kv[d];", "dqv[d] += dS * kv[d];"),
    (C, "full gradient without Delta", "double dS = P * (dP - delta);\n    double* dkv",
     "double dS = P * dP;\n    double* dkv"),
    (C, "full gradient dv halved", "dvv[d] += P * dob[d];", "dvv[d] += P * dob[d] * 0.5;"),
    (C, "mean-pool gradient not divided", "dk[kidx(&p, b, j * blk + i, g, d)] += dkc[kidx(&pc, b, j, g, d)] / blk;",
     "dk[kidx(&p, b, j * blk + i, g, d)] += dkc[kidx(&pc, b, j, g, d)];"),
    (C, "mean-pool gradient of v missing", "dv[kidx(&p, b, j * blk + i, g, d)] += dvc[kidx(&pc, b, j, g, d)] / blk;", ""),
    (C, "full gradient compressed visibility", "int ncv = (t + 1) / blk;\n            for (int j = 0; j < ncv; ++j) keys[j] = j;",
     "int ncv = t / blk;\n            for (int j = 0; j < ncv; ++j) keys[j] = j;"),
    (C, "dgates compression scaled by its gate", "dg[0] = s0;", "dg[0] = s0 * gt[0];"),
    (C, "dgates selection from the compression", "dg[1] = s1;", "dg[1] = s0;"),
    (C, "dgates window offset", "dg[2] = s2;", "dg[2] = s2 + 1e-3;"),
    (C, "full gradient window one longer",
     "for (int s = t - window + 1 > 0 ? t - window + 1 : 0; s <= t; ++s) keys[nw++] = s;",
     "for (int s = t - window > 0 ? t - window : 0; s <= t; ++s) keys[nw++] = s;"),
    (C, "full gradient selection with the window gate", "for (int d = 0; d < D; ++d) dob[d] = gt[1] * dov[d];",
     "for (int d = 0; d < D; ++d) dob[d] = gt[2] * dov[d];"),
    (C, "full gradient selection not causal",
     "for (int s = j * blk; s < (j + 1) * blk && s <= t && s < T; ++s) keys[nk++] = s;\n            }\n"
     "            for (int d = 0; d < D; ++d) dob[d] = gt[1]",
     "for (int s = j * blk; s < (j + 1) * blk && s < T; ++s) keys[nk++] = s;\n            }\n"
     "            for (int d = 0; d < D; ++d) dob[d] = gt[1]"),
    (PY, "decode on the wrong row", "        t = L - 1\n", "        t = L - 2 if L > 1 else 0\n"),
    (PY, "decode drops the window gate", "        gf[0, t] = gates[b]\n",
     "        gf[0, t] = gates[b]\n        gf[0, t, :, 2] = 0.0\n"),
    (PY, "decode importance shifted", "        res[\"scores\"][b, :, :sc.shape[-1]] = sc\n",
     "        res[\"scores\"][b, :, :sc.shape[-1]] = np.roll(sc, 1, axis=-1)\n"),
]


def _stage(tmp):
    for rel in ("oracle/__init__.py", "oracle/nsa_oracle.c", "tests/conftest.py", "tests/test_oracle_pins.py",
                "pytest.ini"):
        os.makedirs(os.path.join(tmp, os.path.dirname(rel)), exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), os.path.join(tmp, rel))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tmp, "tests", "golden"))


def run(selected=()):
    survivors = []
    with tempfile.TemporaryDirectory() as tmp:
        _stage(tmp)
        originals = {f: open(os.path.join(tmp, f)).read() for f in (C, PY)}
        for f, name, old, new in MUTANTS:
            if selected and not any(s in name for s in selected):
                continue
            n = originals[f].count(old)
            if n != 1:
                raise SystemExit(f"mutant '{name}': its text occurs {n} times in {f}")
            for g, text in originals.items():
                open(os.path.join(tmp, g), "w").write(text.replace(old, new) if g == f else text)
            subprocess.run([sys.executable, "-c", "import oracle; oracle.build(force=True)"], cwd=tmp,
                           check=True, capture_output=True)
            r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q",
                                "-m", "not gpu", "-p", "no:cacheprovider"], cwd=tmp, capture_output=True,
                               text=True)
            verdict = "killed" if r.returncode != 0 else "SURVIVED"
            if r.returncode == 0:
                survivors.append(name)
            tail = [x for x in r.stdout.splitlines() if " passed" in x or " failed" in x]
            print(f"{name:46s} {verdict:9s} {tail[-1] if tail else ''}", flush=True)
    print(f"{len(survivors)} survivor(s)" + (": " + ", ".join(survivors) if survivors else ""))
    return survivors


if __name__ == "__main__":
    sys.exit(1 if run(sys.argv[1:]) else 0)
