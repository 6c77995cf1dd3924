"""The oracle's pins catch plausible mistakes.  Each case plants one mistake in a copy of
oracle/tra_oracle.c (a dropped term, a wrong sign, base or index, a transposed operand, a
loop order swapped), builds that copy, and runs the oracle's pin tests against it in a
process of their own: at least one pin must fail (and fail as a test, not a crash).  Nothing
here touches the oracle the other tests use.

Not planted: the disk test's inclusive bound (<= against <).  The two differ only where
ln d^2 equals H_i + lambda exactly in fp64, which would need an fp32 entropy to land on a
transcendental value; no input the tests can build tells them apart."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tra_oracle.c")
PINS = [os.path.join(ROOT, "tests", f) for f in
        ("test_oracle_attention.py", "test_oracle_mask.py", "test_oracle_window.py")]

MISTAKES = [
    # attention (section 2, pipeline step 1: the warm-up pass and its entropy)
    ("entropy in bits instead of nats", "h -= p * log(p);", "h -= p * log2(p);"),
    ("softmax scale dropped", "s[j] = c->scale * acc;", "s[j] = acc;"),
    ("queries read from k", "const double *qi = c->q + (int64_t)i * D;", "const double *qi = c->k + (int64_t)i * D;"),
    ("lse without the row max", "c->lse[r] = mx + log(z);", "c->lse[r] = log(z);"),
    ("block mask column from block_q", "c->block_mask[(int64_t)(i / c->bq) * c->nkb + j / c->bk]",
     "c->block_mask[(int64_t)(i / c->bq) * c->nkb + j / c->bq]"),
    # Insight I and II: budget, frame normaliser, radius
    ("budget from exp(-H)", "return tau * exp(H);", "return tau * exp(-H);"),
    ("frame normaliser decays with gamma, not 2 gamma", "acc += exp(-(2.0 * gamma) * (double)delta);",
     "acc += exp(-gamma * (double)delta);"),
    ("area matching without sqrt", "return sqrt(orc_token_budget(H, tau) / (M_PI * S_f));",
     "return orc_token_budget(H, tau) / (M_PI * S_f);"),
    ("decay sign flipped in the threshold table", "(log(t) - (2.0 * g) * (double)delta)",
     "(log(t) + (2.0 * g) * (double)delta)"),
    ("pi dropped from the threshold table", "- log(M_PI * S[f]);", "- log(S[f]);"),
    # pipeline step 3: tile-major order, coordinates, voting
    ("tile columns before tile rows",
     "for (int y0 = 0; y0 < H; y0 += th)\n            for (int x0 = 0; x0 < W; x0 += tw)",
     "for (int x0 = 0; x0 < W; x0 += tw)\n            for (int y0 = 0; y0 < H; y0 += th)"),
    ("row coordinate keeps the frame", "g->hy[p] = (int32_t)((n / W) % H);", "g->hy[p] = (int32_t)(n / W);"),
    ("votes count key tokens, not queries", "if (orc_mask_member(c, i, j)) touched[j / c->bk] = 1;",
     "if (orc_mask_member(c, i, j)) vt[j / c->bk] += 1;"),
    ("diagonal guard dropped", "mk[kb] = (uint8_t)(vt[kb] >= c->vote || diagonal);",
     "mk[kb] = (uint8_t)(vt[kb] >= c->vote);"),
    # the 1D-distance ablation (section 4)
    ("window half-width without the factor 2", "return log((double)tau) - log(2.0);", "return log((double)tau);"),
]


@pytest.mark.parametrize("name,old,new", MISTAKES, ids=[m[0] for m in MISTAKES])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "the planted site must be unique: %s" % name
    mutant = tmp_path / "tra_oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    "-o", str(lib), str(mutant), "-lm"], check=True)
    env = dict(os.environ, TRA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    failed = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
    assert r.returncode == 1 and failed, "%s: no pin failed (exit %d)\n%s" % (name, r.returncode, r.stdout[-2000:])
    print("%s: %d pin(s) fail, e.g. %s" % (name, len(failed), failed[0].split(" - ")[0]))
