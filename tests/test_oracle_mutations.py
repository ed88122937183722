"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/oracle.c inside a temporary
directory (on the CPU; the repository's oracle is never touched), rebuilds the
copy, and runs the oracle pins (tests/test_oracle.py) against it.  Every
planted mistake must make at least one pin fail.  The mistakes are the kinds a
restatement of the pages could plausibly contain: a dropped scale, a wrong GQA
head map or page slot, a merge that forgets a factor, a wrong split boundary,
a one-sided or inclusive range check, sign flips, V read from K, a wrong fp16
exponent bias, and a fallback that keeps the unified constant.
"""
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]

# (name, text in oracle.c, replacement); every occurrence is replaced
MUTATIONS = [
    ("dropped score scale", "s[t - t0] = dot * p->scale;", "s[t - t0] = dot;"),
    ("GQA map h % Hkv", "int kvh = h / (p->Hq / p->Hkv);", "int kvh = h % p->Hkv;"),
    ("page slot off by one", "int slot = t % p->page_size;", "int slot = (t + 1) % p->page_size;"),
    ("lse without the max", "lse[r] = m + log(z);", "lse[r] = log(z);"),
    ("merged l without l_s", "if (pl[s] > 0.0) l += pl[s] * exp(pm[s] - m);",
     "if (pl[s] > 0.0) l += exp(pm[s] - m);"),
    ("merge weight without l_s", "double w = pl[s] * exp(pm[s] - m);", "double w = exp(pm[s] - m);"),
    ("split boundary one short", "int t0 = sp * split, t1 = t0 + split < n ? t0 + split : n;",
     "int t0 = sp * split, t1 = t0 + split - 1 < n ? t0 + split - 1 : n;"),
    ("inclusive range check", "return s < lo || s > hi;", "return s <= lo || s >= hi;"),
    ("one-sided range check", "return s < lo || s > hi;", "return s > hi;"),
    ("unified exponent sign", "s[t - t0] = exp(s[t - t0] - c);", "s[t - t0] = exp(c - s[t - t0]);"),
    ("LSE merge sign", "double alpha = exp(Ls[s] - L);", "double alpha = exp(L - Ls[s]);"),
    ("V read from K", "double z = weighted_v(p, v, block_table", "double z = weighted_v(p, k, block_table"),
    ("online rescale sign", "double corr = m == -INFINITY ? 0.0 : exp(m - m_new);",
     "double corr = m == -INFINITY ? 0.0 : exp(m_new - m);"),
    ("fp16 exponent bias", "v = ldexp((double)(m | 0x400), e - 25);", "v = ldexp((double)(m | 0x400), e - 24);"),
    ("fallback keeps phi", "c = s[0];", "c = phi;"),
    ("fallback partial m keeps phi", "part_m[slot] = c;", "part_m[slot] = phi;"),
    ("whole-row fallback only recomputes the flagged split", "if (whole_row ? row_bad : bad) {", "if (bad) {"),
    ("per-head K scale by query head", "double ks = k_scale_of(p, kvh);", "double ks = k_scale_of(p, h % p->Hkv);"),
    ("per-head V scale of head 0", "double vs = v_scale_of(p, kvh);", "double vs = v_scale_of(p, 0);"),
    ("causal limit one short", "int lim = n - p->q_len + i + 1;", "int lim = n - p->q_len + i;"),
    ("causal window from the first token", "int lim = n - p->q_len + i + 1;", "int lim = i + 1;"),
]


def _pins_on_copy(tmp_path, old=None, new=None):
    """Copy the oracle, synth and tests into tmp_path, optionally replace text
    in the copied oracle.c, and run the oracle pins there."""
    for d in ("oracle", "synth", "tests"):
        shutil.copytree(ROOT / d, tmp_path / d, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    if old is not None:
        src = tmp_path / "oracle" / "oracle.c"
        text = src.read_text()
        assert old in text, "the text to mutate is not in oracle.c"
        src.write_text(text.replace(old, new))
    return subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle.py", "-x", "-q", "-p", "no:cacheprovider"],
                          cwd=tmp_path, capture_output=True, text=True, timeout=600)


def test_unmutated_copy_passes_the_pins(tmp_path):
    """The control: the copied tree itself is sound, so a failure below is the mistake's."""
    r = _pins_on_copy(tmp_path)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    r = _pins_on_copy(tmp_path, old, new)
    assert r.returncode != 0, f"planted mistake '{name}' survived every pin:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, f"'{name}': the pins did not run to a failure:\n{r.stdout[-2000:]}{r.stderr[-2000:]}"
