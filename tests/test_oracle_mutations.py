"""The oracle's pins are strong enough: plant plausible mistakes in copies of the
oracle source (on the CPU, in a temporary directory) and check that the pin suite
fails for every one of them.  The real oracle is never modified."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, planted mistake)
MUTATIONS = [
    ("nibble order swapped",
     "(c & 1) ? (row[c / 2] >> 4) : (row[c / 2] & 0x0f)",
     "(c & 1) ? (row[c / 2] & 0x0f) : (row[c / 2] >> 4)"),
    ("bias dropped", "return s * (double)q + b;", "return s * (double)q;"),
    ("wrong group index", "int64_t gi = R * (cols / 64) + c / 64;",
     "int64_t gi = R * (cols / 64) + (c / 64 + 1) % (cols / 64);"),
    ("silu sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("no renormalisation", "w[j] = p[sel[j]] / zs;", "w[j] = p[sel[j]];"),
    ("ties to the higher id", "(l[a] == l[b] && a < b)", "(l[a] == l[b] && a > b)"),
    ("down operand transposed", "acc += weight(d, L->bits, e, n, i, I) * h[i];",
     "acc += weight(d, L->bits, e, i % L->hidden, n % L->inter, I) * h[i];"),
    ("shared expert half weight", "yt[c] += gs * o[c];", "yt[c] += 0.5 * gs * o[c];"),
    ("gate and up swapped", "h[i] = silu(gi) * ui;", "h[i] = silu(ui) * gi;"),
    ("router bias ignored", "if (L->router_bias) acc += (double)L->router_bias[e];", ""),
    ("tile rows not interleaved", "return (int64_t)(c / 4) * 64 + r * 4 + (c % 4);",
     "return (int64_t)r * 32 + c;"),
    ("q8 code read unsigned", "dot += (double)(int8_t)blk[2 + c]", "dot += (double)blk[2 + c]"),
    ("activation codes rounded to nearest even", "roundf(v[c] / db)", "rintf(v[c] / db)"),
    ("activation max without abs", "if (fabsf(v[c]) > amax) amax = fabsf(v[c]);", "if (v[c] > amax) amax = v[c];"),
    ("activation scale dropped", "acc += orc_f16_to_double(rd16(blk)) * orc_f16_to_double(xd[b]) * (double)dot;",
     "acc += orc_f16_to_double(rd16(blk)) * (double)dot;"),
    ("activation code read unsigned", "(int64_t)xq[b * 32 + c]", "(int64_t)(uint8_t)xq[b * 32 + c]"),
    ("bf16 scales decoded as fp16",
     "double s = m->sb_bf16 ? orc_bf16_to_double(m->scales[gi]) : orc_f16_to_double(m->scales[gi]);",
     "double s = orc_f16_to_double(m->scales[gi]);"),
    ("shared gate sign", "gs = 1.0 / (1.0 + exp(-z));", "gs = 1.0 / (1.0 + exp(z));"),
    ("shared gate ignored", "yt[c] += gs * o[c];", "yt[c] += o[c];"),
    ("fp16 encoder ties away from zero", "if (rem > 0.5 || (rem == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;",
     "if (rem >= 0.5) r += 1.0;"),
    ("fp16 encoder truncates", "if (rem > 0.5 || (rem == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;", ""),
    ("fp16 encoder subnormal step", "if (expo < -14) expo = -14;", "if (expo < -15) expo = -15;"),
]


@pytest.mark.parametrize("name,orig,bad", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, orig, bad):
    text = open(SRC).read()
    assert text.count(orig) == 1, name
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(text.replace(orig, bad))
    lib = oracle.build(force=True, src=str(mutated), out=str(tmp_path / "liboracle_mut.so"))
    env = dict(os.environ, QSMOE_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch: {name}\n{r.stdout[-2000:]}"
