"""Plant plausible mistakes in copies of the oracle and require the pin suite
to catch every one.  Each mutant is one textual edit of moe_oracle.c (a dropped
term, a wrong sign, index or operand, a swapped nibble ...), compiled with gcc
into a temporary library; all mutants stay in bounds, so a caught mutant fails
an assertion rather than crashing.  Runs on the CPU only."""
import os

import pytest

from oracle import oracle as oracle_mod
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle_mod.__file__), "moe_oracle.c")

MUTANTS = [
    ("bias dropped", "l[e] += (double)bias[e];", "l[e] += 0.0 * (double)bias[e];"),
    ("gumbel sign", "return -log(-log(u));", "return log(-log(u));"),
    ("tau multiplies", "z[e] = v / tau;", "z[e] = v * tau;"),
    ("noise not tempered", "z[e] = v / tau;", "z[e] = (v - g) / tau + g;"),
    ("ties to higher index", "return a < b;", "return a > b;"),
    ("NaN ranks first", "return nb; /* the non-NaN one wins */", "return na;"),
    ("ascending selection", "return z[a] > z[b];", "return z[a] < z[b];"),
    ("softmax mass lost", "p[e] /= s;", "p[e] /= (s + 1.0);"),
    ("softmax on logits", "p[e] = exp(z[e] - m);", "p[e] = exp(l[e] - m);"),
    ("gate from slot index", "gates[t * k + j] = (float)p[best];", "gates[t * k + j] = (float)p[j];"),
    ("gate_p from slot index", "gate_p[t * k + j] = p[best];", "gate_p[t * k + j] = p[j];"),
    ("gelu tanh form", "return 0.5 * h * erfc(-h / sqrt(2.0));",
     "return 0.5 * h * (1.0 + tanh(0.7978845608028654 * (h + 0.044715 * h * h * h)));"),
    ("gelu half dropped", "return 0.5 * h * erfc(-h / sqrt(2.0));", "return h * erfc(-h / sqrt(2.0));"),
    ("gelu sqrt2 dropped", "return 0.5 * h * erfc(-h / sqrt(2.0));", "return 0.5 * h * erfc(-h);"),
    ("gelu tail lost to cancellation", "return 0.5 * h * erfc(-h / sqrt(2.0));",
     "return 0.5 * h * (1.0 + erf(h / sqrt(2.0)));"),
    ("W1 reads x reversed", "h += load_w(W1e, S1e, w_dtype, d, n, i) * xr[i];",
     "h += load_w(W1e, S1e, w_dtype, d, n, i) * xr[d - 1 - i];"),
    ("GeLU skipped", "a[n] = oracle_gelu(h);", "a[n] = h;"),
    ("SwiGLU gate and up swapped", "a[n] = oracle_silu(g) * u;", "a[n] = oracle_silu(u) * g;"),
    ("SwiGLU interleaved in blocks of 8", "int64_t rg = 32 * (n / 16) + n % 16, ru = rg + 16;",
     "int64_t rg = 16 * (n / 8) + n % 8, ru = rg + 8;"),
    ("SiLU sign", "return a / (1.0 + exp(-a));", "return a / (1.0 + exp(a));"),
    ("router encoder skips GeLU", "double a = oracle_gelu(r);", "double a = r;"),
    ("router encoder drops its bias", "r += (double)b_in[j];", "r += 0.0;"),
    ("router encoder reads W_in transposed", "load_act(W_in, act_dtype, j * d + i)",
     "load_act(W_in, act_dtype, i * d_r + j)"),
    ("bf16 midpoint always rounds up", "up = (int)(hi & 1u);", "up = 1;"),
    ("bf16 rounded twice", "else if (fabs(v) != fabs((double)f))", "else if (0)"),
    ("SiLU expert computes GeLU", "a[n] = oracle_silu(h);", "a[n] = oracle_gelu(h);"),
    ("W2 reads hidden reversed", "acc += load_w(W2e, S2e, w_dtype, d_ff, c, n) * a[n];",
     "acc += load_w(W2e, S2e, w_dtype, d_ff, c, n) * a[d_ff - 1 - n];"),
    ("int4 nibble order", "int nib = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
     "int nib = (c % 2 == 0) ? (byte >> 4) : (byte & 0x0F);"),
    ("int4 unsigned", "return nib >= 8 ? nib - 16 : nib;", "return nib;"),
    ("int4 group order", "s = bf16_to_double(((const uint16_t *)scales)[n * (K / 128) + c / 128]);",
     "s = bf16_to_double(((const uint16_t *)scales)[n * (K / 128) + (K / 128 - 1 - c / 128)]);"),
    ("philox 9 rounds", "for (int r = 0; r < 10; ++r) {", "for (int r = 0; r < 9; ++r) {"),
    ("philox key bump lost", "k1 += W1;", "k1 += 0;"),
    ("uniform from second word", "return ((double)(r[0] >> 11) + 0.5)", "return ((double)(r[1] >> 11) + 0.5)"),
    ("noise ignores token offset", "oracle_gumbel(seed, token_offset + (uint64_t)t, (uint64_t)e)",
     "oracle_gumbel(seed, (uint64_t)t, (uint64_t)e)"),
    ("noise key swapped", "oracle_gumbel(seed, token_offset + (uint64_t)t, (uint64_t)e)",
     "oracle_gumbel(seed, (uint64_t)e, token_offset + (uint64_t)t)"),
    ("unstable scatter", "int32_t slot = offsets[e] + fill[e];", "int32_t slot = offsets[e + 1] - 1 - fill[e];"),
    ("combine uses first gate", "double w = gate_p[t * k + j];", "double w = gate_p[t * k];"),
    ("bf16 widened wrongly", "uint32_t w = (uint32_t)bits << 16;", "uint32_t w = ((uint32_t)bits << 16) | 0x8000u;"),
    ("logits skip last input", "for (int64_t i = 0; i < d; ++i) {\n            double xi",
     "for (int64_t i = 0; i + 1 < d; ++i) {\n            double xi"),
    ("fraction over tokens only", "fraction[e] /= (double)T * (double)k;", "fraction[e] /= (double)T;"),
    ("entropy in bits", "h -= q * log(q);", "h -= q * log2(q);"),
    ("entropy sign", "h -= q * log(q);", "h += q * log(q);"),
    ("balance term on fractions uses probs", "sf += (fraction[e] - 1.0 / E) * (fraction[e] - 1.0 / E);",
     "sf += (mean_prob[e] - 1.0 / E) * (mean_prob[e] - 1.0 / E);"),
    ("std without 1/E", "scalars[3] = sqrt(sf / E);", "scalars[3] = sqrt(sf);"),
    ("product term without E", "scalars[4] = (double)E * fp;", "scalars[4] = fp;"),
    ("renormalisation drops the last chosen", "for (int32_t j = 0; j < k; ++j)\n                den +=",
     "for (int32_t j = 0; j + 1 < k; ++j)\n                den +="),
    ("gaussian noise not scaled by sigma", "v += noise_std * oracle_normal(", "v += oracle_normal("),
    ("box-muller without the factor 2", "return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);",
     "return sqrt(-log(u1)) * cos(two_pi * u2);"),
    ("gaussian reuses the gumbel word", "double u1 = ((double)(r[2] >> 11) + 0.5)",
     "double u1 = ((double)(r[0] >> 11) + 0.5)"),
    ("box-muller sine for cosine", "return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);",
     "return sqrt(-2.0 * log(u1)) * sin(two_pi * u2);"),
    ("gaussian words 2 and 3 swapped",
     "(r[2] >> 11) + 0.5) * (1.0 / 9007199254740992.0);\n    double u2 = ((double)(r[3] >> 11)",
     "(r[3] >> 11) + 0.5) * (1.0 / 9007199254740992.0);\n    double u2 = ((double)(r[2] >> 11)"),
    ("expert linear map skips its last input", "for (int64_t i = 0; i < K; ++i)\n            acc += load_w(We",
     "for (int64_t i = 0; i + 1 < K; ++i)\n            acc += load_w(We"),
    ("product term pairs fraction with itself", "fp += fraction[e] * mean_prob[e];",
     "fp += fraction[e] * fraction[e];"),
    ("mean prob not averaged", "mean_prob[e] /= (double)T;", "mean_prob[e] /= (double)E;"),
    ("capacity rounds down", "return (int64_t)ceil((double)T * (double)k / (double)E * capacity_factor);",
     "return (int64_t)floor((double)T * (double)k / (double)E * capacity_factor);"),
    ("capacity off by one", "if (counts[e] < cap) {", "if (counts[e] <= cap) {"),
    ("reroute to the worst expert", "if (best < 0 || ranks_before(z + t * E, e, best))",
     "if (best < 0 || ranks_before(z + t * E, best, e))"),
    ("reroute reuses the token's expert", "if (ids[t * k + jj] == e)\n                            used = 1;",
     "if (ids[t * k + jj] == e)\n                            used = 0;"),
    ("reroute ignores capacity", "if (counts[e] >= cap)\n                        continue;",
     "if (counts[e] > cap + 100)\n                        continue;"),
    ("dropped slot keeps its gate", "double g = ids[a] >= 0 ? p[(a / k) * E + ids[a]] : 0.0;",
     "double g = ids[a] >= 0 ? p[(a / k) * E + ids[a]] : p[(a / k) * E];"),
    ("reroute in reverse token order",
     "for (int64_t t = 0; t < T; ++t)\n            for (int32_t j = 0; j < k; ++j) {\n                if (!overflow",
     "for (int64_t t = T - 1; t >= 0; --t)\n            for (int32_t j = 0; j < k; ++j) {\n                if (!overflow"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, source, name, old, new):
    assert source.count(old) == 1, f"mutation site for '{name}' not unique in moe_oracle.c"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(source.replace(old, new))
    lib = oracle_mod.build(src=str(mutated), out=str(tmp_path / "libmutant.so"))
    orc = oracle_mod.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the mutant '{name}'"
