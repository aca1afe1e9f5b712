"""Mutation tests: each plausible mistake planted in a copy of the oracle's C
source must make at least one pin fail. This shows the pins constrain every
part of the oracle (bit order, word index, group index, affine sign, the
fp16 decode, the summation range, operand indexing, the bound A).

The mistakes are planted on the CPU, in a temporary copy; the oracle itself
is never modified.
"""
import pytest

import oracle
from tests import _pins

MUTANTS = [
    ("tiled layout: lane block and row swapped",
     "const int64_t L = 16 * c + i;",
     "const int64_t L = 4 * i + c;"),
    ("tiled layout: groups not in stream order",
     "const int64_t p = (g * (G / 4) + j) * bits + e;",
     "const int64_t p = ((g ^ 1) * (G / 4) + j) * bits + e;"),
    ("tiled (s, b) words: scale and bias halves swapped",
     "(uint32_t)s[n * Kg + g] | ((uint32_t)b[n * Kg + g] << 16);",
     "(uint32_t)b[n * Kg + g] | ((uint32_t)s[n * Kg + g] << 16);"),
    ("unpack MSB-first within a word",
     "return (int)((row[t / 32] >> (t % 32)) & 1u);",
     "return (int)((row[t / 32] >> (31 - t % 32)) & 1u);"),
    ("pack MSB-first within a word",
     "row[t / 32] |= ((c >> j) & 1u) << (t % 32);",
     "row[t / 32] |= ((c >> j) & 1u) << (31 - t % 32);"),
    ("unpack drops the top bit of each code",
     "    for (int j = 0; j < bits; ++j)\n        c |= (uint32_t)stream_bit",
     "    for (int j = 0; j < bits - 1; ++j)\n        c |= (uint32_t)stream_bit"),
    ("unpack with a code stride of bits+1",
     "c |= (uint32_t)stream_bit(row, k * bits + j) << j;",
     "c |= (uint32_t)stream_bit(row, k * (bits + 1) + j) << j;"),
    ("scale from the wrong group",
     "double s = decode(jb->dtype, jb->s[n * Kg + k / G]);",
     "double s = decode(jb->dtype, jb->s[n * Kg + (k / G + 1) % Kg]);"),
    ("bias group index from k mod Kg",
     "double b = decode(jb->dtype, jb->b[n * Kg + k / G]);",
     "double b = decode(jb->dtype, jb->b[n * Kg + k % Kg]);"),
    ("subtracted bias",
     "w[k] = s * q + b;",
     "w[k] = s * q - b;"),
    ("zero-point form s*(q+b)",
     "w[k] = s * q + b;",
     "w[k] = s * (q + b);"),
    ("scale and bias swapped",
     "double s = decode(jb->dtype, jb->s[n * Kg + k / G]);\n            double b = decode(jb->dtype, jb->b[n * Kg + k / G]);",
     "double s = decode(jb->dtype, jb->b[n * Kg + k / G]);\n            double b = decode(jb->dtype, jb->s[n * Kg + k / G]);"),
    ("dot skips the last k",
     "for (int64_t k = 0; k < K; ++k) {\n                double p",
     "for (int64_t k = 0; k < K - 1; ++k) {\n                double p"),
    ("activation indexed [k][m]",
     "double p = w[k] * xd[m * K + k];",
     "double p = w[k] * xd[(k * M + m) % (M * K)];"),
    ("weight row stride off by one word",
     "        const uint32_t *row = jb->words + n * W;\n        for (int64_t k = 0; k < K; ++k) {",
     "        const uint32_t *row = jb->words + n * (W > 1 ? W - 1 : W);\n        for (int64_t k = 0; k < K; ++k) {"),
    ("bound without absolute value",
     "mag += fabs(p);",
     "mag += p;"),
    ("subnormal halves decoded with 2^-25",
     "v = ldexp((double)frac, -24);",
     "v = ldexp((double)frac, -25);"),
    ("half exponent bias off by one",
     "v = ldexp((double)(1024 + frac), expo - 25);",
     "v = ldexp((double)(1024 + frac), expo - 24);"),
    ("half sign ignored",
     "v = ldexp((double)(1024 + frac), expo - 25);\n    return sign ? -v : v;",
     "v = ldexp((double)(1024 + frac), expo - 25);\n    return v;"),
    ("bf16 sign ignored",
     "v = ldexp((double)(128 + frac), expo - 134);\n    return sign ? -v : v;",
     "v = ldexp((double)(128 + frac), expo - 134);\n    return v;"),
    ("factored form: group sum of x counts the codes",
     "XS += xd[m * K + k];",
     "XS += (double)read_code(row, k, jb->bits);"),
    ("factored form: bias times P",
     "+ decode(jb->dtype, jb->b[n * Kg + g]) * XS;",
     "+ decode(jb->dtype, jb->b[n * Kg + g]) * P;"),
    ("bf16 exponent bias off by one",
     "v = ldexp((double)(128 + frac), expo - 134);",
     "v = ldexp((double)(128 + frac), expo - 133);"),
    ("bf16 read with an 8-bit fraction",
     "int frac = h & 0x7f;",
     "int frac = h & 0xff;"),
    ("bf16 subnormals decoded with 2^-134",
     "v = ldexp((double)frac, -133);",
     "v = ldexp((double)frac, -134);"),
    ("bf16 operands: scales decoded as fp16",
     "double s = decode(jb->dtype, jb->s[n * Kg + k / G]);",
     "double s = qo_half_to_double(jb->s[n * Kg + k / G]);"),
    ("bf16 operands: activations decoded as fp16",
     "    decode_array(jb->dtype, jb->x, xd, M * K);\n    for (int64_t i = jb->n_begin; i < jb->n_end; ++i) {\n        const int64_t n = job_row(jb, i);\n        const uint32_t *row = jb->words + n * W;\n        for (int64_t k = 0; k < K; ++k) {",
     "    decode_array(QO_F16, jb->x, xd, M * K);\n    for (int64_t i = jb->n_begin; i < jb->n_end; ++i) {\n        const int64_t n = job_row(jb, i);\n        const uint32_t *row = jb->words + n * W;\n        for (int64_t k = 0; k < K; ++k) {"),
    ("output row stride N instead of the list stride",
     "jb->y[m * jb->out_stride + i] = acc;\n            if (jb->absum)",
     "jb->y[m * jb->out_stride + (i + m) % jb->out_stride] = acc;\n            if (jb->absum)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = oracle.SOURCE.read_text()
    assert src.count(old) == 1, f"mutation anchor for '{name}' not found exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(source=mutated, output=tmp_path / "libmutant.so")
    results = _pins.run_all(oracle.Oracle(lib))
    caught = [pin for pin, fails in results.items() if fails]
    assert caught, f"no pin caught the planted mistake '{name}'"
