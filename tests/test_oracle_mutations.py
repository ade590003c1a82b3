"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Every mutation is applied to a temporary copy of oracle/oracle.c (the real file is never
touched), compiled with gcc and run through the pins on the CPU."""
import os

import pytest

import oracle

from oracle_pins import ALL_PINS

MUTATIONS = {
    "sink dropped from the denominator": ("double z = has_sink ? exp(sink - m) : 0.0;", "double z = 0.0;"),
    "sink multiplied by the logit scale": ("double m = has_sink ? sink : -INFINITY;",
                                           "sink *= scale; double m = has_sink ? sink : -INFINITY;"),
    "sink given a unit value": ("if (n == 0 || isinf(m)) return m;",
                                "if (n == 0 || isinf(m)) return m; if (has_sink) out[0] += 0.0 + exp(sink - m) / (exp(sink - m) + 1.0) * 0.5;"),
    "window one key too wide": ("(i - window + 1 > 0 ? i - window + 1 : 0) : 0;\n            int cnt = 0;",
                                "(i - window > 0 ? i - window : 0) : 0;\n            int cnt = 0;"),
    "causal mask excludes self": ("for (int64_t j = jlo; j <= i; ++j, ++cnt) {",
                                  "for (int64_t j = jlo; j < i; ++j, ++cnt) {"),
    "GQA head interleaved": ("const int64_t g = h / G;\n            const int64_t jlo", "const int64_t g = h % Hkv;\n            const int64_t jlo"),
    "wrong exponent sign": ("double s = exp(a[t] - m) / z;", "double s = exp(m - a[t]) / z;"),
    "logit scale dropped": ("a[t] = scale * dot;\n        if (a[t] > m) m = a[t];\n    }\n    if (n == 0",
                            "a[t] = dot;\n        if (a[t] > m) m = a[t];\n    }\n    if (n == 0"),
    "max without the row logits": ("if (a[t] > m) m = a[t];\n    }\n    if (n == 0", "\n    }\n    if (n == 0"),
    "ring slot off by one": ("const int64_t slot = j % window;", "const int64_t slot = (j + 1) % window;"),
    "page offset from the wrong end": ("const int64_t off = j % page_size;", "const int64_t off = page_size - 1 - j % page_size;"),
    "decode query position off by one": ("const int64_t i = nb - q_len + r % q_len;",
                                         "const int64_t i = nb - q_len + r % q_len - 1;"),
    "drafted tokens all at the last position": ("const int64_t i = nb - q_len + r % q_len;",
                                                "const int64_t i = nb - 1 + 0 * (r % q_len);"),
    "drafted tokens in reverse order": ("const int64_t i = nb - q_len + r % q_len;",
                                       "const int64_t i = nb - 1 - r % q_len;"),
    "chunk rows placed at the sequence start": ("const int64_t i = (int64_t)Lk - Lq + r; /* position of this query */",
                                                "const int64_t i = r;"),
    "E4M3 exponent bias off by one": ("else x = ldexp(1.0 + m / 8.0, e - 7);", "else x = ldexp(1.0 + m / 8.0, e - 8);"),
    "E4M3 subnormals without the 2^-9 scale": ("if (e == 0) x = ldexp((double)m, -9);", "if (e == 0) x = ldexp((double)m, -6);"),
    "cache scale applied to the value twice": ("if (t < kl->n) return kl->vscale * load(kl->v, kl->vidx[t] + e, kl->kvdtype);",
                                               "if (t < kl->n) return kl->vscale * kl->vscale * load(kl->v, kl->vidx[t] + e, kl->kvdtype);"),
    "drafts beside the cache taken one token late": ("const int64_t t = j - nc;", "const int64_t t = (j - nc + 1) % q_len;"),
    "drafts beside the cache ignored (cache read instead)": ("if (j >= nc) { /* a new token beside the cache */",
                                                             "if (0) { /* a new token beside the cache */"),
    "log-sum-exp without the row max": ("    return m + log(z);", "    return log(z);"),
    "rotary sine with the wrong sign": ("out[base + i] = a * c - b * sn;", "out[base + i] = a * c + b * sn;"),
    "rotary frequencies over all 192 dimensions": ("pow(theta, -2.0 * i / rot)", "pow(theta, -2.0 * i / dim)"),
    "rotary pairs interleaved": ("const double a = load(x, base + i, dtype), b = load(x, base + i + half, dtype);",
                                 "const double a = load(x, base + 2 * (i % (half / 2)) + (i >= half / 2) * half, dtype), b = load(x, base + 2 * (i % (half / 2)) + 1 + (i >= half / 2) * half, dtype);"),
    "sink gradient with the wrong sign": ("dsink_part[b * Hq + h] += -psink * Dsum;", "dsink_part[b * Hq + h] += psink * Dsum;"),
    "score gradient without the row term D": ("return p * (dp - D);", "return p * dp;"),
    "key gradient without the logit scale": ("dk[j * dqk + d] += scale * ds * load(q, qrow * dqk + d, dtype);",
                                             "dk[j * dqk + d] += ds * load(q, qrow * dqk + d, dtype);"),
    "E4M3 encoder multiplies by the scale": ("const float y = (float)x / (float)scale;",
                                             "const float y = (float)x * (float)scale;"),
    "E4M3 encoder clamps at 240": ("if (a > 448.0) a = 448.0;", "if (a > 240.0) a = 240.0;"),
    "E4M3 encoder rounds ties up": ("(frac == 0.5 && fmod(r, 2.0) != 0.0)", "(frac == 0.5)"),
    "E4M3 encoder drops the sign of zero": ("return (uint8_t)(c | (neg << 7));",
                                            "return (uint8_t)(c | ((neg && c) << 7));"),
    "value row from the query position": ("vi[cnt] = (size_t)(((b * Hkv + g) * Lk + j) * dv);",
                                          "vi[cnt] = (size_t)(((b * Hkv + g) * Lk + i) * dv);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {name}"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "liboracle_mut.so")
    oracle.build(str(mutated), lib_path)
    lib = oracle.load(lib_path)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake: {name}"
