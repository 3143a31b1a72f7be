"""The pins must bite: copies of the oracle with one planted mistake each are
compiled (gcc, on the CPU) and every copy must fail at least one pin."""
import os

import pytest

import oracle
import oracle_checks as oc

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")

# (name, original text, planted text): each a plausible slip
MUTATIONS = [
    ("nibble_order", "(i & 1) ? (byte >> 4) : (byte & 15)", "(i & 1) ? (byte & 15) : (byte >> 4)"),
    ("group_index", "(size_t)(i / G);", "(size_t)((i / 2) / G);"),
    ("bias_sign", "* (double)code_at(m, cols, n, i) + bf16_value", "* (double)code_at(m, cols, n, i) - bf16_value"),
    ("rounding_truncates", "u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0u;"),
    ("rounding_half_up", "u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    ("tie_to_higher_id", "L[e] > L[best]", "L[e] >= L[best]"),
    ("softmax_sign", "exp((double)L[ids[(size_t)t * k + j]] - lmax)", "exp(lmax - (double)L[ids[(size_t)t * k + j]])"),
    ("unstable_scatter", "for (int64_t a = 0; a < A; ++a)\n            if (ids[a] == e)",
     "for (int64_t a = A - 1; a >= 0; --a)\n            if (ids[a] == e)"),
    ("exclusive_scan_off_by_one", "offsets[e + 1] = offsets[e] + counts[e];",
     "offsets[e + 1] = offsets[e] + counts[e] + (e == 0);"),
    ("tile_rows_full", "(counts[e] - r0 < tile_m) ? counts[e] - r0 : tile_m", "tile_m"),
    ("silu_sign", "z / (1.0 + exp(-z))", "z / (1.0 + exp(z))"),
    ("gate_up_swapped", "h[n] = silu(g) * u;", "h[n] = silu(u) * g;"),
    ("shared_dropped", "yt[i] += gamma * o[i];", "yt[i] += 0.0 * gamma * o[i];"),
    ("shared_gate_sign", "return 1.0 / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(z));"),
    ("shared_gate_ignored", "const double gamma = shared_weight(xt, shared_gate, d);",
     "const double gamma = shared_weight(xt, NULL, d);"),
    ("routing_weight_dropped", "yt[i] += w[(size_t)t * k + j] * o[i];", "yt[i] += o[i];"),
    ("down_transposed", "weight_at(down, Fw, G, i, n)", "weight_at(down, Fw, G, n % d, i % Fw)"),
    ("x_index", "xt[i] = bf16_value(x[(size_t)t * d + i]);", "xt[i] = bf16_value(x[(size_t)t + i]);"),
    ("router_transposed", "(double)W[(size_t)i * E + e]", "(double)W[((size_t)e * d + i) % ((size_t)d * E)]"),
    ("router_bias_dropped", "if (bias) acc += (double)bias[e];", "if (bias) acc += 0.0;"),
    ("attn_scale_dropped", "s[t] = acc / sqrt((double)D);", "s[t] = acc;"),
    ("attn_group_modulo", "const int g = h / G;", "const int g = h % Hkv;"),
    ("attn_not_normalised", "out[(size_t)h * D + i] = acc / den;", "out[(size_t)h * D + i] = acc;"),
    ("attn_v_dim_reversed", "acc += s[t] * bf16_value(v[((size_t)g * L + t) * D + i]);",
     "acc += s[t] * bf16_value(v[((size_t)g * L + t) * D + (D - 1 - i)]);"),
    ("attn_last_token_dropped", "for (int t = 0; t < L; ++t) {\n            s[t] = exp(s[t] - smax);",
     "for (int t = 0; t < L; ++t) {\n            s[t] = (t == L - 1 && L > 1) ? 0.0 : exp(s[t] - smax);"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: " + name
    mutated = tmp_path / "moe_oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / "libmut.so")
    import subprocess
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o", so,
                    str(mutated), "-lm"], check=True)
    lib = oracle.load(so)
    caught = []
    for check in oc.ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError, IndexError) as e:  # a pin failed
            caught.append(check.__name__)
    assert caught, "planted mistake %r passed every pin" % name
