"""The pins are strong enough: every planted mistake in a copy of the oracle fails one.

Each case takes the oracle's C source, replaces one expression with a
plausible mistake (a dropped term, a wrong sign, a wrong index, a reversed
order, an off-by-one), compiles the copy, binds the `oracle` wrapper to it and
runs the pins until one fails.  The real oracle is rebound afterwards.  CPU only.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

MUTANTS = [
    ("plane_offset_sign", "b[r] = L - zo_dot(rv, mr, d);", "b[r] = L + zo_dot(rv, mr, d);"),
    ("mean_key_not_normalised", "double w = exp(zo_dot(rv, K + t * d, d) - L);",
     "double w = exp(zo_dot(rv, K + t * d, d) - mx);"),
    ("lse_drops_max", "double L = mx + log(s);\n        double* mr", "double L = log(s);\n        double* mr"),
    ("node_range_off_by_one", "int64_t t1 = (j + 1) * span < Nc ? (j + 1) * span : Nc;",
     "int64_t t1 = (j + 1) * span + 1 < Nc ? (j + 1) * span + 1 : Nc;"),
    ("level_count_floor", "return (Nc + span - 1) / span;", "return Nc / span;"),
    ("tail_chunk_in_tree", "return (N / C) * C;", "return N;"),
    ("merge_child_weight", "double w = exp(lse_out[(child_off + c) * R + r] - LP);",
     "double w = exp(lse_out[(child_off + c) * R + r] - mx);"),
    ("merge_child_range", "int64_t c0 = j * C, c1 = (j + 1) * C < nchild ? (j + 1) * C : nchild;",
     "int64_t c0 = j * C, c1 = (j + 1) * C - 1 < nchild ? (j + 1) * C - 1 : nchild;"),
    ("score_min_over_planes", "if (v > best) best = v;", "if (best == -INFINITY || v < best) best = v;"),
    ("score_drops_offset", "double v = b_node[r] + zo_dot(qh, m_node + (int64_t)r * d, d);",
     "double v = zo_dot(qh, m_node + (int64_t)r * d, d);"),
    ("order_ascending", "if (a->w > b->w) return -1;\n    if (a->w < b->w) return 1;",
     "if (a->w < b->w) return -1;\n    if (a->w > b->w) return 1;"),
    ("kstar_off_by_one", "kstar = k + 1;", "kstar = k;"),
    ("kstar_one_too_many", "kstar = k + 1;", "kstar = k + 2 < nF ? k + 2 : nF;"),
    ("no_per_head_normalisation", "w += exp(s[(int64_t)h * nF + i] - lse[h]);",
     "w += exp(s[(int64_t)h * nF + i] - lse[0]);"),
    ("frontier_position_as_id", "const double* mn = m_l + (int64_t)F[i] * R * d;",
     "const double* mn = m_l + (int64_t)i * R * d;"),
    ("children_index", "int64_t id = (int64_t)kept[k] * C + c;", "int64_t id = (int64_t)kept[k] + c;"),
    ("top_frontier_short", "for (int64_t j = 0; j < nL; ++j) F_out[off[L] + j] = (int32_t)j;\n    int64_t nF = nL;",
     "for (int64_t j = 0; j < nL; ++j) F_out[off[L] + j] = (int32_t)j;\n    int64_t nF = nL > 1 ? nL - 1 : nL;"),
    ("sink_dropped", "in[0] = 1;", "in[0] = 0;"),
    ("tail_dropped", "for (int64_t t = Nc; t < N; ++t) in[t] = 1;", ""),
    ("attention_not_normalised", "double w = exp(zo_dot(qh, K + S[i] * d, d) - L);",
     "double w = exp(zo_dot(qh, K + S[i] * d, d) - mx);"),
    ("attention_value_index", "for (int j = 0; j < d; ++j) o[j] += w * V[S[i] * d + j];",
     "for (int j = 0; j < d; ++j) o[j] += w * V[S[i] * d + (d - 1 - j)];"),
    ("e4m3_ties_away", "if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;",
     "if (frac >= 0.5) r += 1.0;"),
    ("e4m3_two_mantissa_bits", "step = ldexp(1.0, (e - 1) - 3);", "step = ldexp(1.0, (e - 1) - 2);"),
    ("e4m3_no_subnormals", "step = ldexp(1.0, -9);                 /* subnormal spacing */",
     "step = ldexp(1.0, -6);                 /* subnormal spacing */"),
    ("fp8_scale_not_minimal", "while (ldexp(amax, -s) > 448.0) ++s;", "while (ldexp(amax, -s) > 224.0) ++s;"),
    ("block_tail_short", "for (int64_t x = Nc; x < E; ++x) in[x] = 1;", "for (int64_t x = Nc; x < E - 1; ++x) in[x] = 1;"),
    ("block_tail_skips_partial_chunk", "for (int64_t x = Nc; x < E; ++x) in[x] = 1;",
     "for (int64_t x = N; x < E; ++x) in[x] = 1;"),
    ("block_tail_to_block_end", "int64_t E = N + t + 1;          /* positions 0 .. N+t may be read */",
     "int64_t E = N + t + 2;          /* positions 0 .. N+t may be read */"),
    ("e2m1_ties_away", "    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;\n    const double v = r * step;\n    return x < 0 ? -v : v;\n}\n\n/* Scale exponent s of a block",
     "    if (frac >= 0.5) r += 1.0;\n    const double v = r * step;\n    return x < 0 ? -v : v;\n}\n\n/* Scale exponent s of a block"),
    ("e2m1_uniform_step", "const double step = a < 2.0 ? 0.5 : (a < 4.0 ? 1.0 : 2.0);", "const double step = 0.5;"),
    ("fp4_scale_not_minimal", "while (ldexp(amax, -s) > 6.0) ++s;", "while (ldexp(amax, -s) > 3.0) ++s;"),
    ("fp4_one_scale_per_row", "for (int k = 0; k < 32; ++k) amax = fmax(amax, fabs(mb[k]));",
     "for (int k = 0; k < d; ++k) amax = fmax(amax, fabs(m[i * d + k]));"),
    ("fp8_plane_offset_from_exact_mean",
     "b[i * R + r] = lse[i * R + r] - zo_dot(refs + (int64_t)r * d, mq + (i * R + r) * d, d);",
     "b[i * R + r] = lse[i * R + r] - zo_dot(refs + (int64_t)r * d, m + (i * R + r) * d, d);"),
    ("fp4_plane_offset_sign", "b[i * R + r] = lse[i * R + r] - zo_dot(refs + (int64_t)r * d, stored, d);",
     "b[i * R + r] = lse[i * R + r] + zo_dot(refs + (int64_t)r * d, stored, d);"),
    ("attention_one_head", "const double* qh = q + (int64_t)h * d;\n        double mx = -INFINITY;\n        for (int64_t i = 0; i < nS; ++i) {",
     "const double* qh = q;\n        double mx = -INFINITY;\n        for (int64_t i = 0; i < nS; ++i) {"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    with open(oracle._SRC, encoding="utf-8") as f:
        src = f.read()
    assert old in src, f"mutation site for {name} not found"
    path = tmp_path / "zha_oracle_mutant.c"
    path.write_text(src.replace(old, new, 1), encoding="utf-8")
    so = str(tmp_path / f"lib_{name}.so")
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", so, str(path), "-lm"])
    prev = oracle.use_library(so)
    caught = None
    try:
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError) as e:  # a pin rejecting the output
                caught = f"{pin.__name__}: {str(e)[:80]}"
                break
    finally:
        oracle.restore_library(prev)
    assert caught, f"planted mistake {name} passed every pin"
    print(f"{name} caught by {caught}")
    assert os.path.exists(so)
