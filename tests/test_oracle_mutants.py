"""Plant plausible mistakes in copies of the oracle (on the CPU) and show
that the pin suite catches every one of them.

Each mutant is oracle.c with one textual change (or one changed compiler
flag), built into a temporary library; the real oracle is never modified.
A mutant that passes every pin would mean the pins cannot tell that
mistake from the definition.
"""
import os
import shutil

import pytest

import oracle
import pins

ORACLE_DIR = os.path.dirname(oracle.__file__)

COUNT_LOOP = ("    for (int64_t j = 0; j < n; ++j)\n"
              "      if (within(form, p, d, norms, i, j, eps2)) ++c;\n"
              "    count[i] = (int32_t)c;")
GRAPH_TEST = "if (within(form, p, d, norms, i, j, eps2)) tmp[c++] = (int32_t)j;"

MUTANTS = {
    # comparison at the radius made strict
    "strict_radius": [("<= eps2", "< eps2")],
    # a point no longer counts itself
    "self_excluded": [(COUNT_LOOP, COUNT_LOOP.replace(
        "if (within", "if (j != i && within"))],
    # core test made strict
    "core_strict": [("count[i] >= min_pts", "count[i] > min_pts")],
    # radius not squared
    "eps_not_squared": [("float e2 = eps * eps;", "float e2 = eps;")],
    # last dimension dropped from the distance
    "dropped_dim": [("for (int32_t k = 0; k < d; ++k) {",
                     "for (int32_t k = 0; k + 1 < d; ++k) {")],
    # sign error in the difference
    "wrong_sign": [("float t = a[k] - b[k];", "float t = a[k] + b[k];")],
    # dimensions summed in reverse order
    "reversed_sum": [("for (int32_t k = 0; k < d; ++k) {",
                      "for (int32_t k = d - 1; k >= 0; --k) {")],
    # row stride forgotten (transposed operand indexing)
    "bad_stride": [("const float* b = p + j * (int64_t)d;", "const float* b = p + j;")],
    # clusters merged through non-core points
    "merge_through_border": [("          if (!core[j]) continue;\n", "")],
    # border point takes its highest-index core neighbour
    "border_last_core": [("        bmin[i] = (int32_t)c;\n        break;\n",
                          "        bmin[i] = (int32_t)c;\n")],
    # label is the union-find root (smallest core) instead of the smallest member
    "label_is_root": [("labels[i] = first[r];", "labels[i] = r;")],
    # noise labelled 0 instead of -1
    "noise_zero": [("else { labels[i] = -1; continue; }",
                    "else { labels[i] = 0; continue; }")],
    # relabelled noise becomes cluster 0
    "relabel_noise_zero": [("out[i] = l < 0 ? -1 : id[l];",
                            "out[i] = l < 0 ? 0 : id[l];")],
    # graph rows leave out the point itself
    "graph_no_self": [(GRAPH_TEST, GRAPH_TEST.replace("if (within", "if (j != i && within"))],
    # graph rows scanned in descending order
    "graph_descending": [("        for (int64_t j = 0; j < n; ++j)\n          " + GRAPH_TEST,
                          "        for (int64_t j = n - 1; j >= 0; --j)\n          " + GRAPH_TEST)],
    # graph radius made strict (only in the graph)
    "graph_strict": [(GRAPH_TEST, "if (within(form, p, d, norms, i, j, eps2) && "
                                  "oracle_d2(p + i * (int64_t)d, p + j * (int64_t)d, d) != eps2) "
                                  "tmp[c++] = (int32_t)j;")],
    # graph offsets shifted by one row
    "graph_offsets": [("row_ptr[i + 1] = row_ptr[i] + len[i];",
                       "row_ptr[i + 1] = row_ptr[i] + (i + 1 < n ? len[i + 1] : len[0]);")],
    # hoisted-norm form: the goal point's coordinates not doubled
    "expanded_not_doubled": [("float inner = (2.0f * a[0]) * b[0];", "float inner = a[0] * b[0];"),
                             ("float q = (2.0f * a[k]) * b[k];", "float q = a[k] * b[k];")],
    # hoisted-norm form: the inner sum added instead of subtracted
    "expanded_plus": [("return s - inner;", "return s + inner;")],
    # hoisted-norm form: one norm used twice
    "expanded_one_norm": [("float s = ta + pb;", "float s = ta + ta;")],
    # hoisted-norm form: inner products summed in descending dimension order
    "expanded_inner_reversed": [(
        "float inner = (2.0f * a[0]) * b[0];\n  for (int32_t k = 1; k < d; ++k) {",
        "float inner = (2.0f * a[d - 1]) * b[d - 1];\n  for (int32_t k = d - 2; k >= 0; --k) {")],
    # hoisted-norm form: (T - inner) + P instead of (T + P) - inner
    "expanded_regrouped": [("float s = ta + pb;\n  return s - inner;",
                            "float s = ta - inner;\n  return s + pb;")],
    # hoisted-norm form: norms summed from the last dimension
    "expanded_norm_reversed": [(
        "float s = a[0] * a[0];\n  for (int32_t k = 1; k < d; ++k) {\n    float q = a[k] * a[k];",
        "float s = a[d - 1] * a[d - 1];\n  for (int32_t k = d - 2; k >= 0; --k) {\n    float q = a[k] * a[k];")],
    # the border step always uses the direct form
    "expanded_border_direct": [("if (core[c] && within(form, p, d, norms, i, c, eps2)) {",
                                "if (core[c] && within(ORACLE_FORM_DIRECT, p, d, norms, i, c, eps2)) {")],
    # the graph always uses the direct form
    "expanded_graph_direct": [(GRAPH_TEST, GRAPH_TEST.replace("within(form,", "within(ORACLE_FORM_DIRECT,"))],
    # the form ignored in the merge of core pairs
    "expanded_merge_direct": [("          if (within(form, p, d, norms, i, j, eps2))\n            if (edge_push",
                               "          if (within(ORACLE_FORM_DIRECT, p, d, norms, i, j, eps2))\n            if (edge_push")],
    # border points treated as noise
    "no_borders": [("else if (bmin[i] >= 0) r = uf_find(parent, bmin[i]);",
                    "else if (0) r = 0;")],
}

FLAG_MUTANTS = {
    # s + t*t fused into one rounding
    "fused_multiply_add": ["-ffp-contract=fast", "-mfma"],
}


def build_mutant(tmp_path, name):
    shutil.copy(os.path.join(ORACLE_DIR, "oracle.h"), tmp_path / "oracle.h")
    with open(os.path.join(ORACLE_DIR, "oracle.c")) as f:
        src = f.read()
    for old, new in MUTANTS.get(name, []):
        assert src.count(old) >= 1, (name, old)
        src = src.replace(old, new)
    path = tmp_path / "oracle.c"
    path.write_text(src)
    lib = oracle.build(force=True, src=str(path), out=str(tmp_path / "lib.so"),
                       extra=FLAG_MUTANTS.get(name))
    return oracle.Oracle(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS) + sorted(FLAG_MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    o = build_mutant(tmp_path, name)
    caught = None
    for check in pins.ALL_CHECKS:
        try:
            check(o)
        except Exception as exc:  # AssertionError, or an error status
            caught = (check.__name__, type(exc).__name__)
            break
    assert caught is not None, f"mutant {name} passed every pin"
