"""Plant plausible mistakes in copies of oracle.c; every one must fail some pin.

Each mutant is a textual edit of the oracle source (a dropped term, a wrong
index or sign, a swapped operand, a reversed tie-break, a missing step),
compiled with gcc to a temporary library and run against the pins in
oracle_pins.py.  All edits keep memory accesses in bounds.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "dot drops the last channel": ("for (int d = 0; d < ORC_D; ++d)\n        s +=",
                                   "for (int d = 0; d < ORC_D - 1; ++d)\n        s +="),
    "dot subtracts": ("s += bf16_value(qrow[d]) * bf16_value(krow[d]);",
                      "s -= bf16_value(qrow[d]) * bf16_value(krow[d]);"),
    "dot reads channel d+1 of the key": ("bf16_value(krow[d]);", "bf16_value(krow[(d + 1) % ORC_D]);"),
    "slot index off by one": ("int64_t slot = j % ORC_PAGE;", "int64_t slot = (j + 1) % ORC_PAGE;"),
    "page index ignores the page table": (
        "int64_t page = c->page_table[(int64_t)b * c->max_pages + j / ORC_PAGE];",
        "int64_t page = (int64_t)b * c->max_pages + j / ORC_PAGE;"),
    "kv head by modulo instead of group": ("g = h / G;\n        const uint16_t *qrow",
                                           "g = h % num_kv_heads;\n        const uint16_t *qrow"),
    "attend kv head by modulo": ("attend_one(&c, b, h / G, q + bh * ORC_D, idx",
                                 "attend_one(&c, b, h % num_kv_heads, q + bh * ORC_D, idx"),
    "tie-break prefers higher index": ("return (a->j > b->j) - (a->j < b->j);",
                                       "return (a->j < b->j) - (a->j > b->j);"),
    "selection keeps lowest scores": ("if (a->s > b->s) return -1;\n    if (a->s < b->s) return 1;",
                                      "if (a->s < b->s) return -1;\n    if (a->s > b->s) return 1;"),
    "output not sorted by index": ("qsort(row, (size_t)kk, sizeof *row, by_index);", ""),
    "k-th score off by one": ("kth_out[bh] = kk > 0 ? all[kk - 1].s", "kth_out[bh] = kk > 0 ? all[kk > 1 ? kk - 2 : 0].s"),
    "softmax scale dropped": ("double w = exp(scale * dot_q_k(", "double w = exp(dot_q_k("),
    "no normalisation": ("out[d] = z > 0.0 ? acc[d] / z : 0.0;", "out[d] = acc[d];"),
    "values read from the key cache": ("const uint16_t *vrow = row_of(c->v,", "const uint16_t *vrow = row_of(c->k,"),
    "weights not exponentiated": ("double w = exp(scale * dot_q_k(qrow, row_of(c->k, c, b, g, sel[i])) - m);",
                                  "double w = 1.0 + scale * dot_q_k(qrow, row_of(c->k, c, b, g, sel[i])) - m;"),
    "dense skips the last token": ("for (int64_t j = 0; j < n; ++j) all[j] = (int32_t)j;\n        attend_one(&c, b, h / G, q + bh * ORC_D, all, n,",
                                   "for (int64_t j = 0; j < n; ++j) all[j] = (int32_t)j;\n        attend_one(&c, b, h / G, q + bh * ORC_D, all, n - 1,"),
    "quest min and max swapped": ("if (v < mn[d]) mn[d] = v;", "if (v > mn[d]) mn[d] = v;"),
    "quest bound takes the smaller product": ("u += lo > hi ? lo : hi;", "u += lo < hi ? lo : hi;"),
    "quest summary reads one row past the sequence": (
        "for (int64_t j = p * ORC_PAGE; j < n && j < (p + 1) * ORC_PAGE; ++j) {",
        "for (int64_t j = p * ORC_PAGE; j <= n && j < (p + 1) * ORC_PAGE; ++j) {"),
    "quest forces the first page instead of the current one": ("prow[taken++] = (int32_t)(P - 1);",
                                                               "prow[taken++] = 0;"),
    "quest tokens past the sequence": (
        "j < n && j < ((int64_t)prow[i] + 1) * ORC_PAGE; ++j)", "j < ((int64_t)prow[i] + 1) * ORC_PAGE; ++j)"),
    "quest bound drops the last channel": ("for (int d = 0; d < ORC_D; ++d) {\n                double qd",
                                           "for (int d = 0; d < ORC_D - 1; ++d) {\n                double qd"),
    "label key channel not mapped": ("bf16_value(qrow[ch[i]]) * bf16_value(krow[ch[i]]);",
                                     "bf16_value(qrow[ch[i]]) * bf16_value(krow[i]);"),
    "label skips the first channel": ("for (int i = 0; i < r; ++i)\n                s += bf16_value(qrow[ch[i]])",
                                      "for (int i = 1; i < r; ++i)\n                s += bf16_value(qrow[ch[i]])"),
    "k not clamped to k_max": ("if (kk > k_max) kk = k_max;\n        if (kk < 0) kk = 0;",
                               "if (kk > k_max) kk = k_max - 1;\n        if (kk < 0) kk = 0;"),
    "sample rank off by one": ("tok = residual[r];", "tok = residual[(r + 1) % M];"),
    "sample draws from the whole context": ("if (!kept[j]) residual[M++] = (int32_t)j;",
                                            "residual[M++] = (int32_t)j;"),
    "sample weight dropped": ("weight_out[bh] = s > 0 ? (double)M / (double)s : 0.0;",
                              "weight_out[bh] = s > 0 ? 1.0 : 0.0;"),
    "sample weight over s + 1 draws": ("weight_out[bh] = s > 0 ? (double)M / (double)s : 0.0;",
                                       "weight_out[bh] = s > 0 ? (double)M / (double)(s + 1) : 0.0;"),
    "sample weight on the kept entries": ("double wt = i < k_max ? 1.0 : weight[bh];",
                                          "double wt = i < k_max ? weight[bh] : 1.0;"),
    "sample weight left out of the denominator": ("            z += p;\n            for (int d = 0; d < ORC_D; ++d)\n                acc[d] += p * bf16_value(vrow[d]);",
                                                  "            z += p / wt;\n            for (int d = 0; d < ORC_D; ++d)\n                acc[d] += p * bf16_value(vrow[d]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name!r} not unique in oracle.c"
    with tempfile.TemporaryDirectory() as tmp:
        c_path = os.path.join(tmp, "mutant.c")
        so_path = os.path.join(tmp, "libmutant.so")
        with open(c_path, "w") as f:
            f.write(src.replace(old, new))
        subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", c_path, "-o", so_path, "-lm"],
                       check=True)
        lib = oracle.load_variant(so_path)
        failed = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(lib)
            except AssertionError:
                failed.append(pin.__name__)
        assert failed, f"no pin caught the planted mistake: {name}"
