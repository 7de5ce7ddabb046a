"""Planted mistakes in the oracle must each be caught by some pin.

Every mutant is a copy of ``oracle/tw_oracle.c`` with one plausible mistake
(a dropped term, a wrong comparison, a wrong index, a transposed operand, a
swapped matrix, a wrong order), compiled into its own library on the CPU.
The pins of ``oracle_pins.py`` run against it and at least one must fail;
otherwise the pins would not notice that kind of mistake in the real oracle.
"""
import os

import pytest

import oracle
import oracle_pins

with open(oracle.SOURCE) as _f:
    _SRC = _f.read()

# (name, exact text in tw_oracle.c, replacement) or (name, [text, repl], [text, repl], ...)
# Every mutant keeps all memory accesses in bounds.
MUTANTS = [
    ("dot drops last term", "for (int k = 0; k < K; ++k)\n        s += a[k] * b[k];",
     "for (int k = 0; k < K - 1; ++k)\n        s += a[k] * b[k];"),
    ("zero counted active", "if (g > 0.0) {\n                    if (n < C)",
     "if (g >= 0.0) {\n                    if (n < C)"),
    ("relu keeps negatives", "return v > 0.0 ? v : 0.0;", "return v;"),
    ("tile-local index", "idx[tile * C + n] = j;", "idx[tile * C + n] = j - t * T;"),
    ("count clipped to capacity", "cnt[tile] = n;", "cnt[tile] = n < C ? n : C;"),
    ("overflow at capacity", "if (n > C)\n                over = 1;",
     "if (n >= C)\n                over = 1;"),
    ("routing list descending", "for (int m = 0; m < M; ++m) {\n        if (flag[m]) {",
     "for (int m = M - 1; m >= 0; --m) {\n        if (flag[m]) {"),
    ("count clipped to R_max", "*ovf_count = r;", "*ovf_count = r < R_max ? r : R_max;"),
    ("up uses gate weights",
     "const double u = dot(xm, wu_t + (size_t)j * K, K);\n        const double h = u * g;\n        const double *wdj",
     "const double u = dot(xm, wg_t + (size_t)j * K, K);\n        const double h = u * g;\n        const double *wdj"),
    ("h adds instead of multiplies",
     "const double h = u * g;\n        const double *wdj = wd + (size_t)j * K;\n        for (int k = 0; k < K; ++k)\n            ym[k] += h * wdj[k];\n    }\n}",
     "const double h = u + g;\n        const double *wdj = wd + (size_t)j * K;\n        for (int k = 0; k < K; ++k)\n            ym[k] += h * wdj[k];\n    }\n}"),
    ("down weights read transposed",
     "for (int k = 0; k < K; ++k)\n            ym[k] += h * wdj[k];\n    }\n}",
     "for (int k = 0; k < K; ++k)\n            ym[k] += h * wd[(size_t)k * N + j];\n    }\n}"),
    ("gate row stride", "z[(size_t)m * N + j] = dot(x + (size_t)m * K, wg_t + (size_t)j * K, K);",
     "z[(size_t)m * N + j] = dot(x + (size_t)m, wg_t + (size_t)j * K, K);"),
    ("sparse drops last slot", "for (int s = 0; s < cnt[tile]; ++s) {\n                const int j",
     "for (int s = 0; s + 1 < cnt[tile]; ++s) {\n                const int j"),
    ("sparse ignores gate value", "const double g = val[tile * C + s];",
     "const double g = 1.0;"),
    # overflow rows evaluated from their truncated packing instead of the
    # dense backup (the slot loop is clamped so the mutant stays in bounds)
    ("no dense backup", ["if (over) {\n            dense_row", "if (0) {\n            dense_row"],
     ["for (int s = 0; s < cnt[tile]; ++s) {\n                const int j",
      "for (int s = 0; s < cnt[tile] && s < C; ++s) {\n                const int j"]),
    ("sparse sign flip", "const double h = u * g;\n                const double *wdj",
     "const double h = -u * g;\n                const double *wdj"),
    # hybrid storage (the copy loop is clamped where a mutant could read past
    # a tile's slots)
    ("hybrid ignores tile overflow",
     ["route[m] = (uint8_t)(over || nnz > P);", "route[m] = (uint8_t)(nnz > P);"],
     ["for (int s = 0; s < cnt[tile]; ++s) {\n                hy_idx",
      "for (int s = 0; s < cnt[tile] && s < C; ++s) {\n                hy_idx"]),
    ("hybrid heavy at capacity", "route[m] = (uint8_t)(over || nnz > P);",
     "route[m] = (uint8_t)(over || nnz >= P);"),
    ("hybrid count clipped", "hy_cnt[m] = nnz;", "hy_cnt[m] = nnz < P ? nnz : P;"),
    ("hybrid slots restart per tile",
     "hy_idx[(size_t)m * P + n] = idx[tile * C + s];\n                hy_val[(size_t)m * P + n]",
     "hy_idx[(size_t)m * P + s] = idx[tile * C + s];\n                hy_val[(size_t)m * P + s]"),
    ("backup list descending", "for (int m = 0; m < M; ++m) {\n        if (route[m]) {",
     "for (int m = M - 1; m >= 0; --m) {\n        if (route[m]) {"),
    ("backup count clipped", "*bk_count = r;", "*bk_count = r < R_max ? r : R_max;"),
    ("hybrid up uses gate weights", "const double u = dot(xm, wu_t + (size_t)hy_idx[e] * K, K);",
     "const double u = dot(xm, wg_t + (size_t)hy_idx[e] * K, K);"),
    ("hybrid product ignores gate", "hy_h[e] = u * hy_g[e];", "hy_h[e] = u;"),
    ("backup gate without ReLU",
     "const double g = relu(dot(xm, wg_t + (size_t)j * K, K));\n            const double u = dot(xm, wu_t + (size_t)j * K, K);\n            bk_g[e] = g;",
     "const double g = dot(xm, wg_t + (size_t)j * K, K);\n            const double u = dot(xm, wu_t + (size_t)j * K, K);\n            bk_g[e] = g;"),
    ("backup reads x by slot", "const double *xm = x + (size_t)bk_rows[r] * K;",
     "const double *xm = x + (size_t)r * K;"),
    ("hybrid down drops last entry",
     "for (int s = 0; s < hy_cnt[m]; ++s) {\n            const size_t e = (size_t)m * P + s;\n            const double *wdj",
     "for (int s = 0; s + 1 < hy_cnt[m]; ++s) {\n            const size_t e = (size_t)m * P + s;\n            const double *wdj"),
    ("hybrid down ignores h", "ym[k] += hy_h[e] * wdj[k];", "ym[k] += wdj[k];"),
    ("backup output to slot row", "double *ym = y + (size_t)bk_rows[r] * K;",
     "double *ym = y + (size_t)r * K;"),
    # backward over hybrid storage
    ("gate gradient misses L1", "hy_dz[e] = dh * hy_u[e] + l1;", "hy_dz[e] = dh * hy_u[e];"),
    ("L1 on inactive backup entries", "bk_dz[e] = bk_g[e] > 0.0 ? dh * bk_u[e] + l1 : 0.0;",
     "bk_dz[e] = dh * bk_u[e] + l1;"),
    ("up gradient scaled by u", "hy_du[e] = dh * hy_g[e];", "hy_du[e] = dh * hy_u[e];"),
    ("dh from up weights", "const double dh = dot(dym, wd + (size_t)hy_idx[e] * K, K);",
     "const double dh = dot(dym, wu_t + (size_t)hy_idx[e] * K, K);"),
    ("dx drops the gate term", "dxm[k] += hy_du[e] * wu[k] + hy_dz[e] * wg[k];",
     "dxm[k] += hy_du[e] * wu[k];"),
    ("dx swaps the weights", "dxm[k] += bk_du[e] * wu[k] + bk_dz[e] * wg[k];",
     "dxm[k] += bk_du[e] * wg[k] + bk_dz[e] * wu[k];"),
    ("down weight gradient from x", "dwd[(size_t)j * K + k] += hy_h[e] * dym[k];",
     "dwd[(size_t)j * K + k] += hy_h[e] * xm[k];"),
    ("up weight gradient from dz", "dwu_t[(size_t)j * K + k] += hy_du[e] * xm[k];",
     "dwu_t[(size_t)j * K + k] += hy_dz[e] * xm[k];"),
    ("backup rows left out of weight gradients", "} else if (r < nbk && bk_rows[r] == m) {",
     "} else if (0) {"),
    ("backup dy by slot", "const double *dym = dy + (size_t)bk_rows[r] * K;",
     "const double *dym = dy + (size_t)r * K;"),
]


def _edits(m):
    if isinstance(m[1], str):
        return [(m[1], m[2])]
    return [tuple(e) for e in m[1:]]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mutant):
    name = mutant[0]
    text = _SRC
    for orig, repl in _edits(mutant):
        assert text.count(orig) == 1, f"mutation anchor for '{name}' not unique in tw_oracle.c"
        text = text.replace(orig, repl)
    src = tmp_path / "mutant.c"
    src.write_text(text)
    lib = oracle.build(str(src), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake '{name}'"
