"""Mutation check of the oracle's pins (CPU only).

Each mutant plants one plausible mistake in a copy of ``oracle/kda_oracle.c``
(a dropped term, a wrong sign, a wrong index or operand, a transposed role),
compiles it to a temporary library and runs the pin suite against it.  Every
mutant must be caught by at least one pin; the unmodified source must pass.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

MUTANTS = {
    "drop_decay": ("S[(size_t)i * dv + j] *= a[i];", "(void)a;"),
    "decay_wrong_index": ("*= a[i];", "*= a[j % dk];"),
    "erase_sign": ("(v[j] - u[j])", "(v[j] + u[j])"),
    "drop_erase": ("(v[j] - u[j])", "(v[j] - 0.0 * u[j])"),
    "drop_beta": ("+= beta * k[i] * (v[j] - u[j])", "+= k[i] * (v[j] - u[j])"),
    "beta_squared": ("+= beta * k[i] * (v[j] - u[j])", "+= beta * beta * k[i] * (v[j] - u[j])"),
    "read_with_q": ("u[j] += k[i] *", "u[j] += q[i] *"),
    "readout_with_k": ("o[j] += q[i] *", "o[j] += k[i] *"),
    "write_key_is_query": ("+= beta * k[i] *", "+= beta * q[i] *"),
    "alpha_shifted_channel": ("aa[i] = load_elem(alpha, dtype, row * dk + i);",
                              "aa[i] = load_elem(alpha, dtype, row * dk + (i + 1) % dk);"),
    "beta_from_first_head": ("const double bt = load_elem(beta, dtype, row);",
                             "const double bt = load_elem(beta, dtype, row - h);"),
    "head_stride_ignored": ("const size_t row = ((size_t)b * T + t) * H + h;",
                            "const size_t row = ((size_t)b * T + t) * H + 0 * h;"),
    "time_reversed": ("const size_t row = ((size_t)b * T + t) * H + h;",
                      "const size_t row = ((size_t)b * T + (T - 1 - t)) * H + h;"),
    "readout_before_update": (
        "    /* 3. erase + write: S <- S + beta k (v - u)^T */",
        "    if (o) { for (int j = j0; j < j1; ++j) { o[j] = 0.0; for (int i = 0; i < dk; ++i) "
        "o[j] += q[i] * S[(size_t)i * dv + j]; } o = NULL; }\n"
        "    /* 3. erase + write: S <- S + beta k (v - u)^T */"),
    "decay_after_write": (
        "    if (!cpx) {\n"
        "        for (int i = 0; i < dk; ++i)\n"
        "            for (int j = j0; j < j1; ++j) S[(size_t)i * dv + j] *= a[i];\n"
        "    } else {",
        "    if (!cpx) {\n    } else {"),
}
# decay_after_write removes the first decay and re-inserts it after the write:
_DECAY_AFTER_WRITE_TAIL = (
    "    /* 4. readout: o = S^T q */",
    "    for (int i = 0; i < dk; ++i) for (int j = j0; j < j1; ++j) S[(size_t)i * dv + j] *= a[i];\n"
    "    /* 4. readout: o = S^T q */")

PIN_TESTS = [
    ("hand", lambda: pins.test_hand_derived_two_tokens()),
    ("explicit", lambda: pins.test_explicit_transition_products(3, 2, 32)),
    ("layout", lambda: pins.test_multi_head_layout_matches_single_heads()),
    ("delta", lambda: pins.test_alpha_one_is_the_delta_rule()),
    ("decay", lambda: pins.test_beta_zero_is_pure_decay()),
    ("rotation", lambda: pins.test_d2_reflection_pair_is_rotation(0.3)),
    ("affine", lambda: pins.test_affine_block_transfer()),
]


def _build_variant(src_text, tmpdir, name):
    path = os.path.join(tmpdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src_text)
    out = os.path.join(tmpdir, f"{name}.so")
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", path, "-o", out],
                   check=True, capture_output=True)
    return oracle.load(out)


def _caught(lib, monkeypatch):
    failed = []
    with monkeypatch.context() as m:
        real_fwd, real_dec = oracle.fwd, oracle.decode
        m.setattr(oracle, "fwd", lambda *a, **kw: real_fwd(*a, lib=lib, **kw))
        m.setattr(oracle, "decode", lambda *a, **kw: real_dec(*a, lib=lib, **kw))
        for name, fn in PIN_TESTS:
            try:
                with np.errstate(all="ignore"):
                    fn()
            except AssertionError:
                failed.append(name)
    return failed


@pytest.fixture(scope="module")
def src_text():
    with open(SRC) as f:
        return f.read()


def test_unmodified_source_passes(src_text, monkeypatch, tmp_path):
    lib = _build_variant(src_text, str(tmp_path), "clean")
    assert _caught(lib, monkeypatch) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src_text, monkeypatch, tmp_path):
    old, new = MUTANTS[name]
    assert src_text.count(old) >= 1, f"mutation anchor for {name} not found"
    text = src_text.replace(old, new, 1)
    if name == "decay_after_write":
        text = text.replace(*_DECAY_AFTER_WRITE_TAIL, 1)
    lib = _build_variant(text, str(tmp_path), name)
    caught = _caught(lib, monkeypatch)
    assert caught, f"mutant {name} passed every pin"


# ---- the Gated DeltaNet-2 token code: plausible mistakes, each must fail a GDN-2 pin
import test_oracle_gdn2 as gpins  # noqa: E402

MUTANTS_GDN2 = {
    "gdn2_erase_gate_dropped": ("const double e = eg[i] * k[i];", "const double e = k[i];"),
    "gdn2_write_gate_dropped": ("(wg[j] * v[j] - u[j])", "(v[j] - u[j])"),
    "gdn2_erase_sign": ("(wg[j] * v[j] - u[j])", "(wg[j] * v[j] + u[j])"),
    "gdn2_gates_swapped_sides": ("+= k[i] * (wg[j] * v[j] - u[j]);", "+= eg[i] * k[i] * (v[j] - u[j]);"),
    "gdn2_write_key_is_erase_key": ("+= k[i] * (wg[j] * v[j] - u[j]);", "+= eg[i] * k[i] * (wg[j] * v[j] - u[j]);"),
    "gdn2_decay_dropped": ("    /* 1. decay: S <- D S */\n    for (int i = 0; i < dk; ++i)\n"
                           "        for (int j = j0; j < j1; ++j) S[(size_t)i * dv + j] *= a[i];",
                           "    /* 1. decay: S <- D S */"),
    "gdn2_erase_channel_shifted": ("ee[i] = load_elem(erase, dtype, tok * dk + i);",
                                   "ee[i] = load_elem(erase, dtype, tok * dk + (i + 1) % dk);"),
    "gdn2_write_channel_shifted": ("ww[j] = load_elem(write, dtype, tok * dv + j);",
                                   "ww[j] = load_elem(write, dtype, tok * dv + (j + 1) % dv);"),
    "gdn2_readout_with_k": ("o[j] += q[i] * S[(size_t)i * dv + j];\n    }\n}\n\n/*\n * Gated DeltaNet-2 forward",
                            "o[j] += k[i] * S[(size_t)i * dv + j];\n    }\n}\n\n/*\n * Gated DeltaNet-2 forward"),
}

PIN_TESTS_GDN2 = [
    ("hand", lambda: gpins.test_gdn2_hand_derived_two_tokens()),
    ("explicit", lambda: gpins.test_gdn2_explicit_transition_products(3, 2, 32)),
    ("tied_kda", lambda: gpins.test_gdn2_with_tied_gates_is_kda()),
    ("readback", lambda: gpins.test_gdn2_full_erase_reads_back_the_write()),
    ("no_erase", lambda: gpins.test_gdn2_without_erase_is_a_decayed_sum_of_writes()),
]


def _caught_gdn2(lib, monkeypatch):
    failed = []
    with monkeypatch.context() as m:
        real = {n: getattr(oracle, n) for n in ("fwd", "decode", "fwd_gdn2", "decode_gdn2")}
        for n, f in real.items():
            m.setattr(oracle, n, (lambda f: lambda *a, **kw: f(*a, lib=lib, **kw))(f))
        for name, fn in PIN_TESTS_GDN2:
            try:
                with np.errstate(all="ignore"):
                    fn()
            except AssertionError:
                failed.append(name)
    return failed


def test_unmodified_source_passes_gdn2_pins(src_text, monkeypatch, tmp_path):
    lib = _build_variant(src_text, str(tmp_path), "clean_gdn2")
    assert _caught_gdn2(lib, monkeypatch) == []


@pytest.mark.parametrize("name", sorted(MUTANTS_GDN2))
def test_gdn2_mutant_is_caught(name, src_text, monkeypatch, tmp_path):
    old, new = MUTANTS_GDN2[name]
    assert src_text.count(old) == 1, f"mutation anchor for {name} not unique"
    lib = _build_variant(src_text.replace(old, new), str(tmp_path), name)
    assert _caught_gdn2(lib, monkeypatch), f"mutant {name} passed every GDN-2 pin"


# ---- the SFDA rotation-decay code: plausible mistakes, each must fail an SFDA pin
import test_oracle_sfda as spins  # noqa: E402

_ROT = ("                S[(size_t)(2 * p) * dv + j] = lr * x - li * y;\n"
        "                S[(size_t)(2 * p + 1) * dv + j] = li * x + lr * y;")
MUTANTS_SFDA = {
    "sfda_conjugate_rotation": (_ROT, _ROT.replace("lr * x - li * y", "lr * x + li * y")
                                .replace("li * x + lr * y", "-li * x + lr * y")),
    "sfda_real_part_only": (_ROT, _ROT.replace("lr * x - li * y", "lr * x").replace("li * x + lr * y", "lr * y")),
    "sfda_re_im_swapped": ("const double lr = a[2 * p], li = a[2 * p + 1];",
                           "const double lr = a[2 * p + 1], li = a[2 * p];"),
    "sfda_rows_mixed_wrong_way": (_ROT, _ROT.replace("lr * x - li * y", "lr * x - li * x")
                                  .replace("li * x + lr * y", "li * y + lr * y")),
    "sfda_pairs_are_halves": (
        "const double x = S[(size_t)(2 * p) * dv + j], y = S[(size_t)(2 * p + 1) * dv + j];\n" + _ROT,
        "const double x = S[(size_t)(p) * dv + j], y = S[(size_t)(p + dk / 2) * dv + j];\n"
        + _ROT.replace("(2 * p) * dv", "(p) * dv").replace("(2 * p + 1) * dv", "(p + dk / 2) * dv")),
    "sfda_gate_from_next_pair": ("const double lr = a[2 * p], li = a[2 * p + 1];",
                                 "const double lr = a[(2 * p + 2) % dk], li = a[(2 * p + 3) % dk];"),
}

PIN_TESTS_SFDA = [
    ("hand", lambda: spins.test_sfda_hand_derived_two_tokens()),
    ("explicit", lambda: spins.test_sfda_explicit_transition_products(4, 2, 32)),
    ("zero_phase_kda", lambda: spins.test_sfda_with_zero_phases_is_kda_with_paired_decay()),
    ("closed_form", lambda: spins.test_sfda_pure_rotation_decay_closed_form()),
    ("counter", lambda: spins.test_sfda_phase_only_cyclic_counter(5)),
]


def _caught_sfda(lib, monkeypatch):
    failed = []
    with monkeypatch.context() as m:
        real = {n: getattr(oracle, n) for n in ("fwd", "decode", "fwd_sfda", "decode_sfda")}
        for n, f in real.items():
            m.setattr(oracle, n, (lambda f: lambda *a, **kw: f(*a, lib=lib, **kw))(f))
        for name, fn in PIN_TESTS_SFDA:
            try:
                with np.errstate(all="ignore"):
                    fn()
            except AssertionError:
                failed.append(name)
    return failed


def test_unmodified_source_passes_sfda_pins(src_text, monkeypatch, tmp_path):
    lib = _build_variant(src_text, str(tmp_path), "clean_sfda")
    assert _caught_sfda(lib, monkeypatch) == []


@pytest.mark.parametrize("name", sorted(MUTANTS_SFDA))
def test_sfda_mutant_is_caught(name, src_text, monkeypatch, tmp_path):
    old, new = MUTANTS_SFDA[name]
    assert src_text.count(old) == 1, f"mutation anchor for {name} not unique"
    lib = _build_variant(src_text.replace(old, new), str(tmp_path), name)
    assert _caught_sfda(lib, monkeypatch), f"mutant {name} passed every SFDA pin"


# ---- the backward (reverse-mode) code: plausible mistakes, each must fail a backward pin
import test_oracle_bwd as bpins  # noqa: E402

MUTANTS_BWD = {
    "bwd_dk_sign_of_read_term": ("dkt[i] = bt * a - c;", "dkt[i] = bt * a + c;"),
    "bwd_dk_read_term_dropped": ("dkt[i] = bt * a - c;", "dkt[i] = bt * a;"),
    "bwd_erase_adjoint_dropped": ("const double g = G[(size_t)i * dv + j] - kk[i] * dd[j];",
                                  "const double g = G[(size_t)i * dv + j];"),
    "bwd_decay_adjoint_dropped": ("G[(size_t)i * dv + j] = aa[i] * g;", "G[(size_t)i * dv + j] = g;"),
    "bwd_dalpha_from_decayed_state": ("a += g * Sprev[(size_t)i * dv + j];", "a += g * Sp[(size_t)i * dv + j];"),
    "bwd_dq_before_update": ("a += (Sp[(size_t)i * dv + j] + bt * kk[i] * del[j]) * dOt[j];",
                             "a += Sp[(size_t)i * dv + j] * dOt[j];"),
    "bwd_dbeta_with_v": ("db += dd[j] * del[j];", "db += dd[j] * vv[j];"),
    "bwd_dv_without_beta": ("        dd[j] *= bt;\n", ""),
    "bwd_stale_block_history": ("for (int t = t0; t < t1 - 1; ++t) {", "for (int t = t0; t < t1 - 2; ++t) {"),
}

PIN_TESTS_BWD = [
    ("secants_short", lambda: bpins.test_bwd_exact_secants(5)),
    ("secants_blocks", lambda: bpins.test_bwd_exact_secants(150)),
    ("key_fd", lambda: bpins.test_bwd_key_central_differences()),
    ("scalar_hand", lambda: bpins.test_bwd_scalar_token_by_hand()),
]


def _caught_bwd(lib, monkeypatch):
    """The forward stays the clean library (the pins measure the backward against it)."""
    failed = []
    with monkeypatch.context() as m:
        real = oracle.bwd
        m.setattr(oracle, "bwd", lambda *a, **kw: real(*a, lib=lib, **kw))
        for name, fn in PIN_TESTS_BWD:
            try:
                with np.errstate(all="ignore"):
                    fn()
            except AssertionError:
                failed.append(name)
    return failed


def test_unmodified_source_passes_bwd_pins(src_text, monkeypatch, tmp_path):
    lib = _build_variant(src_text, str(tmp_path), "clean_bwd")
    assert _caught_bwd(lib, monkeypatch) == []


@pytest.mark.parametrize("name", sorted(MUTANTS_BWD))
def test_bwd_mutant_is_caught(name, src_text, monkeypatch, tmp_path):
    old, new = MUTANTS_BWD[name]
    assert src_text.count(old) == 1, f"mutation anchor for {name} not unique"
    lib = _build_variant(src_text.replace(old, new), str(tmp_path), name)
    assert _caught_bwd(lib, monkeypatch), f"mutant {name} passed every backward pin"


MUTANTS_BWD_GDN2 = {
    "gdn2_bwd_dk_read_side_dropped": ("dkg[i] = w_side + bb[i] * de;", "dkg[i] = w_side;"),
    "gdn2_bwd_dwrite_with_w": ("dwg[j] = vv[j] * dd[j];", "dwg[j] = ww[j] * dd[j];"),
    "gdn2_bwd_derase_without_k": ("dbg[i] = kk[i] * de;", "dbg[i] = de;"),
    "gdn2_bwd_erase_adjoint_dropped": ("const double g = G[(size_t)i * dv + j] - ee[i] * dd[j];",
                                       "const double g = G[(size_t)i * dv + j];"),
    "gdn2_bwd_read_through_key": ("ee[i] = bb[i] * kk[i];", "ee[i] = kk[i];"),
}

PIN_TESTS_BWD_GDN2 = [
    ("secants_short", lambda: bpins.test_gdn2_bwd_exact_secants(5)),
    ("secants_blocks", lambda: bpins.test_gdn2_bwd_exact_secants(150)),
    ("key_fd", lambda: bpins.test_gdn2_bwd_key_central_differences()),
    ("scalar_hand", lambda: bpins.test_gdn2_bwd_scalar_token_by_hand()),
]


def _caught_bwd_gdn2(lib, monkeypatch):
    """The forward stays the clean library (the pins measure the backward against it)."""
    failed = []
    with monkeypatch.context() as m:
        real = oracle.bwd_gdn2
        m.setattr(oracle, "bwd_gdn2", lambda *a, **kw: real(*a, lib=lib, **kw))
        for name, fn in PIN_TESTS_BWD_GDN2:
            try:
                with np.errstate(all="ignore"):
                    fn()
            except AssertionError:
                failed.append(name)
    return failed


def test_unmodified_source_passes_gdn2_bwd_pins(src_text, monkeypatch, tmp_path):
    lib = _build_variant(src_text, str(tmp_path), "clean_bwd_gdn2")
    assert _caught_bwd_gdn2(lib, monkeypatch) == []


@pytest.mark.parametrize("name", sorted(MUTANTS_BWD_GDN2))
def test_gdn2_bwd_mutant_is_caught(name, src_text, monkeypatch, tmp_path):
    old, new = MUTANTS_BWD_GDN2[name]
    assert src_text.count(old) == 1, f"mutation anchor for {name} not unique"
    lib = _build_variant(src_text.replace(old, new), str(tmp_path), name)
    assert _caught_bwd_gdn2(lib, monkeypatch), f"mutant {name} passed every GDN-2 backward pin"


# ---- SFDA backward: planted mistakes in the complex-gate branch of the reverse sweep
MUTANTS_BWD_SFDA = {
    "sfda_bwd_dim_sign": ("dim += g1 * s0 - g0 * s1;", "dim += g0 * s1 - g1 * s0;"),
    "sfda_bwd_dre_drops_odd_row": ("dre += g0 * s0 + g1 * s1;", "dre += g0 * s0;"),
    "sfda_bwd_adjoint_not_transposed": ("G[(size_t)i0 * dv + j] = lr * g0 + li * g1;",
                                        "G[(size_t)i0 * dv + j] = lr * g0 - li * g1;"),
    "sfda_bwd_recompute_real_part_only": ("y0[j] = lr * x0[j] - li * x1[j];", "y0[j] = lr * x0[j];"),
    "sfda_bwd_block_rebuild_real_gates": (
        "kda_token(nx, dk, dv, 0, dv, qq, kk, vv, aa, load_elem(beta, dtype, row), u, NULL, cpx);",
        "kda_token(nx, dk, dv, 0, dv, qq, kk, vv, aa, load_elem(beta, dtype, row), u, NULL, 0);"),
}

PIN_TESTS_BWD_SFDA = [
    ("secants_short", lambda: bpins.test_sfda_bwd_exact_secants(5)),
    ("secants_blocks", lambda: bpins.test_sfda_bwd_exact_secants(150)),
    ("key_fd", lambda: bpins.test_sfda_bwd_key_central_differences()),
    ("closed_form", lambda: bpins.test_sfda_bwd_pure_rotation_closed_form()),
]


def _caught_bwd_sfda(lib, monkeypatch):
    """The forward stays the clean library (the pins measure the backward against it)."""
    failed = []
    with monkeypatch.context() as m:
        real = oracle.bwd_sfda
        m.setattr(oracle, "bwd_sfda", lambda *a, **kw: real(*a, lib=lib, **kw))
        for name, fn in PIN_TESTS_BWD_SFDA:
            try:
                with np.errstate(all="ignore"):
                    fn()
            except AssertionError:
                failed.append(name)
    return failed


def test_unmodified_source_passes_sfda_bwd_pins(src_text, monkeypatch, tmp_path):
    lib = _build_variant(src_text, str(tmp_path), "clean_bwd_sfda")
    assert _caught_bwd_sfda(lib, monkeypatch) == []


@pytest.mark.parametrize("name", sorted(MUTANTS_BWD_SFDA))
def test_sfda_bwd_mutant_is_caught(name, src_text, monkeypatch, tmp_path):
    old, new = MUTANTS_BWD_SFDA[name]
    assert src_text.count(old) == 1, f"mutation anchor for {name} not unique"
    lib = _build_variant(src_text.replace(old, new), str(tmp_path), name)
    assert _caught_bwd_sfda(lib, monkeypatch), f"mutant {name} passed every SFDA backward pin"
