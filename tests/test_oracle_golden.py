"""The oracle against hand-worked examples (tests/golden/*.txt).

Each fixture's expected LSE, O and gradients are derived on paper, in the
fixture's own comments, from the definitions of page "llm.istanbul --
10_backward_attention.wgsl" (header comment and kernel attention_backward).
None of them comes from the oracle or from the GPU path.
"""
import numpy as np
import pytest

from tests.golden_io import golden_files, load_golden

FILES = golden_files()


def test_there_is_a_fixture():
    assert FILES


@pytest.mark.parametrize("path", FILES, ids=lambda p: p.rsplit("/", 1)[-1])
def test_oracle_fp64_matches_hand_worked(oracle_mod, path):
    g = load_golden(path)
    O, LSE = oracle_mod.attn_fwd_f64(g["Q"], g["K"], g["V"], g["seg"], g["scale"])
    np.testing.assert_allclose(LSE, g["LSE"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(O, g["O"], rtol=0, atol=1e-13)
    # row term D = sum_j P*dP, and D = dO.O: both routes reach the same values
    for O_arg in (None, g["O"]):
        dQ, dK, dV = oracle_mod.attn_bwd_f64(g["Q"], g["K"], g["V"], g["dO"], g["LSE"],
                                             g["seg"], g["scale"], O=O_arg)
        for name, got in (("dQ", dQ), ("dK", dK), ("dV", dV)):
            np.testing.assert_allclose(got, g[name], rtol=0, atol=1e-13, err_msg=name)


@pytest.mark.parametrize("path", FILES, ids=lambda p: p.rsplit("/", 1)[-1])
def test_oracle_fp32_accumulates_onto_hand_worked(oracle_mod, path):
    g = load_golden(path)
    rng = np.random.default_rng(5)
    init = [rng.standard_normal(g[n].shape).astype(np.float32) for n in ("dQ", "dK", "dV")]
    out = oracle_mod.attn_bwd(g["Q"], g["K"], g["V"], g["dO"], g["LSE"], g["seg"], g["scale"],
                              *[x.copy() for x in init])
    for name, got, i0 in zip(("dQ", "dK", "dV"), out, init):
        np.testing.assert_allclose(got.astype(np.float64) - i0, g[name], rtol=0, atol=2e-6,
                                   err_msg=name)


def test_fixture_reader_pads_without_changing_the_problem(oracle_mod):
    from tests.golden_io import pad_head_dim
    g = pad_head_dim(load_golden(FILES[0]), 16)
    dQ, dK, dV = oracle_mod.attn_bwd_f64(g["Q"], g["K"], g["V"], g["dO"], g["LSE"], g["seg"],
                                         g["scale"])
    for name, got in (("dQ", dQ), ("dK", dK), ("dV", dV)):
        np.testing.assert_allclose(got, g[name], rtol=0, atol=1e-13, err_msg=name)


def golden_fails(oracle):
    """Names of the hand-worked fixtures whose values the given oracle misses."""
    failed = []
    for path in FILES:
        g = load_golden(path)
        with np.errstate(all="ignore"):
            O, LSE = oracle.attn_fwd_f64(g["Q"], g["K"], g["V"], g["seg"], g["scale"])
            got = [LSE, O] + list(oracle.attn_bwd_f64(g["Q"], g["K"], g["V"], g["dO"], g["LSE"],
                                                      g["seg"], g["scale"]))
        want = [g[n] for n in ("LSE", "O", "dQ", "dK", "dV")]
        if not all(np.allclose(a, b, rtol=0, atol=1e-13) for a, b in zip(got, want)):
            failed.append(path)
    return failed


@pytest.mark.parametrize("name", ["none", "drop_D_term", "flip_dS_sign", "drop_scale_in_dS",
                                  "drop_diagonal_in_dKdV", "ignore_doc_mask_in_dKdV",
                                  "wrong_group_map", "dK_uses_dO", "dV_uses_dS", "P_ignores_LSE",
                                  "fwd_drops_max", "dQ_uses_V"])
def test_hand_worked_examples_alone_catch_planted_mistakes(oracle_mod, tmp_path, name):
    """The same planted mistakes as the other pins face (a copy of the oracle's
    C source, edited, built apart): the fixtures by themselves catch each."""
    from tests.test_oracle_mutants import build_mutant
    so = build_mutant(tmp_path, name)
    with oracle_mod._use_library(so):
        failed = golden_fails(oracle_mod)
    if name == "none":
        assert failed == [], failed
    else:
        assert failed, f"the hand-worked examples miss mutant {name}"
