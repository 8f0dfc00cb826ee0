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
