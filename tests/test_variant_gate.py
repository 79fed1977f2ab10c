"""The variant-agreement gate of the GPU tests, checked on the CPU.

assert_variants_agree must pass two bf16 roundings of the same exact output that
differ only by fp32-sized perturbations, and must fail when one side drops or
doubles a key (a plausible split/pack bookkeeping mistake), which moves every
output of a row by about P_j * |V_j - O|.
"""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import oracle
from _parity import assert_variants_agree, bf16_steps


def _bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


def _case(seed=5):
    B, S, Hq, Hk, d = 2, 96, 4, 2, 64
    q = gi.random_bf16(seed, (B, S, Hq, d)).double().numpy()
    k = gi.random_bf16(seed + 1, (B, S, Hk, d)).double().numpy()
    v = gi.random_bf16(seed + 2, (B, S, Hk, d)).double().numpy()
    return q, k, v


def test_bf16_steps_counts_representable_values():
    a = torch.tensor([1.0, 1.0, -1.0, 0.0, -0.0, 2.0 ** -20], dtype=torch.bfloat16)
    b = torch.tensor([1.0, 1.0078125, -1.0078125, -0.0, 2.0 ** -133, 2.0 ** -20 * 1.015625],
                     dtype=torch.bfloat16)
    assert bf16_steps(a, b).tolist() == [0, 1, 1, 0, 1, 2]


def test_gate_passes_fp32_reassociation():
    q, k, v = _case()
    O, L = oracle.attention_fp64(q, k, v, False, 0.125)
    rng = np.random.default_rng(0)
    Oa = _bf16(O)
    Ob = _bf16(O * (1 + 2.0 ** -22 * rng.standard_normal(O.shape)))
    st = assert_variants_agree(Oa, torch.from_numpy(L), Ob, torch.from_numpy(L + 1e-6), float(np.abs(v).max()),
                               tag="reassociation")
    assert st["n_1step"] > 0  # some values straddle a rounding boundary
    assert st["frac_gt_1e-3"] <= 1e-3


@pytest.mark.parametrize("mistake", ["dropped key", "doubled key"])
def test_gate_catches_key_bookkeeping(mistake):
    q, k, v = _case()
    O, L = oracle.attention_fp64(q, k, v, False, 0.125)
    j = 37
    if mistake == "dropped key":
        k2, v2 = np.delete(k, j, axis=1), np.delete(v, j, axis=1)
    else:
        k2, v2 = np.insert(k, j, k[:, j], axis=1), np.insert(v, j, v[:, j], axis=1)
    O2, L2 = oracle.attention_fp64(q, k2, v2, False, 0.125)
    with pytest.raises(AssertionError):
        assert_variants_agree(_bf16(O), torch.from_numpy(L), _bf16(O2), torch.from_numpy(L2), float(np.abs(v).max()),
                              tag=mistake)
