"""The whole-output property checker used at full sizes must accept a correct
attention output and reject plausible mistakes.

The correct output comes from the oracle on a small causal GQA case (CPU,
float64, rounded to float32 like the library's outputs); each mistake is
planted in a copy of it on the CPU."""

import numpy as np
import pytest

import oracle
from gpu_util import whole_output_properties

torch = pytest.importorskip("torch")


def _case():
    rng = np.random.default_rng(11)
    S, H, HKV, D = 40, 4, 2, 16
    q = rng.standard_normal((S, H, D)).astype(np.float32)
    k = rng.standard_normal((S, HKV, D)).astype(np.float32)
    v = rng.standard_normal((S, HKV, D)).astype(np.float32)
    qb, kb, vb = (torch.from_numpy(x).bfloat16() for x in (q, k, v))
    q64, k64, v64 = (t.double().numpy() for t in (qb, kb, vb))
    scale = 1.0 / np.sqrt(D)
    o, lse = oracle.attention_ref(q64[None], k64[None], v64[None], np.arange(S), np.arange(S),
                                  causal=True, scale=scale)
    return (torch.from_numpy(o[0]).float(), torch.from_numpy(lse[0]).float(), qb, kb, vb,
            torch.arange(S), H // HKV, scale)


def _check(o, lse, q, k, v, pos, group, scale):
    whole_output_properties(o, lse, q, k, v, pos, 0, group, scale, "case")


def test_accepts_the_oracle_output():
    _check(*_case())


@pytest.mark.parametrize("plant", ["nan_o", "inf_lse", "o_out_of_range", "lse_too_low",
                                   "lse_too_high"])
def test_rejects_planted_mistakes(plant):
    o, lse, q, k, v, pos, group, scale = _case()
    o, lse = o.clone(), lse.clone()
    if plant == "nan_o":
        o[7, 1, 3] = float("nan")
    elif plant == "inf_lse":
        lse[5, 0] = float("-inf")
    elif plant == "o_out_of_range":
        o[20, 2, 0] = v[:, 1, 0].float().max() + 0.5       # head 2 reads kv head 1
    elif plant == "lse_too_low":
        lse[30, 3] = -10.0                                  # below every score the row sees
    elif plant == "lse_too_high":
        lse[0, 0] += 50.0                                   # row 0 sees one key: lse = its score
    with pytest.raises(AssertionError):
        _check(o, lse, q, k, v, pos, group, scale)
