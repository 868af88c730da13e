"""The whole-output comparison helper on the CPU: it reports agreement for
the oracle's own rows rounded to bf16, and catches a planted error and an
unwritten (NaN) element, with the (b, h, row) of the worst element."""
import math

import numpy as np
import torch

import full_parity
import oracle
from sparse_causal_attention_band_amd import inputs


def _case():
    q, k, v = inputs.random_qkv(2, 4, 2, 200, 64, torch.bfloat16, seed=3)
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
    want = oracle.attn_fwd(qf, kf, vf, 37, 0, 1 / math.sqrt(64))
    G = 2

    def want_of(bh):
        b, h = bh
        return oracle.attn_fwd(qf[b:b + 1, h:h + 1], kf[b:b + 1, h // G:h // G + 1], vf[b:b + 1, h // G:h // G + 1],
                               37, 0, 1 / math.sqrt(64))[0, 0]

    keys = [(b, h) for b in range(2) for h in range(4)]
    return want, want_of, keys


def test_rounded_oracle_passes():
    want, want_of, keys = _case()
    got = torch.from_numpy(want).to(torch.bfloat16).float().numpy()
    st = full_parity.compare_heads(keys, lambda bh: got[bh], want_of)
    assert st.count == want.size and st.over == 0 and st.nonfinite == 0
    assert 0 < st.max_err <= 2.0 ** -7 and st.mean_err < 1e-3
    full_parity.assert_bf16(st, "rounded oracle")


def test_planted_error_and_nan_are_caught():
    want, want_of, keys = _case()
    got = want.astype(np.float32).copy()
    got[1, 3, 150, 7] += 0.05
    st = full_parity.compare_heads(keys, lambda bh: got[bh], want_of)
    assert st.over == 1 and st.worst == (1, 3, 150)
    got[0, 2, 10, 0] = np.nan
    st = full_parity.compare_heads(keys, lambda bh: got[bh], want_of)
    assert st.nonfinite == 1 and st.worst == (0, 2, 10)
    try:
        full_parity.assert_bf16(st, "nan")
    except AssertionError:
        pass
    else:
        raise AssertionError("a NaN output must fail")


def test_tolerance_helpers():
    """The bf16 bounds: flat 1.5e-2 below |x| = 4, half ulp plus the
    arithmetic share from 4 on; the rounding mean is 0 for values bf16
    holds exactly and equals the known rounding error otherwise."""
    from tolerances import BF16_ARITH, bf16_element_bound, bf16_mean_bound, bf16_rounding_mean

    b = bf16_element_bound(np.array([0.0, 1.0, -3.99, 4.0, -7.9, 8.0]))
    assert np.allclose(b, [1.5e-2, 1.5e-2, 1.5e-2, BF16_ARITH + 2 ** -6, BF16_ARITH + 2 ** -6, BF16_ARITH + 2 ** -5])
    exact = np.array([1.0, -0.5, 3.0, 1 + 2 ** -7])
    assert bf16_rounding_mean(exact) == 0.0
    # 1 + 2^-9 is a quarter ulp above 1: rounds down by 2^-9
    assert bf16_rounding_mean(np.array([1 + 2 ** -9])) == 2 ** -9
    assert bf16_mean_bound(exact) == 1e-3
