"""The logit softcap in its binding regime, on the GPU against the fp64 oracle.

The cap is cap * tanh(z / cap) on the LM head's output z (yelogs.com launch write-up,
architecture answer: logit softcap; cap 15).  With N(0, 0.02) weights every natural logit
has |z / cap| below about 0.2, where the kernels' tanh takes its odd-series branch, so two
stresses drive it through its exponential branch and into saturation:

1. A smaller cap, 15 / 2^7 and 15 / 2^10 (exact in fp32): z is unchanged, z / cap reaches
   tens to hundreds.  The error of a capped logit is sech^2(z / cap) times the error of z, so
   the model's own bars hold unchanged: 1e-4 (fp32), 3e-2 (bf16), and |logit| <= cap.
2. The LM head scaled by s = 2^7 and 2^10 with the cap left at 15.  A power of two keeps the
   bf16 weights exact and scales every partial sum of the head's product exactly, on the GPU
   and in the oracle alike, so the head's argument is exactly s times the unscaled one on
   both sides.  With t = logit / cap, the cap's slope is sech^2(z / cap) = 1 - t^2 (at most
   1), so an unscaled logit's error err_1 is (1 - t_1^2) times its argument's error, and the
   scaled logit's error at most s times that argument error, plus the rounding of the fp32
   tanh and of the fp32 outputs: the bound checked, logit by logit, is
   2e-5 + 1.01 s (|err_1| + 1e-7) / (1 - t_1^2).  Saturated logits must equal +-cap.

Each stress runs through every kernel that applies the cap: the prefill product's epilogue
(rows x positions), the decode LM head with at most 32 rows, and the decode products for
more rows (40)."""

from dataclasses import replace

import numpy as np
import pytest

from dense_decoder_only_bf16_amd.inputs import TINY, Shape, make_tokens, make_weights
from oracle import OracleModel

from gpu_helpers import decode, gpu_model, prefill, report

pytestmark = pytest.mark.gpu

SMALL_BF16 = Shape("small-bf16", n_layer=2, d_model=256, n_head=2, head_dim=128, d_ff=1024,
                   vocab=1000, dtype="bf16", max_seq=320)
TOL = {"f32": 1e-4, "bf16": 3e-2}
T = 24


def _run(shape, w, B):
    """GPU logits of a prefill of B rows x T tokens and of one decode step after it, and
    the oracle's for the same positions (one oracle prefill of T + 1 tokens: prefill and
    decode logits agree by causality)."""
    toks = make_tokens(shape.vocab, B, T + 1, seed=40 + B)
    gm = gpu_model(shape, w)
    kv, got_pre = prefill(gm, toks[:, :T], T + 1)
    got_dec = decode(gm, kv, toks[:, T])
    kv.close()
    gm.close()
    want, _ = OracleModel(shape, w).prefill(toks)
    got = np.concatenate([got_pre, got_dec[:, None]], axis=1)  # [B, T + 1, V]
    return got.astype(np.float64), want


def _base(dtype):
    return (TINY, 0) if dtype == "f32" else (SMALL_BF16, 3)


@pytest.mark.parametrize("B", [8, 40])
@pytest.mark.parametrize("k", [7, 10])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_softcap_binds_with_a_smaller_cap(dtype, k, B):
    shape0, seed = _base(dtype)
    shape = replace(shape0, softcap=15.0 / 2 ** k)
    cap32 = float(np.float32(shape.softcap))
    w = make_weights(shape, seed=seed)
    got, want = _run(shape, w, B)
    err, agree = report(f"{dtype} cap 15/2^{k} B={B}", got, want)
    ratio = np.abs(want) / shape.softcap
    print(f"  |logit|/cap: median {np.median(ratio):.3f}, share above 0.99: "
          f"{np.mean(ratio > 0.99):.3f}", flush=True)
    assert np.mean(ratio > 0.5) > 0.5  # the cap binds for most logits
    assert np.all(np.abs(got) <= cap32)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("B", [8, 40])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_softcap_binds_with_a_scaled_head(dtype, B):
    shape, seed = _base(dtype)
    w = make_weights(shape, seed=seed)
    got1, want1 = _run(shape, w, B)
    err1, _ = report(f"{dtype} head x1 B={B}", got1, want1)
    assert err1 <= TOL[dtype]
    t1 = want1 / shape.softcap
    assert np.max(np.abs(t1)) < 0.5  # unscaled logits sit where the cap is nearly linear
    for k in (7, 10):
        s = 2.0 ** k
        ws = dict(w)
        ws["lm_head"] = (w["lm_head"] * np.float32(s)).astype(np.float32)  # exact: power of 2
        got, want = _run(shape, ws, B)
        report(f"{dtype} head x2^{k} B={B}", got, want)
        bound = 2e-5 + 1.01 * s * (np.abs(got1 - want1) + 1e-7) / (1 - t1 * t1)
        excess = np.abs(got - want) - bound
        print(f"  worst logit vs its bound: {np.max(excess):.3e} (<= 0 passes); "
              f"saturated share {np.mean(np.abs(want) > 0.999 * shape.softcap):.3f}", flush=True)
        assert np.all(excess <= 0)
        assert np.all(np.abs(got) <= shape.softcap)
        sat = np.abs(want) >= shape.softcap * (1 - 1e-9)
        assert np.all(np.abs(got[sat]) == np.float32(shape.softcap))
