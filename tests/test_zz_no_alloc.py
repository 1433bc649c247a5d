"""The allocation-free decode step (nc_decode_step_static) against nc_decode_step.

Both run the same kernels on the same inputs; only the workspace differs (the library's
static device array instead of the kv object's memory), so their logits must agree bit for
bit, and both must match the fp64 oracle within the model's bar.  Two calls in a row through
the static array, the second with a smaller batch (40 rows, the wide split-K projections,
then 8 rows), show that each call clears what must start at zero (attention ready flags,
split-K arrival counters) whatever the last call left."""

from dataclasses import replace

import numpy as np
import pytest

from dense_decoder_only_bf16_amd import nc
from dense_decoder_only_bf16_amd.inputs import TINY, Shape, make_extras, make_lens, make_tokens, make_weights
from oracle import OracleModel

from gpu_helpers import gpu_model, prefill, torch_mod

pytestmark = pytest.mark.gpu

SMALL = Shape("small-bf16", n_layer=2, d_model=256, n_head=2, head_dim=128, d_ff=1024,
              vocab=1000, dtype="bf16", max_seq=320)
TOL = {"bf16": 3e-2, "f32": 1e-4}


def _pair(gm, toks, T, lens, max_seq):
    """Two caches with the same contents: prefill T tokens, then truncate to lens."""
    kv_s, _ = prefill(gm, toks[:, :T], max_seq, logits=False)
    kv_r, _ = prefill(gm, toks[:, :T], max_seq, logits=False)
    kv_s.set_lens(lens)
    kv_r.set_lens(lens)
    return kv_s, kv_r


@pytest.mark.parametrize("shape,seed", [(SMALL, 3), (TINY, 0)], ids=["bf16", "f32"])
def test_static_decode_matches_decode_step(shape, seed):
    torch = torch_mod()
    w = make_weights(shape, seed=seed)
    gm = gpu_model(shape, w)
    orc = OracleModel(shape, w)
    T, steps = 40, 2
    for B in (40, 8):  # two calls in a row, the second smaller
        toks = make_tokens(shape.vocab, B, T + steps, seed=60 + B)
        lens = make_lens(B, 1, T, seed=70 + B)
        kv_s, kv_r = _pair(gm, toks, T, lens, 64)
        got_s, got_r = [], []
        for s in range(steps):
            tok = torch.from_numpy(np.ascontiguousarray(toks[:, T + s])).cuda()
            out_s = torch.empty((B, shape.vocab), device="cuda", dtype=torch.float32)
            out_r = torch.empty_like(out_s)
            kv_s.decode_static(tok, out_s)
            kv_r.decode(tok, out_r)
            torch.cuda.synchronize()
            got_s.append(out_s.cpu().numpy())
            got_r.append(out_r.cpu().numpy())
        for s in range(steps):
            assert np.array_equal(got_s[s], got_r[s]), (B, s)
        assert np.array_equal(kv_s.lens(), lens + steps)
        want = np.stack([orc.prefill(np.concatenate([toks[b, :lens[b]], toks[b, T:T + steps]])[None],
                                     logits_at=np.arange(lens[b], lens[b] + steps))[0][0]
                         for b in range(B)])  # [B, steps, V]
        err = float(np.max(np.abs(np.stack(got_s, 1) - want)))
        print(f"[static decode {shape.dtype} B={B}] max_abs={err:.3e}", flush=True)
        assert err <= TOL[shape.dtype]
        kv_s.close()
        kv_r.close()
    gm.close()


def test_static_decode_errors():
    torch = torch_mod()
    # a workspace beyond the static array: 128 rows over 32768 positions need more
    big = replace(SMALL, max_seq=32768)
    gm = gpu_model(big, make_weights(big, seed=3))
    kv = gm.new_kv(128, 32768)
    tok = torch.zeros(128, dtype=torch.int32, device="cuda")
    out = torch.empty((128, big.vocab), device="cuda", dtype=torch.float32)
    with pytest.raises(nc.NcError) as e:
        kv.decode_static(tok, out)
    assert e.value.code == nc.NC_ERR_CAPACITY and "static array" in str(e.value)
    assert np.array_equal(kv.lens(), np.zeros(128, dtype=np.int32))  # no state change
    kv.close()
    gm.close()
    # the later version's blocks are not taken
    w = make_weights(SMALL, seed=3)
    gm = gpu_model(SMALL, w, extras=make_extras(SMALL, seed=5))
    kv = gm.new_kv(2, 16)
    with pytest.raises(nc.NcError) as e:
        kv.decode_static(torch.zeros(2, dtype=torch.int32, device="cuda"),
                         torch.empty((2, SMALL.vocab), device="cuda", dtype=torch.float32))
    assert e.value.code == nc.NC_ERR_UNSUPPORTED
    kv.close()
    gm.close()
