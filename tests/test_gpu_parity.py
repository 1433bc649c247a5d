"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars: fp32 model max |logit error| <= 1e-4; bf16 models max |logit error| <= 3e-2 and
greedy-argmax agreement >= 99% over the checked positions.  Decode is teacher-forced:
the GPU is fed the oracle's greedy tokens (tiny) or seeded tokens (bf16), so logits are
comparable at every step."""

from dataclasses import replace

import numpy as np
import pytest

from dense_decoder_only_bf16_amd import nc
from dense_decoder_only_bf16_amd.inputs import (TINY, Shape, make_extras, make_tokens, make_weights,
                                                make_lens)
from oracle import OracleModel

from gpu_helpers import (agreement, assert_flips_are_near_ties, decode, gpu_model, prefill,
                         report, torch_mod)

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 3e-2
AGREE = 0.99

# bf16 model small enough for the oracle to check every output, with ragged sizes:
# T not a multiple of any tile, vocab not a multiple of 128.
SMALL_BF16 = Shape("small-bf16", n_layer=2, d_model=256, n_head=2, head_dim=128, d_ff=1024,
                   vocab=1000, dtype="bf16", max_seq=320)


@pytest.fixture(scope="module")
def tiny():
    w = make_weights(TINY, seed=0)
    return w, OracleModel(TINY, w), gpu_model(TINY, w)


def test_tiny_prefill_and_greedy_decode(tiny):
    w, orc, gm = tiny
    prompt = make_tokens(TINY.vocab, 1, 64, seed=1)
    want_pre, _ = orc.prefill(prompt)
    toks, want_steps = orc.greedy(prompt, 16, max_seq=80)
    kv, got_pre = prefill(gm, prompt, 80)
    err, _ = report("tiny prefill", got_pre, want_pre)
    assert err <= F32_TOL
    # greedy continuation on the GPU reproduces the oracle's tokens
    assert np.array_equal(np.argmax(got_pre[:, -1], -1), toks[:, 0])
    for s in range(16):
        got = decode(gm, kv, toks[:, s])
        err, _ = report(f"tiny decode {s}", got, want_steps[:, s])
        assert err <= F32_TOL
        if s + 1 < 16:
            assert np.array_equal(np.argmax(got, -1), toks[:, s + 1])
    assert np.array_equal(kv.lens(), [80])
    kv.close()


def test_tiny_cache_contents(tiny):
    torch = torch_mod()
    w, orc, gm = tiny
    prompt = make_tokens(TINY.vocab, 1, 64, seed=1)
    _, cache = orc.prefill(prompt, max_seq=80)
    kv, _ = prefill(gm, prompt, 80, logits=False)
    for layer in range(TINY.n_layer):
        k = torch.empty((1, 80, 64), device="cuda", dtype=torch.float32)
        v = torch.empty_like(k)
        kv.export(layer, k, v)
        torch.cuda.synchronize()
        k, v = k.cpu().numpy(), v.cpu().numpy()
        assert np.max(np.abs(k[0, :64] - cache["k"][layer, 0, :64, 0])) < 1e-5
        assert np.max(np.abs(v[0, :64] - cache["v"][layer, 0, :64, 0])) < 1e-5
    kv.close()


@pytest.fixture(scope="module")
def small():
    w = make_weights(SMALL_BF16, seed=3)
    return w, OracleModel(SMALL_BF16, w), gpu_model(SMALL_BF16, w)


def test_bf16_small_prefill_ragged(small):
    w, orc, gm = small
    toks = make_tokens(SMALL_BF16.vocab, 3, 200, seed=4)
    want, _ = orc.prefill(toks)
    kv, got = prefill(gm, toks, 320)
    err, agr = report("small bf16 prefill", got, want)
    assert err <= BF16_TOL and agr >= AGREE
    kv.close()


def test_bf16_small_decode_teacher_forced(small):
    w, orc, gm = small
    toks = make_tokens(SMALL_BF16.vocab, 3, 216, seed=5)
    want, _ = orc.prefill(toks)
    kv, _ = prefill(gm, toks[:, :200], 320, logits=False)
    got = np.stack([decode(gm, kv, toks[:, 200 + s]) for s in range(16)], axis=1)
    err, agr = report("small bf16 decode", got, want[:, 200:216])
    assert err <= BF16_TOL and agr >= AGREE
    kv.close()


@pytest.mark.parametrize("B", [40, 100])
def test_bf16_small_decode_many_rows(small, B):
    """Decode with more than 32 rows (the wide, split-K projection path and its reduce
    kernel; B not a multiple of 32), rows at different context lengths, 3 teacher-forced
    steps through the captured graph; every row is checked against the oracle."""
    w, orc, gm = small
    T, steps = 40, 3
    toks = make_tokens(SMALL_BF16.vocab, B, T + steps, seed=20 + B)
    lens = make_lens(B, 1, T, seed=30 + B)
    kv, _ = prefill(gm, toks[:, :T], 64, logits=False)
    kv.set_lens(lens)
    got = np.stack([decode(gm, kv, toks[:, T + s]) for s in range(steps)], axis=1)  # [B, steps, V]
    assert np.array_equal(kv.lens(), lens + steps)
    want = np.empty_like(got, dtype=np.float64)
    for b in range(B):
        seq = np.concatenate([toks[b, :lens[b]], toks[b, T:T + steps]])[None]
        want[b] = orc.prefill(seq, logits_at=np.arange(lens[b], lens[b] + steps))[0][0]
    err, agr = report(f"small bf16 decode B={B}", got, want)
    assert err <= BF16_TOL and agr >= AGREE
    kv.close()


def test_bf16_small_truncated_rows(small):
    # prefill, shrink rows to different lengths, decode: equals shorter prefills
    w, orc, gm = small
    toks = make_tokens(SMALL_BF16.vocab, 3, 300, seed=6)
    lens = np.array([1, 77, 300], dtype=np.int32)
    kv, _ = prefill(gm, toks, 320, logits=False)
    kv.set_lens(lens)
    nxt = make_tokens(SMALL_BF16.vocab, 1, 3, seed=7)[0]
    got = decode(gm, kv, nxt)
    for b in range(3):
        seq = np.concatenate([toks[b, :lens[b]], nxt[b:b + 1]])[None]
        ref, _ = orc.prefill(seq, logits_at=[lens[b]])
        err = np.max(np.abs(got[b] - ref[0, 0]))
        assert err <= BF16_TOL, (b, err)
        assert np.argmax(got[b]) == np.argmax(ref[0, 0])
    assert np.array_equal(kv.lens(), lens + 1)
    kv.close()


def test_prefill_single_token_and_batch_independence(small):
    w, orc, gm = small
    toks = make_tokens(SMALL_BF16.vocab, 4, 1, seed=8)
    want, _ = orc.prefill(toks)
    kv, got = prefill(gm, toks, 8)
    err, agr = report("small bf16 T=1", got, want)
    assert err <= BF16_TOL
    kv.close()
    # row b of a batched prefill equals a batch-1 prefill of row b, bitwise
    toks = make_tokens(SMALL_BF16.vocab, 3, 70, seed=9)
    kv, full = prefill(gm, toks, 80)
    kv.close()
    for b in range(3):
        kv1, one = prefill(gm, toks[b:b + 1], 80)
        kv1.close()
        assert np.array_equal(one[0], full[b])


def test_determinism(small):
    w, orc, gm = small
    toks = make_tokens(SMALL_BF16.vocab, 2, 150, seed=10)
    kv1, a = prefill(gm, toks, 160)
    kv2, b = prefill(gm, toks, 160)
    assert np.array_equal(a, b)
    nxt = make_tokens(SMALL_BF16.vocab, 1, 2, seed=11)[0]
    assert np.array_equal(decode(gm, kv1, nxt), decode(gm, kv2, nxt))
    kv1.close()
    kv2.close()


def test_error_paths_on_gpu(small):
    torch = torch_mod()
    w, orc, gm = small
    toks = make_tokens(SMALL_BF16.vocab, 2, 8, seed=12)
    kv, _ = prefill(gm, toks, 9, logits=False)
    t = torch.zeros(2, dtype=torch.int32, device="cuda")
    out = torch.empty((2, SMALL_BF16.vocab), device="cuda", dtype=torch.float32)
    with pytest.raises(nc.NcError) as e:  # an appended chunk past max_seq (8 + 4 > 9)
        kv.prefill(torch.zeros((2, 4), dtype=torch.int32, device="cuda"), None)
    assert e.value.code == nc.NC_ERR_CAPACITY
    kv.decode(t, out)  # fills position 8 (the last)
    with pytest.raises(nc.NcError) as e:
        kv.decode(t, out)
    assert e.value.code == nc.NC_ERR_CAPACITY
    assert np.array_equal(kv.lens(), [9, 9])  # unchanged by the failed call
    t3 = torch.zeros(3, dtype=torch.int32, device="cuda")
    out3 = torch.empty((3, SMALL_BF16.vocab), device="cuda", dtype=torch.float32)
    with pytest.raises(nc.NcError) as e:  # the library's check: B differs from the cache's
        nc.nc_decode_step(gm.handle, t3, 3, kv.handle, out3)
    assert e.value.code == nc.NC_ERR_INVALID_ARG and "batch" in str(e.value)
    # the binding's checks: buffers too small, wrong dtype, not contiguous, not on the GPU
    bad = [(t, 3, out3), (t.long(), 2, out), (t, 2, out.double()), (t, 2, out.t()),
           (t.cpu(), 2, out)]
    for tt, bb, oo in bad:
        with pytest.raises(nc.NcError) as e:
            nc.nc_decode_step(gm.handle, tt, bb, kv.handle, oo)
        assert e.value.code == nc.NC_ERR_INVALID_ARG
    with pytest.raises(nc.NcError) as e:
        kv.decode(t, out[:, :10].contiguous())
    assert e.value.code == nc.NC_ERR_INVALID_ARG
    assert np.array_equal(kv.lens(), [9, 9])
    with pytest.raises(nc.NcError) as e:
        kv.set_lens([10, 1])  # grow
    assert e.value.code == nc.NC_ERR_INVALID_ARG
    kv.close()
    with pytest.raises(nc.NcError) as e:
        gm.new_kv(1, SMALL_BF16.max_seq + 1)
    assert e.value.code == nc.NC_ERR_INVALID_ARG


def test_argmax_ties_and_nan():
    torch = torch_mod()
    x = torch.zeros((4, 1000), device="cuda", dtype=torch.float32)
    x[0, 5] = 1.0
    x[0, 7] = 1.0          # tie -> lowest index
    x[1, :] = float("nan")
    x[1, 999] = -3.0       # NaN never wins
    x[2, 123] = float("inf")
    x[3, :] = -1.0         # all equal -> 0
    out = torch.empty(4, dtype=torch.int32, device="cuda")
    nc.nc_argmax(x, 4, 1000, out)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [5, 999, 123, 0]


def test_decode_graph_replays_match_eager(small, monkeypatch):
    """The captured decode graph, replayed step after step with eager work in between,
    gives bitwise the same logits as launching the kernels one by one."""
    torch = torch_mod()
    w, orc, gm = small
    toks = make_tokens(SMALL_BF16.vocab, 3, 140, seed=13)
    kv_g, _ = prefill(gm, toks[:, :130], 160, logits=False)
    monkeypatch.setenv("NC_DECODE_GRAPH", "0")
    kv_e, _ = prefill(gm, toks[:, :130], 160, logits=False)
    monkeypatch.delenv("NC_DECODE_GRAPH")
    tok_buf = torch.zeros(3, dtype=torch.int32, device="cuda")
    out_g = torch.empty((3, SMALL_BF16.vocab), device="cuda", dtype=torch.float32)
    want, _ = orc.prefill(toks)
    for s in range(10):
        tok_buf.copy_(torch.from_numpy(toks[:, 130 + s].astype(np.int32)))
        kv_g.decode(tok_buf, out_g)
        torch.cuda.synchronize()
        got_g = out_g.cpu().numpy()
        got_e = decode(gm, kv_e, toks[:, 130 + s])
        assert np.array_equal(got_g, got_e), s
        assert np.max(np.abs(got_g - want[:, 130 + s])) <= BF16_TOL
    assert np.array_equal(kv_g.lens(), [140, 140, 140])
    kv_g.close()
    kv_e.close()


def test_decode_graph_eviction_without_host_syncs(small, monkeypatch):
    """Eleven decode steps, each with its own (tokens, logits) buffer pair, enqueued back to
    back with no host synchronisation: the cache of captured graphs (eight) evicts its oldest
    while earlier replays may still be queued.  Every step's logits equal the eager ones."""
    torch = torch_mod()
    w, orc, gm = small
    B, T, n = 3, 100, 11
    toks = make_tokens(SMALL_BF16.vocab, B, T + n, seed=19)
    kv_g, _ = prefill(gm, toks[:, :T], 128, logits=False)
    monkeypatch.setenv("NC_DECODE_GRAPH", "0")
    kv_e, _ = prefill(gm, toks[:, :T], 128, logits=False)
    monkeypatch.delenv("NC_DECODE_GRAPH")
    tok_bufs = [torch.from_numpy(np.ascontiguousarray(toks[:, T + s])).cuda() for s in range(n)]
    outs = [torch.empty((B, SMALL_BF16.vocab), device="cuda", dtype=torch.float32) for _ in range(n)]
    torch.cuda.synchronize()
    for s in range(n):
        kv_g.decode(tok_bufs[s], outs[s])
    torch.cuda.synchronize()
    for s in range(n):
        assert np.array_equal(outs[s].cpu().numpy(), decode(gm, kv_e, toks[:, T + s])), s
    assert np.array_equal(kv_g.lens(), [T + n] * B)
    kv_g.close()
    kv_e.close()


@pytest.mark.parametrize("in_place", [True, False])
def test_decode_greedy_matches_step_then_argmax(small, in_place):
    """nc_decode_greedy (decode step and argmax in one graph) against nc_decode_step then
    nc_argmax on a second cache: the same picks and bitwise the same logits over 12 greedy
    steps (graph replays), the picks fed back; picks written in place or to another buffer."""
    torch = torch_mod()
    w, orc, gm = small
    B = 4
    toks = make_tokens(SMALL_BF16.vocab, B, 120, seed=17)
    kv_a, _ = prefill(gm, toks, 160, logits=False)
    kv_b, _ = prefill(gm, toks, 160, logits=False)
    V = SMALL_BF16.vocab
    start = torch.from_numpy(make_tokens(V, 1, B, seed=18)[0]).cuda()
    tok_a, tok_b = start.clone(), start.clone()
    nxt_a = tok_a if in_place else torch.empty_like(tok_a)
    log_a = torch.empty((B, V), device="cuda", dtype=torch.float32)
    log_b = torch.empty_like(log_a)
    for s in range(12):
        kv_a.decode_greedy(tok_a, log_a, nxt_a)
        kv_b.decode(tok_b, log_b)
        nc.nc_argmax(log_b, B, V, tok_b)
        torch.cuda.synchronize()
        assert torch.equal(log_a, log_b), s
        assert torch.equal(nxt_a, tok_b), s
        if not in_place:
            tok_a.copy_(nxt_a)
    assert np.array_equal(kv_a.lens(), [132] * B)
    with pytest.raises(nc.NcError):
        nc.nc_decode_greedy(gm.handle, tok_a, B, kv_a.handle, log_a, None)
    kv_a.close()
    kv_b.close()


def test_kernel_timing_counts_launches(small):
    """Timing mode brackets every decode projection (4 per layer + LM head) and every
    prefill projection (4 per layer + LM head) with events and reports the algorithmic
    bytes and flops of those launches; decode stays correct while timed (eager launches)."""
    torch = torch_mod()
    w, orc, gm = small
    s = SMALL_BF16
    toks = make_tokens(s.vocab, 2, 40, seed=14)
    nc.nc_timing_enable(nc.NC_KC_PREFILL_GEMM)
    kv, _ = prefill(gm, toks[:, :32], 64)
    launches, ms, byts, flops = nc.nc_timing_read()
    assert launches == 4 * s.n_layer + 1 and ms > 0
    M = 2 * 32
    want_flops = s.n_layer * 2 * M * s.d_model * ((s.n_head + 2) * s.head_dim + s.d_model + 2 * s.d_ff)
    want_flops += 2 * M * s.d_model * s.vocab
    assert abs(flops - want_flops) / want_flops < 1e-9
    nc.nc_timing_enable(nc.NC_KC_DECODE_GEMM)
    tok_buf = torch.zeros(2, dtype=torch.int32, device="cuda")
    out = torch.empty((2, s.vocab), device="cuda", dtype=torch.float32)
    for step in range(3):
        tok_buf.copy_(torch.from_numpy(toks[:, 32 + step].astype(np.int32)))
        kv.decode(tok_buf, out)
        launches, ms, byts, flops = nc.nc_timing_read()
        # per layer: QKV (with its finish in the epilogue at 32 rows or fewer), O, FC,
        # PROJ; then the LM head
        assert launches == (step + 1) * (4 * s.n_layer + 1)
        assert ms > 0 and byts > 0
    want = orc.prefill(toks[:, :35], logits_at=[34])[0][:, 0]
    assert np.max(np.abs(out.cpu().numpy() - want)) <= BF16_TOL  # timed graph still correct
    nc.nc_timing_enable(nc.NC_KC_NONE)
    kv.close()


# head_dim 64 in bf16 (the other bf16 models use 128), vocab not a multiple of 32
SMALL_HD64 = Shape("small-hd64", n_layer=2, d_model=256, n_head=4, head_dim=64, d_ff=1024,
                   vocab=777, dtype="bf16", max_seq=200)
# the most query heads the decode kernel takes (16: no padded head slots)
WIDE_H16 = Shape("h16", n_layer=1, d_model=2048, n_head=16, head_dim=128, d_ff=2048,
                 vocab=512, dtype="bf16", max_seq=96)
# grouped-query attention: 8 query heads over 2 K/V heads (groups of 4)
GQA_8_2 = Shape("gqa8x2", n_layer=2, d_model=1024, n_head=8, head_dim=128, d_ff=2048,
                vocab=640, dtype="bf16", max_seq=160, n_kv_head=2)
# plain multi-head attention (a K/V head per query head), head_dim 64
MHA_4 = Shape("mha4", n_layer=2, d_model=256, n_head=4, head_dim=64, d_ff=512,
              vocab=300, dtype="bf16", max_seq=100, n_kv_head=4)
# the widest group with more than one K/V head: 32 query heads over 2 (groups of 16)
GQA_32_2 = Shape("gqa32x2", n_layer=1, d_model=2048, n_head=32, head_dim=64, d_ff=1024,
                 vocab=256, dtype="bf16", max_seq=96, n_kv_head=2)


@pytest.mark.parametrize("shape", [SMALL_HD64, WIDE_H16, GQA_8_2, MHA_4, GQA_32_2], ids=lambda s: s.name)
def test_bf16_other_head_shapes(shape):
    """Prefill of ragged rows, then decode from rows truncated to 0 (empty context: the new
    key is the only one), 1 and a middle length, compared with the oracle everywhere."""
    w = make_weights(shape, seed=8)
    orc = OracleModel(shape, w)
    gm = gpu_model(shape, w)
    T = 70
    toks = make_tokens(shape.vocab, 3, T + 4, seed=9)
    want, _ = orc.prefill(toks[:, :T])
    kv, got = prefill(gm, toks[:, :T], shape.max_seq)
    err, agr = report(f"{shape.name} prefill", got, want)
    assert err <= BF16_TOL and agr >= AGREE
    lens = np.array([0, 1, 41], dtype=np.int32)
    kv.set_lens(lens)
    got = np.stack([decode(gm, kv, toks[:, T + s]) for s in range(4)], axis=1)
    for b in range(3):
        seq = np.concatenate([toks[b, :lens[b]], toks[b, T:T + 4]])[None]
        ref, _ = orc.prefill(seq, logits_at=np.arange(lens[b], lens[b] + 4))
        err, agr = report(f"{shape.name} decode row {b} from length {lens[b]}", got[b], ref[0])
        assert err <= BF16_TOL
        srt = np.sort(ref[0], -1)  # any argmax disagreement must be a near tie
        flip = np.argmax(got[b], -1) != np.argmax(ref[0], -1)
        assert not np.any(flip & (srt[:, -1] - srt[:, -2] >= 2 * err))
    assert np.array_equal(kv.lens(), lens + 4)
    kv.close()
    gm.close()


# Prefill products with K >= 2048 whose tiles leave the last round of workgroups at most
# half full run that round's tiles as two K halves, joined through a partial-sum buffer.
# M = 2 x 1100 rows (9 row tiles, ragged), d 2048: O (72 tiles, the plain kernel), PROJ (72,
# K 8192) and the LM head (36) have every tile split; FC's 288 tiles leave 32 tail tiles
# after 256 whole ones (the compensated kernel); QKV (216 tiles, a round over half full) is
# not split.
TAIL = Shape("tail-split", n_layer=1, d_model=2048, n_head=16, head_dim=128, d_ff=8192, vocab=1000,
             dtype="bf16", max_seq=1104)


def test_bf16_prefill_tail_split():
    w = make_weights(TAIL, seed=21)
    orc = OracleModel(TAIL, w)
    gm = gpu_model(TAIL, w)
    toks = make_tokens(TAIL.vocab, 2, 1100, seed=22)
    want, _ = orc.prefill(toks)
    kv, got = prefill(gm, toks, TAIL.max_seq)
    err, agr = report("tail-split prefill", got, want)
    assert err <= BF16_TOL and agr >= AGREE
    kv.close()
    kv, got2 = prefill(gm, toks, TAIL.max_seq)  # the join's counters are left at zero
    assert np.array_equal(got, got2)
    kv.close()
    gm.close()


# fp32 grouped-query model: 4 query heads over 2 K/V heads, checked at the fp32 bar
TINY_GQA = replace(TINY, name="tiny-gqa", d_model=256, n_head=4, n_kv_head=2, d_ff=512)


def test_fp32_gqa_prefill_decode_and_cache():
    """Grouped-query attention in fp32: prefill logits, teacher-forced decode logits and
    every K/V head of the cache against the oracle at the fp32 bar."""
    torch = torch_mod()
    shape = TINY_GQA
    w = make_weights(shape, seed=40)
    orc = OracleModel(shape, w)
    gm = gpu_model(shape, w)
    B, T, steps = 2, 50, 6
    toks = make_tokens(shape.vocab, B, T + steps, seed=41)
    want, cache = orc.prefill(toks, max_seq=shape.max_seq)
    kv, got = prefill(gm, toks[:, :T], shape.max_seq)
    err, _ = report("tiny-gqa prefill", got, want[:, :T])
    assert err <= F32_TOL
    nkv, hd, S = shape.n_kv_head, shape.head_dim, shape.max_seq
    for layer in range(shape.n_layer):
        k = torch.empty((B, nkv, S, hd), device="cuda", dtype=torch.float32)
        v = torch.empty_like(k)
        kv.export(layer, k, v)
        torch.cuda.synchronize()
        k, v = k.cpu().numpy(), v.cpu().numpy()
        # oracle cache: [layer][row][position][K/V head][hd]
        ck = np.transpose(cache["k"][layer, :, :T], (0, 2, 1, 3))
        cv = np.transpose(cache["v"][layer, :, :T], (0, 2, 1, 3))
        assert np.max(np.abs(k[:, :, :T] - ck)) < 1e-5
        assert np.max(np.abs(v[:, :, :T] - cv)) < 1e-5
    got = np.stack([decode(gm, kv, toks[:, T + s]) for s in range(steps)], axis=1)
    err, _ = report("tiny-gqa decode", got, want[:, T:T + steps])
    assert err <= F32_TOL
    kv.close()
    gm.close()


# The narrowest model the library takes: d_model 64 (one 64-wide head), so the QKV, FC and
# LM-head products have K = 64, four 16-deep steps: the prefill GEMMs' short pipeline
# paths (prologue and drain with fewer stages than the ring holds).
NARROW = Shape("narrow", n_layer=2, d_model=64, n_head=1, head_dim=64, d_ff=256, vocab=300,
               dtype="bf16", max_seq=140)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_narrow_model_prefill_and_decode(dtype):
    """K = 64 products end to end: ragged prefill of 3 rows (T = 70), then 4 teacher-forced
    decode steps, against the oracle at the bar of the dtype."""
    shape = replace(NARROW, name=f"narrow-{dtype}", dtype=dtype)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    w = make_weights(shape, seed=50)
    orc = OracleModel(shape, w)
    gm = gpu_model(shape, w)
    B, T, steps = 3, 70, 4
    toks = make_tokens(shape.vocab, B, T + steps, seed=51)
    want, _ = orc.prefill(toks)
    kv, got = prefill(gm, toks[:, :T], shape.max_seq)
    err, agr = report(f"{shape.name} prefill", got, want[:, :T])
    assert err <= tol
    if dtype == "bf16":
        assert agr >= AGREE
    got = np.stack([decode(gm, kv, toks[:, T + s]) for s in range(steps)], axis=1)
    err, _ = report(f"{shape.name} decode", got, want[:, T:T + steps])
    assert err <= tol
    assert_flips_are_near_ties(got, want[:, T:T + steps], err)
    kv.close()
    gm.close()


# MLP width 2880: decode's down-projection (K = 2880, 180 16-deep steps) is split over 3
# workgroups per column tile, 60 steps each (7 or 8 per wave)
TINY_WIDE_MLP = replace(TINY, name="tiny-mlp2880", d_ff=2880)
SMALL_WIDE_MLP = replace(SMALL_BF16, name="small-mlp2880", d_ff=2880)


def test_fp32_split_k_decode():
    """Decode with the down-projection split over workgroups (the last of a tile to finish
    adds the slices), 8 teacher-forced steps at the fp32 bar; the slice counters return to
    zero, so every step (graph replays included) sees the same result as the oracle."""
    shape = TINY_WIDE_MLP
    w = make_weights(shape, seed=44)
    orc = OracleModel(shape, w)
    gm = gpu_model(shape, w)
    B, T, steps = 2, 20, 8
    toks = make_tokens(shape.vocab, B, T + steps, seed=45)
    want, _ = orc.prefill(toks)
    kv, got = prefill(gm, toks[:, :T], shape.max_seq)
    err, _ = report("tiny-mlp2880 prefill", got, want[:, :T])
    assert err <= F32_TOL
    got = np.stack([decode(gm, kv, toks[:, T + s]) for s in range(steps)], axis=1)
    err, _ = report("tiny-mlp2880 decode", got, want[:, T:T + steps])
    assert err <= F32_TOL
    kv.close()
    gm.close()


@pytest.mark.parametrize("B", [1, 32])
def test_bf16_split_k_decode(B):
    """The split down-projection in bf16 at 1 row and at a full 32-row block, 3 steps."""
    shape = SMALL_WIDE_MLP
    w = make_weights(shape, seed=46)
    orc = OracleModel(shape, w)
    gm = gpu_model(shape, w)
    T, steps = 33, 3
    toks = make_tokens(shape.vocab, B, T + steps, seed=47)
    want, _ = orc.prefill(toks, logits_at=np.arange(T, T + steps))
    kv, _ = prefill(gm, toks[:, :T], shape.max_seq)
    got = np.stack([decode(gm, kv, toks[:, T + s]) for s in range(steps)], axis=1)
    err, agr = report(f"small-mlp2880 decode B={B}", got, want)
    assert err <= BF16_TOL
    assert_flips_are_near_ties(got, want, err)
    kv.close()
    gm.close()


@pytest.mark.parametrize("B", [3, 40])
def test_bf16_gqa_decode_many_rows(B):
    """Grouped-query decode at mixed context lengths up to 600 (B = 40: 80 (row, K/V head)
    units, many of them cut between workgroup runs and merged; B = 3: units spread over many
    short runs), 2 teacher-forced steps; every row is checked against the oracle."""
    shape = replace(GQA_8_2, n_layer=1, max_seq=640)
    w = make_weights(shape, seed=42)
    orc = OracleModel(shape, w)
    gm = gpu_model(shape, w)
    T, steps = 600, 2
    toks = make_tokens(shape.vocab, B, T + steps, seed=43 + B)
    lens = make_lens(B, 1, T, seed=44 + B)
    kv, _ = prefill(gm, toks[:, :T], shape.max_seq, logits=False)
    kv.set_lens(lens)
    got = np.stack([decode(gm, kv, toks[:, T + s]) for s in range(steps)], axis=1)
    assert np.array_equal(kv.lens(), lens + steps)
    want = np.empty_like(got, dtype=np.float64)
    for b in range(B):
        seq = np.concatenate([toks[b, :lens[b]], toks[b, T:T + steps]])[None]
        want[b] = orc.prefill(seq, logits_at=np.arange(lens[b], lens[b] + steps))[0][0]
    err, agr = report(f"gqa decode B={B}", got, want)
    assert err <= BF16_TOL  # 2 B positions: each argmax disagreement must be a near tie
    assert_flips_are_near_ties(got, want, err)
    kv.close()
    gm.close()


# ---------------------------------------------------------------- sliding windows ------
def test_fp32_windows_prefill_and_decode():
    """Sliding windows in fp32 (layer 0: 7 keys back, layer 1: the whole context) over a
    prefill that spans several 64-key blocks, then decode steps, at the fp32 bar."""
    shape = replace(TINY, max_seq=160)
    wins = [7, -1]
    w = make_weights(shape, seed=50)
    orc = OracleModel(shape, w, windows=wins)
    gm = gpu_model(shape, w, windows=wins)
    B, T, steps = 2, 150, 6
    toks = make_tokens(shape.vocab, B, T + steps, seed=51)
    want, _ = orc.prefill(toks)
    kv, got = prefill(gm, toks[:, :T], shape.max_seq)
    err, _ = report("tiny windows prefill", got, want[:, :T])
    assert err <= F32_TOL
    got = np.stack([decode(gm, kv, toks[:, T + s]) for s in range(steps)], axis=1)
    err, _ = report("tiny windows decode", got, want[:, T:T + steps])
    assert err <= F32_TOL
    kv.close()
    gm.close()


SSSL = Shape("sssl", n_layer=4, d_model=512, n_head=4, head_dim=128, d_ff=1024, vocab=500,
             dtype="bf16", max_seq=640, n_kv_head=2)


@pytest.mark.parametrize("short", [0, 70, 300])
def test_bf16_window_pattern_prefill(short):
    """Pattern SSSL with short windows of 0 keys back (each query sees itself only), 70
    (not a block multiple) and 300 (longer than a 256-query tile) over a 520-token prefill."""
    wins = nc.layer_windows("SSSL", SSSL.n_layer, short)
    w = make_weights(SSSL, seed=52)
    orc = OracleModel(SSSL, w, windows=wins)
    gm = gpu_model(SSSL, w, windows=wins)
    toks = make_tokens(SSSL.vocab, 2, 520, seed=53)
    want, _ = orc.prefill(toks)
    kv, got = prefill(gm, toks, SSSL.max_seq)
    err, agr = report(f"sssl w={short} prefill", got, want)
    assert err <= BF16_TOL and agr >= AGREE
    kv.close()
    gm.close()


@pytest.mark.parametrize("B", [3, 40])
def test_bf16_window_pattern_decode_many_rows(B):
    """SSSL decode with a 100-key short window at mixed context lengths up to 600: the
    decode attention counts only the blocks the window touches (B = 40: 80 units; B = 3:
    units spread over many short runs); every row is checked."""
    wins = nc.layer_windows("SSSL", SSSL.n_layer, 100)
    w = make_weights(SSSL, seed=54)
    orc = OracleModel(SSSL, w, windows=wins)
    gm = gpu_model(SSSL, w, windows=wins)
    T, steps = 600, 2
    toks = make_tokens(SSSL.vocab, B, T + steps, seed=55 + B)
    lens = make_lens(B, 1, T, seed=56 + B)
    kv, _ = prefill(gm, toks[:, :T], SSSL.max_seq, logits=False)
    kv.set_lens(lens)
    got = np.stack([decode(gm, kv, toks[:, T + s]) for s in range(steps)], axis=1)
    want = np.empty_like(got, dtype=np.float64)
    for b in range(B):
        seq = np.concatenate([toks[b, :lens[b]], toks[b, T:T + steps]])[None]
        want[b] = orc.prefill(seq, logits_at=np.arange(lens[b], lens[b] + steps))[0][0]
    err, agr = report(f"sssl decode B={B}", got, want)
    assert err <= BF16_TOL  # 2 B positions: each argmax disagreement must be a near tie
    assert_flips_are_near_ties(got, want, err)
    kv.close()
    gm.close()


def test_windows_only_change_without_kv():
    w = make_weights(SMALL_BF16, seed=57)
    gm = gpu_model(SMALL_BF16, w)
    kv = gm.new_kv(1, 16)
    with pytest.raises(nc.NcError) as e:
        nc.nc_model_set_windows(gm.handle, [4, -1])
    assert e.value.code == nc.NC_ERR_STATE
    kv.close()
    nc.nc_model_set_windows(gm.handle, [4, -1])
    gm.close()


# ---------------------------------------------------------------- appended prefill -----
def test_fp32_append_chunks_with_windows():
    """A prompt prefilled in three chunks (37, 64 and 1 tokens after the first 48) equals
    one prefill of the whole, with a 20-key window in layer 0, at the fp32 bar; then a
    decode step continues from the appended cache."""
    torch = torch_mod()
    shape = replace(TINY, max_seq=160)
    wins = [20, -1]
    w = make_weights(shape, seed=60)
    orc = OracleModel(shape, w, windows=wins)
    gm = gpu_model(shape, w, windows=wins)
    B = 2
    toks = make_tokens(shape.vocab, B, 151, seed=61)
    want, _ = orc.prefill(toks)
    kv, got0 = prefill(gm, toks[:, :48], shape.max_seq)
    parts = [got0]
    for a, b in ((48, 85), (85, 149), (149, 150)):
        out = torch.empty((B, b - a, shape.vocab), device="cuda", dtype=torch.float32)
        kv.prefill(torch.from_numpy(np.ascontiguousarray(toks[:, a:b])).cuda(), out)
        torch.cuda.synchronize()
        parts.append(out.cpu().numpy())
    assert np.array_equal(kv.lens(), [150, 150])
    err, _ = report("tiny append chunks", np.concatenate(parts, 1), want[:, :150])
    assert err <= F32_TOL
    got = decode(gm, kv, toks[:, 150])
    err, _ = report("tiny decode after append", got, want[:, 150])
    assert err <= F32_TOL
    kv.close()
    gm.close()


def test_bf16_append_at_ragged_lengths():
    """Rows truncated to lengths 0, 1, 77 and 260, then a 300-token chunk appended to all
    of them (queries at different positions per row, two query tiles), then one decode
    step: every row equals the oracle's prefill of its own concatenated sequence."""
    torch = torch_mod()
    shape = replace(SMALL_BF16, max_seq=600)
    w = make_weights(shape, seed=64)
    orc = OracleModel(shape, w)
    gm = gpu_model(shape, w)
    B, T0, T = 4, 260, 300
    toks = make_tokens(shape.vocab, B, T0, seed=62)
    more = make_tokens(shape.vocab, B, T + 1, seed=63)
    lens = np.array([0, 1, 77, 260], dtype=np.int32)
    kv, _ = prefill(gm, toks, 600, logits=False)
    kv.set_lens(lens)
    out = torch.empty((B, T, shape.vocab), device="cuda", dtype=torch.float32)
    kv.prefill(torch.from_numpy(np.ascontiguousarray(more[:, :T])).cuda(), out)
    got = out.cpu().numpy()
    dec = decode(gm, kv, more[:, T])
    assert np.array_equal(kv.lens(), lens + T + 1)
    for b in range(B):
        seq = np.concatenate([toks[b, :lens[b]], more[b]])[None]
        ref, _ = orc.prefill(seq, logits_at=np.arange(lens[b], lens[b] + T + 1))
        err, agr = report(f"small append row {b} from length {lens[b]}", got[b], ref[0, :T])
        assert err <= BF16_TOL and agr >= AGREE
        err = np.max(np.abs(dec[b] - ref[0, T]))
        assert err <= BF16_TOL
    kv.close()
    gm.close()


# ---------------------------------------------------------------- cache row copies -----
def test_copy_rows_bit_exact_and_lengths():
    """Copied rows hold exactly the source's keys and values (every layer and K/V head,
    across caches of different capacity, and within one cache) and take its length."""
    torch = torch_mod()
    shape = replace(TINY_GQA, max_seq=200)
    w = make_weights(shape, seed=70)
    gm = gpu_model(shape, w)
    toks = make_tokens(shape.vocab, 3, 90, seed=71)
    src, _ = prefill(gm, toks, 120, logits=False)
    src.set_lens([90, 17, 64])
    dst = gm.new_kv(5, 200)
    dst.copy_rows_from(src, [1, 0, 2, 0], [4, 0, 1, 3])
    assert np.array_equal(dst.lens(), [90, 64, 0, 90, 17])
    nkv, hd = shape.n_kv_head, shape.head_dim

    def export(kv, rows, cap):
        out = []
        for layer in range(shape.n_layer):
            k = torch.empty((rows, nkv, cap, hd), device="cuda", dtype=torch.float32)
            v = torch.empty_like(k)
            kv.export(layer, k, v)
            torch.cuda.synchronize()
            out.append((k.cpu().numpy(), v.cpu().numpy()))
        return out

    before, copied = export(src, 3, 120), export(dst, 5, 200)
    src.copy_rows_from(src, [0], [1])  # within one cache
    assert np.array_equal(src.lens(), [90, 90, 64])
    after = export(src, 3, 120)
    for layer in range(shape.n_layer):
        (ks, vs), (kd, vd), (ka, va) = before[layer], copied[layer], after[layer]
        for d, s, n in ((4, 1, 17), (0, 0, 90), (1, 2, 64), (3, 0, 90)):
            assert np.array_equal(kd[d, :, :n], ks[s, :, :n]), (layer, d)
            assert np.array_equal(vd[d, :, :n], vs[s, :, :n]), (layer, d)
        assert np.array_equal(ka[1, :, :90], ks[0, :, :90])
        assert np.array_equal(va[1, :, :90], vs[0, :, :90])
        assert np.array_equal(ka[2], ks[2]) and np.array_equal(ka[0], ks[0])  # others untouched
    dst.close()
    src.close()
    gm.close()


def test_copy_rows_then_sample_independently(small):
    """Batch generation: one prompt prefilled once, copied to four rows, each continued
    with its own tokens (decode steps and an appended chunk) against the oracle."""
    torch = torch_mod()
    w, orc, gm = small
    prompt = make_tokens(SMALL_BF16.vocab, 1, 100, seed=72)
    one, _ = prefill(gm, prompt, 101, logits=False)
    many = gm.new_kv(4, 200)
    many.copy_rows_from(one, [0, 0, 0, 0], [3, 0, 2, 1])
    one.close()
    nxt = make_tokens(SMALL_BF16.vocab, 4, 8, seed=73)
    got = [decode(gm, many, nxt[:, s]) for s in range(3)]
    out = torch.empty((4, 5, SMALL_BF16.vocab), device="cuda", dtype=torch.float32)
    many.prefill(torch.from_numpy(np.ascontiguousarray(nxt[:, 3:])).cuda(), out)
    got = np.concatenate([np.stack(got, 1), out.cpu().numpy()], 1)  # [4, 8, V]
    assert np.array_equal(many.lens(), [108] * 4)
    for b in range(4):
        seq = np.concatenate([prompt[0], nxt[b]])[None]
        ref, _ = orc.prefill(seq, logits_at=np.arange(100, 108))
        err, agr = report(f"copied row {b}", got[b], ref[0])
        assert err <= BF16_TOL
        assert_flips_are_near_ties(got[b], ref[0], err)
    many.close()


def test_copy_rows_errors(small):
    w, orc, gm = small
    a = gm.new_kv(3, 50)
    b = gm.new_kv(2, 10)
    toks = make_tokens(SMALL_BF16.vocab, 3, 20, seed=74)
    a.prefill(torch_mod().from_numpy(toks).cuda(), None)
    for dst, src, code in (
        ([0, 0], [1, 2], nc.NC_ERR_INVALID_ARG),   # a destination twice
        ([2], [3], nc.NC_ERR_INVALID_ARG),         # source row out of range
        ([0], [1], nc.NC_ERR_CAPACITY),            # 20 positions into a 10-position cache
    ):
        with pytest.raises(nc.NcError) as e:
            (a if code != nc.NC_ERR_CAPACITY else b).copy_rows_from(a, src, dst)
        assert e.value.code == code
    with pytest.raises(nc.NcError) as e:  # within one cache, a row both read and written
        a.copy_rows_from(a, [0, 1], [1, 2])
    assert e.value.code == nc.NC_ERR_INVALID_ARG
    assert np.array_equal(a.lens(), [20, 20, 20]) and np.array_equal(b.lens(), [0, 0])
    a.close()
    b.close()


# ---------------------------------------------------------------- sampling -------------
def _check_samples(logits, temperature, top_k, u, got, tol=1e-4):
    """Every pick equals the oracle's, or u lies within tol of the boundary between the two
    picks in the oracle's fp64 cumulative distribution; every pick has probability > 0."""
    from oracle import sample
    want = sample(logits, temperature, top_k, u.astype(np.float64))
    z = np.where(np.isnan(logits), -np.inf, logits.astype(np.float64))
    n_diff = 0
    for b in range(z.shape[0]):
        if got[b] == want[b]:
            continue
        n_diff += 1
        row = z[b]
        if 0 < top_k < row.shape[0]:
            kth = np.sort(row)[::-1][top_k - 1]
            row = np.where(row >= kth, row, -np.inf)
        p = np.exp((row - np.max(row)) / temperature)
        cdf = np.cumsum(p) / np.sum(p)
        g = int(got[b])
        assert p[g] > 0, (b, g)
        lo = cdf[g - 1] if g > 0 else 0.0
        assert lo - tol <= u[b] <= cdf[g] + tol, (b, g, int(want[b]), float(u[b]), lo, cdf[g])
    return n_diff


@pytest.mark.parametrize("V", [65536, 1000, 1, 100003])  # 100003: two register tiles
def test_sampling_against_oracle(V):
    torch = torch_mod()
    rng = np.random.default_rng(80 + V)
    B = 64
    logits = (rng.standard_normal((B, V)) * 2.0).astype(np.float32)
    if V > 1:
        logits[:8] = np.round(logits[:8] * 4) / 4  # rows with many ties
        logits[8, ::3] = -np.inf
        logits[9, 1::5] = np.nan
    u = rng.random(B).astype(np.float32)
    u[0], u[1] = 0.0, np.nextafter(np.float32(1), np.float32(0))
    dl = torch.from_numpy(logits).cuda()
    du = torch.from_numpy(u).cuda()
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    diffs = 0
    for temperature in (0.7, 1.0, 1.8):
        for top_k in (0, 1, 7, 50, V):
            nc.nc_sample(dl, B, V, temperature, top_k, du, out)
            got = out.cpu().numpy()
            diffs += _check_samples(logits, temperature, top_k, u, got)
    print(f"[sampling V={V}] picks differing from the oracle (near a boundary): {diffs}", flush=True)
    assert diffs <= 3
    # temperature 0: the greedy pick, u not needed
    nc.nc_sample(dl, B, V, 0.0, 0, None, out)
    ref = torch.empty_like(out)
    nc.nc_argmax(dl, B, V, ref)
    assert torch.equal(out, ref)


def test_sampling_frequencies_on_a_grid():
    """u on a grid of 4096 points over one row: the picks reproduce the distribution's
    slices (counts within 1 of N p_i, up to boundary rounding)."""
    torch = torch_mod()
    rng = np.random.default_rng(90)
    V, N, t, k = 300, 4096, 1.2, 20
    z = (rng.standard_normal(V) * 1.5).astype(np.float32)
    logits = np.ascontiguousarray(np.broadcast_to(z, (N, V)))
    u = ((np.arange(N) + 0.5) / N).astype(np.float32)
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    nc.nc_sample(torch.from_numpy(logits).cuda(), N, V, t, k, torch.from_numpy(u).cuda(), out)
    got = out.cpu().numpy()
    _check_samples(logits, t, k, u, got)
    keep = np.argsort(z.astype(np.float64))[::-1][:k]
    e = np.exp(z[keep].astype(np.float64) / t)
    probs = np.zeros(V)
    probs[keep] = e / e.sum()
    counts = np.bincount(got, minlength=V)
    assert np.all(np.abs(counts - N * probs) <= 2.0)
    assert set(np.nonzero(counts)[0]) <= set(keep)


# ---------------------------------------------------------------- later-version blocks -
EXTRAS_TINY = replace(TINY, name="tiny-extras", n_layer=3, d_model=256, n_head=4, n_kv_head=2,
                      max_seq=96)


def test_fp32_extras_prefill_decode_append_copy():
    """Value embeddings (layers 0 and 2), residual lambdas, smear and backout in fp32: a
    prefill, decode steps (smear reading the cached previous token), a truncated row, an
    appended chunk and a copied row, all against the oracle at the fp32 bar."""
    torch = torch_mod()
    shape = EXTRAS_TINY
    w = make_weights(shape, seed=100)
    ex = make_extras(shape, seed=101, ve_layers=(0, 2), smear_ch=24, ve_ch=40)
    orc = OracleModel(shape, w, extras=ex)
    gm = gpu_model(shape, w, extras=ex)
    B, T = 2, 60
    toks = make_tokens(shape.vocab, B, 80, seed=102)
    want, _ = orc.prefill(toks)
    kv, got = prefill(gm, toks[:, :T], shape.max_seq)
    err, _ = report("tiny extras prefill", got, want[:, :T])
    assert err <= F32_TOL
    got = np.stack([decode(gm, kv, toks[:, T + s]) for s in range(4)], axis=1)
    err, _ = report("tiny extras decode", got, want[:, T:T + 4])
    assert err <= F32_TOL
    kv.set_lens([30, 64])
    out = torch.empty((B, 5, shape.vocab), device="cuda", dtype=torch.float32)
    kv.prefill(torch.from_numpy(np.ascontiguousarray(toks[:, 70:75])).cuda(), out)
    got = out.cpu().numpy()
    for b, n in enumerate((30, 64)):
        seq = np.concatenate([toks[b, :n], toks[b, 70:75]])[None]
        ref, _ = orc.prefill(seq, logits_at=np.arange(n, n + 5))
        err, _ = report(f"tiny extras append row {b} at {n}", got[b], ref[0])
        assert err <= F32_TOL
    other = gm.new_kv(3, shape.max_seq)
    other.copy_rows_from(kv, [1], [2])
    got = decode(gm, other, np.array([0, 0, toks[1, 75]], dtype=np.int32))[2]
    seq = np.concatenate([toks[1, :64], toks[1, 70:76]])[None]
    ref, _ = orc.prefill(seq, logits_at=[69])
    err = float(np.max(np.abs(got - ref[0, 0])))
    print(f"[tiny extras copied row] max_abs={err:.3e}", flush=True)
    assert err <= F32_TOL
    other.close()
    kv.close()
    gm.close()


@pytest.mark.parametrize("B", [3, 40])
def test_bf16_extras_prefill_and_decode(B):
    """The blocks on a bf16 model (4 layers, value embeddings on the odd ones): ragged
    prefill, then decode of B rows at mixed lengths (B = 40: the split-K decode path, whose
    reduce kernel runs the residual epilogue)."""
    shape = replace(SMALL_BF16, name="small-extras", n_layer=4, n_kv_head=2, max_seq=400)
    w = make_weights(shape, seed=103)
    ex = make_extras(shape, seed=104)
    orc = OracleModel(shape, w, extras=ex)
    gm = gpu_model(shape, w, extras=ex)
    T = 300
    toks = make_tokens(shape.vocab, B, T + 2, seed=105 + B)
    kv, got = prefill(gm, toks[:, :T], shape.max_seq)
    want, _ = orc.prefill(toks[:2, :T])
    err, agr = report(f"small extras prefill B={B}", got[:2], want)
    assert err <= BF16_TOL and agr >= AGREE
    lens = make_lens(B, 1, T, seed=106 + B)
    kv.set_lens(lens)
    got = np.stack([decode(gm, kv, toks[:, T + s]) for s in range(2)], axis=1)
    want = np.empty_like(got, dtype=np.float64)
    for b in range(B):
        seq = np.concatenate([toks[b, :lens[b]], toks[b, T:T + 2]])[None]
        want[b] = orc.prefill(seq, logits_at=np.arange(lens[b], lens[b] + 2))[0][0]
    err, agr = report(f"small extras decode B={B}", got, want)
    assert err <= BF16_TOL
    assert_flips_are_near_ties(got, want, err)
    kv.close()
    gm.close()


def test_extras_switch_off_and_errors(small):
    """Setting the blocks requires no live cache; clearing them gives the plain model."""
    w, orc, gm = small
    kv = gm.new_kv(1, 8)
    ex = make_extras(SMALL_BF16, seed=107)
    with pytest.raises(nc.NcError) as e:
        nc.nc_model_set_extras(gm.handle, ex, SMALL_BF16.n_layer, "bf16")
    assert e.value.code == nc.NC_ERR_STATE
    kv.close()
    bad = dict(ex, backout_layer=SMALL_BF16.n_layer)
    with pytest.raises(nc.NcError) as e:
        nc.nc_model_set_extras(gm.handle, bad, SMALL_BF16.n_layer, "bf16")
    assert e.value.code == nc.NC_ERR_INVALID_ARG
    nc.nc_model_set_extras(gm.handle, ex, SMALL_BF16.n_layer, "bf16")
    nc.nc_model_set_extras(gm.handle, None, SMALL_BF16.n_layer, "bf16")
    toks = make_tokens(SMALL_BF16.vocab, 1, 20, seed=108)
    _, got = prefill(gm, toks, 20)
    want, _ = orc.prefill(toks)
    assert np.max(np.abs(got - want)) <= BF16_TOL


def test_diagnostic_rates_are_physical():
    """The sustained-rate probes return values below MI355X's published peaks."""
    rnd, const = nc.nc_diag_mfma_rate(True), nc.nc_diag_mfma_rate(False)
    hbm = nc.nc_diag_hbm_read_rate()
    print(f"[diag] mfma random {rnd:.0f} constant {const:.0f} TFLOP/s, hbm read {hbm:.2f} TB/s", flush=True)
    assert 100.0 < rnd <= 2516.6 * 1.05 and 100.0 < const <= 2516.6 * 1.05
    assert 0.5 < hbm <= 8.0 * 1.05
