"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and by the oracle's tests.

This module holds the workload shapes and the random draws only: no step of the model's
arithmetic lives here.  Weights, token ids and per-row context lengths are drawn from
numpy's PCG64 generator so that both sides of a parity test receive identical values.

Weight recipe: every matrix (token embedding, Wq, Wk, Wv, Wo, Wfc, Wproj per layer, LM
head) is drawn as standard normals times 0.02 in float64, in that canonical order from one
generator seeded with `seed`, then rounded to float32 and, for bf16 models, rounded again
to bfloat16 (round to nearest even on the float32 bit pattern).  The arrays returned are
float32 and hold exactly the values the model uses; `bf16_bits` gives their 16-bit
encoding for upload.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Shape:
    """Model shape.  dtype is "f32" or "bf16" (the storage type of weights, activations
    that feed matrix products, and the KV cache)."""
    name: str
    n_layer: int
    d_model: int
    n_head: int
    head_dim: int
    d_ff: int
    vocab: int
    dtype: str
    max_seq: int
    n_kv_head: int = 1
    rope_base: float = 10000.0
    softcap: float = 15.0
    norm_eps: float = 1e-6


@dataclass(frozen=True)
class Workload:
    """A run on one model: prefill batch x T, then decode steps."""
    shape: Shape
    prefill_batch: int
    prefill_len: int
    decode_batch: int
    decode_steps: int
    decode_context: int          # context length before the first decode step
    mixed_lengths: bool = False  # per-row context lengths drawn from U{256..2048}
    window_pattern: str = ""     # per-layer sliding windows, e.g. "SSSL" ("" = none)
    short_window: int = 0        # window of the pattern's S layers (keys back)
    temperature: float = 0.0     # decode picks: > 0 samples (with top_k), else greedy
    top_k: int = 0
    extras_seed: int = -1        # >= 0: the later version's blocks from make_extras(seed)


def from_depth(depth, vocab=65536, dtype="bf16", max_seq=2048, name=None):
    """The single-knob rule: width 64*depth, heads of 128, MLP 4x width."""
    d = 64 * depth
    return Shape(name or f"d{depth}", depth, d, d // 128, 128, 4 * d, vocab, dtype, max_seq)


TINY = Shape("tiny", 2, 128, 2, 64, 512, 512, "f32", 80)
D12 = replace(from_depth(12), max_seq=2304)
D20 = replace(from_depth(20), max_seq=2176)
D26 = replace(from_depth(26), max_seq=2048)
D30 = replace(from_depth(30), max_seq=2304)

WORKLOADS = {
    "tiny": Workload(TINY, 1, 64, 1, 16, 64),
    "d12": Workload(D12, 8, 2048, 8, 256, 2048),
    "d20": Workload(D20, 32, 2048, 64, 128, 2048),
    "d26": Workload(D26, 16, 2048, 0, 0, 0),
    "d30": Workload(D30, 0, 0, 128, 256, 2048, mixed_lengths=True),
    # the later version's attention options on the d20 model and run: 5 K/V heads (groups
    # of 2 query heads), and an SSSL window pattern with 512-key short windows
    "d20-gqa": Workload(replace(D20, name="d20-gqa", n_kv_head=5), 32, 2048, 64, 128, 2048),
    "d20-sssl": Workload(replace(D20, name="d20-sssl"), 32, 2048, 64, 128, 2048,
                         window_pattern="SSSL", short_window=512),
    # the later version's learned blocks on the d20 model and run (value embeddings on the
    # odd layers, residual lambdas, smear, backout at layer 10)
    "d20-blocks": Workload(replace(D20, name="d20-blocks"), 32, 2048, 64, 128, 2048, extras_seed=5),
    # the d12 run with sampled instead of greedy decode picks (temperature 1, top-50)
    "d12-sample": Workload(D12, 8, 2048, 8, 256, 2048, temperature=1.0, top_k=50),
}


def round_bf16(a):
    """float32 -> nearest bfloat16 value (ties to even), returned as float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bf16_bits(a):
    """16-bit encoding of float32 values that are exactly representable in bfloat16."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def weight_shapes(s: Shape):
    """(name, [out, in]) of every weight matrix, in canonical order."""
    hq, hkv = s.n_head * s.head_dim, s.n_kv_head * s.head_dim
    out = [("wte", (s.vocab, s.d_model))]
    for i in range(s.n_layer):
        out += [(f"l{i}.wq", (hq, s.d_model)), (f"l{i}.wk", (hkv, s.d_model)),
                (f"l{i}.wv", (hkv, s.d_model)), (f"l{i}.wo", (s.d_model, hq)),
                (f"l{i}.wfc", (s.d_ff, s.d_model)), (f"l{i}.wproj", (s.d_model, s.d_ff))]
    out.append(("lm_head", (s.vocab, s.d_model)))
    return out


def make_weights(s: Shape, seed=0, std=0.02):
    """Seeded N(0, std^2) weights in canonical order.

    Returns {"wte", "layers": [{"wq","wk","wv","wo","wfc","wproj"}], "lm_head"} of float32
    arrays holding the exact values of the model's storage dtype."""
    rng = np.random.default_rng(seed)
    flat = {}
    for name, shp in weight_shapes(s):
        w = (rng.standard_normal(shp) * std).astype(np.float32)
        flat[name] = round_bf16(w) if s.dtype == "bf16" else w
    layers = [{k: flat[f"l{i}.{k}"] for k in ("wq", "wk", "wv", "wo", "wfc", "wproj")}
              for i in range(s.n_layer)]
    return {"wte": flat["wte"], "layers": layers, "lm_head": flat["lm_head"]}


def canonical_list(weights):
    """The 6L+2 weight arrays in canonical order."""
    out = [weights["wte"]]
    for lw in weights["layers"]:
        out += [lw["wq"], lw["wk"], lw["wv"], lw["wo"], lw["wfc"], lw["wproj"]]
    out.append(weights["lm_head"])
    return out


def make_extras(s: Shape, seed=5, ve_layers=None, smear_ch=24, ve_ch=32, ve_std=0.5):
    """Seeded parameters of the later version's blocks (value embeddings, residual lambdas,
    smear, backout) in the dict form both sides take: per-layer lambdas as float32 values,
    tables and gates as float32 arrays holding exact values of the storage dtype.  Value
    embeddings sit on the odd layers unless ve_layers says otherwise; backout takes the
    middle layer."""
    rng = np.random.default_rng(seed)
    L, kvd = s.n_layer, s.n_kv_head * s.head_dim
    rnd = (lambda a: round_bf16(a)) if s.dtype == "bf16" else (lambda a: a)
    ve_layers = list(range(1, L, 2)) if ve_layers is None else list(ve_layers)
    f32 = lambda a: np.asarray(a, dtype=np.float32)  # noqa: E731
    ex = {"resid_lambda": [float(v) for v in f32(rng.uniform(0.8, 1.2, L))],
          "x0_lambda": [float(v) for v in f32(rng.uniform(0.0, 0.3, L))],
          "smear_gate": rnd(f32(rng.standard_normal(smear_ch) * 0.3)),
          "smear_lambda": float(np.float32(0.5)),
          "backout_layer": L // 2, "backout_lambda": float(np.float32(0.3)),
          "ve": {}, "ve_gate": {}}
    for l in ve_layers:
        ex["ve"][l] = rnd(f32(rng.standard_normal((s.vocab, kvd)) * ve_std))
        ex["ve_gate"][l] = rnd(f32(rng.standard_normal((s.n_kv_head, ve_ch)) * 0.3))
    return ex


def make_tokens(vocab, batch, length, seed=1):
    """Uniform random token ids in [0, vocab), int32 [batch, length]."""
    return np.random.default_rng(seed).integers(0, vocab, (batch, length)).astype(np.int32)


def make_lens(batch, lo=256, hi=2048, seed=2):
    """Per-row context lengths uniform in {lo..hi} (inclusive), int32 [batch]."""
    return np.random.default_rng(seed).integers(lo, hi + 1, batch).astype(np.int32)
