"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random bytes and numbers; it holds none of the method's
arithmetic (no decoding, no quantization, no dot products).

Recipe (the pages measured a LLaMA-7B q4_K_M model on a 3314-token prefill; no
model file is available, so inputs of the same shapes and field distributions
stand in for it):
  * one ``numpy.random.default_rng(seed)`` stream per case, drawn in a fixed
    order: the weight fields in block-struct order (each field for all blocks at
    once), then the activations, then the outlier mask;
  * q6_K blocks (210 B): ql and qh uniform bytes; the sixteen int8 scales
    uniform in [-32, 31]; d = f16(|N(0,1)| * 1e-3);
  * q4_K blocks (144 B): d and dmin = f16(|N(0,1)| * 1e-3) each; the twelve
    packed scale/min bytes and the 128 qs bytes uniform;
  * activations f32 N(0,1); with ``outliers`` every element is multiplied by 20
    with probability 0.01 (Bernoulli draws from the same stream).
"""
from __future__ import annotations

import numpy as np

Q4_K = 4
Q6_K = 6
Q4_K_PACKED = 14  # the same q4_K input blocks, registered with packed codes
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, Q4_K_PACKED: 144}
TYPE_NAMES = {Q4_K: "q4_K", Q6_K: "q6_K", Q4_K_PACKED: "q4_K packed"}


def _f16_scale(rng: np.random.Generator, n: int) -> np.ndarray:
    """n binary16 bit patterns of |N(0,1)| * 1e-3 (float16 rounding by numpy)."""
    v = (np.abs(rng.standard_normal(n)) * 1e-3).astype(np.float16)
    return v.view(np.uint16)


def q6k_weights(rng: np.random.Generator, od: int, id_: int) -> np.ndarray:
    """Raw q6_K bytes, row-major od x (id/256) blocks of 210 bytes."""
    nb = od * (id_ // 256)
    ql = rng.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    qh = rng.integers(0, 256, size=(nb, 64), dtype=np.uint8)
    sc = rng.integers(-32, 32, size=(nb, 16), dtype=np.int8)
    d = _f16_scale(rng, nb)
    blk = np.empty((nb, 210), np.uint8)
    blk[:, 0:128] = ql
    blk[:, 128:192] = qh
    blk[:, 192:208] = sc.view(np.uint8)
    blk[:, 208:210] = d.astype("<u2").view(np.uint8).reshape(nb, 2)
    return blk.reshape(-1)


def q4k_weights(rng: np.random.Generator, od: int, id_: int) -> np.ndarray:
    """Raw q4_K bytes, row-major od x (id/256) blocks of 144 bytes."""
    nb = od * (id_ // 256)
    d = _f16_scale(rng, nb)
    dmin = _f16_scale(rng, nb)
    scales = rng.integers(0, 256, size=(nb, 12), dtype=np.uint8)
    qs = rng.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    blk = np.empty((nb, 144), np.uint8)
    blk[:, 0:2] = d.astype("<u2").view(np.uint8).reshape(nb, 2)
    blk[:, 2:4] = dmin.astype("<u2").view(np.uint8).reshape(nb, 2)
    blk[:, 4:16] = scales
    blk[:, 16:144] = qs
    return blk.reshape(-1)


def weights(rng: np.random.Generator, type_: int, od: int, id_: int) -> np.ndarray:
    if type_ == Q6_K:
        return q6k_weights(rng, od, id_)
    if type_ in (Q4_K, Q4_K_PACKED):
        return q4k_weights(rng, od, id_)
    raise ValueError(f"unknown type {type_}")


def activations(rng: np.random.Generator, n_tok: int, id_: int,
                outliers: bool = False) -> np.ndarray:
    """f32 [n_tok][id] N(0,1), optionally with 1% of elements scaled by 20."""
    x = rng.standard_normal((n_tok, id_), dtype=np.float32)
    if outliers:
        mask = rng.random((n_tok, id_)) < 0.01
        x = np.where(mask, x * np.float32(20.0), x).astype(np.float32)
    return x


def block_format(type_: int) -> int:
    """The block format a registration type reads (both q4_K types read q4_K)."""
    return Q4_K if type_ == Q4_K_PACKED else type_


def case(type_: int, od: int, id_: int, n_tok: int, seed: int = 0,
         outliers: bool = False):
    """(raw weight bytes, f32 activations) for one GEMM, drawn in recipe order."""
    rng = np.random.default_rng(seed)
    raw = weights(rng, type_, od, id_)
    x = activations(rng, n_tok, id_, outliers)
    return raw, x


# The five workloads: (name, type, od, id, n_tok, outliers).
SMALL_Q6K = ("q6_K 256x512 T=64", Q6_K, 256, 512, 64, False)
FFN_DOWN = ("q6_K ffn_down 4096x11008 T=512", Q6_K, 4096, 11008, 512, False)
FFN_DOWN_ODD = ("q6_K ffn_down od=4097 T=509", Q6_K, 4097, 11008, 509, False)
ATTN = ("q4_K attn 4096x4096 T=512", Q4_K, 4096, 4096, 512, False)
GATE_UP = ("q4_K ffn gate/up 11008x4096 T=512", Q4_K, 11008, 4096, 512, False)
HEAD = ("q6_K head 32000x4096 T=2048", Q6_K, 32000, 4096, 2048, True)

# One LLaMA-7B q4_K_M-style layer at a 3314-token prefill: (name, type, od, id).
LAYER_TOKENS = 3314
LAYER_GEMMS = (
    ("attn_q", Q4_K, 4096, 4096),
    ("attn_k", Q4_K, 4096, 4096),
    ("attn_v", Q6_K, 4096, 4096),
    ("attn_output", Q4_K, 4096, 4096),
    ("ffn_gate", Q4_K, 11008, 4096),
    ("ffn_up", Q4_K, 11008, 4096),
    ("ffn_down", Q6_K, 4096, 11008),
)
