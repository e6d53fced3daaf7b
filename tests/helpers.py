"""Shared test helpers: fixture loaders and parity comparisons (no selector arithmetic)."""
import json
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
K = 16


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def stutter_inputs(zero_pair=False):
    """Arrays of the hand-worked stutter example (golden/stutter_walk.json)."""
    g = load_golden("stutter_walk.json")
    V, d, r, B, L = g["vocab"], g["d"], g["r"], g["batch"], g["block"]
    logits = np.zeros((B, L, V), np.float32)
    for t, tok, val in g["logit_entries"]:
        logits[0, t, tok] = val
    eye = np.eye(V, d, dtype=np.float32)
    W_A = np.zeros((r, d), np.float32) if zero_pair else -4.0 * np.eye(r, d, dtype=np.float32)
    inp = dict(
        logits=logits,
        E=synth.f32_to_bf16_bits(eye),
        W_A=synth.f32_to_bf16_bits(W_A),
        W_B=synth.f32_to_bf16_bits(np.eye(r, d, dtype=np.float32)),
        W_H=synth.f32_to_bf16_bits(np.zeros((r, d), np.float32)),
        h=synth.f32_to_bf16_bits(np.zeros((B, L, d), np.float32)),
        verified=np.array(g["verified"], np.int32),
        uniforms=np.zeros((B, L), np.float32),
    )
    return inp, g["expected"]
