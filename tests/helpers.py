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


# ---------------------------------------------------------------- GPU side ---
def bf16_dev(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def to_dev(inp, dev):
    """Host arrays drawn by synth (or built by a test) -> device tensors."""
    return synth.to_device(inp, dev)


def sub_inputs(inp, blocks):
    """The inputs of a subset of blocks (every block is independent)."""
    return synth.sub_blocks(inp, blocks)


def ulp32(x):
    x = np.abs(np.asarray(x, np.float64))
    return np.spacing(x.astype(np.float32)).astype(np.float64)


def check_scores(S_gpu, S_ref, cand_u):
    """The matching rule for scores: max |dS| <= 2e-3 max|S| over the finite
    entries, the same relative bound on the pair term P = S - U, and identical
    -inf padding.  Returns (eps_S, tol_S, eps_P, tol_P)."""
    S_g = np.asarray(S_gpu, np.float64)
    fin = np.isfinite(S_ref)
    assert np.array_equal(np.isneginf(S_g), np.isneginf(S_ref)), "-inf padding differs"
    assert np.all(np.isfinite(S_g[fin])), "non-finite GPU score where the oracle is finite"
    eps = float(np.abs(S_g[fin] - S_ref[fin]).max()) if fin.any() else 0.0
    tol = 2e-3 * float(np.abs(S_ref[fin]).max()) if fin.any() else 0.0
    U = np.asarray(cand_u, np.float64)[:, :, None, :]
    P_g, P_r = (S_g - U)[fin], (S_ref - U)[fin]
    eps_p = float(np.abs(P_g - P_r).max()) if fin.any() else 0.0
    tol_p = 2e-3 * float(np.abs(P_r).max()) + 1e-30 if fin.any() else 0.0
    assert eps <= tol, f"max |dS| {eps} > {tol}"
    assert eps_p <= tol_p, f"max |dP| {eps_p} > {tol_p}"
    return eps, tol, eps_p, tol_p


def check_walk(ora, gpu, S_ref, S_gpu, cand_id, mode, uniforms=None, T=1.0, eps=0.0):
    """Walk parity with teacher forcing: at every step the GPU's slot must equal
    the oracle's choice from the GPU's own predecessor, except at steps whose
    top-2 gap (greedy) or CDF margin (sampled) is within the score error; those
    are counted as flagged.  Also checks path_tok / path_s against the GPU's own
    scores and, for greedy, that each slot is the arg-max of the GPU's own row.
    Returns the number of flagged steps."""
    choice, aux = ora.step_table(S_ref, mode, uniforms, T)
    slot = gpu["path_slot"]
    B, L = slot.shape
    S_g = np.asarray(S_gpu, np.float32) if S_gpu is not None else None
    flagged = 0
    for b in range(B):
        row = 0
        for t in range(L):
            g = int(slot[b, t])
            assert 0 <= g < K
            assert gpu["path_tok"][b, t] == cand_id[b, t, g]
            if S_g is not None:
                assert gpu["path_s"][b, t] == S_g[b, t, row, g]
                if mode == 0:
                    assert g == int(np.argmax(S_g[b, t, row])), "greedy slot is not the arg-max of its own row"
            o = int(choice[b, t, row])
            if g != o:
                a = float(aux[b, t, row])
                if mode == 0:
                    best = float(np.max(S_ref[b, t, row]))
                    bound = 2.0 * eps + 16.0 * float(ulp32(best))
                else:
                    bound = 2.0 * eps / T + 64.0 * 2.0 ** -24
                assert a <= bound, f"walk differs at block {b} position {t}: gpu {g} oracle {o}, aux {a} > {bound}"
                flagged += 1
            row = g
    return flagged
