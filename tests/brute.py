"""Brute-force restatement of the attention step for tiny inputs.

Written separately from the oracle, in plain Python floats and loops, with an
explicit dense causal mask and exact rational rounding, so that it can pin
the oracle: logical K/V rows come from the workload's own logical arrays
(not from the paged pool), so the paged scatter/gather of the oracle is
checked end to end.  Only for inputs small enough that Python loops finish
in well under a second.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np


def round_bf16(x: float) -> float:
    """Round a binary64 value to bf16 (8 significant bits, RNE) exactly."""
    if x == 0.0 or math.isnan(x) or math.isinf(x):
        return x
    a = abs(Fraction(x))
    e = 0
    while Fraction(2) ** e <= a:
        e += 1
    while Fraction(2) ** (e - 1) > a:
        e -= 1
    e = max(e, -125)
    q = a / (Fraction(2) ** (e - 8))
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = float(fl * Fraction(2) ** (e - 8))
    return -v if x < 0 else v


def round_f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def widen(bits_or_f32, dtype: str) -> list:
    a = np.asarray(bits_or_f32)
    if dtype == "bf16":
        flat = [struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in a.reshape(-1)]
    else:
        flat = [float(v) for v in a.reshape(-1)]
    return np.array(flat, dtype=np.float64).reshape(a.shape).tolist()


def rotate(vec: list, pos: int, theta: float) -> list:
    d = len(vec)
    h = d // 2
    out = [0.0] * d
    for i in range(h):
        ang = pos * theta ** (-(2.0 * i) / d)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = vec[i] * c - vec[i + h] * s
        out[i + h] = vec[i + h] * c + vec[i] * s
    return out


def run(batch):
    """Return (q_rot_rounded [T][H][d] floats, out [T][H][d] floats) for a
    small workload batch with logical pre-existing K/V kept."""
    sh = batch.shape
    H, Hkv, d, dt = sh.num_heads, sh.num_kv_heads, sh.head_dim, sh.dtype
    G = H // Hkv
    rnd = round_bf16 if dt == "bf16" else round_f32
    rows = widen(batch.qkv, dt)
    T = len(rows)
    q_rot, k_new, v_new = [], [], []
    for t in range(T):
        r = rows[t]
        p = int(batch.positions[t])
        q_rot.append([[rnd(v) for v in rotate(r[h * d:(h + 1) * d], p, sh.rope_theta)]
                      for h in range(H)])
        k_new.append([[rnd(v) for v in rotate(r[(H + g) * d:(H + g + 1) * d], p, sh.rope_theta)]
                      for g in range(Hkv)])
        v_new.append([r[(H + Hkv + g) * d:(H + Hkv + g + 1) * d] for g in range(Hkv)])

    out = [[[0.0] * d for _ in range(H)] for _ in range(T)]
    row0 = 0
    for s in range(batch.num_seqs):
        n = int(batch.query_lens[s])
        c = int(batch.context_lens[s])
        K = widen(batch.pre_k[s], dt) if batch.pre_k[s].size else []
        V = widen(batch.pre_v[s], dt) if batch.pre_v[s].size else []
        K = list(K) + [k_new[row0 + i] for i in range(n)]
        V = list(V) + [v_new[row0 + i] for i in range(n)]
        assert len(K) == c
        mask = [[(j <= c - n + i) for j in range(c)] for i in range(n)]
        for g in range(Hkv):
            for h in range(g * G, (g + 1) * G):
                for i in range(n):
                    qv = q_rot[row0 + i][h]
                    sc = []
                    for j in range(c):
                        if mask[i][j]:
                            sc.append(sum(qv[e] * K[j][g][e] for e in range(d)) / math.sqrt(d))
                        else:
                            sc.append(None)
                    mx = max(v for v in sc if v is not None)
                    w = [math.exp(v - mx) if v is not None else 0.0 for v in sc]
                    tot = sum(w)
                    for e in range(d):
                        out[row0 + i][h][e] = sum(w[j] * V[j][g][e] for j in range(c)) / tot
        row0 += n
    return q_rot, out
