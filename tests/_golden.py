"""Readers for the hand-worked fixtures under tests/golden/ (each fixture
file states its source passage in its header)."""
from __future__ import annotations

import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield [c.strip() for c in line.split("|")]


def _expand_signs(spec: str) -> str:
    """'64+ -' -> 64 '+' then '-'; '35+-' -> 35 copies of '+-'."""
    out = []
    for tok in spec.split():
        i = 0
        while i < len(tok) and tok[i].isdigit():
            i += 1
        count = int(tok[:i]) if i else 1
        out.append(tok[i:] * count)
    return "".join(out)


def signs_to_f32(signs: str) -> np.ndarray:
    return np.array([1.0 if c == "+" else -1.0 for c in signs], dtype=np.float32).reshape(1, -1)


def worked_examples():
    """(n, x_signs, w_signs, x_words, w_words, d, dot)."""
    for n, xs, ws, xw, ww, d, dot in _rows("worked_examples.txt"):
        xs, ws = _expand_signs(xs), _expand_signs(ws)
        n = int(n)
        assert len(xs) == n and len(ws) == n, (n, xs, ws)
        yield (n, xs, ws, [int(t, 16) for t in xw.split()], [int(t, 16) for t in ww.split()],
               int(d), int(dot))


def scaled_examples():
    """(dot, alpha, expected)."""
    for dot, alpha, exp in _rows("scaled_examples.txt"):
        yield int(dot), np.float32(float(alpha)), np.float32(float(exp))


def _f32_from_bits(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b))[0]


def projection_f32():
    """(bits, description, expected bit)."""
    for bits, desc, bit in _rows("projection_f32.txt"):
        yield int(bits, 16), desc, int(bit)


def projection_bf16():
    for bits, desc, bit in _rows("projection_bf16.txt"):
        yield int(bits, 16), desc, int(bit)


def repack_examples():
    """(K, [dots], [words])."""
    for k, dots, words in _rows("repack_examples.txt"):
        vals = []
        for tok in dots.split():
            if "*" in tok:
                c, v = tok.split("*")
                vals += [int(v)] * int(c)
            else:
                vals.append(int(tok))
        yield int(k), vals, [int(t, 16) for t in words.split()]


def pair_rows_for_dots(k: int, dots):
    """float32 x (1, k) all +1 and W (len(dots), k) whose row n holds
    (k - dots[n]) / 2 entries -1, so that <x, w_n> = dots[n]."""
    x = np.ones((1, k), dtype=np.float32)
    w = np.ones((len(dots), k), dtype=np.float32)
    for n, d in enumerate(dots):
        assert (k - d) % 2 == 0 and abs(d) <= k, (k, d)
        w[n, : (k - d) // 2] = -1.0
    return x, w


def _expand_values(spec: str) -> list:
    out = []
    for tok in spec.split():
        if "*" in tok:
            c, v = tok.split("*")
            out += [float(v)] * int(c)
        else:
            out.append(float(tok))
    return out


def signw_examples():
    """(x values as float64 array, sign string, expected s)."""
    for xs, ws, exp in _rows("signw_examples.txt"):
        x = np.array(_expand_values(xs), dtype=np.float64)
        signs = _expand_signs(ws)
        assert len(signs) == x.size, (xs, ws)
        yield x, signs, float(exp)
