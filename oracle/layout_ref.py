"""Definition-level evaluation of a Shape:Stride layout, for tests.

TEST INFRASTRUCTURE ONLY.  A layout maps a coordinate to the inner product of
the coordinate with the stride; a one-dimensional coordinate is first split
colexicographically (mode 0 fastest) over the shape's leaves, the last leaf
taking whatever remains ("CuTe's layout algebra", section "A layout: shape and
stride").  This module evaluates that definition directly (no algebra), so
the C++ module's symbolic results can be checked point by point.
"""
from __future__ import annotations

import re


def parse(text: str):
    """'(4,(2,4)):(2,(1,8))' -> (shape, stride) as nested Python tuples/ints."""
    text = text.replace("_", "").replace(" ", "")

    def tup(s, i):
        if s[i] == "(":
            items, i = [], i + 1
            while True:
                v, i = tup(s, i)
                items.append(v)
                if s[i] == ",":
                    i += 1
                    continue
                assert s[i] == ")"
                return tuple(items), i + 1
        m = re.match(r"-?\d+", s[i:])
        return int(m.group()), i + len(m.group())

    shape_txt, stride_txt = text.split(":")
    shape, i = tup(shape_txt, 0)
    assert i == len(shape_txt)
    stride, j = tup(stride_txt, 0)
    assert j == len(stride_txt)
    return shape, stride


def leaves(t):
    return [t] if isinstance(t, int) else [x for c in t for x in leaves(c)]


def size(shape) -> int:
    n = 1
    for x in leaves(shape):
        n *= x
    return n


def evaluate(text: str, coord: int) -> int:
    """L(coord) for a one-dimensional coordinate: split over the flattened
    leaves with mode 0 fastest, the last leaf unbounded."""
    shape, stride = parse(text)
    ext, st = leaves(shape), leaves(stride)
    idx, c = 0, coord
    for k, (e, d) in enumerate(zip(ext, st)):
        if k == len(ext) - 1:
            idx += c * d
        else:
            idx += (c % e) * d
            c //= e
    return idx


def table(text: str):
    """Every index of the layout, for coordinates 0 .. size-1."""
    shape, _ = parse(text)
    return [evaluate(text, c) for c in range(size(shape))]
