"""Readers for the cited fixtures under tests/golden/."""
import os

import numpy as np

_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(_DIR, name)) as f:
        return [l.strip() for l in f if l.strip() and not l.startswith("#")]


def kv(name):
    out = {}
    for l in lines(name):
        k, v = l.split(None, 1)
        out[k] = v
    return out


def kv_share_map_e2b():
    return [int(t) for t in lines("kv_share_map_e2b.txt")[0].split()]


def nibble_case():
    d = kv("nibble_order.txt")
    words = np.array([int(w, 16) for w in d["words"].split()], dtype=np.uint32).view(np.int32)
    q = np.array([int(t) for t in d["q"].split()], dtype=np.int64)
    return words, q
