"""Reader for the hand-worked fixtures under tests/golden/ (test helper)."""
import os
import re
import struct

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _expand(text):
    """Expand 'V*N' and '(a b c)*N' repeat tokens into a flat token list."""
    out = []
    pos = 0
    tokens = re.findall(r"\([^)]*\)\*\d+|\S+", text)
    for tok in tokens:
        m = re.fullmatch(r"\(([^)]*)\)\*(\d+)", tok)
        if m:
            inner = _expand(m.group(1))
            out.extend(inner * int(m.group(2)))
            continue
        m = re.fullmatch(r"([^*]+)\*(\d+)", tok)
        if m:
            out.extend([m.group(1)] * int(m.group(2)))
            continue
        out.append(tok)
    del pos
    return out


def _stanzas(path):
    cur = None
    res = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            m = re.fullmatch(r"\[(\w+)\]", line)
            if m:
                cur = {}
                res[m.group(1)] = cur
                continue
            key, _, val = line.partition("=")
            cur[key.strip()] = val.strip()
    return res


def load_blocks():
    """Return {id: (type, 34-byte np.uint8 block, expected fp32 bit array)}."""
    res = {}
    for gid, st in _stanzas(os.path.join(GOLDEN_DIR, "blocks.txt")).items():
        if "bytes" in st:
            raw = bytes(int(t, 16) for t in _expand(st["bytes"]))
        else:
            words = [int(t, 16) for t in _expand(st["words"])]
            assert len(words) == 8, gid
            raw = struct.pack("<H8I", int(st["scale"], 16), *words)
        assert len(raw) == 34, gid
        expect = np.array([int(t, 16) for t in _expand(st["expect"])], dtype=np.uint32)
        res[gid] = (st["type"], np.frombuffer(raw, np.uint8).copy(), expect)
    return res


def load_gemv():
    """Return {id: dict(type, k, w (uint8 rows), x (fp16), y, a)}."""
    blocks = load_blocks()
    res = {}
    for gid, st in _stanzas(os.path.join(GOLDEN_DIR, "gemv.txt")).items():
        k = int(st["k"])
        rows = []
        for spec in st["rows"].split():
            rows.append(np.concatenate([blocks[b][1] for b in spec.split("+")]))
        w = np.stack(rows)
        if "x" in st:
            xb = np.array([int(t, 16) for t in _expand(st["x"])], dtype=np.uint16)
        else:
            xb = np.zeros(k, np.uint16)
            idx, _, val = st["onehot"].partition(":")
            xb[int(idx)] = int(val, 16)
        assert xb.size == k, gid
        res[gid] = dict(type=st["type"], k=k, w=w, x=xb.view(np.float16),
                        y=np.array([float(v) for v in st["y"].split()]),
                        a=np.array([float(v) for v in st["a"].split()]))
    return res
