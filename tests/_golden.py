"""Readers for the hand-derived fixtures in tests/golden/."""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(tok):
    tok = tok.strip()
    if "p" in tok.lower() and tok.lower().lstrip("-").startswith("0x"):
        return float.fromhex(tok)
    if tok.lower().lstrip("-").startswith("0x"):
        return int(tok, 16)
    return float(tok)


def lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            s = raw.split("#", 1)[0].strip()
            if s:
                yield s.split()


def code_table(name):
    """[(code, value)] from a two-column table."""
    return [(int(c, 16), _num(v)) for c, v in lines(name)]


def mx_blocks(name="mx_worked_blocks.txt"):
    """[(name, fmt, scale_byte, {index: (value, code)})]."""
    out = []
    for tok in lines(name):
        if tok[0] == "block":
            out.append((tok[1], tok[2], int(tok[3]), {}))
        else:
            out[-1][3][int(tok[0])] = (_num(tok[1]), int(tok[2], 16))
    return out


def keyed(name):
    """{key: [numbers]} for 'key v1 v2 ...' lines."""
    return {tok[0]: [_num(t) for t in tok[1:]] for tok in lines(name)}


def rows(name):
    return [tok for tok in lines(name)]
