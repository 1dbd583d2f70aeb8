"""Readers for the text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


def quant_rows():
    cases, cur = [], {}
    for ln in _lines("quant_rows.txt"):
        key, vals = ln.split(":", 1)
        cur[key.strip()] = [float(v) for v in vals.split()]
        if key.strip() == "q":
            cases.append((cur["x"], cur["s"][0], [int(v) for v in cur["q"]]))
            cur = {}
    return cases


def kv_bytes():
    per_token, totals = [], []
    for ln in _lines("kv_bytes_workshop.txt"):
        key, vals = ln.split(":", 1)
        v = vals.split()
        if key == "per_token":
            per_token.append(tuple(int(x) for x in v))
        else:
            totals.append((int(v[0]), int(v[1]), int(v[2]), int(v[3]), int(v[4]), int(v[5]),
                           float(v[6]), int(v[7])))
    return per_token, totals


def prefix_cache_cases():
    """[(bs, capacity, [(op, tokens, expected)])]; op in match / insert /
    state / evicted (see tests/golden/prefix_cache_lru.txt)."""
    cases = []
    for ln in _lines("prefix_cache_lru.txt"):
        op, _, rest = ln.partition(" ")
        if op == "case":
            bs, cap = (int(x) for x in rest.split())
            cases.append((bs, cap, []))
        elif op in ("match", "insert"):
            toks, _, res = rest.partition("=")
            cases[-1][2].append((op, [int(x) for x in toks.split()], [int(x) for x in res.split()]))
        elif op == "state":
            blocks = [tuple(int(x) for x in part.split()) for part in rest.split("|")]
            cases[-1][2].append((op, None, sorted(blocks)))
        elif op == "evicted":
            cases[-1][2].append((op, None, int(rest)))
        else:
            raise ValueError(f"prefix_cache_lru.txt: unknown line {ln!r}")
    return cases
