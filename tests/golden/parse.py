"""Parsers for the text fixtures in this folder (no arithmetic of the method)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def page_figures():
    rows = []
    with open(os.path.join(HERE, "page_figures.txt"), encoding="utf-8") as f:
        for line in f:
            body, _, cite = line.partition("#")
            body = body.strip()
            if not body:
                continue
            name, *kvs = body.split()
            d = {}
            for kv in kvs:
                k, v = kv.split("=")
                d[k] = float(v)
            rows.append((name, d, cite.strip()))
    return rows


def lloyd_max_table():
    out = {}
    with open(os.path.join(HERE, "lloyd_max_gaussian.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            d = {}
            for kv in line.split():
                k, v = kv.split("=")
                d[k] = [float(t) for t in v.split(",") if t] if k in ("thresholds", "outputs") else float(v)
            out[int(d["levels"])] = d
    return out
