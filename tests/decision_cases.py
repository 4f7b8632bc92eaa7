"""Loader of the hand-worked compress-or-acquire cases in
tests/golden/growpage_decision.txt (shared by the oracle pins and the GPU
parity test)."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "growpage_decision.txt")
DECISIONS = {"none": 0, "acquire": 1, "compress": 2}
PAGE = 16


def load():
    """List of dicts: name, Hkv, tau, ctx, page_max [2, 1, Hkv, npg] (fp64),
    and the expected ws_size [2, Hkv], union [2], decision, victim."""
    cases, cur = [], None
    with open(GOLDEN) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(" ")
            rest = rest.strip()
            if key == "case":
                cur = {"name": rest, "fast": {}, "slow": {}}
            elif key in ("hkv", "ctx"):
                cur[key] = int(rest)
            elif key == "tau":
                cur["tau"] = float(rest)
            elif key in ("fast", "slow"):
                g, _, vals = rest.partition(":")
                cur[key][int(g)] = [float(v) for v in vals.split()]
            elif key in ("ws_size", "union", "victim"):
                cur[key] = [int(v) for v in rest.lstrip(":").split()]
            elif key == "decision":
                cur["decision"] = DECISIONS[rest.lstrip(":").strip()]
            elif key == "end":
                hkv = cur["hkv"]
                npg = -(-cur["ctx"] // PAGE)
                pm = np.full((2, 1, hkv, max(npg, 1)), -np.inf)
                for k, which in enumerate(("fast", "slow")):
                    for g in range(hkv):
                        assert len(cur[which][g]) == npg, (cur["name"], which, g)
                        pm[k, 0, g, :npg] = cur[which][g]
                cases.append({"name": cur["name"], "Hkv": hkv, "tau": cur["tau"],
                              "ctx": cur["ctx"], "page_max": pm,
                              "ws_size": np.array(cur["ws_size"]).reshape(2, hkv),
                              "union": np.array(cur["union"]), "decision": cur["decision"],
                              "victim": cur["victim"][0]})
                cur = None
    return cases
