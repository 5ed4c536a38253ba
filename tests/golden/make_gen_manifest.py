"""Writes gen_manifest.json: SHA-256 of every array the seeded generators
produce for each named workload at seed 0. Calls only the generators."""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import gen  # noqa: E402


def main():
    out = {}
    for name in gen.CONFIG_NAMES:
        case = gen.make_config(name, seed=0)
        out[name] = gen.sha256_manifest(case.arrays())
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gen_manifest.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
