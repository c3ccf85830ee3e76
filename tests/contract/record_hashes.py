"""Writes the record of the current contract version into hashes.json (run
on a GPU after an intended bit change, together with a new contract
version):

    python -m tests.contract.record_hashes [--out PATH]

(--out writes the updated record elsewhere, e.g. to copy back from a remote
GPU run, instead of overwriting hashes.json.)
"""
import json
import sys

import selected_token_lm_amd as rlk
from tests.contract.cases import RECORD, compute, load


def main():
    v = str(rlk.contract_version())
    rec = load()
    if v in rec and "--force" not in sys.argv:
        raise SystemExit(f"contract version {v} is already recorded; a bit change needs a new version")
    rec[v] = compute()
    out = sys.argv[sys.argv.index("--out") + 1] if "--out" in sys.argv else RECORD
    with open(out, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec[v], indent=1))


if __name__ == "__main__":
    main()
