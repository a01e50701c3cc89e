"""Record that an earlier revision of oracle/swiftkv_oracle.py computes what the current one does.

The stored full-size oracle results (tests/golden/fullsize/*.npz) name the
SHA-256 of the oracle source that wrote them.  A later edit that touches only
comments or docstrings leaves every result the same, but changes that hash.
This script takes the earlier revision's source from git, checks that its
code (the module's syntax tree with docstrings removed) is identical to the
current file's, and records the earlier raw hash against the code hash in
tests/golden/fullsize/oracle_equivalents.json, which the fixture tests accept
in place of a matching raw hash.  It refuses when the code differs: then the
stored results must be written again by make_fullsize_fixtures.py.

Usage (from the repository root): python tests/golden/record_oracle_equivalence.py <git revision>
"""
import hashlib
import json
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from tests.helpers import oracle_code_sha256  # noqa: E402

ORACLE = "oracle/swiftkv_oracle.py"
OUT = os.path.join(HERE, "fullsize", "oracle_equivalents.json")


def main(rev: str) -> None:
    old = subprocess.run(["git", "show", f"{rev}:{ORACLE}"], cwd=ROOT, check=True, capture_output=True).stdout
    cur = open(os.path.join(ROOT, ORACLE), "rb").read()
    old_code, cur_code = oracle_code_sha256(old), oracle_code_sha256(cur)
    if old_code != cur_code:
        sys.exit(f"{ORACLE} at {rev} differs in code from the current file: write the stored results again")
    table = json.load(open(OUT)) if os.path.exists(OUT) else {}
    table[hashlib.sha256(old).hexdigest()] = cur_code
    with open(OUT, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"recorded {hashlib.sha256(old).hexdigest()} -> code {cur_code}")


if __name__ == "__main__":
    main(sys.argv[1])
