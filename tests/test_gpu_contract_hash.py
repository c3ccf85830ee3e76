"""The numerical contract's bits, pinned per contract version: sha256 of the
GPU outputs on fixed seeded inputs must equal the record of the library's
rlk_contract_version() ("vLLM RL-Kernel v0.1.0: Bitwise Train-Rollout
Consistency on ROCm", "The Numerical Execution Contract": equal version and
equal inputs give identical bits).  A self-pin on the GPU's own bits, not a
parity reference (tests/contract/cases.py)."""
import pytest

import selected_token_lm_amd as rlk
from tests.contract.cases import compute, load
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_outputs_match_the_contract_record():
    v = str(rlk.contract_version())
    rec = load().get(v)
    assert rec is not None, (f"no bit record for contract version {v}: record one with "
                             f"`python -m tests.contract.record_hashes` on a GPU")
    got = compute()
    diff = [f"{c}.{o}" for c in rec for o in rec[c] if got.get(c, {}).get(o) != rec[c][o]]
    say(f"  contract v{v}: {sum(len(x) for x in rec.values())} digests, {len(diff)} differ {diff}")
    assert not diff, f"bits changed under contract version {v}: {diff}"
    assert set(got) == set(rec)
