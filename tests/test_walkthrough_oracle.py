"""The pages' worked example (nine-step RadixAttention walkthrough) on the
oracle tree.  CPU only."""
from oracle.radix import OracleTree
from tests import walkthrough


def test_nine_steps_oracle():
    walkthrough.run(lambda P: OracleTree(P))
