"""Host-side check that the row top-k's branch rows (topk_branch_rows) take
the branch of the sampled pass each is named after; no GPU."""
from topk_branch_rows import branch_rows, sampled_branch


def test_topk_branch_rows_take_their_branch():
    for name, (row, k) in branch_rows().items():
        assert sampled_branch(row, k) == name, (name, sampled_branch(row, k))
