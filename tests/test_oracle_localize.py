"""Pins of the localisation oracle (fla ``get_cp_cu_seqlens``).

* hand-worked examples under tests/golden/ (derived step by step from the
  page's algorithm);
* per-token brute-force enumeration (owner of every token, clip-and-drop
  pieces as in h3-blackwell-runtime ``localize_segments``) on random
  cu_seqlens with repeats, boundaries on shard edges and sequences spanning
  three or more shards;
* the numpy restatement and the C oracle agree everywhere.
"""
import os

import numpy as np
import pytest

from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "localize_hand_examples.txt")
FIELDS = ("rank_start", "rank_end", "num_local_seqs", "first_seq_global_idx", "is_first_rank",
          "is_last_rank", "pre_num_ranks", "post_num_ranks", "pre_num_conv_tokens", "n_halo")


def _golden():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, local, meta = (p.strip() for p in line.split("|"))
        cu, ws, rank, K = lhs.split()
        out.append(([int(c) for c in cu.split(",")], int(ws), int(rank), int(K),
                     [int(c) for c in local.split(",")], dict(zip(FIELDS, map(int, meta.split())))))
    return out


@pytest.mark.parametrize("case", _golden(), ids=lambda c: "cu%s_ws%d_r%d" % (len(c[0]), c[1], c[2]))
def test_golden_examples(case, oracle_lib):
    cu, ws, rank, K, local, meta = case
    for fn in (oracle_lib.localize, ref.localize_p1, ref.localize_bruteforce):
        got_local, got_meta = fn(cu, ws, rank, K)
        assert list(got_local) == local, fn
        assert got_meta == meta, fn


def random_cu(rng, n_seqs, ws, allow_empty=True, edge_align=True):
    """Random cu_seqlens whose total divides by ws; some boundaries are
    forced onto shard edges and some sequences are empty."""
    part = int(rng.integers(1, 40))
    total = part * ws
    cuts = sorted(int(c) for c in rng.integers(0, total + 1, size=n_seqs - 1))
    if edge_align and n_seqs > 2:
        for i in range(min(2, len(cuts))):
            cuts[int(rng.integers(len(cuts)))] = part * int(rng.integers(0, ws + 1))
        cuts.sort()
    if not allow_empty:
        cuts = sorted(set(c for c in cuts if 0 < c < total))
    return [0] + cuts + [total]


@pytest.mark.parametrize("ws", [1, 2, 3, 4, 8])
def test_bruteforce_random(ws, oracle_lib):
    rng = np.random.default_rng(100 + ws)
    n_cases = 0
    for trial in range(150):
        cu = random_cu(rng, int(rng.integers(1, 9)), ws, allow_empty=bool(trial % 2))
        for rank in range(ws):
            K = int(rng.integers(1, 6))
            bl, bm = ref.localize_bruteforce(cu, ws, rank, K)
            pl, pm = ref.localize_p1(cu, ws, rank, K)
            cl, cm = oracle_lib.localize(cu, ws, rank, K)
            assert list(bl) == list(pl) == list(cl), (cu, ws, rank)
            assert bm == pm == cm, (cu, ws, rank, bm, pm, cm)
            n_cases += 1
    assert n_cases >= 150 * ws


def test_long_sequence_spanning_ranks(oracle_lib):
    # one sequence over every shard: ranks in the middle neither start nor end it
    cu = [0, 3, 77, 80]
    for rank in range(8):
        local, meta = oracle_lib.localize(cu, 8, rank, 4)
        bl, bm = ref.localize_bruteforce(cu, 8, rank, 4)
        assert list(local) == list(bl) and meta == bm
    _, m = oracle_lib.localize(cu, 8, 4, 4)
    assert m["pre_num_ranks"] == 4 and m["post_num_ranks"] == 3
    assert m["is_first_rank"] == 0 and m["is_last_rank"] == 0
    assert m["pre_num_conv_tokens"] == 40 - 3 and m["n_halo"] == 3


def test_rejects_undefined_splits(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.localize([0, 5, 7], 2, 0, 4)      # 7 % 2 != 0
    with pytest.raises(ValueError):
        oracle_lib.localize([0, 4], 2, 2, 4)         # rank out of range
    with pytest.raises(ValueError):
        oracle_lib.localize([0, 0], 1, 0, 4)         # empty part
