"""GPU localisation (gdn_localize_cu_seqlens) against the oracle: bit-exact
local cu_seqlens and metadata on random packed batches, device-side status
codes, and the sharded benchmark workload."""
import numpy as np
import pytest
import torch

from linear_attention_sequence_causal_amd import gdn, workloads
from oracle import capi
from tests.test_oracle_localize import random_cu

pytestmark = pytest.mark.gpu


def _run(cu, ws, rank, K):
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    local, meta = gdn.gdn_localize_cu_seqlens(cu_d, int(cu[-1]), ws, rank, K)
    return local.cpu().numpy(), gdn.read_meta(meta)


def _compare(cu, ws, rank, K):
    local, meta = _run(cu, ws, rank, K)
    want_local, want = capi.localize(cu, ws, rank, K)
    n = meta["num_local_seqs"]
    assert meta["status"] == gdn.META_OK
    assert list(local[:n + 1]) == list(want_local), (cu, ws, rank)
    part = cu[-1] // ws
    assert all(int(x) == part for x in local[n + 1:])  # padding = empty trailing sequences
    for key, val in want.items():
        assert meta[key] == val, (key, cu, ws, rank)


@pytest.mark.parametrize("ws", [1, 2, 3, 4, 8])
def test_random_batches_bit_exact(ws):
    rng = np.random.default_rng(200 + ws)
    for trial in range(40):
        cu = random_cu(rng, int(rng.integers(1, 12)), ws, allow_empty=bool(trial % 2))
        for rank in range(ws):
            _compare(cu, ws, rank, int(rng.integers(1, 6)))


def test_many_sequences_multiple_tiles():
    # more sequences than one workgroup pass (256) exercises the tiled scan
    rng = np.random.default_rng(7)
    lengths = rng.integers(0, 5, size=1000)
    lengths[-1] += 8 - (lengths.sum() % 8)
    cu = [0] + list(np.cumsum(lengths))
    for rank in range(8):
        _compare(cu, 8, rank, 4)


def test_device_status_codes():
    _, meta = _run([0, 5, 3, 8], 2, 0, 4)
    assert meta["status"] == gdn.META_NOT_MONOTONE
    cu_d = torch.tensor([0, 4, 8], dtype=torch.int32, device="cuda")
    _, m = gdn.gdn_localize_cu_seqlens(cu_d, 10, 2, 0, 4)  # total disagrees with cu[-1]
    assert gdn.read_meta(m)["status"] == gdn.META_BAD_TOTAL


def test_host_errors():
    cu_d = torch.tensor([0, 4, 9], dtype=torch.int32, device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_localize_cu_seqlens(cu_d, 9, 2, 0, 4)
    assert e.value.code == gdn.GDN_EINVAL


def test_sharded_workload():
    spec = workloads.config("shard3of8_32k_h16_d128_bf16")
    rng = np.random.default_rng(spec.seed)
    lengths = workloads._draw_lengths(rng, spec.length_rule)
    cu = [0] + list(np.cumsum(lengths))
    assert cu[-1] == 32768
    _compare(cu, spec.world_size, spec.rank, spec.K)
    _, meta = _run(cu, 8, 3, 4)
    assert meta["num_local_seqs"] >= 2 and meta["pre_num_ranks"] >= 1
    print("  sharded workload seed %d: %s" % (spec.seed, meta))
