"""Grouping stage on the GPU, bit-exact against the oracle (moe_align)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from mixture_experts_expert_02_amd import binding as B

pytestmark = pytest.mark.gpu


def run_and_compare(ids: np.ndarray, E: int):
    T, k = ids.shape
    dev = torch.device("cuda")
    print(f"[align] T={T} k={k} E={E}", flush=True)
    counts, cu, perm, inv, ws = B.align(torch.from_numpy(ids.astype(np.int32)).to(dev), E)
    torch.cuda.synchronize()
    ref = oracle.align(ids, E)
    M = int(ref["offsets"][E])
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(cu.cpu().numpy(), ref["cu_seqlens"])
    p = perm.cpu().numpy()
    assert np.array_equal(p[:M], ref["perm"])
    assert np.all(p[M:] == -1)
    assert np.array_equal(inv.cpu().numpy(), ref["inv_perm"])
    assert B.moe_device_error(ws) == ref["n_bad"]


@pytest.mark.parametrize("name", ["tiny", "mixtral_prefill", "fine_grained_prefill", "mxfp4_decode"])
def test_align_workload_routing(name):
    wl = synth.workload(name)
    ids, _ = synth.make_routing(wl)
    run_and_compare(ids, wl.E)


@pytest.mark.parametrize("T,k,E,kind", [
    (1, 1, 1, "random"),
    (1, 4, 8, "random"),
    (1000, 1, 16, "one_expert"),          # every slot on one expert
    (5, 2, 300, "random"),                # more experts than slots
    (333, 3, 7, "masked_bad"),            # -1 and out-of-range ids mixed in
    (3000, 1, 2000, "random"),            # E > 1024: multi-workgroup path
    (1500, 3, 64, "masked_bad"),          # M > 4096: multi-workgroup path, ragged last chunk
    (100000, 4, 64, "random"),            # many chunks
    (5000, 8, 4096, "random"),            # largest supported E
    (257, 2, 3, "dups"),                  # duplicate ids in a token's row
    (64, 2, 8, "all_masked"),
])
def test_align_adversarial(T, k, E, kind):
    rng = np.random.default_rng(T * 31 + k * 7 + E)
    if kind == "one_expert":
        ids = np.full((T, k), E // 2)
    elif kind == "masked_bad":
        ids = rng.integers(-1, E + 3, size=(T, k))
        ids[rng.random((T, k)) < 0.1] = -7
    elif kind == "dups":
        ids = rng.integers(0, E, size=(T, k))
    elif kind == "all_masked":
        ids = np.full((T, k), -1)
    else:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if k <= E else rng.integers(0, E, (T, k))
    run_and_compare(ids.astype(np.int32), E)


def test_align_reuses_workspace_with_smaller_input():
    dev = torch.device("cuda")
    rng = np.random.default_rng(9)
    big = rng.integers(0, 32, size=(6000, 2)).astype(np.int32)
    small = rng.integers(-1, 40, size=(700, 2)).astype(np.int32)
    ws = B.alloc_workspace(B.moe_align_workspace_bytes(6000, 2, 32), dev)
    for ids in (big, small):
        counts, cu, perm, inv, _ = B.align(torch.from_numpy(ids).to(dev), 32, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.align(ids, 32)
        assert np.array_equal(inv.cpu().numpy(), ref["inv_perm"])
        assert B.moe_device_error(ws) == ref["n_bad"]
