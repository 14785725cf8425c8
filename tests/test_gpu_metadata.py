"""GPU metadata value checks (lora_check_metadata, through the C ABI) against the oracle's rules:
the number of the first rule broken must be the same, on the valid workloads and on planted
violations of each rule (every device access of the check is bounded, so invalid values are
safe inputs)."""

import numpy as np
import pytest
import torch

import lora_inputs as li
from oracle import validate_metadata

pytestmark = pytest.mark.gpu


def _check(T, L, R, N, indptr, widx, perm, ranks, offs):
    alp = __import__("adapter_lora_projection_amd")
    g = lambda a: None if a is None else torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    got = alp.check_metadata(g(indptr), g(widx), g(ranks), R, T, permutation=g(perm),
                             slice_offsets=g(offs), N=N)
    ref = validate_metadata(T, L, R, N, indptr, widx, np.arange(T) if perm is None else perm, ranks,
                            offs)
    assert got == ref, (got, ref)
    return got


def _base():
    c = li.config_decode_qkv(T=200)
    return dict(T=c.T, L=c.L, R=c.R, N=c.N, indptr=c.seg_indptr.numpy().copy(),
                widx=c.weight_indices.numpy().copy(), perm=c.permutation.numpy().copy(),
                ranks=c.lora_ranks.numpy().copy(), offs=c.slice_offsets.numpy().copy())


@pytest.mark.parametrize("maker", [li.config_tiny_f32, li.config_decode_qkv, li.config_irregular])
def test_valid_workloads(maker):
    c = maker()
    print("case", c.name, flush=True)
    assert _check(c.T, c.L, c.R, c.N, c.seg_indptr.numpy(), c.weight_indices.numpy(),
                  c.permutation.numpy(), c.lora_ranks.numpy(), c.slice_offsets.numpy()) == 0


def _mut(name):
    d = _base()
    if name == "indptr_start":
        d["indptr"][0] = 1
    elif name == "indptr_end":
        d["indptr"][-1] = d["T"] - 1
    elif name == "indptr_decreasing":
        d["indptr"][2] = d["indptr"][1] - 1
    elif name == "index_high":
        d["widx"][1] = d["L"]
    elif name == "index_negative":
        d["widx"][0] = -1
    elif name == "rank_high":
        d["ranks"][2] = d["R"] + 1
    elif name == "rank_negative":
        d["ranks"][0] = -3
    elif name == "perm_duplicate":
        d["perm"][5] = d["perm"][6]
    elif name == "perm_out_of_range":
        d["perm"][7] = d["T"]
    elif name == "perm_negative":
        d["perm"][3] = -1
    elif name == "slices_end":
        d["offs"][-1] = d["N"] + 1
    elif name == "slices_decreasing":
        d["offs"][2] = d["offs"][1] - 1
    elif name == "two_rules":  # the lower rule number is reported
        d["ranks"][0] = -1
        d["perm"][1] = d["perm"][0]
    return d


@pytest.mark.parametrize("name", ["indptr_start", "indptr_end", "indptr_decreasing", "index_high",
                                  "index_negative", "rank_high", "rank_negative", "perm_duplicate",
                                  "perm_out_of_range", "perm_negative", "slices_end",
                                  "slices_decreasing", "two_rules"])
def test_planted_violations(name):
    print("case", name, flush=True)
    d = _mut(name)
    assert _check(**d) != 0


def test_unchecked_parts():
    d = _base()
    print("case unchecked", flush=True)
    # the permutation and the slices are not checked when not given
    d["perm"] = None
    assert _check(**d) == 0
    alp = __import__("adapter_lora_projection_amd")
    g = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    assert alp.check_metadata(g(d["indptr"]), g(d["widx"]), g(d["ranks"]), d["R"], d["T"]) == 0
