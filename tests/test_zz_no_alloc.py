"""moe_route_align_noalloc (the library's static device scratch in place of a
workspace) against moe_route_align with a caller workspace, through the C ABI:
every output bit-identical, on two calls in a row of which the second is
smaller (the scratch keeps the first call's contents), and the ids equal to
the oracle's."""

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle

import mixture_experts_routing_moe_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda"

KEYS = ("topk_w", "topk_ids", "counts", "offsets", "sorted_token_ids", "sorted_slot_ids",
        "slot_to_sorted")
MH_KEYS = ("multihot", "probs_in_multihot", "position_map")


def _logits(T, E, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((T, E)).astype(np.float32)
    x += (g.standard_normal(E) * np.sqrt(0.5)).astype(np.float32)[None, :]
    return x


def _check_pair(logits_np, k, with_multihot):
    T, E = logits_np.shape
    lg = torch.from_numpy(logits_np).to(DEV)
    ref = moe.moe_route_align(lg, k, True, with_multihot=with_multihot)
    # Outputs pre-filled with a pattern no call writes, so an unwritten entry shows.
    out = {key: torch.full_like(v, -7) for key, v in ref.items()}
    got = moe.moe_route_align_noalloc(lg, k, True, with_multihot=with_multihot, out=out)
    torch.cuda.synchronize()
    for key in KEYS + (MH_KEYS if with_multihot else ()):
        a, b = got[key], ref[key]
        if a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)
        assert torch.equal(a, b), f"T={T} E={E} k={k}: {key} differs"
    _, oids = oracle.route(logits_np, k, True)
    np.testing.assert_array_equal(got["topk_ids"].cpu().numpy(), oids)
    ra = oracle.align(oids, E)
    for key in ("counts", "offsets", "sorted_token_ids", "slot_to_sorted"):
        np.testing.assert_array_equal(got[key].cpu().numpy(), ra[key], err_msg=key)


@pytest.mark.parametrize("T1,T2,E,k,mh", [
    (16384, 3000, 64, 8, True),    # the routing workload, then a smaller batch (fused launches)
    (5000, 700, 128, 6, False),    # separate route and alignment launches
    (3000, 40, 64, 8, True),       # then a batch that needs no scratch (one block)
])
def test_noalloc_matches_workspace_call(T1, T2, E, k, mh):
    print(f"noalloc route_align T={T1} then T={T2}, E={E}, k={k}, multihot={mh}", flush=True)
    _check_pair(_logits(T1, E, T1 + E), k, mh)
    _check_pair(_logits(T2, E, T2 + E + 1), k, mh)


def test_noalloc_routing_workload():
    w = mi.WORKLOADS["routing"]
    print("noalloc route_align on the routing workload", flush=True)
    _check_pair(mi.gating_logits(w), w.k, True)
    _check_pair(mi.gating_logits(w)[:1111], w.k, True)
