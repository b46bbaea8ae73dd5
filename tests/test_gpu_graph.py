"""GPU: the forward calls captured in a HIP graph replay to the same bytes as eager launches.

Each replay is checked against the eager result, with the program's own eager work
(other launches of the library, a torch matmul, fresh inputs written into the captured
buffers) and synchronizations between the replays; the eager results themselves are
checked against the fp64 oracle."""

import numpy as np
import pytest
import torch

from oracle import pair_update_ref, tri_mul_ref
from pair_rep_triangle_amd.inputs import make_random, make_weights
from pair_rep_triangle_amd.trimul import TriMul
from tests.gpu_util import TOL, note, rel_err, to_device

pytestmark = pytest.mark.gpu


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype,n,c_z,c", [("bf16", 129, 128, 128), ("fp32", 70, 64, 32),
                                           ("bf16", 512, 128, 128)])
def test_graph_replays_match_eager(dtype, n, c_z, c):
    note(f"graph replay {dtype} n={n} cz={c_z} c={c}")
    d = make_random(1, n, c_z, c, seed=n, mask="block", random_affine=True)
    w_in = make_weights(np.random.default_rng(5), c_z, c, random_affine=True)
    z, m, z_host, m_host = to_device(d, dtype)
    mods = [("outgoing", TriMul(d["weights"], c_z, c, dtype)), ("incoming", TriMul(w_in, c_z, c, dtype))]
    ws = mods[0][1].new_workspace(1, n)
    outs = [torch.empty_like(z) for _ in mods]

    def step():
        for (direction, mod), out in zip(mods, outs):
            mod.forward(z, m, out=out, direction=direction, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    if n <= 129:  # the eager result itself against the oracle (the large case is covered elsewhere)
        for (direction, _), got, w in zip(mods, eager, (d["weights"], w_in)):
            ref = tri_mul_ref(z_host, m_host, w, direction)
            assert rel_err(got.to(torch.float64).cpu().numpy(), ref) <= TOL[dtype]

    g = _capture(step)
    other = make_random(1, n, c_z, c, seed=n + 1, mask="random_pairs")
    z2, m2, _, _ = to_device(other, dtype)
    a = torch.randn(256, 256, device="cuda")
    for r in range(4):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {r} differs from the eager result"
        # eager work between replays: other inputs through the same modules and workspace,
        # an unrelated torch kernel, then the captured inputs rewritten with their values
        mods[0][1].forward(z2, m2, direction="outgoing", workspace=ws)
        _ = a @ a
        torch.cuda.synchronize()
    # new values written into the captured input buffer are picked up by the replay
    z_saved = z.clone()
    z.copy_(z2)
    g.replay()
    torch.cuda.synchronize()
    for (direction, mod), o in zip(mods, outs):
        assert torch.equal(o, mod.forward(z2, m, direction=direction, workspace=ws))
    z.copy_(z_saved)


def test_graph_chained_pair_update_in_place():
    """The in-place chained pair update (outgoing then incoming, each with its residual add)
    captured once; each replay starts from a fresh copy of z written eagerly."""
    note("graph chained in place")
    n, c_z, c = 96, 64, 64
    d = make_random(1, n, c_z, c, seed=3, mask="random_residues", random_affine=True)
    w_in = make_weights(np.random.default_rng(9), c_z, c, random_affine=True)
    z, m, z_host, m_host = to_device(d, "bf16")
    out_mod, in_mod = TriMul(d["weights"], c_z, c, "bf16"), TriMul(w_in, c_z, c, "bf16")
    ws = out_mod.new_workspace(1, n)
    zi = z.clone()

    def step():
        out_mod.forward_residual(zi, m, out=zi, direction="outgoing", workspace=ws)
        in_mod.forward_residual(zi, m, out=zi, direction="incoming", workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = zi.clone()
    want = pair_update_ref(z_host, m_host, d["weights"], w_in)
    assert rel_err(eager.to(torch.float64).cpu().numpy(), want) <= TOL["bf16"]
    zi.copy_(z)
    g = _capture(step)  # the warm-up run and the capture leave zi changed
    for r in range(3):
        zi.copy_(z)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(zi, eager), f"replay {r} differs from the eager chained update"
