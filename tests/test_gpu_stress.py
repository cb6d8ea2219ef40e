"""The persistent kernel's exchange protocol under stress (through the C ABI):
flint_stack_decode_stress injects pseudo-random delays before every exchange
store and permutes the workgroups' roles inside each XCD.  With the normal
wait limit the results must be bit-identical to flint_stack_decode's (the
arithmetic and every reduction order are unchanged); with a tiny limit every
wait must give up, the watchdog flag must be raised and the kernel must
return (no hang), and after the workspace is zeroed the plan decodes
correctly again."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    from nvfp4_bit_projection_amd import flint, workload
    torch.cuda.set_device(0)
    return flint, workload


def make_stack(F, E, L, V):
    flint, workload = F
    dims = synth.MoEDims(n_experts=E)
    layers = [workload.build_layer(dims, seed=l) for l in range(L)]
    head = workload.build_head(V, dims.hidden)
    d = flint.dims_struct(dims.hidden, dims.n_experts, dims.expert_width, dims.top_k, dims.shared_width)
    return flint.Stack(d, layers, head, V, schedule=flint.SCHEDULE_PERSISTENT), dims


@pytest.mark.parametrize("E,L,V,T,seeds", [(32, 3, 4099, 3, (1, 2)), (256, 4, 16385, 2, (7,))])
def test_stress_identical(F, E, L, V, T, seeds):
    _, workload = F
    stack, dims = make_stack(F, E, L, V)
    x = workload.tokens(range(300, 300 + T), dims.hidden)
    r0 = torch.zeros((T, L, dims.top_k), dtype=torch.int32, device="cuda")
    lg0, am0 = stack.decode(x, routes=r0)
    torch.cuda.synchronize()
    assert stack.error() == 0
    for seed in seeds:
        print(f"stress decode E={E} L={L} T={T} seed={seed}", flush=True)
        r1 = torch.zeros_like(r0)
        lg1, am1 = stack.decode_stress(x, seed, 1 << 22, routes=r1)
        torch.cuda.synchronize()
        assert stack.error() == 0
        assert torch.equal(r1, r0)
        assert torch.equal(am1, am0)
        assert torch.equal(lg1.view(torch.int32), lg0.view(torch.int32))


def test_stress_watchdog_gives_up_and_recovers(F):
    """A wait limit of 4 polls with delays of microseconds: the waits give up,
    the flag is raised and every workgroup leaves the kernel; zeroing the
    workspace makes the plan usable again."""
    _, workload = F
    stack, dims = make_stack(F, 32, 3, 4099)
    x = workload.tokens(range(400, 402), dims.hidden)
    lg0, am0 = stack.decode(x)
    torch.cuda.synchronize()
    assert stack.error() == 0
    print("stress decode with a wait limit of 4 polls", flush=True)
    stack.decode_stress(x, 3, 4)
    torch.cuda.synchronize()
    assert stack.error() != 0
    stack.ws.zero_()
    lg1, am1 = stack.decode(x)
    torch.cuda.synchronize()
    assert stack.error() == 0
    assert torch.equal(am1, am0) and torch.equal(lg1, lg0)
