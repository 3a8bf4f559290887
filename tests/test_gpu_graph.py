"""The step's entry points inside a HIP graph.

zs_adamw_step and zs_gather_unit allocate nothing and never synchronize, so a
caller can capture them (here with torch.cuda.graph) and replay the launches.
One fused step on a rank's shard plus the gather of its unit is captured once
and replayed three times, with eager work and synchronizations between the
replays; after every replay the state, the working shard and the unit buffer
equal the same calls made eagerly on a second copy of the inputs, bit for
bit, and the oracle."""
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
import workloads as W
from gpu_util import check_bf16, check_bits, check_f32, device, to_np
from oracle import zs_oracle as O

pytestmark = pytest.mark.gpu


def test_step_and_gather_replay_from_a_graph():
    dev = device()
    D = 8
    S = 100_008          # 97 tile pairs and a tail of 680; 16-byte shards for the gather
    hp = zs.AdamWHP(step=1, **W.ADAMW_HP)
    ohp = O.AdamWHP(step=1, **W.ADAMW_HP)
    cs = [W.as_bf16_bits(W.normal_f32(S, W.GRAD_SCALE, 40 + k, dev)) for k in range(D)]
    peers = [W.as_bf16_bits(W.normal_f32(S, 0.02, 80 + r, dev)) for r in range(D - 1)]

    def state():
        return (W.master_init(S, 9, dev), torch.zeros(S, device=dev), torch.zeros(S, device=dev),
                torch.zeros(S, dtype=torch.int16, device=dev))

    # the same launches once, eagerly, on scratch buffers: the library's code
    # is loaded before the capture starts
    sp, sm, sv, sw = state()
    zs.zs_adamw_step(sp, sm, sv, sw, cs, hp)
    zs.zs_gather_unit([sw] + peers, torch.empty(D * S, dtype=torch.int16, device=dev))
    torch.cuda.synchronize()

    gp, gm, gv, gw = state()                 # advanced by the graph
    ep, em, ev, ew = state()                 # advanced eagerly
    gflat = torch.zeros(D * S, dtype=torch.int16, device=dev)
    eflat = torch.zeros(D * S, dtype=torch.int16, device=dev)
    op, om, ov = to_np(ep), to_np(em), to_np(ev)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        zs.zs_adamw_step(gp, gm, gv, gw, cs, hp)
        zs.zs_gather_unit([gw] + peers, gflat)
    torch.cuda.synchronize()
    # capturing ran nothing: the graph's copy still holds the initial state
    check_bits(to_np(gp), op, "p after capture")
    assert not to_np(gflat).any()

    for rep in range(3):
        graph.replay()
        zs.zs_adamw_step(ep, em, ev, ew, cs, hp)
        zs.zs_gather_unit([ew] + peers, eflat)
        torch.cuda.synchronize()
        for a, b, what in ((gp, ep, "p"), (gm, em, "m"), (gv, ev, "v"), (gw, ew, "w"),
                           (gflat, eflat, "unit")):
            check_bits(to_np(a), to_np(b), f"replay {rep}: {what}, graph against eager")
        op, om, ov, ow = O.rank_step(op, om, ov, [to_np(c) for c in cs], O.BF16, ohp)
        check_f32(to_np(gp), op, f"replay {rep} p", exact=True)
        check_f32(to_np(gm), om, f"replay {rep} m", exact=True)
        check_f32(to_np(gv), ov, f"replay {rep} v", exact=True)
        check_bf16(to_np(gw), ow, f"replay {rep} w", exact=True)
        check_bits(to_np(gflat), O.gather_unit([ow] + [to_np(x) for x in peers]),
                   f"replay {rep} unit")
