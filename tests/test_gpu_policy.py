"""The adaptive residency loop on the GPU: counter -> snapshot -> policy ->
swaps, over a domain shift.

Two layers at the pages' geometry (384 experts, 295 hot / 89 cold rows; small
expert shapes, H = 256, I = 128), 16 tokens per step, traffic from the map's
own ranking (phase A), then from an independent ranking (B), then A again
("We Built the Counter", section 3: prose, then agent, then prose). Every
step runs the whole layer through the C ABI with the counter on
(moe_route_split); every `read_every` steps the table is snapshotted
(moe_usage_counts), the policy with the pages' rules decides, and its swaps
are applied with moe_swap_rows between steps ("We Built the Counter",
sections 2 and 5). After every barrier:
 - the device counter equals the host's count of the same picks;
 - both banks and the row map equal the oracle's swaps on host byte arrays;
 - one step's layer output is within tolerance of the oracle and
   bit-identical to the same step on an all-hot bank.
Then: the cold share of picks falls during phase B; a control-file freeze
stops all swaps; a control-file restore_map brings back every layer's
boot-time hot set."""
import json

import numpy as np
import pytest
import torch

import expert_weight_residency_amd as moe
import oracle
import synth
from expert_weight_residency_amd.layer import LayerBuffers, ResidencyLayer
from expert_weight_residency_amd.policy import (AdaptivePolicy, PolicyConfig, RuntimeControl,
                                                restore_swaps)
from gpu_util import MAX_REL, REL_L2, device_bank, host_bank, pinned_bank, rel_errors

pytestmark = pytest.mark.gpu

E, N_COLD, K, H, I, T, L, SEED = 384, 89, 6, 256, 128, 16, 2, 91
READ = 16          # steps per policy read (the pages read every 64 at larger step counts)
PHASE = 12 * READ  # steps per phase


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield


def _bank_equals(gbank, obank):
    return all(np.array_equal(getattr(gbank, t).cpu().numpy(), getattr(obank, t))
               for t in synth.TENSORS)


def test_policy_loop_domain_shift(tmp_path):
    perm_a = [synth.layer_permutation(E, SEED, l) for l in range(L)]
    perm_b = [synth.layer_permutation(E, SEED ^ 0x0FFD0, l) for l in range(L)]
    hot, cold, ob_hot, ob_cold, rm_dev, rm_host, ho, co, allhot, layers = ([] for _ in range(10))
    all_map, all_owner, _ = synth.all_hot_map(E)
    for l in range(L):
        rm, h_own, c_own = synth.fitted_map(E, N_COLD, SEED, l)
        hb, cb = host_bank(h_own, SEED, l, H, I), host_bank(c_own, SEED, l, H, I)
        hot.append(device_bank(hb))
        cold.append(pinned_bank(cb))
        ob_hot.append(oracle.Bank(**{k: v.copy() for k, v in hb.items()}))
        ob_cold.append(oracle.Bank(**{k: v.copy() for k, v in cb.items()}))
        rm_dev.append(torch.from_numpy(rm.copy()).cuda())
        rm_host.append(rm.copy())
        ho.append(h_own.copy())
        co.append(c_own.copy())
        allhot.append(device_bank(host_bank(all_owner, SEED, l, H, I)))
        layers.append(ResidencyLayer(hot[l], cold[l], rm_dev[l], H, I))
    boot_hot = [h.copy() for h in ho]
    all_dev = torch.from_numpy(all_map).cuda()
    empty_cold = moe.Bank(*[torch.empty(s, dtype=torch.uint8, device="cuda")
                            for s in synth.tensor_shapes(0, H, I).values()])
    counts = torch.zeros((L, E), dtype=torch.int32, device="cuda")
    snap = torch.empty((L, E), dtype=torch.int32, pin_memory=True)
    host_counts = np.zeros((L, E), np.int64)
    staging = torch.empty(moe.moe_expert_bytes(H, I), dtype=torch.uint8, device="cuda")
    bufs = LayerBuffers.allocate(T, K, H, I, E - N_COLD, N_COLD)
    bufs_all = LayerBuffers.allocate(T, K, H, I, E, 0)
    policy = AdaptivePolicy(L, E, PolicyConfig(read_every=READ, half_life=4 * READ))
    ctrl_path = tmp_path / "ctrl.json"
    control = RuntimeControl(policy, str(ctrl_path))
    x = synth.activations(T, H, SEED)
    x_d = torch.from_numpy(x.view(np.int16)).cuda()

    def routing(step, phase):
        out = []
        for l in range(L):
            pm = perm_b[l] if phase == 1 else perm_a[l]
            out.append(synth.skewed_routing(T, K, E, SEED, l, step, perm=pm))
        return out

    def run_step(step, phase, check=False):
        cold_picks = 0
        for l, (ids, w) in enumerate(routing(step, phase)):
            np.add.at(host_counts[l], ids.ravel(), 1)
            cold_picks += int((rm_host[l][ids] < 0).sum())
            ids_d = torch.from_numpy(ids).cuda()
            w_d = torch.from_numpy(w).cuda()
            layers[l].forward(x_d, ids_d, w_d, bufs, counts_layer=counts[l])
            if check:
                torch.cuda.synchronize()
                out = bufs.out[:T].cpu().numpy().view(np.uint16).copy()
                ResidencyLayer(allhot[l], empty_cold, all_dev, H, I).forward(
                    x_d, ids_d, w_d, bufs_all)
                torch.cuda.synchronize()
                out_all = bufs_all.out[:T].cpu().numpy().view(np.uint16)
                assert np.array_equal(out, out_all), (step, l)
                _, ref, bad = oracle.moe_layer(ob_hot[l], ob_cold[l], rm_host[l], ids, w, x, H, I)
                assert bad == 0
                e = rel_errors(out, ref)
                assert e[0] <= REL_L2 and e[1] <= MAX_REL, (step, l, e)
        return cold_picks

    applied_total = [0]

    def barrier(step):
        control.poll()
        moe.moe_usage_counts(counts, snap)
        torch.cuda.synchronize()
        assert np.array_equal(snap.numpy().astype(np.int64), host_counts), step
        policy.observe(snap.numpy())
        if control.restore_pending:
            props = restore_swaps(ho, co, boot_hot, limit=policy.cfg.swaps_per_barrier)
            if not props:
                control.restore_pending = False
        else:
            props = policy.decide(ho, co)
        for sw in props:
            l, a, b = sw.layer, sw.hot_row, sw.cold_row
            e_h, e_c = sw.expect_hot_expert, sw.expect_cold_expert
            moe.moe_swap_rows(hot[l], cold[l], a, b, e_h, e_c, rm_dev[l], ho[l], co[l], staging,
                              H, I)
            oh, oc = ho[l].copy(), co[l].copy()   # the mirrors before this swap
            oh[a], oc[b] = e_h, e_c
            oracle.swap_rows(ob_hot[l], ob_cold[l], a, b, e_h, e_c, rm_host[l], oh, oc)
        torch.cuda.synchronize()
        for l in range(L):
            assert np.array_equal(rm_dev[l].cpu().numpy(), rm_host[l]), (step, l)
            assert _bank_equals(hot[l], ob_hot[l]) and _bank_equals(cold[l], ob_cold[l]), (step, l)
        applied_total[0] += len(props)
        return len(props)

    share, swaps = [], []          # per read window: cold share of picks, swaps applied
    step = 0
    for phase in (0, 1, 0):
        for _ in range(PHASE // READ):
            cold_picks = 0
            for i in range(READ):
                cold_picks += run_step(step, phase, check=(i == READ - 1))
                step += 1
            share.append(cold_picks / (READ * L * T * K))
            swaps.append(barrier(step))
    n = PHASE // READ
    a1, b, a2 = share[:n], share[n:2 * n], share[2 * n:]
    print(f"cold share per window: A {np.round(a1, 3)} B {np.round(b, 3)} A {np.round(a2, 3)}; "
          f"swaps {swaps}", flush=True)
    assert max(a1) < 0.06                       # the fitted map: a few % cold
    assert b[0] > 0.15                          # the new ranking: far more cold
    assert np.mean(b[-3:]) < 0.7 * b[0]         # the policy follows the traffic
    assert sum(swaps[n:2 * n]) > 0

    # freeze: B traffic again, no swaps however skewed the counts
    ctrl_path.write_text(json.dumps({"freeze": True}))
    for _ in range(3):
        for i in range(READ):
            run_step(step, 1, check=(i == READ - 1))
            step += 1
        assert barrier(step) == 0
    assert policy.frozen

    # restore to the boot-time map (a queued restore runs even while frozen)
    ctrl_path.write_text(json.dumps({"freeze": True, "restore_map": True}))
    for _ in range(100):
        barrier(step)
        if not control.restore_pending:
            break
    assert not control.restore_pending
    for l in range(L):
        assert set(ho[l].tolist()) == set(boot_hot[l].tolist()), l
    run_step(step, 0, check=True)
    print(f"{applied_total[0]} swaps applied in all", flush=True)
