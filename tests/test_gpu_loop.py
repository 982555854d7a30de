"""The decode loop (32 sequences x 1,085 committed tokens, Zipf-skewed
routing, output hidden rows fed back as the next step's input, finished
sequences compacted out) on the GPU, with oracle spot checks: steps 0-2,
every 50th step and the first step after a compaction are checked
teacher-forced (every layer on the GPU's own input, the LM head on the GPU's
final rows, the accept rule on the oracle's argmax), and every step's input
rows are checked to be the previous step's output rows, row for row."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from parity import Tally, forced_stack
from speculative_decode_verification_router_amd import decode_loop, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd(gpu_lib):
    from speculative_decode_verification_router_amd import binding

    return binding


def _feedback_ok(prev, cur, K_prev):
    """cur's input rows are, per sequence in cur, the first K+1 output rows of
    that sequence in prev (last repeated), and nothing else."""
    pos = {int(s): i for i, s in enumerate(prev.seqs)}
    K = cur.K
    d = prev.outputs["h_out"].shape[1]
    out_prev = prev.outputs["h_out"].reshape(len(prev.seqs), K_prev + 1, d)
    want = np.stack([out_prev[pos[int(s)], np.minimum(np.arange(K + 1), K_prev)] for s in cur.seqs])
    return np.array_equal(want.reshape(-1, d), cur.h_in_host)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("K", [3])
def test_zipf_decode_loop_spot_checks(bd, K):
    import torch

    dims = synth.DS3B_BF16
    wl = synth.WORKLOADS["zipf_loop_c32"]
    W = synth.workload_weights(wl)
    model = bd.DeviceModel(dims, W, max_tokens=wl.batch * (K + 1))
    B0, target, p = wl.batch, 1085, 0.6
    h0 = bd.to_device(synth.make_hidden(dims, B0 * (K + 1), 0, wl.code))

    def draw(step, g, seqs):
        return synth.make_drafts(g, p, dims.vocab, seed=0, step=step, code=wl.code)

    res = decode_loop.run_loop(bd, model, h0, B0, target, decode_loop.FixedK(K), K, draw_drafts=draw,
                               record=lambda s, c: True)
    torch.cuda.synchronize()
    steps = res.steps
    assert res.committed == B0 * target
    for st in steps:
        st.h_in_host = bd.to_host(st.h_in)
    # every step's input rows are the previous step's output rows
    for prev, cur in zip(steps, steps[1:]):
        assert _feedback_ok(prev, cur, prev.K), f"step {cur.index}: input rows are not the previous outputs"
    # commits add up per sequence and the loop stops each one at its target
    done = np.zeros(B0, np.int64)
    for st in steps:
        done[st.seqs] += st.outputs["n_committed"]
    assert np.all(done >= target) and np.all(done - target <= K)

    first_compacted = next(st.index for st in steps if st.compacted and st.index > 0)
    check = sorted({0, 1, 2, first_compacted} | set(range(50, len(steps), 50)))
    print(f"{len(steps)} steps, first compaction at step {first_compacted}; checking steps {check}")
    total_checked = total = 0
    for i in check:
        st = steps[i]
        B = len(st.seqs)
        pick = np.unique([0, B - 1])               # first and last running sequence
        rows = (pick[:, None] * (K + 1) + np.arange(K + 1)[None, :]).reshape(-1)
        label = f"loop step {i} (B={B})"
        tally, h_fin, lm = forced_stack(bd, torch, dims, W, model, st.h_in, rows, label)
        assert np.array_equal(h_fin, st.outputs["h_out"]), f"{label}: chain and step end in different states"
        tally.argmax(st.outputs["argmax"][rows], lm["argmax"], lm["margin"])
        g_ref = np.asarray(lm["argmax"]).reshape(len(pick), K + 1)
        drafts = bd.to_host(st.drafts)[pick]
        r_acc, r_com, r_ncom = O.spec_accept(g_ref, drafts)
        gpu_c = {k: st.outputs[k][pick] for k in ("n_accepted", "committed", "n_committed")}
        tally.commits(len(pick), K, gpu_c, dict(n_accepted=r_acc, committed=r_com, n_committed=r_ncom))
        tally.assert_ok(label, min_checked=0.5)
        total_checked += tally.checked
        total += tally.T
    print(f"loop spot checks: {total_checked}/{total} tokens checked to the end")
    assert total_checked >= 0.75 * total
