"""ca_cluster enqueues the query trees' levels on the caller's stream and the
key trees' levels on a library side stream, forked from the caller's stream
and joined back to it by events, so the call must be ordered on the caller's
stream as a whole. Checked by calling it from two host threads at once, each
on its own stream, and reading the outputs on that stream right after each
call (no device-wide synchronisation in between): every result must equal the
sequential run on the default stream bit for bit."""
import threading

import pytest

import synth

pytestmark = pytest.mark.gpu


def _inputs(dev, h0):
    import torch
    w = synth.WORKLOADS["video_32760"]
    Qn, Kn, _ = synth.generate(w, heads=slice(h0, h0 + 2), N=4000)
    return tuple(torch.from_numpy(x).to(torch.bfloat16).to(dev).contiguous() for x in (Qn, Kn))


def _outputs(cr):
    return [t.clone() for t in (cr.perm_q, cr.perm_k, cr.cent_q, cr.cent_k, cr.counts)]


@pytest.mark.parametrize("opts", [{}, {"cluster_size_k": 256}, {"split_mode": "diag"}])
def test_cluster_two_threads_match_sequential(ca, opts):
    import torch
    dev = torch.device("cuda:0")
    ins = [_inputs(dev, 0), _inputs(dev, 2)]
    ref = [_outputs(ca.cluster(Q, K, 128, seed=3, **opts)) for Q, K in ins]
    torch.cuda.synchronize()

    out, err = [None, None], []
    barrier = threading.Barrier(2)

    def work(i):
        try:
            s = torch.cuda.Stream()
            res = []
            with torch.cuda.stream(s):
                Q, K = ins[i]
                barrier.wait(timeout=120)
                for _ in range(3):
                    res.append(_outputs(ca.cluster(Q, K, 128, seed=3, **opts)))
            s.synchronize()
            out[i] = res
        except Exception as e:      # reported by the main thread
            err.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=240)
    assert not any(t.is_alive() for t in threads), "a clustering thread did not finish"
    assert not err, err
    for i in range(2):
        for rep, res in enumerate(out[i]):
            for a, b in zip(res, ref[i]):
                assert torch.equal(a, b), (opts, i, rep)
