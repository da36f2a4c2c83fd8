"""GPU parity of lowbit_gemv_chain (dependent GEMV stages in one persistent
launch) against the CPU oracle, through the C ABI.

Stages are chained for real: the y of one stage is the x of the next, every
output buffer starts as NaN, and a second run with a different first input
must not see the first run's values -- so a stage that read its input before
the previous stage finished would show up as a mismatch.  Each stage is
compared with the oracle applied to the input that stage actually read
(rel-L2 <= 1e-3, max |error| <= 1e-2 * max |y_ref|)."""
import numpy as np
import pytest
import torch

import bit_weight_only_pack_amd as lb
import oracle
from bit_weight_only_pack_amd import synth
from gpu_util import assert_close, dev, f16_to_f64, pack_w4

pytestmark = pytest.mark.gpu

WL = 600


def _ref(w, x_bits, G):
    _, yb = oracle.w4_matmul(x_bits.view(np.float16), "f16", w["qweight"], w["scales"], w["zeros"], G, "f16")
    return f16_to_f64(yb)


class Chain:
    """A chain built from [(stage, N, K)] with weights drawn per problem.
    inputs: problem index -> 'x0' (an external input) or the index of the
    problem whose y it reads."""

    def __init__(self, M, G, asym, probs, inputs, spin_limit=0, seed=0):
        self.M, self.G, self.asym = M, G, asym
        self.w, self.packed, self.x, self.y = [], [], [], []
        self.fmt = lb.LOWBIT_W4_ASYM if asym else lb.LOWBIT_W4_SYM
        self.ext = {}
        for i, (st, N, K) in enumerate(probs):
            w = synth.w4_weights(N, K, G, asym=asym, scale_range=(0.01, 0.03), workload_id=WL, layer=seed, part=i)
            self.w.append(w)
            self.packed.append(pack_w4(w, G)[1])
            self.y.append(torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda"))
        for i, (st, N, K) in enumerate(probs):
            src = inputs[i]
            if src == "x0":
                xb = torch.empty((M, K), dtype=torch.float16, device="cuda")
                self.ext[i] = xb
                self.x.append(xb)
            else:
                assert probs[src][1] == K and probs[src][0] == st - 1
                self.x.append(self.y[src])
        self.probs = probs
        self.items = lb.make_gemv_problems([(self.packed[i], self.x[i], self.y[i], N, K)
                                            for i, (_, N, K) in enumerate(probs)])
        stages = [p[0] for p in probs]
        nb = lb.lowbit_gemv_chain_bytes(len(probs), stages[-1] + 1)
        assert nb > 0
        self.buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
        self.chain = lb.lowbit_gemv_chain()
        lb.check(lb.lowbit_gemv_chain_init(self.chain, self.fmt, M, G, len(probs), self.items, stages, spin_limit,
                                           self.buf, nb))

    def set_inputs(self, seed):
        for i, xb in self.ext.items():
            K = self.probs[i][2]
            x = synth.activations_f16(self.M, K, workload_id=WL, layer=seed, part=i)
            xb.copy_(dev(x))

    def run(self):
        lb.check(lb.lowbit_gemv_chain_run(self.chain))
        torch.cuda.synchronize()

    def outputs(self):
        return [y.cpu().numpy().view(np.uint16) for y in self.y]


def _check(ch, inputs, seed):
    ch.set_inputs(seed)
    ext = {i: xb.cpu().numpy().view(np.uint16) for i, xb in ch.ext.items()}
    for y in ch.y:
        y.fill_(float("nan"))
    ch.run()
    st, err = lb.lowbit_gemv_chain_error(ch.chain)
    assert st == 0 and err == 0
    outs = ch.outputs()
    for i, (s, N, K) in enumerate(ch.probs):
        x_bits = ext[i] if inputs[i] == "x0" else outs[inputs[i]]
        assert_close(f16_to_f64(outs[i]), _ref(ch.w[i], x_bits, ch.G), "problem %d (stage %d)" % (i, s))
    return outs


DEP = [(0, 384, 256), (1, 512, 384), (2, 256, 512), (2, 72, 512), (3, 96, 256)]
DEP_IN = ["x0", 0, 1, 1, 2]


@pytest.mark.parametrize("M,G,asym", [(1, 128, False), (1, 32, True), (2, 64, False), (3, 32, True), (4, 128, True)])
def test_chain_dependent_stages(M, G, asym):
    ch = Chain(M, G, asym, DEP, DEP_IN, seed=M)
    a = _check(ch, DEP_IN, seed=1)
    b = _check(ch, DEP_IN, seed=2)               # new input: no stage may see run 1's values
    assert not np.array_equal(a[-1], b[-1])


def test_chain_deterministic_and_replayable():
    ch = Chain(1, 128, False, DEP, DEP_IN, seed=7)
    ch.set_inputs(5)
    ch.run()
    first = ch.outputs()
    for _ in range(3):
        for y in ch.y:
            y.fill_(float("nan"))
        ch.run()
        assert all(np.array_equal(u, v) for u, v in zip(first, ch.outputs()))
    # replayed from a HIP graph, with eager work between replays
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        lb.check(lb.lowbit_gemv_chain_run(ch.chain, stream))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            lb.check(lb.lowbit_gemv_chain_run(ch.chain, stream))
    torch.cuda.synchronize()
    for rep in range(3):
        for y in ch.y:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert all(np.array_equal(u, v) for u, v in zip(first, ch.outputs())), "replay %d" % rep
    st, err = lb.lowbit_gemv_chain_error(ch.chain)
    assert st == 0 and err == 0


def test_chain_ragged_and_long_k():
    """Ragged N (not a multiple of 16), K not a multiple of 128 or of the 4096-K
    round, and K above one round (several rounds per strip)."""
    probs = [(0, 33, 160), (0, 96, 9216), (1, 1000, 96)]
    inputs = ["x0", "x0", 1]
    ch = Chain(2, 32, True, probs, inputs, seed=3)
    _check(ch, inputs, seed=4)


def test_chain_decode_layer_shapes_sampled():
    """Two Llama-3-8B layers at M=1, G=128, as the decode step runs them:
    q+k+v | o | gate+up | down per layer (8 stages, 14 GEMVs, independent
    inputs).  Every output row is computed; 64 seeded rows per problem are
    checked against the oracle."""
    projs = {name: (K, N) for name, K, N in synth.LLAMA3_8B_PROJS}
    groups = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    probs, names = [], []
    for layer in range(2):
        for gi, g in enumerate(groups):
            for name in g:
                K, N = projs[name]
                probs.append((layer * 4 + gi, N, K))
                names.append(name)
    ch = Chain(1, 128, False, probs, ["x0"] * len(probs), seed=11)
    ch.set_inputs(12)
    ext = {i: xb.cpu().numpy().view(np.uint16) for i, xb in ch.ext.items()}
    ch.run()
    st, err = lb.lowbit_gemv_chain_error(ch.chain)
    assert st == 0 and err == 0
    outs = ch.outputs()
    r = np.random.default_rng(13)
    for i, (s, N, K) in enumerate(probs):
        rows = np.sort(r.choice(N, size=64, replace=False))
        w = ch.w[i]
        _, yb = oracle.w4_matmul(ext[i].view(np.float16), "f16", w["qweight"][rows], w["scales"][rows], None, 128,
                                 "f16")
        assert_close(f16_to_f64(outs[i][:, rows]), f16_to_f64(yb), "%s (stage %d)" % (names[i], s))


def test_chain_wait_timeout_is_reported_and_run_completes():
    """A spin limit of one poll makes dependency waits give up (the condition
    is set from the host; every kernel still ends normally) and the error word
    reports it.  Stage 0 is a single 16-row strip with K = 65536 (16 rounds on
    one workgroup), so every other workgroup's stage-1 wait lasts far longer
    than one poll.  A chain re-initialised with the default limit on the same
    buffer then runs correctly."""
    probs = [(0, 16, 65536), (1, 4096, 4096)]
    inputs = ["x0", "x0"]
    ch = Chain(1, 128, False, probs, inputs, spin_limit=1, seed=21)
    ch.set_inputs(22)
    ch.run()
    st, err = lb.lowbit_gemv_chain_error(ch.chain)
    assert st == 0 and err & 1
    nb = lb.lowbit_gemv_chain_bytes(len(probs), 2)
    lb.check(lb.lowbit_gemv_chain_init(ch.chain, ch.fmt, 1, 128, len(probs), ch.items, [0, 1], 0, ch.buf, nb))
    _check(ch, inputs, seed=23)
