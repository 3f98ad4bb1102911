"""Host logic of bench.py's graph timing (no GPU): the captured graphs
replay exactly the requested number of steps, in cycle order, each graph
from its first step, and the timed steps start where the warm-up's whole
cycles end."""

import contextlib
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


class _FakeTorch:
    """Just what graph_replay_seconds touches: streams, graph capture (the
    steps called while capturing are recorded into the graph) and replay
    (which appends the recorded step indices to `ran`)."""

    def __init__(self):
        self.ran, self.sizes, self._rec = [], [], None
        fake = self

        class Graph:
            def __init__(self):
                self.steps = []

            def replay(self):
                fake.ran.extend(self.steps)
                fake.sizes.append(len(self.steps))

        class Cuda:
            CUDAGraph = Graph

            @staticmethod
            def Stream():
                return type("S", (), {"wait_stream": lambda self, o: None})()

            @staticmethod
            def current_stream():
                return type("S", (), {"wait_stream": lambda self, o: None})()

            @staticmethod
            def stream(s):
                return contextlib.nullcontext()

            @staticmethod
            @contextlib.contextmanager
            def graph(g, stream=None):
                fake._rec = g
                yield
                fake._rec = None

            @staticmethod
            def synchronize():
                pass

        self.cuda = Cuda

    def step(self, i):
        assert self._rec is not None, "a step ran outside capture"
        self._rec.steps.append(i)


def _run(n_cycle, steps, warmup, per_graph=4):
    b = _bench()
    t = _FakeTorch()
    b.graph_replay_seconds(t, t.step, n_cycle, steps, warmup, per_graph=per_graph)
    return t.ran, t.sizes


def test_graph_replay_counts_and_order():
    for n_cycle, steps, warmup, per_graph in [(4, 20, 5, 4), (32, 20, 5, 4), (9, 7, 3, 4), (8, 20, 5, 8), (1, 3, 0, 4)]:
        ran, _ = _run(n_cycle, steps, warmup, per_graph)
        warm = -(-warmup // n_cycle) * n_cycle
        assert len(ran) == warm + steps, (n_cycle, steps, warmup)
        # every step in cycle order, the timed ones continuing from index 0
        assert ran == [i % n_cycle for i in range(warm + steps)], (n_cycle, steps, warmup)


def test_graph_replay_launches_whole_graphs():
    # the headline step: 20 timed steps are five replays of the 4-step graph
    # after two warm-up replays; the 64K step (32 copies) replays graphs of
    # four from index 0 after its 32-step warm-up
    _, sizes = _run(4, 20, 5)
    assert sizes == [4] * 7
    _, sizes = _run(32, 20, 5)
    assert sizes == [4] * 8 + [4] * 5
    _, sizes = _run(9, 7, 3)  # graphs of 4, 4, 1 steps; 7 = 4 + 3 singles
    assert sizes == [4, 4, 1] + [4, 1, 1, 1]
