"""Per-token weight sweep over a 27B-shaped decoder stack (64 layers x
q, k, v, o, gate, up, down), the decode workload of the tensorless pages
("Why the P100", "Why memory bandwidth sets the pace": every weight is read
once per token).

The executor places every packed matrix in HBM once, then runs one token's
GEMVs on the current stream in one of these launch schedules:
  token  one grouped launch for all GEMVs of the token (pn_group_run);
  layer  four launches per layer, the groups a real decoder can form because
         their inputs are ready together: {q, k, v}, {o}, {gate, up}, {down};
  gemv   one pn_gemv launch per matrix;
  token_rot  the token plan with every input in the model's unrotated basis
         (PN_DESC_ROTATE: one rotation launch over all inputs, then the
         grouped GEMV launch).
With M > 1 the token schedule is one pn_group_create_smallm plan and the gemv
schedule one pn_gemm_smallm launch per matrix.  A schedule can be captured
once into a HIP graph (torch.cuda.CUDAGraph) and replayed.
"""
import numpy as np
import torch

from . import _binding as B
from . import synth

LAYER_GROUPS = ((0, 1, 2), (3,), (4, 5), (6,))


class Sweep:
    def __init__(self, layers=synth.SWEEP_LAYERS, m=None, device="cuda", threads=16,
                 sample=None, unused_bits=False):
        """Generate and upload the sweep.  `sample(rec)` (optional) sees each
        matrix on the host before it is dropped, e.g. to keep some rows.
        `unused_bits`: pn3t words keep random bits 15 and 31."""
        self.layers = layers
        self.m = m
        self.device = torch.device(device)
        self.mats = []
        self.weight_bytes = 0
        self.act_bytes = 0

        def consume(rec):
            if sample is not None:
                sample(rec)
            w = torch.from_numpy(rec["W"]).to(self.device)
            x = torch.from_numpy(rec["x"]).to(self.device)
            n = rec["N"]
            y = torch.empty((n,) if m is None else (m, n), dtype=torch.float32, device=self.device)
            self.mats.append(dict(name=rec["name"], layer=rec["layer"], mat=rec["mat"], type=rec["type"],
                                  N=n, K=rec["K"], W=w, x=x, y=y))
            self.weight_bytes += w.numel()
            self.act_bytes += x.numel() * 2 + y.numel() * 4

        synth.sweep_matrices(layers=layers, m=m, config=3 if m is None else 4, threads=threads,
                             consume=consume, unused_bits=unused_bits)
        self.groups = {}
        self.graph = None

    def batch_view(self, m):
        """The same resident weights with an M-row activation batch per matrix
        (drawn from config 4's streams, as a Sweep(m=m) would) and its own
        outputs: the M = 8 workload without a second copy of the weights."""
        v = Sweep.__new__(Sweep)
        v.layers, v.m, v.device = self.layers, m, self.device
        v.mats, v.weight_bytes, v.act_bytes = [], self.weight_bytes, 0
        for e in self.mats:
            n, k = e["N"], e["K"]
            x = torch.from_numpy(synth.activation(synth.rng(4, e["layer"], e["mat"]), k, m)).to(self.device)
            y = torch.empty((m, n), dtype=torch.float32, device=self.device)
            v.mats.append(dict(e, x=x, y=y))
            v.act_bytes += x.numel() * 2 + y.numel() * 4
        v.groups, v.graph = {}, None
        return v

    # -- schedules --------------------------------------------------------
    def _problem(self, e):
        if self.m is not None:
            return (e["type"], e["W"], e["N"], e["K"], e["x"], e["K"], self.m, e["y"], e["N"])
        return (e["type"], e["W"], e["N"], e["K"], e["x"], e["y"])

    def prepare(self, schedule):
        if self.m is not None and schedule == "layer":
            raise ValueError("M > 1 runs the token and gemv schedules")
        if schedule == "token" and "token" not in self.groups:
            self.groups["token"] = [B.Group([self._problem(e) for e in self.mats],
                                            smallm=self.m is not None)]
        if schedule == "token_rot" and "token_rot" not in self.groups:
            if self.m is not None:
                raise ValueError("rotated inputs: M = 1 plans only")
            self.groups["token_rot"] = [B.Group([self._problem(e) for e in self.mats], rotate=True)]
        if schedule == "layer" and "layer" not in self.groups:
            gl = []
            per = len(synth.SWEEP_LAYER)
            for l in range(self.layers):
                for grp in LAYER_GROUPS:
                    gl.append(B.Group([self._problem(self.mats[l * per + j]) for j in grp]))
            self.groups["layer"] = gl

    def launches(self, schedule):
        if schedule == "token_rot":
            return 2
        if schedule in ("token", "layer"):
            return len(self.groups[schedule])
        return len(self.mats)

    def step(self, schedule="layer"):
        """Enqueue one token's GEMVs on the current stream."""
        if schedule in ("token", "layer", "token_rot"):
            self.prepare(schedule)
            for g in self.groups[schedule]:
                g.run()
        elif schedule == "gemv":
            if self.m is None:
                for e in self.mats:
                    B.pn_gemv(e["type"], e["W"], e["N"], e["K"], e["x"], e["y"])
            else:
                for e in self.mats:
                    B.pn_gemm_smallm(e["type"], e["W"], e["N"], e["K"], e["x"], e["K"], self.m,
                                     e["y"], e["N"])
        else:
            raise ValueError(schedule)

    def capture(self, schedule="layer"):
        """Capture one step into a HIP graph; returns the graph."""
        if schedule in ("token", "layer", "token_rot"):
            self.prepare(schedule)
        self.step(schedule)  # warm: first launches, occupancy queries
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(schedule)
        torch.cuda.synchronize()
        self.graph = g
        return g

    def outputs(self):
        return [e["y"] for e in self.mats]

    def close(self):
        for gl in self.groups.values():
            for g in gl:
                g.close()
        self.groups = {}
        self.graph = None


def sample_rows(rec, rows_per_matrix, store):
    """A `sample` callback body: keep rows (first, last and seeded random ones)
    and the activation of one matrix for later checks."""
    n = rec["N"]
    g = np.random.default_rng([rec["layer"], rec["mat"], 99])
    rows = sorted(set([0, n - 1] + list(g.integers(0, n, size=max(rows_per_matrix - 2, 0)))))
    store[(rec["layer"], rec["mat"])] = dict(rows=np.array(rows), W=rec["W"][rows].copy(),
                                             x=rec["x"].copy(), type=rec["type"], K=rec["K"])
