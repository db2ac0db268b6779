"""Layer frames on the libpg calls: the decode frame at one position and the
prefill frame over one pass of up to 64 positions.

Stage order follows the embryo token frame (embryo_wide.wgsl: norm, mixer
projections, residual + norm, FFN up with its activation, FFN down, residual
+ norm, head) with the mixer left out: the first `hidden` outputs of the QKV
product stand in for the mixer output added into the residual.

    qkv = W_qkv x0            h1 = h0 + qkv[:, :hidden];   x1 = rmsnorm(h1) w1
    u   = relu^2(W_up x1)     d  = W_down u
    h2  = h1 + d;  x2 = rmsnorm(h2) w2                     logits = W_head x2

The two residual + norm sites run inside the products around them, so a
frame is four product calls.  Decode: the QKV and down GEMVs add their output
into the residual and leave w * h and partial sums of squares
(gemv_q8_residual); the up and head GEMVs apply 1/rms to their dot products
(gemv_q8_normed) -- four GEMV launches back to back.  Prefill: one
prefill_frame_q8 call (five launches: the staging of x0 and the four
matrix-core passes, each finishing the add + norm work around it in its
epilogue).  ``capture()`` records
the whole frame once into a HIP graph (through torch.cuda.CUDAGraph) so
replays pay one launch for the frame.  ``Prompt`` goes further: its frame
reads the pass size {n, pos0} from a device buffer, so one recording serves
every pass of a prompt (nemotron_prefill.rs builds its bind groups once and
keeps n and pos0 in its `Meta` uniform for the same reason).
"""
from __future__ import annotations

import torch

from ._lib import (Q8Weight, gemv_q8, gemv_q8_normed, gemv_q8_residual, norm_parts, prefill_frame_q8,
                   prefill_frame_q8_meta, prefill_frame_q8_workspace_bytes, prefill_gemm_q8,
                   prefill_gemm_q8_workspace_bytes)

PB_MAX = 64


class Frame:
    """One layer frame over n positions (n == 1 runs the decode GEMVs)."""

    def __init__(self, qkv: Q8Weight, up: Q8Weight, down: Q8Weight, head: Q8Weight,
                 w1: torch.Tensor, w2: torch.Tensor, eps: float, n: int = 1):
        if not 1 <= n <= PB_MAX:
            raise ValueError(f"n must be in [1, {PB_MAX}]")
        self.W = {"qkv": qkv, "up": up, "down": down, "head": head}
        self.w1, self.w2, self.eps, self.n = w1, w2, eps, n
        self.hidden = qkv.cols
        dev = qkv.q.device
        f32 = dict(dtype=torch.float32, device=dev)
        self.buf = {"qkv": torch.empty(n, qkv.rows, **f32), "u": torch.empty(n, up.rows, **f32),
                    "d": torch.empty(n, self.hidden, **f32), "logits": torch.empty(n, head.rows, **f32)}
        if n == 1:   # decode: w * h and the sum-of-squares parts handed between GEMVs
            for k in ("xw1", "xw2"):
                self.buf[k] = torch.empty(self.hidden, **f32)
            for k in ("p1", "p2"):
                self.buf[k] = torch.empty(norm_parts(self.hidden), **f32)
        if n > 1:
            need = max(max(prefill_gemm_q8_workspace_bytes(w.rows, w.cols, n) for w in self.W.values()),
                       prefill_frame_q8_workspace_bytes(self.hidden, qkv.rows, up.rows, head.rows, n))
            self.workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        self.graph = None

    def weight_bytes(self) -> int:
        return sum(w.nbytes() for w in self.W.values())

    def _mm(self, name: str, x: torch.Tensor, y: torch.Tensor, act: int = 0):
        if self.n == 1:
            gemv_q8(self.W[name], x.view(-1), y.view(-1), act)
        else:
            prefill_gemm_q8(self.W[name], x, y, act, workspace=self.workspace)

    def stages(self, x0: torch.Tensor, h: torch.Tensor):
        """The frame as its library calls (zero-argument callables, in order): four
        GEMV calls at one position, one prefill_frame_q8 call for a pass."""
        b = self.buf
        H = self.hidden
        W = self.W
        if self.n == 1:
            hv = h.view(-1)
            return [lambda: gemv_q8_residual(W["qkv"], x0.view(-1), hv, self.w1, b["xw1"], b["p1"],
                                             y=b["qkv"].view(-1), h_out=hv),
                    lambda: gemv_q8_normed(W["up"], b["xw1"], b["p1"], self.eps, y=b["u"].view(-1), act=1),
                    lambda: gemv_q8_residual(W["down"], b["u"].view(-1), hv, self.w2, b["xw2"], b["p2"],
                                             y=b["d"].view(-1), h_out=hv),
                    lambda: gemv_q8_normed(W["head"], b["xw2"], b["p2"], self.eps, y=b["logits"].view(-1))]
        ws = self.workspace
        return [lambda: prefill_frame_q8(W["qkv"], W["up"], W["down"], W["head"], self.w1, self.w2, self.eps, x0, h,
                                         {"qkv": b["qkv"], "u": b["u"], "d": b["d"], "logits": b["logits"]},
                                         ws)]

    def run(self, x0: torch.Tensor, h: torch.Tensor) -> torch.Tensor:
        """Run the frame on x0 [n][hidden]; h [n][hidden] is the residual, updated in place
        (h ends as h + qkv[:, :hidden] + d)."""
        for st in self.stages(x0, h):
            st()
        return self.buf["logits"]

    def capture(self, x0: torch.Tensor, h: torch.Tensor):
        """Record run(x0, h) into a graph; replay() then reruns it on the same buffers."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run(x0, h)      # warm-up outside the graph (kernel attributes, allocator)
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run(x0, h)
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()


class Prompt:
    """A prompt of ``rows`` positions through the layer frame in passes of at most 64,
    from ONE recorded launch sequence: the frame is captured once as
    prefill_frame_q8_meta, whose kernels read the pass's {n, pos0} from a device
    buffer at launch, and each pass is a replay after that buffer is set
    (nemotron_prefill.rs, module doc: bind groups built once, n and pos0 in the
    `Meta` uniform).  X0 and H are the prompt's [rows][hidden] buffers; H is the
    residual, updated in place; ``buf`` holds qkv, u, d and logits for every row."""

    def __init__(self, qkv: Q8Weight, up: Q8Weight, down: Q8Weight, head: Q8Weight,
                 w1: torch.Tensor, w2: torch.Tensor, eps: float, X0: torch.Tensor, H: torch.Tensor):
        self.W = {"qkv": qkv, "up": up, "down": down, "head": head}
        self.w1, self.w2, self.eps = w1, w2, eps
        self.X0, self.H = X0, H
        self.rows, hidden = X0.shape
        dev = X0.device
        f32 = dict(dtype=torch.float32, device=dev)
        R = self.rows
        self.buf = {"qkv": torch.empty(R, qkv.rows, **f32), "u": torch.empty(R, up.rows, **f32),
                    "d": torch.empty(R, hidden, **f32), "logits": torch.empty(R, head.rows, **f32)}
        self.workspace = torch.empty(prefill_frame_q8_workspace_bytes(hidden, qkv.rows, up.rows, head.rows, PB_MAX),
                                     dtype=torch.uint8, device=dev)
        self.passes = [(min(PB_MAX, R - p0), p0) for p0 in range(0, R, PB_MAX)]
        # one {n, pos0} row per pass, on the device; the launch reads `meta`
        self.metas = torch.tensor(self.passes, dtype=torch.int32, device=dev)
        self.meta = self.metas[0].clone()
        self.graph = None

    def _call(self):
        prefill_frame_q8_meta(self.W["qkv"], self.W["up"], self.W["down"], self.W["head"], self.w1, self.w2,
                              self.eps, self.X0, self.H, self.meta, self.buf, self.workspace)

    def capture(self):
        """Record the frame once; the recording is replayed for every pass."""
        self.meta.zero_()            # n = 0: the warm-up call below changes nothing
        self._call()                 # outside the graph: kernel attributes, allocator
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            self._call()
        torch.cuda.current_stream().wait_stream(s)
        self.graph = g
        return g

    def run_pass(self, i: int):
        """Pass i (rows pos0 .. pos0 + n - 1): set the device meta, then replay (or call)."""
        self.meta.copy_(self.metas[i])
        if self.graph is not None:
            self.graph.replay()
        else:
            self._call()

    def run(self):
        """Every pass in order (H ends as the residual after the frame for every row)."""
        for i in range(len(self.passes)):
            self.run_pass(i)
        return self.buf["logits"]
