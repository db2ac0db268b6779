"""Layer frames on the libpg calls: the decode frame at one position and the
prefill frame over one pass of up to 64 positions.

Stage order follows the embryo token frame (embryo_wide.wgsl: norm, mixer
projections, residual + norm, FFN up with its activation, FFN down, residual
+ norm, head) with the mixer left out: the first `hidden` outputs of the QKV
product stand in for the mixer output added into the residual.

    qkv = W_qkv x0            h1 = h0 + qkv[:, :hidden];   x1 = rmsnorm(h1) w1
    u   = relu^2(W_up x1)     d  = W_down u
    h2  = h1 + d;  x2 = rmsnorm(h2) w2                     logits = W_head x2

Every stage is one libpg call on the current stream; ``capture()`` records the
whole frame once into a HIP graph (through torch.cuda.CUDAGraph) so replays
pay one launch for the frame (nemotron_prefill.rs builds its bind groups once
and keeps the pass size in a device buffer for the same reason).
"""
from __future__ import annotations

import torch

from ._lib import Q8Weight, add_rmsnorm, gemv_q8, prefill_gemm_q8, prefill_gemm_q8_workspace_bytes

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
        self.buf = {"qkv": torch.empty(n, qkv.rows, **f32), "x1": torch.empty(n, self.hidden, **f32),
                    "u": torch.empty(n, up.rows, **f32), "d": torch.empty(n, self.hidden, **f32),
                    "x2": torch.empty(n, self.hidden, **f32), "logits": torch.empty(n, head.rows, **f32)}
        if n > 1:
            need = max(prefill_gemm_q8_workspace_bytes(w.rows, w.cols, n) for w in self.W.values())
            self.workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        self.graph = None

    def weight_bytes(self) -> int:
        return sum(w.nbytes() for w in self.W.values())

    def _mm(self, name: str, x: torch.Tensor, y: torch.Tensor, act: int = 0):
        if self.n == 1:
            gemv_q8(self.W[name], x.view(-1), y.view(-1), act)
        else:
            prefill_gemm_q8(self.W[name], x, y, act, workspace=self.workspace)

    def run(self, x0: torch.Tensor, h: torch.Tensor) -> torch.Tensor:
        """Run the frame on x0 [n][hidden]; h [n][hidden] is the residual, updated in place."""
        b = self.buf
        H = self.hidden
        self._mm("qkv", x0, b["qkv"])
        add_rmsnorm(h, b["qkv"][:, :H], self.w1, self.eps, out=b["x1"], delta_stride=b["qkv"].shape[1])
        self._mm("up", b["x1"], b["u"], act=1)
        self._mm("down", b["u"], b["d"])
        add_rmsnorm(h, b["d"], self.w2, self.eps, out=b["x2"])
        self._mm("head", b["x2"], b["logits"])
        return b["logits"]

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
