"""Graph-captured autoregressive decode loop.

The cached decode of "Compiler-First State Space Duality and Portable O(1)
Autoregressive Caching for Inference" (abstract) runs the per-token step in an
on-device loop instead of one host launch per token.  Here the loop is a HIP
graph (captured through torch.cuda.CUDAGraph): `steps` consecutive
``ssd_decode_step`` launches on static buffers, replayed as one unit.  Each
replay advances the state in place by `steps` tokens; the per-token inputs of a
replay are whatever the static input buffers hold when it is launched.

The graph holds kernel launches only (the library allocates, clears and
synchronizes nothing), so a replay does exactly what the same eager calls do.
"""
from __future__ import annotations

from typing import Optional

import mamba_ssd_chunked_02_amd as ssd


class DecodeLoop:
    """`steps` decode steps of a batch, captured once, replayed many times.

    Static buffers (allocated here, filled by the caller before ``replay``):
      state [b, H, P, N] fp32 (advanced in place by every replay),
      x [steps, b, H, P], dt [steps, b, H] fp32, B and C [steps, b, G, N]
      (x, B, C in ``dtype``), and the outputs y [steps, b, H, P] (``y_dtype``).
    A and D [H] fp32 are captured by reference.
    """

    def __init__(self, steps: int, batch: int, H: int, P: int, N: int, G: int, A, D, *, dtype=None,
                 y_dtype=None, device=None, dt_softplus: bool = False, dt_bias=None, dt_limit=None):
        import torch
        dtype = dtype or torch.bfloat16
        y_dtype = y_dtype or torch.float32
        device = device or A.device
        self.steps = steps
        self.state = torch.zeros((batch, H, P, N), dtype=torch.float32, device=device)
        self.x = torch.zeros((steps, batch, H, P), dtype=dtype, device=device)
        self.dt = torch.zeros((steps, batch, H), dtype=torch.float32, device=device)
        self.B = torch.zeros((steps, batch, G, N), dtype=dtype, device=device)
        self.C = torch.zeros((steps, batch, G, N), dtype=dtype, device=device)
        self.y = torch.zeros((steps, batch, H, P), dtype=y_dtype, device=device)
        self.A, self.D = A, D
        self._act = dict(dt_softplus=dt_softplus, dt_bias=dt_bias, dt_limit=dt_limit)
        # one eager pass first (the library's first call loads the module),
        # then capture on a side stream as torch requires
        saved = self.state.clone()
        self._steps_eager()
        self.state.copy_(saved)
        torch.cuda.synchronize(device)
        self.graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=device)
        side.wait_stream(torch.cuda.current_stream(device))
        with torch.cuda.stream(side):
            with torch.cuda.graph(self.graph, stream=side):
                self._steps_eager()
        torch.cuda.current_stream(device).wait_stream(side)
        torch.cuda.synchronize(device)
        self.state.copy_(saved)

    def _steps_eager(self):
        for k in range(self.steps):
            ssd.decode_step(self.state, self.x[k], self.dt[k], self.A, self.B[k], self.C[k], self.D,
                            y=self.y[k], **self._act)

    def replay(self):
        """Advance ``state`` by ``steps`` tokens (asynchronous, current stream)."""
        self.graph.replay()

    def run_eager(self):
        """The same steps as ordinary launches (for checks and comparison)."""
        self._steps_eager()
