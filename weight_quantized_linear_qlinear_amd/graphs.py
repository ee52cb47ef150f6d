"""Decode-batch graph buckets: one captured HIP graph per bucketed batch size.

A serving engine replays captured graphs for its decode steps and pads the batch
up to the next captured size ("tiny-vLLM" README, "Decode-Heavy Scaling": decode
throughput stops rising past the range covered by captured graphs; "Nano-vLLM-MoE"
README, Highlights: CUDA-graph capture in the runtime).  `GraphBuckets` does this
for any chain of library calls: for every bucket size b it owns a static input
[b, in_features] and output [b, out_features] (bf16) and captures `fn(x, out)`
once; a call with M rows copies x into the bucket's input, zeroes the pad rows,
replays the graph and returns the first M output rows.

Pad rows never change the real rows: every scheme here computes each output row
from its own input row only (W8A16; W8A8 static with one fixed input scale; W8A8
dynamic with one scale per row), and zero pad rows stay finite.  `fn` must enqueue
only library calls on the current stream and keep everything it writes in
buffers it owns (captured graphs reuse the same addresses on every replay),
including its split-K workspace.
"""
from __future__ import annotations

import torch

DEFAULT_BUCKETS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512)


class GraphBuckets:
    """Captured graphs of `fn(x, out)` for each bucket size; calls pad M up to a bucket."""

    def __init__(self, fn, in_features: int, out_features: int, buckets=DEFAULT_BUCKETS,
                 device: torch.device | None = None):
        self.fn = fn
        self.in_features = int(in_features)
        self.out_features = int(out_features)
        self.buckets = tuple(sorted(set(int(b) for b in buckets)))
        if not self.buckets or self.buckets[0] < 1:
            raise ValueError("buckets must be positive sizes")
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self._x = {}
        self._y = {}
        self._graphs = {}
        self._stream = torch.cuda.Stream(device=self.device)
        for b in self.buckets:
            self._capture(b)

    def bucket_for(self, M: int) -> int:
        """Smallest bucket that holds M rows."""
        for b in self.buckets:
            if M <= b:
                return b
        raise ValueError(f"batch of {M} rows above the largest bucket ({self.buckets[-1]})")

    def _capture(self, b: int):
        x = torch.zeros((b, self.in_features), dtype=torch.bfloat16, device=self.device)
        y = torch.zeros((b, self.out_features), dtype=torch.bfloat16, device=self.device)
        self.fn(x, y)                                   # eager run: kernel set-up outside capture
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self._stream):
            self.fn(x, y)
        torch.cuda.synchronize(self.device)
        self._x[b], self._y[b], self._graphs[b] = x, y, g

    def __call__(self, x: torch.Tensor) -> torch.Tensor:
        """Run the chain on x [M, in_features] bf16; returns a view of the bucket's
        output rows [M, out_features], valid until the next call on the same bucket."""
        if x.dim() != 2 or x.dtype != torch.bfloat16 or x.shape[1] != self.in_features:
            raise ValueError(f"x must be bf16 [M, {self.in_features}]")
        M = x.shape[0]
        b = self.bucket_for(M)
        xs = self._x[b]
        xs[:M].copy_(x)
        if M < b:
            xs[M:].zero_()
        self._graphs[b].replay()
        return self._y[b][:M]
