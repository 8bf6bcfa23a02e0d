"""Whole block steps replayed from a HIP graph.

A block step issues a few dozen library calls.  At small token counts the
host's time on them (10-20 us per call through ctypes) exceeds the GPU's time,
and the GPU waits for the host.  StepGraph records one step (every kernel and
every fork to and join from the block's second stream) into a HIP graph
through torch.cuda.CUDAGraph, and replays it with no host work per launch.

What capture needs, and how it is met here:
  * the step runs on a stream of its own (the capture stream), and every
    library handle it uses exists before capture: a few eager steps on that
    stream first create them and size their workspaces;
  * no call may allocate or synchronise during capture or afterwards under
    the graph (its kernels hold the workspace addresses of capture time): the
    workspaces of the capture stream's handle and of the block's second
    streams are then fixed until close() releases the graph (a call that
    would need more fails instead of allocating);
  * inputs and outputs keep their addresses between replays: a block reuses
    its buffers, and the caller refills its input tensors in place.
The library records no memset in a step, so replays do not depend on memset
nodes.
"""
import torch

from . import ops


class StepGraph:
    """step: a callable running one block step on the current stream.
    side_streams: the block's second streams (their handles' workspaces are
    fixed with the capture stream's)."""

    def __init__(self, step, side_streams=(), device: int = 0, warmup: int = 3):
        self.stream = torch.cuda.Stream(device=device)
        cur = torch.cuda.current_stream(device)
        self.stream.wait_stream(cur)
        with torch.cuda.stream(self.stream):
            for _ in range(warmup):
                step()
        self.stream.synchronize()
        self._fixed = (self.stream, *side_streams)
        for s in self._fixed:
            ops.set_stream_option(s, "workspace_fixed", 1)
        self.graph = torch.cuda.CUDAGraph()
        try:
            with torch.cuda.graph(self.graph, stream=self.stream):
                step()
        except BaseException:
            self.graph = None
            for s in self._fixed:
                ops.set_stream_option(s, "workspace_fixed", 0)
            raise
        cur.wait_stream(self.stream)

    def close(self):
        """Release the graph, then let the handles' workspaces grow again
        (torch reuses streams, so a handle left fixed would refuse a later
        block's larger calls)."""
        if self.graph is None:
            return
        torch.cuda.synchronize()
        self.graph.reset()
        self.graph = None
        for s in self._fixed:
            ops.set_stream_option(s, "workspace_fixed", 0)

    def replay(self):
        """One step, ordered after the current stream's earlier work; later
        work on the current stream is ordered after it."""
        if self.graph is None:
            raise RuntimeError("StepGraph.replay after close")
        cur = torch.cuda.current_stream()
        self.stream.wait_stream(cur)
        with torch.cuda.stream(self.stream):
            self.graph.replay()
        cur.wait_stream(self.stream)
