"""Decode-loop scheduling with the window's prune overlapped with decoding.

Streams and events over the C ABI only: every step runs in the library's
kernels, and nothing here computes.

The prune runs once per window of generated tokens (yeyulingfeng.com
TriAttention page, section 主要方法: compression is triggered every 128
generated tokens).  It needs the window's last appended token and nothing the
decode steps compute, and the next window's attention over layer l needs only
layer l pruned.  So the prune of a window runs out of place on a stream of its
own (default priority, like the decode stream), in groups of consecutive
layers:
  * it starts once the window's last append has been issued and runs beside
    that step's attention (both only read the source cache);
  * the next window's first step appends and attends group by group, each
    group after that group's prune (`first_step`);
  * the steps after it run over every layer, as before.
The caller keeps the prune's inputs (source cache, positions t, workspace)
unchanged until the next window's first step has been issued, which waits for
every group.  The source and destination are distinct caches (an in-place
prune would rewrite rows the last step's attention still reads).
"""
from __future__ import annotations

import torch

from . import triattn as T


class LayerGroups:
    """Descriptors of groups of consecutive layers of one dense cache held in
    torch tensors k/v [n_seg, capacity, d], pos [n_seg, capacity], lengths
    [n_seg] (segment = (layer, sequence, KV head), layer-major, so a group of
    layers is one contiguous range of segments)."""

    def __init__(self, cache, *, n_layers, n_seq, n_kv_heads, n_groups):
        if not 1 <= n_groups <= n_layers:
            raise ValueError(f"n_groups must be in 1..{n_layers}")
        per_l = n_seq * n_kv_heads
        edges = [n_layers * g // n_groups for g in range(n_groups + 1)]
        self.layers = list(zip(edges[:-1], edges[1:]))
        self.segs = [(a * per_l, b * per_l) for a, b in self.layers]
        self.lengths = [cache["lengths"][s0:s1] for s0, s1 in self.segs]
        self.descs = [T.cache_desc(cache["k"][s0:s1], cache["v"][s0:s1], cache["pos"][s0:s1], ln,
                                   n_layers=b - a, n_seq=n_seq, n_kv_heads=n_kv_heads, layer0=a)
                      for (a, b), (s0, s1), ln in zip(self.layers, self.segs, self.lengths)]


class OverlappedPrune:
    """Prunes `src` into `dst` (two LayerGroups of the same shape) on a second
    stream (`prune_stream`, else a new one), group by group, ordered after what
    `decode_stream` has issued."""

    def __init__(self, calib, src, dst, budget, ws, decode_stream, prune_stream=None):
        if len(src.descs) != len(dst.descs):
            raise ValueError("source and destination need the same layer groups")
        self.calib, self.src, self.dst, self.budget, self.ws = calib, src, dst, budget, ws
        self.decode = decode_stream
        self.stream = prune_stream or torch.cuda.Stream(device=decode_stream.device)   # default priority
        self.ready = torch.cuda.Event()
        self.done = [torch.cuda.Event() for _ in src.descs]

    def launch(self, t):
        """Issue the prune of every group, after the work issued so far on the
        decode stream (the window's last append); t: [n_seq] int32 positions."""
        self.ready.record(self.decode)
        self.stream.wait_event(self.ready)
        for g, (s, d, n) in enumerate(zip(self.src.descs, self.dst.descs, self.dst.lengths)):
            T.tri_prune_window(self.calib, s, t, self.budget, d, n, self.ws, stream=self.stream)
            self.done[g].record(self.stream)

    def wait(self, g):
        """Order the decode stream's next work after group g's prune."""
        self.decode.wait_event(self.done[g])


def first_step(pruned, groups, n_q_heads, k_new, v_new, pos_new, q, scale, out, stream):
    """The first decode step of a window whose cache (`groups`) is being
    written by `pruned`: append and attention per layer group, each after that
    group's prune.  k_new/v_new [n_seg, d], pos_new [n_seq], q/out [L, n_seq,
    Hq, d] as for tri_append / tri_decode_attn."""
    for g, ((a, b), (s0, s1), desc) in enumerate(zip(groups.layers, groups.segs, groups.descs)):
        pruned.wait(g)
        T.tri_append(desc, k_new[s0:s1], v_new[s0:s1], pos_new, stream=stream)
        T.tri_decode_attn(desc, n_q_heads, q[a:b], scale, out[a:b], stream=stream)
