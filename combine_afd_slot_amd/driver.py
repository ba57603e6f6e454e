"""Convenience driver over the C ABI for callers that hold torch tensors.

It allocates device buffers with torch (plumbing only), creates one window,
and issues afd_slot_pack / afd_ffn_run / afd_slot_unpack through the ctypes
binding.  Simulated attention peers run on their own HIP streams, the FFN on
another; every step of the path runs in libafd.so.
"""
from __future__ import annotations

import numpy as np

from . import afd


def _dev_bf16(torch, a: np.ndarray, dev):
    """bf16 bit patterns (uint16) -> a torch.bfloat16 tensor on `dev`."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(dev).view(torch.bfloat16)


class FfnSession:
    """One FFN replica window with P simulated peers on separate streams."""

    def __init__(self, wl, inputs: dict, device="cuda:0", poll_timeout_us=5_000_000, weights=True,
                 static_window=False):
        import torch
        self.torch = torch
        self.wl = wl
        self.dev = torch.device(device)
        torch.cuda.set_device(self.dev)
        self.cfg = afd.make_config(wl.num_peers, wl.token_cap, wl.hidden, wl.num_experts, wl.top_k,
                                   wl.intermediate, wl.shared_intermediate, ring_depth=wl.ring_depth,
                                   routed_scaling_factor=wl.routed_scaling_factor, renormalize=wl.renormalize,
                                   poll_timeout_us=poll_timeout_us, attention_routes=wl.attention_routes,
                                   route_experts=wl.route_experts, expert_offset=wl.expert_offset,
                                   w1_fp8=wl.w1_fp8)
        # static_window: the window in the library's static device array
        # (afd_window_create_static: no device allocation)
        self.win = (afd.afd_window_create_static if static_window else afd.afd_window_create)(self.cfg)
        self.layout = afd.afd_window_layout(self.win)
        self.peer_streams = [torch.cuda.Stream(device=self.dev) for _ in range(wl.num_peers)]
        self.ffn_stream = torch.cuda.Stream(device=self.dev)
        self.set_inputs(inputs)
        if weights:
            self.set_weights(inputs)

    # ---------------------------------------------------------------- data
    def set_inputs(self, inputs: dict):
        torch = self.torch
        self.x = [_dev_bf16(torch, a, self.dev) if a.shape[0] else torch.empty((0, self.wl.hidden),
                  dtype=torch.bfloat16, device=self.dev) for a in inputs["x"]]
        self.l = [torch.from_numpy(np.ascontiguousarray(a)).to(self.dev) for a in inputs["l"]]
        self.out = [torch.empty((n, self.wl.hidden), dtype=torch.bfloat16, device=self.dev)
                    for n in self.wl.seq_lens]

    def set_weights(self, inputs: dict):
        torch = self.torch
        self.w13 = _dev_bf16(torch, inputs["W13"], self.dev)
        self.w2 = _dev_bf16(torch, inputs["W2"], self.dev)
        if self.wl.shared_intermediate > 0:
            self.ws13 = _dev_bf16(torch, inputs["Ws13"], self.dev)
            self.ws2 = _dev_bf16(torch, inputs["Ws2"], self.dev)
        else:
            self.ws13 = self.ws2 = None
        # the layer's weights in GEMM tile order (what afd_ffn_run reads)
        nbytes = self.layout.packed_weight_bytes
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device=self.dev)
        torch.cuda.synchronize(self.dev)
        afd.afd_weights_pack(self.win, self.w13.data_ptr(), self.w2.data_ptr(),
                             self.ws13.data_ptr() if self.ws13 is not None else 0,
                             self.ws2.data_ptr() if self.ws2 is not None else 0,
                             self.packed.data_ptr(), nbytes, self.ffn_stream.cuda_stream)
        self.ffn_stream.synchronize()

    # ---------------------------------------------------------------- steps
    def pack(self, peer, stage=0, layer=0, flags=0, seq_len=None):
        n = self.wl.seq_lens[peer] if seq_len is None else seq_len
        return afd.afd_slot_pack(self.win, peer, stage, layer, n, self.x[peer].data_ptr() if n else 0,
                                 self.l[peer].data_ptr() if n else 0, flags,
                                 self.peer_streams[peer].cuda_stream)

    def pack_all(self, stage=0, layer=0, sync=True):
        for p in range(self.wl.num_peers):
            self.pack(p, stage, layer)
        if sync:
            for s in self.peer_streams:
                s.synchronize()

    def run(self, stage=0, layer=0):
        return afd.afd_ffn_run(self.win, stage, layer, self.packed.data_ptr(), self.ffn_stream.cuda_stream)

    def unpack(self, peer, stage=0):
        n = self.wl.seq_lens[peer]
        return afd.afd_slot_unpack(self.win, peer, stage, n, self.out[peer].data_ptr() if n else 0,
                                   self.peer_streams[peer].cuda_stream)

    def unpack_all(self, stage=0, sync=True):
        for p in range(self.wl.num_peers):
            self.unpack(p, stage)
        if sync:
            for s in self.peer_streams:
                s.synchronize()

    def step(self, stage=0, layer=0):
        """pack all peers -> run -> unpack all peers, fully synchronized."""
        self.pack_all(stage, layer)
        self.run(stage, layer)
        self.ffn_stream.synchronize()
        self.unpack_all(stage)

    def status(self, stage=0):
        return afd.afd_window_status(self.win, stage, self.ffn_stream.cuda_stream)

    def peer_status(self, peer, stage=0):
        return afd.afd_peer_status(self.win, peer, stage, self.peer_streams[peer].cuda_stream)

    def routing(self):
        wl = self.wl
        maxp = wl.num_peers * wl.token_cap * wl.top_k
        r = afd.afd_debug_routing(self.win, self.ffn_stream.cuda_stream, maxp, wl.num_experts, wl.num_peers)
        T = int(r["off"][-1])
        n = T * wl.top_k
        for k in ("ids", "w", "perm", "inv"):
            r[k] = r[k][:n]
        r["ids"] = r["ids"].reshape(T, wl.top_k)
        r["w"] = r["w"].reshape(T, wl.top_k)
        return r

    def outputs_f32(self):
        return [o.float().cpu().numpy() for o in self.out]

    def close(self):
        if self.win:
            afd.afd_window_destroy(self.win)
            self.win = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
