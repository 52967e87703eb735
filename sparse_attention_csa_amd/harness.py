"""Device-side sessions for a decode step or a prefill chunk of one layer.

A session takes inputs given *by position* (a dict of NumPy arrays: bf16 as
uint16 bit patterns, e4m3 as uint8 codes with float32 scales, float32 as is)
and lays them into the library's state layout: the window ring (position p in
slot p % n_win), the compression tail ring (slot p % R, R = 3m with overlap
and 2m without), the compressed caches and their entry counts.  It then calls
the C-ABI entry points.  Pure marshalling: all arithmetic runs in libcsa.so.
"""

import numpy as np
import torch

from . import _lib as L

_KV = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(arr, kind, device="cuda"):
    """Upload a host array in its storage format."""
    a = np.ascontiguousarray(arr)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if kind == "e4m3":
        return torch.from_numpy(a.view(np.uint8)).to(device)
    if kind == "f32":
        return torch.from_numpy(a.astype(np.float32)).to(device)
    if kind in ("i32", "i64"):
        return torch.from_numpy(a.astype(np.int32 if kind == "i32" else np.int64)).to(device)
    raise ValueError(kind)


def to_host_bits(t):
    """Device tensor -> NumPy in storage format (bf16 as uint16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


DTYPE_CODE = {"f32": L.CSA_F32, "bf16": L.CSA_BF16, "e4m3": L.CSA_E4M3}


def make_desc(g):
    d = L.LayerDesc()
    d.kind = L.CSA_LAYER_CSA if g["kind"] == "csa" else L.CSA_LAYER_HCA
    d.H, d.c, d.m = g["H"], g["c"], g["m"]
    d.H_I = g.get("H_I") or 0
    d.d_I = g.get("d_I") or 0
    d.overlap = 1 if g["overlap"] else 0
    d.k = g.get("k") or 0
    d.n_win = g["n_win"]
    d.vis = g["vis"]
    d.kv_dtype = DTYPE_CODE[g["kv_dtype"]]
    d.idx_dtype = DTYPE_CODE[g["idx_dtype"]] if g.get("idx_dtype") else 0
    d.scale = g["scale"]
    return d


class _State:
    """Layer state tensors (caches, rings, tails, parameters)."""

    def __init__(self, g, B, E_cap, device):
        kvk = g["kv_dtype"]
        c, m = g["c"], g["m"]
        self.R = 3 * m if g["overlap"] else 2 * m
        self.S = 4 if g["overlap"] else 2
        tdt = _KV[kvk]
        self.kv_cache = torch.zeros((B, E_cap, c), dtype=tdt, device=device)
        self.n_entries = torch.zeros(B, dtype=torch.int32, device=device)
        self.win_ring = torch.zeros((B, g["n_win"], c), dtype=tdt, device=device)
        self.tail = torch.zeros((B, self.S, self.R, c), dtype=tdt, device=device)
        self.bias_a = dev(g["bias_a"], "f32", device) if g.get("bias_a") is not None else None
        self.bias_b = dev(g["bias_b"], "f32", device) if g.get("bias_b") is not None else None
        self.sink = dev(g["sink"], "f32", device) if g.get("sink") is not None else None
        self.idx_cache = self.idx_scale = self.idx_tail = self.ibias_a = self.ibias_b = None
        if g["kind"] == "csa":
            d_I = g["d_I"]
            idt = torch.uint8 if g["idx_dtype"] == "e4m3" else _KV[g["idx_dtype"]]
            self.idx_cache = torch.zeros((B, E_cap, d_I), dtype=idt, device=device)
            if g["idx_dtype"] == "e4m3":
                self.idx_scale = torch.ones((B, E_cap), dtype=torch.float32, device=device)
            self.idx_tail = torch.zeros((B, 4, self.R, d_I), dtype=tdt, device=device)
            self.ibias_a = dev(g["ibias_a"], "f32", device)
            self.ibias_b = dev(g["ibias_b"], "f32", device)
        self.B, self.E_cap = B, E_cap

    def struct(self):
        s = L.LayerState()
        s.B, s.E_cap = self.B, self.E_cap
        for name in ("kv_cache", "idx_cache", "idx_scale", "n_entries", "win_ring", "tail",
                     "idx_tail", "bias_a", "bias_b", "ibias_a", "ibias_b", "sink"):
            setattr(s, name, L.ptr(getattr(self, name)))
        return s


class DecodeSession:
    """One decode step (one new token per sequence) of a CSA or HCA layer."""

    def __init__(self, g, device="cuda"):
        self.g = g
        B, E_cap, c, m, n_win = g["B"], g["E_cap"], g["c"], g["m"], g["n_win"]
        kvk = g["kv_dtype"]
        self.desc = make_desc(g)
        st = _State(g, B, E_cap, device)
        self.state = st
        st.kv_cache.copy_(dev(g["kv_cache"], kvk, device))
        st.n_entries.copy_(dev(g["n_entries"], "i32", device))
        pos = np.asarray(g["pos"], np.int64)
        # window ring: positions t-(n_win-1) .. t-1
        ring = torch.zeros_like(st.win_ring)
        wh = dev(g["win_hist"], kvk, device)
        for b in range(B):
            t = int(pos[b])
            for j in range(wh.shape[1]):
                p = t - wh.shape[1] + j
                if p >= 0:
                    ring[b, p % n_win] = wh[b, j]
        st.win_ring.copy_(ring)
        streams = ("ca", "za", "cb", "zb")[:st.S]
        tail0 = np.asarray(g["tail_pos0"], np.int64)
        tail = torch.zeros_like(st.tail)
        for si, sname in enumerate(streams):
            src = dev(g["tail_" + sname], kvk, device)
            for b in range(B):
                for j in range(src.shape[1]):
                    tail[b, si, int(tail0[b] + j) % st.R] = src[b, j]
        st.tail.copy_(tail)
        io = {}
        io["pos"] = dev(pos, "i64", device)
        io["q"] = dev(g["q"], kvk, device)
        io["x_new"] = dev(g["x_new"], kvk, device)
        io["streams"] = torch.stack([dev(g["new_" + s], kvk, device) for s in streams], dim=1)
        H = g["H"]
        io["out"] = torch.empty((B, H, c), dtype=_KV[kvk], device=device)
        io["lse"] = torch.empty((B, H), dtype=torch.float32, device=device)
        if g["kind"] == "csa":
            idk = g["idx_dtype"]
            st.idx_cache.copy_(dev(g["idx_cache"], idk, device))
            if idk == "e4m3":
                st.idx_scale.copy_(dev(g["idx_scale"], "f32", device))
            itail = torch.zeros_like(st.idx_tail)
            for si, sname in enumerate(("ica", "iza", "icb", "izb")):
                src = dev(g["tail_" + sname], kvk, device)
                for b in range(B):
                    for j in range(src.shape[1]):
                        itail[b, si, int(tail0[b] + j) % st.R] = src[b, j]
            st.idx_tail.copy_(itail)
            io["idx_streams"] = torch.stack(
                [dev(g["new_" + s], kvk, device) for s in ("ica", "iza", "icb", "izb")], dim=1)
            io["q_idx"] = dev(g["q_idx"], idk, device)
            io["q_scale"] = dev(g["q_scale"], "f32", device) if idk == "e4m3" else None
            io["w_idx"] = dev(g["w_idx"], "f32", device)
            io["topk_idx"] = torch.empty((B, g["k"]), dtype=torch.int32, device=device)
            io["topk_cnt"] = torch.empty((B,), dtype=torch.int32, device=device)
        self.io = io
        self.ws = torch.zeros(max(256, L.hybrid_layer_workspace(self.desc, B, 1, E_cap)),
                              dtype=torch.uint8, device=device)
        self._io_struct = self._make_io()
        self._state_struct = st.struct()

    def _make_io(self):
        s = L.DecodeIO()
        for name in ("pos", "q", "q_idx", "q_scale", "w_idx", "x_new", "streams", "idx_streams",
                     "out", "lse", "topk_idx", "topk_cnt"):
            setattr(s, name, L.ptr(self.io.get(name)))
        return s

    def run(self, stream=None):
        L.hybrid_layer_decode(self.desc, self._state_struct, self._io_struct, self.ws, stream)


class PrefillSession:
    """One prefill chunk of a CSA or HCA layer (all sequences aligned)."""

    def __init__(self, g, device="cuda"):
        self.g = g
        B, E_cap, c, m, T = g["B"], g["E_cap"], g["c"], g["m"], g["T"]
        kvk = g["kv_dtype"]
        self.desc = make_desc(g)
        st = _State(g, B, E_cap, device)
        self.state = st
        st.kv_cache.copy_(dev(g["kv_cache"], kvk, device))
        st.n_entries.copy_(dev(g["n_entries"], "i32", device))
        pos0 = int(g["pos0"])
        if g["overlap"] and pos0 > 0:
            for si, sname in ((2, "prev_cb"), (3, "prev_zb")):
                src = dev(g[sname], kvk, device)
                for j in range(m):
                    st.tail[:, si, (pos0 - m + j) % st.R] = src[:, j]
        streams = ("ca", "za", "cb", "zb")[:st.S]
        io = {"q": dev(g["q"], kvk, device), "win": dev(g["win"], kvk, device)}
        io["streams"] = torch.stack([dev(g[s], kvk, device) for s in streams], dim=1)
        H = g["H"]
        io["out"] = torch.empty((B, T, H, c), dtype=_KV[kvk], device=device)
        io["lse"] = torch.empty((B, T, H), dtype=torch.float32, device=device)
        if g["kind"] == "csa":
            idk = g["idx_dtype"]
            st.idx_cache.copy_(dev(g["idx_cache"], idk, device))
            if pos0 > 0:
                for si, sname in ((2, "prev_icb"), (3, "prev_izb")):
                    src = dev(g[sname], kvk, device)
                    for j in range(m):
                        st.idx_tail[:, si, (pos0 - m + j) % st.R] = src[:, j]
            io["idx_streams"] = torch.stack([dev(g[s], kvk, device) for s in ("ica", "iza", "icb", "izb")],
                                            dim=1)
            io["q_idx"] = dev(g["q_idx"], idk, device)
            io["q_scale"] = None
            io["w_idx"] = dev(g["w_idx"], "f32", device)
            io["topk_idx"] = torch.empty((B, T, g["k"]), dtype=torch.int32, device=device)
            io["topk_cnt"] = torch.empty((B, T), dtype=torch.int32, device=device)
        self.io = io
        self.pos0, self.T = pos0, T
        self.ws = torch.zeros(max(256, L.hybrid_layer_workspace(self.desc, B, T, E_cap)),
                              dtype=torch.uint8, device=device)
        s = L.PrefillIO()
        s.pos0, s.T = pos0, T
        for name in ("q", "q_idx", "q_scale", "w_idx", "win", "streams", "idx_streams", "out", "lse",
                     "topk_idx", "topk_cnt"):
            setattr(s, name, L.ptr(io.get(name)))
        self._io_struct = s
        self._state_struct = st.struct()

    def run(self, stream=None):
        L.hybrid_layer_prefill(self.desc, self._state_struct, self._io_struct, self.ws, stream)
