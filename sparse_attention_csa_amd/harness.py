"""Device-side sessions for a decode step or a prefill chunk of one layer.

A session takes inputs given *by position* (a dict of NumPy arrays: bf16 as
uint16 bit patterns, e4m3 as uint8 codes with float32 scales, mxfp4 as packed
uint8 codes with uint8 E8M0 block scales, float32 as is)
and lays them into the library's state layout: the window ring (position p in
slot p % n_win), the compression tail ring (slot p % R, R = 3m with overlap
and 2m without), the compressed caches and their entry counts.  It then calls
the C-ABI entry points.  Pure marshalling: all arithmetic runs in libcsa.so.
"""

import numpy as np
import torch

from . import _lib as L

_KV = {"f32": torch.float32, "bf16": torch.bfloat16}


def act_kind(kvk):
    """Storage of the activations (queries, window rows, token streams,
    outputs): bf16 under the 576-byte FP8 + BF16 cache entry."""
    return "bf16" if kvk == "fp8bf16" else kvk


def dev(arr, kind, device="cuda"):
    """Upload a host array in its storage format."""
    a = np.ascontiguousarray(arr)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if kind in ("e4m3", "mxfp4", "u8", "fp8bf16"):
        return torch.from_numpy(a.view(np.uint8)).to(device)
    if kind == "f32":
        return torch.from_numpy(a.astype(np.float32)).to(device)
    if kind == "f64":
        return torch.from_numpy(a.astype(np.float64)).to(device)
    if kind in ("i32", "i64"):
        return torch.from_numpy(a.astype(np.int32 if kind == "i32" else np.int64)).to(device)
    raise ValueError(kind)


def to_host_bits(t):
    """Device tensor -> NumPy in storage format (bf16 as uint16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


DTYPE_CODE = {"f32": L.CSA_F32, "bf16": L.CSA_BF16, "e4m3": L.CSA_E4M3, "mxfp4": L.CSA_MXFP4,
              "fp8bf16": L.CSA_FP8BF16}
SCALE_KIND = {"e4m3": "f32", "mxfp4": "u8"}  # storage of the scales of a scaled format


def scales_dev(arr, idk, device):
    """Upload the scales of a scaled indexer format (None otherwise)."""
    return dev(arr, SCALE_KIND[idk], device) if idk in SCALE_KIND else None


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
    d.split_rows = int(g.get("split_rows") or 0)
    d.score_bf16 = 1 if g.get("score_dtype") == "bf16" else 0
    if g.get("norm_rope"):
        d.norm_rope = 1
        d.rope_dims = int(g["rope_dims"])
        d.norm_eps = float(g["norm_eps"])
    return d


class _State:
    """Layer state tensors (caches, rings, tails, parameters)."""

    def __init__(self, g, B, E_cap, device):
        kvk = g["kv_dtype"]
        c, m = g["c"], g["m"]
        self.R = 3 * m if g["overlap"] else 2 * m
        self.S = 4 if g["overlap"] else 2
        tdt = _KV[act_kind(kvk)]
        self.kv_scale = None
        if kvk == "fp8bf16":  # 576-byte entries and their scales
            self.kv_cache = torch.zeros((B, E_cap, 576), dtype=torch.uint8, device=device)
            self.kv_scale = torch.ones((B, E_cap), dtype=torch.float32, device=device)
        else:
            self.kv_cache = torch.zeros((B, E_cap, c), dtype=tdt, device=device)
        self.n_entries = torch.zeros(B, dtype=torch.int32, device=device)
        self.win_ring = torch.zeros((B, g["n_win"], c), dtype=tdt, device=device)
        self.tail = torch.zeros((B, self.S, self.R, c), dtype=tdt, device=device)
        self.bias_a = dev(g["bias_a"], "f32", device) if g.get("bias_a") is not None else None
        self.bias_b = dev(g["bias_b"], "f32", device) if g.get("bias_b") is not None else None
        self.sink = dev(g["sink"], "f32", device) if g.get("sink") is not None else None
        self.q_norm_w = self.kv_norm_w = self.rope_inv_freq = None
        if g.get("norm_rope"):
            self.q_norm_w = dev(g["q_norm_w"], "f32", device)
            self.kv_norm_w = dev(g["kv_norm_w"], "f32", device)
            self.rope_inv_freq = dev(g["rope_inv_freq"], "f64", device)
        self.idx_cache = self.idx_scale = self.idx_tail = self.ibias_a = self.ibias_b = None
        if g["kind"] == "csa":
            d_I = g["d_I"]
            idk = g["idx_dtype"]
            if idk == "mxfp4":
                self.idx_cache = torch.zeros((B, E_cap, d_I // 2), dtype=torch.uint8, device=device)
                self.idx_scale = torch.zeros((B, E_cap, d_I // 32), dtype=torch.uint8, device=device)
            else:
                idt = torch.uint8 if idk == "e4m3" else _KV[idk]
                self.idx_cache = torch.zeros((B, E_cap, d_I), dtype=idt, device=device)
            if idk == "e4m3":
                self.idx_scale = torch.ones((B, E_cap), dtype=torch.float32, device=device)
            self.idx_tail = torch.zeros((B, 4, self.R, d_I), dtype=tdt, device=device)
            self.ibias_a = dev(g["ibias_a"], "f32", device)
            self.ibias_b = dev(g["ibias_b"], "f32", device)
        self.B, self.E_cap = B, E_cap
        self.pools = {}  # paged: the pools behind the per-sequence caches
        self.table = None
        self.page_entries = 0
        self.auto_gather = True  # paged: refresh the per-sequence views after each call

    _PAGED = ("kv_cache", "kv_scale", "idx_cache", "idx_scale")

    def page_in(self, g):
        """Paged cache (g["block_table"], g["page_entries"], g["n_pages"]):
        move the per-sequence caches into pools of pages (rows no sequence
        owns hold all-ones bytes, NaN in every float format), which the
        library then reads and writes; the per-sequence tensors become views
        refreshed by gather()."""
        P = int(g["page_entries"])
        table = np.asarray(g["block_table"], np.int32)
        B, E = self.B, self.E_cap
        assert table.shape == (B, E // P) and E % P == 0
        e = np.arange(E)
        rows = table[:, e // P].astype(np.int64) * P + e % P
        device = self.kv_cache.device
        self.rows = torch.from_numpy(rows).to(device)
        self.table = dev(table, "i32", device)
        self.page_entries = P
        for name in self._PAGED:
            x = getattr(self, name)
            if x is None:
                continue
            pool = torch.empty((int(g["n_pages"]) * P,) + tuple(x.shape[2:]), dtype=x.dtype, device=device)
            pool.view(torch.uint8).fill_(0xFF)
            pool[self.rows.reshape(-1)] = x.reshape((-1,) + tuple(x.shape[2:]))
            self.pools[name] = pool

    def gather(self):
        """Paged: refresh the per-sequence caches from the pools (stream-ordered)."""
        for name, pool in self.pools.items():
            getattr(self, name).copy_(pool[self.rows])

    def struct(self):
        s = L.LayerState()
        s.B, s.E_cap = self.B, self.E_cap
        for name in ("kv_cache", "idx_cache", "idx_scale", "n_entries", "win_ring", "tail",
                     "idx_tail", "bias_a", "bias_b", "ibias_a", "ibias_b", "sink", "q_norm_w",
                     "kv_norm_w", "rope_inv_freq", "kv_scale"):
            setattr(s, name, L.ptr(self.pools.get(name, getattr(self, name))))
        s.block_table = L.ptr(self.table)
        s.page_entries = self.page_entries
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
        if st.kv_scale is not None:
            st.kv_scale.copy_(dev(g["kv_scale"], "f32", device))
        kvk = act_kind(kvk)  # the state's rows below are activations
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
        if g["kind"] == "csa":
            idk = g["idx_dtype"]
            st.idx_cache.copy_(dev(g["idx_cache"], idk, device))
            if idk in SCALE_KIND:
                st.idx_scale.copy_(scales_dev(g["idx_scale"], idk, device))
            itail = torch.zeros_like(st.idx_tail)
            for si, sname in enumerate(("ica", "iza", "icb", "izb")):
                src = dev(g["tail_" + sname], kvk, device)
                for b in range(B):
                    for j in range(src.shape[1]):
                        itail[b, si, int(tail0[b] + j) % st.R] = src[b, j]
            st.idx_tail.copy_(itail)
        self.io, self._io_struct = decode_io(g, device)
        self.ws = torch.zeros(max(256, L.hybrid_layer_workspace(self.desc, B, 1, E_cap)),
                              dtype=torch.uint8, device=device)
        if g.get("block_table") is not None:
            st.page_in(g)
        self._state_struct = st.struct()

    def run(self, stream=None):
        L.hybrid_layer_decode(self.desc, self._state_struct, self._io_struct, self.ws, stream)
        _after(self.state, stream)


def decode_io(g, device="cuda"):
    """The per-step inputs and outputs of a decode step (one token per
    sequence) of workload ``g``: a dict of device tensors and the DecodeIO
    structure pointing at them."""
    B, c, H = g["B"], g["c"], g["H"]
    kvk = act_kind(g["kv_dtype"])
    streams = ("ca", "za", "cb", "zb") if g["overlap"] else ("ca", "za")
    io = {}
    io["pos"] = dev(np.asarray(g["pos"], np.int64), "i64", device)
    io["q"] = dev(g["q"], kvk, device)
    io["x_new"] = dev(g["x_new"], kvk, device)
    io["streams"] = torch.stack([dev(g["new_" + s], kvk, device) for s in streams], dim=1)
    io["out"] = torch.empty((B, H, c), dtype=_KV[kvk], device=device)
    io["lse"] = torch.empty((B, H), dtype=torch.float32, device=device)
    if g["kind"] == "csa":
        idk = g["idx_dtype"]
        io["idx_streams"] = torch.stack(
            [dev(g["new_" + s], kvk, device) for s in ("ica", "iza", "icb", "izb")], dim=1)
        io["q_idx"] = dev(g["q_idx"], idk, device)
        io["q_scale"] = scales_dev(g["q_scale"], idk, device)
        io["w_idx"] = dev(g["w_idx"], "f32", device)
        io["topk_idx"] = torch.empty((B, g["k"]), dtype=torch.int32, device=device)
        io["topk_cnt"] = torch.empty((B,), dtype=torch.int32, device=device)
    s = L.DecodeIO()
    for name in ("pos", "q", "q_idx", "q_scale", "w_idx", "x_new", "streams", "idx_streams",
                 "out", "lse", "topk_idx", "topk_cnt"):
        setattr(s, name, L.ptr(io.get(name)))
    return io, s


class PrefillSession:
    """Prefill chunks of a CSA or HCA layer: the state built from workload g
    (its cache, entry counts and, with overlap, the previous block's branch-b
    streams), the first chunk from g's inputs; later chunks (``prefill``) and
    decode steps (``decode``) continue on the library's own state.  A chunk
    with ``seq_pos0`` / ``seq_len`` is a variable-length batch."""

    def __init__(self, g, device="cuda"):
        self.g = g
        B, E_cap, c, m, T = g["B"], g["E_cap"], g["c"], g["m"], g["T"]
        kvk = g["kv_dtype"]
        self.desc = make_desc(g)
        st = _State(g, B, E_cap, device)
        self.state = st
        st.kv_cache.copy_(dev(g["kv_cache"], kvk, device))
        if st.kv_scale is not None:
            st.kv_scale.copy_(dev(g["kv_scale"], "f32", device))
        kvk = act_kind(kvk)
        st.n_entries.copy_(dev(g["n_entries"], "i32", device))
        pos0 = int(g["pos0"])
        if g["overlap"] and pos0 > 0:
            for si, sname in ((2, "prev_cb"), (3, "prev_zb")):
                src = dev(g[sname], kvk, device)
                for j in range(m):
                    st.tail[:, si, (pos0 - m + j) % st.R] = src[:, j]
        if g["kind"] == "csa":
            idk = g["idx_dtype"]
            st.idx_cache.copy_(dev(g["idx_cache"], idk, device))
            if pos0 > 0:
                for si, sname in ((2, "prev_icb"), (3, "prev_izb")):
                    src = dev(g[sname], kvk, device)
                    for j in range(m):
                        st.idx_tail[:, si, (pos0 - m + j) % st.R] = src[:, j]
            if idk in SCALE_KIND:
                st.idx_scale.copy_(scales_dev(g["idx_scale"], idk, device))
        self.io, self._io_struct = prefill_io(g, device)
        self.pos0, self.T = pos0, T
        self.ws = torch.zeros(max(256, L.hybrid_layer_workspace(self.desc, B, T, E_cap)),
                              dtype=torch.uint8, device=device)
        if g.get("block_table") is not None:
            st.page_in(g)
        self._state_struct = st.struct()
        self.dec_ws = None

    def run(self, stream=None):
        L.hybrid_layer_prefill(self.desc, self._state_struct, self._io_struct, self.ws, stream)
        _after(self.state, stream)

    def prefill(self, g_chunk, stream=None):
        """Another chunk on the same state, with the per-token inputs of
        workload ``g_chunk`` (its cache and state fields are not used).
        Returns the chunk's io tensors."""
        device = self.state.kv_cache.device
        io, s = prefill_io(g_chunk, device)
        ws = torch.zeros(max(256, L.hybrid_layer_workspace(self.desc, self.g["B"], int(g_chunk["T"]),
                                                             self.g["E_cap"])), dtype=torch.uint8, device=device)
        L.hybrid_layer_prefill(self.desc, self._state_struct, s, ws, stream)
        _after(self.state, stream)
        io["_ws"] = ws
        return io

    def decode(self, g_step, stream=None):
        """Continue the same layer state with one decode step whose per-token
        inputs are those of decode workload ``g_step`` (its cache and state
        fields are not used: the state is the one this session holds).
        Returns the step's io tensors."""
        if self.dec_ws is None:
            self.dec_ws = torch.zeros(
                max(256, L.hybrid_layer_workspace(self.desc, self.g["B"], 1, self.g["E_cap"])),
                dtype=torch.uint8, device=self.state.kv_cache.device)
        io, s = decode_io(g_step, self.state.kv_cache.device)
        L.hybrid_layer_decode(self.desc, self._state_struct, s, self.dec_ws, stream)
        _after(self.state, stream)
        return io


def prefill_io(g, device="cuda"):
    """The inputs and outputs of a prefill chunk of workload ``g`` ([B][T]
    rows; with ``seq_pos0`` / ``seq_len`` a variable-length batch): a dict of
    device tensors and the PrefillIO structure pointing at them."""
    B, c, H, T = g["B"], g["c"], g["H"], int(g["T"])
    kvk = act_kind(g["kv_dtype"])
    streams = ("ca", "za", "cb", "zb") if g["overlap"] else ("ca", "za")
    io = {"q": dev(g["q"], kvk, device), "win": dev(g["win"], kvk, device)}
    io["streams"] = torch.stack([dev(g[s], kvk, device) for s in streams], dim=1)
    io["out"] = torch.empty((B, T, H, c), dtype=_KV[kvk], device=device)
    io["lse"] = torch.empty((B, T, H), dtype=torch.float32, device=device)
    if g["kind"] == "csa":
        idk = g["idx_dtype"]
        io["idx_streams"] = torch.stack([dev(g[s], kvk, device) for s in ("ica", "iza", "icb", "izb")], dim=1)
        io["q_idx"] = dev(g["q_idx"], idk, device)
        io["q_scale"] = scales_dev(g["q_scale"], idk, device)
        io["w_idx"] = dev(g["w_idx"], "f32", device)
        io["topk_idx"] = torch.empty((B, T, g["k"]), dtype=torch.int32, device=device)
        io["topk_cnt"] = torch.empty((B, T), dtype=torch.int32, device=device)
    if g.get("seq_pos0") is not None:
        io["seq_pos0"] = dev(np.asarray(g["seq_pos0"], np.int64), "i64", device)
        io["seq_len"] = dev(np.asarray(g["seq_len"], np.int32), "i32", device)
    s = L.PrefillIO()
    s.pos0, s.T = int(g["pos0"]), T
    for name in ("q", "q_idx", "q_scale", "w_idx", "win", "streams", "idx_streams", "out", "lse",
                 "topk_idx", "topk_cnt", "seq_pos0", "seq_len"):
        setattr(s, name, L.ptr(io.get(name)))
    return io, s


def _after(st, stream):
    """Paged state: the per-sequence views follow the pools after a call."""
    if not st.pools or not st.auto_gather:
        return
    if stream is None:
        st.gather()
    else:
        with torch.cuda.stream(stream):
            st.gather()
