"""Device buffers for one eviction pass and the four library calls in order.

PyTorch only provides device memory and the stream; every step runs in
libadakv's kernels through the ctypes binding.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import lib
from .configs import Workload

_SCORERS = {"snapkv": lib.ADAKV_SCORE_SNAPKV, "lava": lib.ADAKV_SCORE_LAVA, "criticalkv": lib.ADAKV_SCORE_CRITICALKV,
            "laprox": lib.ADAKV_SCORE_LAPROX}
_MODES = {"snapkv": lib.ADAKV_ALLOC_ADA, "lava": lib.ADAKV_ALLOC_LAVA_LAYERS,
          "criticalkv": lib.ADAKV_ALLOC_ADA_CRITICALKV, "laprox": lib.ADAKV_ALLOC_GLOBAL}
_ALLOC_NAMES = {"ada": lib.ADAKV_ALLOC_ADA, "lava": lib.ADAKV_ALLOC_LAVA_LAYERS,
                "criticalkv": lib.ADAKV_ALLOC_ADA_CRITICALKV, "global": lib.ADAKV_ALLOC_GLOBAL,
                "floor": lib.ADAKV_ALLOC_ADA_FLOOR, "streaming": lib.ADAKV_ALLOC_STREAMING}


def make_shape(cfg: Workload, n_inst: Optional[int] = None, n: Optional[int] = None) -> lib.AdakvShape:
    return lib.AdakvShape(
        n_inst=cfg.instances if n_inst is None else n_inst, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d,
        n=cfg.n if n is None else n, w=cfg.w, pool=cfg.pool,
        dtype=lib.ADAKV_BF16 if cfg.dtype == "bf16" else lib.ADAKV_F32, scorer=_SCORERS[cfg.scorer],
        hidden=cfg.hidden, eps=cfg.eps, reserved0=0)


def make_alloc(cfg: Workload, budget: Optional[int] = None, inst_budget=None) -> lib.AdakvAlloc:
    """Allocation settings of a workload.  inst_budget: per-instance budgets
    (preset layer budgets, Ada-KV mode); the ctypes array is kept on the
    returned struct so it lives as long as the struct."""
    mode = _ALLOC_NAMES[cfg.alloc] if cfg.alloc else _MODES[cfg.scorer]
    a = lib.AdakvAlloc(mode=mode, alpha_num=cfg.alpha[0], alpha_den=cfg.alpha[1], ck_num=cfg.ck[0],
                       ck_den=cfg.ck[1], sinks=cfg.stream_sinks, budget=cfg.budget if budget is None else budget)
    if inst_budget is not None:
        arr = (ctypes.c_int64 * len(inst_budget))(*[int(x) for x in inst_budget])
        a.inst_budget = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64))
        a._keep = arr
    return a


def selected_rows(shape: lib.AdakvShape, alloc: lib.AdakvAlloc) -> int:
    if alloc.mode in (lib.ADAKV_ALLOC_LAVA_LAYERS, lib.ADAKV_ALLOC_GLOBAL):
        return alloc.budget - shape.n_inst * shape.w * shape.hkv
    if alloc.inst_budget:
        return sum(int(alloc.inst_budget[i]) - shape.w * shape.hkv for i in range(shape.n_inst))
    return shape.n_inst * (alloc.budget - shape.w * shape.hkv)


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    """Storage array (bf16 bits as uint16, or float32) -> device tensor."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_host_f64(t) -> np.ndarray:
    """Device tensor (bf16 or f32) -> float64 values, exactly."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


class Eviction:
    """Output buffers and workspace for one call sequence score -> allocate ->
    compact -> decode over I instances."""

    def __init__(self, cfg: Workload, n_inst: Optional[int] = None, n: Optional[int] = None,
                 budget: Optional[int] = None, reserve: Optional[int] = None, device="cuda", inst_budget=None):
        import torch
        self.cfg = cfg
        self.shape = make_shape(cfg, n_inst, n)
        self.alloc = make_alloc(cfg, budget, inst_budget)
        self.reserve = cfg.reserve if reserve is None else reserve
        s = self.shape
        I, hkv, p = s.n_inst, s.hkv, s.n - s.w
        self.tdtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        ws_bytes = lib.adakv_workspace_bytes(s, self.alloc, self.reserve)
        if ws_bytes == 0:
            raise ValueError("invalid shape or allocation settings")
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        self.score = torch.empty((I, hkv, p), dtype=torch.float32, device=device)
        self.score2 = (torch.empty((I, hkv, p), dtype=torch.float32, device=device)
                       if cfg.scorer == "criticalkv" else None)
        self.budgets = torch.empty((I, hkv), dtype=torch.int32, device=device)
        self.n_sel = selected_rows(s, self.alloc)
        self.sel = torch.empty((max(self.n_sel, 4),), dtype=torch.int32, device=device)
        self.sel_off = torch.empty((I + 1,), dtype=torch.int64, device=device)
        self.rows = self.n_sel + I * hkv * (s.w + self.reserve)
        self.k_flat = torch.empty((self.rows, s.d), dtype=self.tdtype, device=device)
        self.v_flat = torch.empty((self.rows, s.d), dtype=self.tdtype, device=device)
        self.seg_start = torch.empty((I * hkv + 1,), dtype=torch.int64, device=device)
        self.seg_len = torch.empty((I * hkv,), dtype=torch.int32, device=device)
        self.out = torch.empty((I, s.hq, s.d), dtype=torch.float32, device=device)
        self.step = 0

    def run_score(self, q_win, k, v=None, w_o=None, stream=None, row_lse=None):
        """Window scores; with row_lse [I, hq, w] (float32 log-sum-exp of each
        window row over its domain) the single-pass entry point is used.  A
        w_o with a leading instance dimension ([I, hidden, hq*d]: one output
        projection per layer) is scored one instance per call."""
        if w_o is not None and w_o.dim() == 3:
            one = make_shape(self.cfg, 1, self.shape.n)
            for i in range(self.shape.n_inst):
                lse = None if row_lse is None else row_lse[i]
                s2 = None if self.score2 is None else self.score2[i]
                if lse is None:
                    lib.adakv_score(one, q_win[i], k[i], v[i], w_o[i], self.score[i], s2, self.ws, stream)
                else:
                    lib.adakv_score_lse(one, q_win[i], k[i], v[i], w_o[i], lse, self.score[i], s2, self.ws,
                                        stream)
            return
        if row_lse is None:
            lib.adakv_score(self.shape, q_win, k, v, w_o, self.score, self.score2, self.ws, stream)
        else:
            lib.adakv_score_lse(self.shape, q_win, k, v, w_o, row_lse, self.score, self.score2, self.ws, stream)

    def lse_from_causal(self, q_win, k, lse_causal, out=None, row_flag=None, stream=None):
        """The scorer's window-row log-sum-exp [I, hq, w] (float32) from the
        causal one a prefill leaves (keys 0 .. p + r for window row r), for
        run_score's row_lse.  out may be lse_causal (in place); row_flag, an
        int32 [I, hq, w] tensor or None, receives 0 (well conditioned), 1
        (the prefix keeps less than 2^-7 of the causal mass) or 2 (not
        finite) per row."""
        import torch
        if out is None:
            out = torch.empty_like(lse_causal)
        lib.adakv_lse_from_causal(self.shape, q_win, k, lse_causal, out, row_flag, stream)
        return out

    def scores_invalid(self) -> bool:
        """Whether the last allocation read a negative, NaN or infinite score
        (the int32 the library keeps at the start of the workspace).  Waits
        for the device."""
        import torch
        torch.cuda.synchronize(self.ws.device)
        return bool(self.ws[:4].view(torch.int32).item())

    def run_allocate(self, stream=None):
        lib.adakv_allocate(self.shape, self.alloc, self.score, self.score2, self.budgets, self.sel, self.sel_off,
                           self.ws, stream)

    def run_compact(self, k, v, stream=None):
        lib.adakv_compact(self.shape, self.alloc, k, v, self.budgets, self.sel, self.sel_off, self.reserve,
                          self.k_flat, self.v_flat, self.seg_start, self.seg_len, stream)
        self.step = 0

    def run_decode(self, q, k_new=None, v_new=None, stream=None):
        lib.adakv_decode_attn(self.shape, self.alloc, q, k_new, v_new, self.k_flat, self.v_flat, self.seg_start,
                              self.seg_len, self.reserve, self.step, self.out, self.ws, stream)
        if k_new is not None:
            self.step += 1

    def evict(self, q_win, k, v=None, w_o=None, stream=None, row_lse=None):
        self.run_score(q_win, k, v, w_o, stream, row_lse)
        self.run_allocate(stream)
        self.run_compact(k, v, stream)

    # host views -------------------------------------------------------------
    def host_selection(self):
        """Per instance, per head: the selected token indices (numpy)."""
        b = self.budgets.cpu().numpy().astype(np.int64)
        sel = self.sel.cpu().numpy().astype(np.int64)
        off = self.sel_off.cpu().numpy()
        res = []
        for i in range(b.shape[0]):
            pos = int(off[i])
            heads = []
            for g in range(b.shape[1]):
                heads.append(sel[pos:pos + b[i, g]])
                pos += int(b[i, g])
            res.append(heads)
        return b, off, res


class LavaOnline:
    """LAVa's online prefill over the layers of one sequence: after each layer
    is prefilled, score it, re-allocate every layer so far under the shared
    total, and rebuild the flat cache from the new layer's dense K/V and the
    previous flat cache (two buffers used in turn).  Only the newest layer's
    dense cache is read at each step.  Each layer's entropy is kept from the
    step that added it; with `incremental` (the default) the older layers are
    re-selected from their previous kept entries, otherwise from their full
    scores (the same result)."""

    def __init__(self, cfg: Workload, n: Optional[int] = None, total: Optional[int] = None, device="cuda"):
        import torch
        if cfg.scorer != "lava" or cfg.batch != 1:
            raise ValueError("the online prefill runs the LAVa scorer on the layers of one sequence")
        self.cfg = cfg
        self.L = cfg.layers
        self.n = cfg.n if n is None else n
        self.total = cfg.budget if total is None else total
        s = make_shape(cfg, self.L, self.n)
        self.hkv, self.w, self.p = s.hkv, s.w, s.n - s.w
        self.tdtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        lava = lib.AdakvAlloc(mode=lib.ADAKV_ALLOC_LAVA_LAYERS, alpha_num=0, alpha_den=1, ck_num=0, ck_den=1, sinks=0,
                              budget=self.L * self.w * self.hkv)
        ws = max(lib.adakv_workspace_bytes(s, lava, 0), lib.adakv_workspace_bytes(make_shape(cfg, 1, self.n), None, 0))
        self.ws = torch.empty(ws, dtype=torch.uint8, device=device)
        self.score = torch.empty((self.L, self.hkv, self.p), dtype=torch.float32, device=device)
        cap = max(self.total - self.w * self.hkv, 4)         # B'(0), the largest selection of any step
        rows = max(self.total, 1)                            # B'(l) + (l+1)*w*hkv = total at every step
        self.bufs = []
        for _ in range(2):
            self.bufs.append({
                "budgets": torch.empty((self.L * self.hkv,), dtype=torch.int32, device=device),
                "sel": torch.empty((cap,), dtype=torch.int32, device=device),
                "sel_off": torch.empty((self.L + 1,), dtype=torch.int64, device=device),
                "k_flat": torch.empty((rows, s.d), dtype=self.tdtype, device=device),
                "v_flat": torch.empty((rows, s.d), dtype=self.tdtype, device=device),
                "seg_start": torch.empty((self.L * self.hkv + 1,), dtype=torch.int64, device=device),
                "seg_len": torch.empty((self.L * self.hkv,), dtype=torch.int32, device=device),
            })
        self.layer_ent = torch.zeros((self.L,), dtype=torch.float64, device=device)
        self.max_rows = rows
        self.layers_done = 0

    def current(self):
        return self.bufs[(self.layers_done - 1) % 2]

    def step(self, q_win, k, v, stream=None, incremental=True):
        """Prefill-time eviction after the next layer: q_win [hq, w, d],
        k, v [hkv, n, d] of that layer."""
        l = self.layers_done
        if l >= self.L:
            raise ValueError("every layer is already prefilled")
        one = make_shape(self.cfg, 1, self.n)
        lib.adakv_score(one, q_win, k, v, None, self.score[l], None, self.ws, stream)
        cur, prev = self.bufs[l % 2], self.bufs[(l + 1) % 2]
        sh = make_shape(self.cfg, l + 1, self.n)
        inc = incremental and l > 0
        lib.adakv_lava_online_allocate(sh, self.total, self.score[:l + 1], prev["sel_off"] if l else None,
                                       prev["budgets"] if inc else None, prev["sel"] if inc else None,
                                       self.layer_ent, cur["budgets"], cur["sel"], cur["sel_off"], self.ws, stream)
        old = (lambda key: prev[key] if l else None)
        lib.adakv_lava_online_compact(sh, k, v, old("k_flat"), old("v_flat"), old("seg_start"), old("sel"),
                                      old("sel_off"), cur["budgets"], cur["sel"], cur["sel_off"], self.max_rows,
                                      cur["k_flat"], cur["v_flat"], cur["seg_start"], cur["seg_len"], stream)
        self.layers_done = l + 1

    def host_selection(self):
        """Per layer present, per head: the selected token indices (numpy)."""
        cur = self.current()
        I = self.layers_done
        b = cur["budgets"][:I * self.hkv].cpu().numpy().astype(np.int64).reshape(I, self.hkv)
        sel = cur["sel"].cpu().numpy().astype(np.int64)
        off = cur["sel_off"][:I + 1].cpu().numpy()
        res = []
        for i in range(I):
            pos, heads = int(off[i]), []
            for g in range(self.hkv):
                heads.append(sel[pos:pos + b[i, g]])
                pos += int(b[i, g])
            res.append(heads)
        return b, off, res
