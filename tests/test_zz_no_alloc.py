"""The allocation-free decode entry point against adakv_decode_attn, through
the C ABI: bit-identical outputs on two calls in a row, the second with a
smaller input, both in the split regime that uses the scratch partials."""
import numpy as np
import pytest
import torch

from adaptive_head_budget_amd import configs, lib, pipeline, synth
from adaptive_head_budget_amd.configs import scaled
from parity_util import log

pytestmark = pytest.mark.gpu


def _evicted(cfg, n, seed_name):
    c = scaled(cfg, name=seed_name, decode_steps=2, reserve=2)
    insts = [synth.make_instance(c, i, n_override=n) for i in range(c.instances)]
    st = {k: np.ascontiguousarray(np.stack([x[k] for x in insts])) for k in ("q_win", "k", "v", "q_dec", "k_new",
                                                                               "v_new")}
    q, k, v = (pipeline.to_device(st[x], "bf16") for x in ("q_win", "k", "v"))
    ev = pipeline.Eviction(c, n=n, budget=c.hkv * c.w + (c.hkv * (n - c.w)) // 5, reserve=2)
    ev.evict(q, k, v)
    return c, ev, st


def _split_count(ev):
    """Workgroups per segment the decode launch uses (the partials live in the
    scratch only when there is more than one)."""
    s = ev.shape
    S = s.n_inst * s.hkv
    return S < 512


@pytest.mark.parametrize("first,second", [((2, 6000), (1, 2500))])
def test_noalloc_decode_matches_workspace_decode(gpu_lib, first, second):
    for I, n in (first, second):
        cfg = scaled(configs.LLAMA8B_LAYER, layers=I)
        c, ev, st = _evicted(cfg, n, f"noalloc_I{I}_n{n}")
        assert _split_count(ev), "this case must use split partials"
        out_ws = torch.empty_like(ev.out)
        for t in range(2):
            qd = pipeline.to_device(np.ascontiguousarray(st["q_dec"][:, t]), "bf16")
            kn = pipeline.to_device(np.ascontiguousarray(st["k_new"][:, t]), "bf16")
            vn = pipeline.to_device(np.ascontiguousarray(st["v_new"][:, t]), "bf16")
            # the workspace entry point first (it appends row t), then the
            # allocation-free one on the same state (the same row appended again)
            lib.adakv_decode_attn(ev.shape, ev.alloc, qd, kn, vn, ev.k_flat, ev.v_flat, ev.seg_start, ev.seg_len,
                                  ev.reserve, t, out_ws, ev.ws)
            ev.out.fill_(float("nan"))
            lib.adakv_decode_attn_noalloc(ev.shape, ev.alloc, qd, kn, vn, ev.k_flat, ev.v_flat, ev.seg_start,
                                          ev.seg_len, ev.reserve, t, ev.out)
            torch.cuda.synchronize()
            assert torch.equal(ev.out, out_ws), f"I={I} n={n} step {t}: outputs differ"
            assert torch.isfinite(ev.out).all()
        log(f"  noalloc decode I={I} n={n}: two steps bit-identical to the workspace entry point")
        del ev
        torch.cuda.empty_cache()
