"""GPU parity of the HIP path against the oracle, through the C ABI.

Sizes: the tiny workload in full; the Llama-3.1-8B layer in full; the other
workloads at reduced cache length or instance count (several tiles plus a
ragged tail) with every output checked, and at full size in the benchmark's
launch configuration: every instance of the 32-layer Llama and LAVa workloads,
the CriticalKV composite on two whole KV heads and at every stage-2 cut-off,
LaProx on sampled keys.
"""
import numpy as np
import pytest
import torch

from adaptive_head_budget_amd import configs, lib, pipeline, synth
from adaptive_head_budget_amd.configs import scaled
from oracle import allocation, cache, scoring
from parity_util import (assert_decode_close, assert_scores_close, check_flat, check_lava_layer_budgets,
                         check_selection, jaccard, log, oracle_scores)

pytestmark = pytest.mark.gpu


def _stack(cfg, I, n):
    insts = [synth.make_instance(cfg, i, n_override=n) for i in range(I)]
    keys = [k for k in insts[0] if k not in ("w_o", "tau")]
    return insts, {k: np.ascontiguousarray(np.stack([x[k] for x in insts])) for k in keys}


def _w(x, dtype):
    return synth.widen(x, dtype)


def run_case(cfg, I, n, budget, reserve, steps, label, check_scores_of=None, single_pass=False, inst_budget=None,
             causal_lse=False):
    """Run score -> allocate -> compact -> decode on numpy-drawn inputs and
    check every stage.  Returns the Eviction object.  single_pass: score
    through adakv_score_lse with the oracle's window-row log-sum-exp (rounded
    to float32, the same input for both sides).  causal_lse: the same, but the
    input is the causal statistic a prefill leaves (keys 0 .. p + r, rounded
    to float32), turned into the scorer's own by adakv_lse_from_causal on the
    device and by the oracle's lse_from_causal on the host.  inst_budget:
    per-instance budgets (preset layer budgets) instead of `budget`."""
    log(f"case {label}: {cfg.name} I={I} n={n} budget={budget} reserve={reserve} steps={steps}")
    if steps != cfg.decode_steps:
        cfg = scaled(cfg, decode_steps=steps)       # draws of q, k, v do not depend on this
    dt = cfg.dtype
    insts, st = _stack(cfg, I, n)
    q = pipeline.to_device(st["q_win"], dt)
    k = pipeline.to_device(st["k"], dt)
    v = pipeline.to_device(st["v"], dt)
    if cfg.scorer == "criticalkv":
        w_o = pipeline.to_device(insts[0]["w_o"], dt)
    elif cfg.scorer == "laprox":                                  # one projection per layer
        w_o = pipeline.to_device(np.stack([x["w_o"] for x in insts]), dt)
    else:
        w_o = None
    wo_of = (lambda i: insts[i]["w_o"]) if cfg.scorer == "laprox" else (lambda i: insts[0]["w_o"])
    ev = pipeline.Eviction(cfg, n_inst=I, n=n, budget=budget, reserve=reserve, inst_budget=inst_budget)
    w = cfg.w
    k64 = [_w(x["k"], dt) for x in insts]
    v64 = [_w(x["v"], dt) for x in insts]
    lse32 = lse_ref = lse_dev = None
    if causal_lse:
        lc32 = np.stack([scoring.window_lse(_w(insts[i]["q_win"], dt), k64[i], causal=True)
                         for i in range(I)]).astype(np.float32)
        lse_dev = ev.lse_from_causal(q, k, torch.from_numpy(lc32).cuda())
        lse_ref = np.stack([scoring.lse_from_causal(lc32[i].astype(np.float64), _w(insts[i]["q_win"], dt), k64[i],
                                                    cfg.scorer)[0] for i in range(I)])
    elif single_pass:
        lse32 = np.stack([scoring.window_lse(_w(insts[i]["q_win"], dt), k64[i], causal=cfg.scorer == "lava",
                                             full=cfg.scorer == "laprox")
                          for i in range(I)]).astype(np.float32)
        lse_dev = torch.from_numpy(lse32).cuda()
        lse_ref = lse32.astype(np.float64)
    ev.run_score(q, k, v if cfg.scorer != "snapkv" else None, w_o, row_lse=lse_dev)
    torch.cuda.synchronize()
    score = ev.score.cpu().numpy()
    score2 = ev.score2.cpu().numpy() if ev.score2 is not None else None
    for i in (range(I) if check_scores_of is None else check_scores_of):
        ref, ref2 = oracle_scores(cfg.scorer, _w(insts[i]["q_win"], dt), k64[i], v64[i],
                                  _w(wo_of(i), dt) if w_o is not None else None, cfg.pool, cfg.eps,
                                  None if lse_ref is None else lse_ref[i])
        worst = assert_scores_close(score[i], ref, f"{label} score inst {i}")
        if ref2 is not None:
            assert_scores_close(score2[i], ref2, f"{label} composite inst {i}")
        log(f"  scores inst {i}: worst rel {worst:.2e}")

    ev.run_allocate()
    torch.cuda.synchronize()
    b, off, sel = ev.host_selection()
    if cfg.scorer == "lava":
        r = allocation.lava_allocate(score.astype(np.float64), budget, w)
        lb = np.array([off[l + 1] - off[l] for l in range(I)])
        if not check_lava_layer_budgets(lb, r["layer_budgets"], r["entropy"], budget - I * w * cfg.hkv, label):
            r = allocation.lava_allocate(score.astype(np.float64), budget, w, layer_budgets=lb)
        for l in range(I):
            check_selection(b[l], off[l], sel[l], r["budgets"][l], r["sel"][l], f"{label} layer {l}")
    elif cfg.scorer == "laprox":
        r = allocation.global_allocate(score.astype(np.float64), budget, w)
        base = 0
        for i in range(I):
            check_selection(b[i], int(off[i]), sel[i], r["budgets"][i], r["sel"][i], f"{label} inst {i}",
                            off_ref=base)
            base += int(r["budgets"][i].sum())
        assert int(off[I]) == r["Bp"]
    else:
        base = 0
        for i in range(I):
            bi = budget if inst_budget is None else int(inst_budget[i])
            if cfg.alloc == "floor":
                r = allocation.ada_floor_allocate(score[i].astype(np.float64), bi, w, cfg.alpha)
            elif cfg.alloc == "streaming":
                r = allocation.streaming_allocate(cfg.hkv, n - w, bi, w, cfg.stream_sinks)
            elif cfg.scorer == "criticalkv":
                r = allocation.criticalkv_allocate(score[i].astype(np.float64), score2[i].astype(np.float64),
                                                   bi, w, cfg.alpha, cfg.ck)
            else:
                r = allocation.ada_allocate(score[i].astype(np.float64), bi, w, cfg.alpha)
            check_selection(b[i], int(off[i]), sel[i], r["budgets"], r["sel"], f"{label} inst {i}", off_ref=base)
            base += bi - w * cfg.hkv
        assert int(off[I]) == base

    ev.run_compact(k, v)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):     # reserve rows are not written yet: any bits, NaN patterns included
        kf = pipeline.to_host_f64(ev.k_flat)
        vf = pipeline.to_host_f64(ev.v_flat)
    ss = ev.seg_start.cpu().numpy()
    sl = ev.seg_len.cpu().numpy()
    hats = [check_flat(kf, vf, ss, sl, i, cfg.hkv, k64[i], v64[i], sel[i], w, label) for i in range(I)]
    log(f"  selection + flat cache exact")

    for t in range(steps):
        qd = pipeline.to_device(np.ascontiguousarray(st["q_dec"][:, t]), dt)
        if cfg.append:
            kn = np.ascontiguousarray(st["k_new"][:, t])
            vn = np.ascontiguousarray(st["v_new"][:, t])
            ev.run_decode(qd, pipeline.to_device(kn, dt), pipeline.to_device(vn, dt))
            hats = [cache.append(kh, vh, _w(kn[i], dt), _w(vn[i], dt)) for i, (kh, vh) in enumerate(hats)]
        else:
            ev.run_decode(qd)
        torch.cuda.synchronize()
        out = ev.out.cpu().numpy()
        if t in (0, steps - 1):
            for i in range(I):
                ref = cache.decode(_w(st["q_dec"][i, t], dt), hats[i][0], hats[i][1])
                ma, rl = assert_decode_close(out[i], ref, f"{label} decode step {t} inst {i}")
            log(f"  decode step {t}: max-abs {ma:.2e} rel-L2 {rl:.2e}")
    return ev


# ------------------------------------------------------------------ workloads
def test_tiny_mha_full(gpu_lib):
    cfg = configs.TINY_MHA
    run_case(cfg, 1, cfg.n, cfg.budget, cfg.reserve, cfg.decode_steps, "tiny")


def test_llama_layer_reduced(gpu_lib):
    cfg = configs.LLAMA8B_LAYER
    n = 2000                                   # 1968 prefix keys: 15 full tiles + a ragged tail
    run_case(cfg, 1, n, (20 * cfg.hkv * n) // 100, 2, 2, "llama-layer n2000")


def test_llama_layer_full(gpu_lib):
    cfg = configs.LLAMA8B_LAYER
    run_case(cfg, 1, cfg.n, cfg.budget, cfg.reserve, cfg.decode_steps, "llama-layer full")


def test_llama_model_reduced(gpu_lib):
    cfg = scaled(configs.LLAMA8B_MODEL, layers=2, batch=2)
    run_case(cfg, 4, 3000, 8 * 200, 4, 4, "llama-model I4 n3000")


def test_lava_reduced(gpu_lib):
    cfg = scaled(configs.MISTRAL7B_LAVA, layers=4)
    n = 3000
    run_case(cfg, 4, n, 4 * 8 * (32 + 96), 0, 0, "lava L4 n3000")


def test_criticalkv_reduced(gpu_lib):
    cfg = scaled(configs.QWEN32B_CK, hidden=1024)
    n = 2100
    run_case(cfg, 1, n, (40 * cfg.hkv * n) // 100, 0, 0, "criticalkv n2100 D1024")


def test_laprox_reduced(gpu_lib):
    cfg = scaled(configs.MISTRAL7B_LAPROX, layers=3, hidden=1024)
    n = 2100                                   # 2068 prefix keys: 16 full tiles + a ragged tail
    run_case(cfg, 3, n, 3 * 32 * 8 + (3 * 8 * (n - 32)) // 10, 0, 0, "laprox L3 n2100 D1024")


# ------------------------------------------------------------------ single pass (row statistics supplied)
@pytest.mark.parametrize("draw", range(3))
@pytest.mark.parametrize("scorer", ["snapkv", "lava", "criticalkv", "laprox"])
def test_fresh_draws(gpu_lib, scorer, draw):
    """Every scorer on three more seeded draws (the seed follows the workload
    name), at reduced sizes with a ragged last tile."""
    if scorer == "snapkv":
        cfg = scaled(configs.LLAMA8B_MODEL, layers=2, batch=2, name=f"draw{draw}_snapkv")
        run_case(cfg, 4, 1500, 8 * 120, 2, 2, f"snapkv draw {draw}")
    elif scorer == "lava":
        cfg = scaled(configs.MISTRAL7B_LAVA, layers=3, name=f"draw{draw}_lava")
        run_case(cfg, 3, 1300, 3 * 8 * (32 + 60), 0, 0, f"lava draw {draw}")
    elif scorer == "criticalkv":
        cfg = scaled(configs.QWEN32B_CK, hidden=512, name=f"draw{draw}_ck")
        run_case(cfg, 1, 1300, (40 * cfg.hkv * 1300) // 100, 0, 0, f"criticalkv draw {draw}")
    else:
        cfg = scaled(configs.MISTRAL7B_LAPROX, layers=2, hidden=512, name=f"draw{draw}_laprox")
        run_case(cfg, 2, 1300, 2 * 32 * 8 + (2 * 8 * 1268) // 10, 0, 0, f"laprox draw {draw}")


def test_single_pass_tiny(gpu_lib):
    cfg = configs.TINY_MHA
    run_case(cfg, 1, cfg.n, cfg.budget, cfg.reserve, cfg.decode_steps, "tiny single-pass", single_pass=True)


def test_single_pass_llama_reduced(gpu_lib):
    cfg = scaled(configs.LLAMA8B_MODEL, layers=2, batch=2)
    run_case(cfg, 4, 3000, 8 * 200, 1, 1, "llama-model I4 n3000 single-pass", single_pass=True)


def test_single_pass_lava_reduced(gpu_lib):
    cfg = scaled(configs.MISTRAL7B_LAVA, layers=4)
    run_case(cfg, 4, 3000, 4 * 8 * (32 + 96), 0, 0, "lava L4 n3000 single-pass", single_pass=True)


def test_single_pass_criticalkv_reduced(gpu_lib):
    cfg = scaled(configs.QWEN32B_CK, hidden=1024)
    n = 2100
    run_case(cfg, 1, n, (40 * cfg.hkv * n) // 100, 0, 0, "criticalkv n2100 D1024 single-pass", single_pass=True)


def test_single_pass_laprox_reduced(gpu_lib):
    cfg = scaled(configs.MISTRAL7B_LAPROX, layers=2, hidden=512)
    run_case(cfg, 2, 1500, 2 * 32 * 8 + 900, 0, 0, "laprox L2 n1500 D512 single-pass", single_pass=True)


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("hq,hkv,w,pool,d,dtype", [
    (8, 8, 7, 5, 64, "bf16"),      # MHA, w < 16, pool 5, d 64
    (40, 8, 40, 1, 128, "bf16"),   # G = 5, w = 40 (padded window rows), no pooling
    (8, 1, 16, 3, 64, "f32"),      # G = 8, fp32 d 64
])
def test_geometries(gpu_lib, hq, hkv, w, pool, d, dtype):
    cfg = scaled(configs.LLAMA8B_LAYER, hq=hq, hkv=hkv, w=w, pool=pool, d=d, dtype=dtype,
                 name=f"geom_{hq}_{hkv}_{w}_{pool}_{d}_{dtype}", reserve=1, decode_steps=1)
    n = 1000
    run_case(cfg, 2, n, (30 * hkv * n) // 100, 1, 1, cfg.name)


# The register-K scoring kernels (bf16, d = 128, w <= 32) engage only when a
# call gives every resident workgroup several 64-key blocks; many short
# instances in one call do, so these cases reach their edges: group sizes 1,
# 2, 5, 8, one or two 16-row window blocks (padded rows), every pool width,
# ragged last blocks, causal statistics, the supplied-statistics mode.
KR_CASES = [
    # scorer, hq, hkv, w, pool, n
    ("snapkv", 32, 8, 32, 7, 1000),
    ("snapkv", 8, 8, 16, 3, 777),
    ("snapkv", 16, 8, 20, 5, 1500),
    ("snapkv", 40, 8, 32, 1, 900),
    ("snapkv", 64, 8, 12, 7, 1100),
    ("lava", 32, 8, 32, 7, 1000),
]


@pytest.mark.parametrize("scorer,hq,hkv,w,pool,n", KR_CASES)
def test_register_k_path(gpu_lib, scorer, hq, hkv, w, pool, n):
    base = configs.MISTRAL7B_LAVA if scorer == "lava" else configs.LLAMA8B_LAYER
    cfg = scaled(base, hq=hq, hkv=hkv, w=w, pool=pool, name=f"kr_{scorer}_{hq}_{hkv}_{w}_{pool}", reserve=1,
                 decode_steps=1)
    I = 256
    if scorer == "lava":   # the layers share at most one layer's prefix entries (B' <= hkv * p)
        run_case(cfg, I, n, I * hkv * w + (hkv * (n - w)) // 2, 1, 1, cfg.name)
    else:
        run_case(cfg, I, n, hkv * w + (hkv * (n - w)) // 5, 1, 1, cfg.name)


def test_register_k_single_pass(gpu_lib):
    cfg = scaled(configs.LLAMA8B_LAYER, name="kr_single_pass", reserve=1, decode_steps=1)
    n = 1000
    run_case(cfg, 256, n, cfg.hkv * cfg.w + (cfg.hkv * (n - cfg.w)) // 5, 1, 1, cfg.name, single_pass=True)


# scorer, dtype, hq, hkv, d, w, n: GQA groups 1..8, window lengths with a
# ragged last chunk of eight keys, up to 512 rows (and 64 KiB of window keys)
# per workgroup
CAUSAL_CASES = [
    ("snapkv", "bf16", 32, 8, 128, 32, 300),
    ("criticalkv", "bf16", 40, 8, 128, 32, 257),
    ("laprox", "bf16", 32, 8, 128, 32, 300),
    ("lava", "bf16", 32, 8, 128, 32, 300),
    ("snapkv", "bf16", 64, 8, 128, 64, 200),
    ("laprox", "bf16", 64, 8, 64, 64, 200),
    ("snapkv", "bf16", 8, 8, 64, 13, 150),
    ("snapkv", "f32", 4, 4, 16, 4, 64),
    ("laprox", "f32", 12, 4, 64, 21, 90),
    ("snapkv", "bf16", 10, 2, 128, 1, 40),
]


def _causal_inputs(scorer, dtype, hq, hkv, d, w, n, I, window_gain=0.0):
    """Instances of a scaled Llama layer, the window keys optionally pulled
    towards each head group's first query head (gain a: row j's own key gets
    a * (j+1)/w * 4 sqrt(d) along that query), so the window holds most of
    the causal mass of the later rows."""
    base = configs.TINY_MHA if dtype == "f32" else configs.LLAMA8B_LAYER
    cfg = scaled(base, name=f"causal_{scorer}_{hq}_{hkv}_{d}_{w}", hq=hq, hkv=hkv, d=d, w=w, scorer=scorer,
                 tau=("loguniform", 0.1, 3.0), hidden=256 if scorer in ("criticalkv", "laprox") else 0)
    insts, st = _stack(cfg, I, n)
    q64 = _w(st["q_win"], dtype)
    k64 = _w(st["k"], dtype)
    if window_gain:
        G, p = hq // hkv, n - w
        for i in range(I):
            for g in range(hkv):
                for j in range(w):
                    qj = q64[i, g * G, j]
                    k64[i, g, p + j] = (window_gain * (j + 1) / w * 4 * np.sqrt(d)) * qj / np.linalg.norm(qj)
        k_st = synth._store(k64.astype(np.float32), dtype)
        k64 = _w(k_st, dtype)
        st["k"] = k_st
    return cfg, st, q64, k64


def _check_causal(cfg, st, q64, k64, label, in_place=False):
    dt, I = cfg.dtype, q64.shape[0]
    lc32 = np.stack([scoring.window_lse(q64[i], k64[i], causal=True) for i in range(I)]).astype(np.float32)
    ref, keep = zip(*[scoring.lse_from_causal(lc32[i].astype(np.float64), q64[i], k64[i], cfg.scorer)
                      for i in range(I)])
    ref, keep = np.stack(ref), np.stack(keep)
    lc = torch.from_numpy(lc32).cuda()
    flag = torch.full(lc.shape, -1, dtype=torch.int32, device="cuda")
    out = lc if in_place else torch.full_like(lc, float("nan"))
    lib.adakv_lse_from_causal(pipeline.make_shape(cfg, I, k64.shape[2]), pipeline.to_device(st["q_win"], dt),
                              pipeline.to_device(st["k"], dt), lc, out, flag)
    torch.cuda.synchronize()
    got, fl = out.cpu().numpy().astype(np.float64), flag.cpu().numpy()
    want_flag = np.where(keep < 2.0 ** -7, 1, 0)
    # the flag is a float64 comparison on both sides: no row may sit at the threshold
    assert np.all(np.abs(keep - 2.0 ** -7) > 1e-12), f"{label}: a row sits at the flag threshold"
    assert np.array_equal(fl, want_flag), f"{label}: flags differ at {np.argwhere(fl != want_flag)[:5]}"
    assert np.isfinite(got).all(), f"{label}: non-finite statistic"
    tight = keep >= 2.0 ** -20
    ulp = np.spacing(np.abs(ref[tight]).astype(np.float32)).astype(np.float64)
    err = np.abs(got[tight] - ref[tight])
    assert np.all(err <= ulp), f"{label}: worst {np.max(err / ulp):.2f} float32 ulp"
    lost = keep <= 2.0 ** -60
    assert np.array_equal(got[lost], (lc32.astype(np.float64) + np.log(2.0 ** -60)).astype(np.float32)[lost])
    log(f"  {label}: {tight.sum()} rows within 1 float32 ulp, {int(want_flag.sum())} flagged, "
        f"{int(lost.sum())} with no prefix share left")
    return int(want_flag.sum()), int(lost.sum())


@pytest.mark.parametrize("scorer,dtype,hq,hkv,d,w,n", CAUSAL_CASES)
def test_lse_from_causal(gpu_lib, scorer, dtype, hq, hkv, d, w, n):
    """Every corrected window-row statistic against the oracle's, to one
    float32 ulp (both sides correct in float64 and the device rounds once),
    and every row's precision flag."""
    cfg, st, q64, k64 = _causal_inputs(scorer, dtype, hq, hkv, d, w, n, 3)
    log(f"case lse_from_causal {cfg.name} n={n}")
    _check_causal(cfg, st, q64, k64, cfg.name)


@pytest.mark.parametrize("in_place", [False, True])
def test_lse_from_causal_window_dominated(gpu_lib, in_place):
    """Window keys that carry most of the later rows' causal mass: rows below
    the 2^-7 prefix share are flagged, rows where the float32 input leaves no
    share get L - 60 ln 2, the rest match; also written over the input."""
    cfg, st, q64, k64 = _causal_inputs("snapkv", "bf16", 32, 8, 128, 32, 300, 2, window_gain=0.4)
    log(f"case lse_from_causal window-dominated in_place={in_place}")
    flagged, lost = _check_causal(cfg, st, q64, k64, "window-dominated", in_place=in_place)
    assert flagged > 0 and lost > 0


@pytest.mark.parametrize("scorer", ["snapkv", "laprox", "lava"])
def test_lse_from_causal_non_finite_rows(gpu_lib, scorer):
    """Rows whose causal statistic is not finite are passed through with flag
    2; every other row is corrected as usual (one float32 ulp of the oracle)."""
    cfg, st, q64, k64 = _causal_inputs(scorer, "bf16", 32, 8, 128, 32, 300, 2)
    I = q64.shape[0]
    lc32 = np.stack([scoring.window_lse(q64[i], k64[i], causal=True) for i in range(I)]).astype(np.float32)
    bad = np.zeros(lc32.shape, dtype=bool)
    bad[0, 3, 5] = bad[1, 30, 0] = bad[1, 7, 31] = True
    lc32[0, 3, 5], lc32[1, 30, 0], lc32[1, 7, 31] = np.inf, np.nan, -np.inf
    lc = torch.from_numpy(lc32).cuda()
    out = torch.full_like(lc, 7.0)
    flag = torch.full(lc.shape, -1, dtype=torch.int32, device="cuda")
    log(f"case lse_from_causal non-finite rows {scorer}")
    lib.adakv_lse_from_causal(pipeline.make_shape(cfg, I, k64.shape[2]), pipeline.to_device(st["q_win"], "bf16"),
                              pipeline.to_device(st["k"], "bf16"), lc, out, flag)
    torch.cuda.synchronize()
    got, fl = out.cpu().numpy(), flag.cpu().numpy()
    assert np.all(fl[bad] == 2)
    np.testing.assert_array_equal(got[bad], lc32[bad])     # passed through (NaN stays NaN)
    ref, keep = zip(*[scoring.lse_from_causal(np.where(bad[i], 0.0, lc32[i]).astype(np.float64), q64[i], k64[i],
                                              scorer) for i in range(I)])
    ref, keep = np.stack(ref), np.stack(keep)
    ok = ~bad & (keep >= 2.0 ** -20)
    ulp = np.spacing(np.abs(ref[ok]).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got[ok].astype(np.float64) - ref[ok]) <= ulp)
    assert np.all(fl[~bad] == np.where(keep[~bad] < 2.0 ** -7, 1, 0))


@pytest.mark.parametrize("scorer", ["snapkv", "criticalkv", "laprox", "lava"])
def test_causal_single_pass(gpu_lib, scorer):
    """The whole path scored from a prefill's causal statistic: corrected on
    the device, then adakv_score_lse; scores against the oracle's scores from
    the oracle's correction of the same float32 input."""
    if scorer == "snapkv":     # enough instances for the register-K emit pass
        cfg = scaled(configs.LLAMA8B_LAYER, name="causal_e2e_snapkv", reserve=1, decode_steps=1)
        n = 1000
        run_case(cfg, 256, n, cfg.hkv * cfg.w + (cfg.hkv * (n - cfg.w)) // 5, 1, 1, cfg.name, causal_lse=True)
    elif scorer == "criticalkv":
        cfg = scaled(configs.QWEN32B_CK, name="causal_e2e_ck", hidden=256)
        n = 700
        run_case(cfg, 1, n, cfg.hkv * cfg.w + (cfg.hkv * (n - cfg.w)) // 4, 0, 0, cfg.name, causal_lse=True)
    elif scorer == "laprox":
        cfg = scaled(configs.MISTRAL7B_LAPROX, layers=2, hidden=256, name="causal_e2e_laprox")
        n = 600
        run_case(cfg, 2, n, 2 * cfg.w * cfg.hkv + cfg.hkv * (n - cfg.w) // 3, 0, 0, cfg.name, causal_lse=True)
    else:
        cfg = scaled(configs.MISTRAL7B_LAVA, layers=3, name="causal_e2e_lava")
        n = 500
        run_case(cfg, 3, n, 3 * cfg.w * cfg.hkv + cfg.hkv * (n - cfg.w) // 2, 0, 0, cfg.name, causal_lse=True)


def test_budget_extremes(gpu_lib):
    base = scaled(configs.LLAMA8B_LAYER, name="extremes", decode_steps=1, reserve=1)
    n = 700
    run_case(base, 1, n, base.w * base.hkv, 1, 1, "window only")            # P = 0
    run_case(base, 1, n, base.n * 0 + n * base.hkv, 1, 1, "keep all")       # P = hkv * p


def test_global_budget_extremes(gpu_lib):
    cfg = scaled(configs.MISTRAL7B_LAPROX, layers=2, hidden=256, name="global_extremes")
    n = 700
    win = 2 * cfg.w * cfg.hkv
    run_case(cfg, 2, n, win, 0, 0, "model-wide: windows only")                          # B' = 0
    run_case(cfg, 2, n, win + 2 * cfg.hkv * (n - cfg.w), 0, 0, "model-wide: keep all")  # B' = I*hkv*p


def test_global_ties_across_instances(gpu_lib):
    """Two identical layers with constant keys and values: every score of a
    head is the same, and the two layers tie entry for entry, so the
    model-wide selection is decided by the flat-index tie-break alone (ties
    shared out across heads and instances)."""
    cfg = scaled(configs.MISTRAL7B_LAPROX, layers=2, hidden=256, name="global_ties", sinks=0)
    n = 600
    inst = synth.make_instance(cfg, 0, n_override=n)
    kc = np.broadcast_to(inst["k"][:, :1, :], inst["k"].shape).copy()
    vc = np.broadcast_to(inst["v"][:, :1, :], inst["v"].shape).copy()
    q = pipeline.to_device(np.stack([inst["q_win"]] * 2), "bf16")
    k = pipeline.to_device(np.stack([kc] * 2), "bf16")
    v = pipeline.to_device(np.stack([vc] * 2), "bf16")
    w_o = pipeline.to_device(np.stack([inst["w_o"]] * 2), "bf16")
    budget = 2 * cfg.w * cfg.hkv + 3 * (n - cfg.w) + 123
    ev = pipeline.Eviction(cfg, n_inst=2, n=n, budget=budget, reserve=0)
    ev.evict(q, k, v, w_o)
    torch.cuda.synchronize()
    s = ev.score.cpu().numpy()
    assert np.all(s == s[:, :, :1]) and np.array_equal(s[0], s[1])
    b, off, sel = ev.host_selection()
    r = allocation.global_allocate(s.astype(np.float64), budget, cfg.w)
    base = 0
    for i in range(2):
        check_selection(b[i], int(off[i]), sel[i], r["budgets"][i], r["sel"][i], f"ties inst {i}", off_ref=base)
        base += int(r["budgets"][i].sum())


@pytest.mark.parametrize("alpha", [(0, 1), (1, 1), (1, 2), (4, 5)])   # (4, 5): the other reading of alpha = 0.2
def test_safeguard_settings(gpu_lib, alpha):
    cfg = scaled(configs.LLAMA8B_LAYER, alpha=alpha, name=f"alpha{alpha[0]}_{alpha[1]}", decode_steps=0)
    run_case(cfg, 2, 1500, 8 * 100, 0, 0, f"alpha {alpha}")


@pytest.mark.parametrize("alpha", [(1, 5), (0, 1), (1, 1), (4, 5)])
def test_floor_reading(gpu_lib, alpha):
    cfg = scaled(configs.LLAMA8B_LAYER, alpha=alpha, alloc="floor", name=f"floor{alpha[0]}_{alpha[1]}",
                 decode_steps=1, reserve=1)
    run_case(cfg, 3, 1900, 8 * 32 + 8 * 150 + 5, 1, 1, f"floor alpha {alpha}")


def test_floor_reading_ties(gpu_lib):
    """Constant keys: every score of a head is equal, so both stages are
    decided by the index tie-break alone."""
    cfg = scaled(configs.LLAMA8B_LAYER, name="floor_ties", sinks=0, decode_steps=0, alloc="floor", alpha=(1, 2))
    n = 600
    inst = synth.make_instance(cfg, 0, n_override=n)
    kconst = np.broadcast_to(inst["k"][:, :1, :], inst["k"].shape).copy()
    q = pipeline.to_device(inst["q_win"][None], "bf16")
    k = pipeline.to_device(kconst[None], "bf16")
    v = pipeline.to_device(inst["v"][None], "bf16")
    budget = 8 * 32 + 901
    ev = pipeline.Eviction(cfg, n_inst=1, n=n, budget=budget, reserve=0)
    ev.evict(q, k, v)
    torch.cuda.synchronize()
    s = ev.score.cpu().numpy()[0]
    b, off, sel = ev.host_selection()
    r = allocation.ada_floor_allocate(s.astype(np.float64), budget, cfg.w, cfg.alpha)
    check_selection(b[0], int(off[0]), sel[0], r["budgets"], r["sel"], "floor ties")


@pytest.mark.parametrize("n", [2500, 1200])      # the chunked selection path, and one workgroup per instance
@pytest.mark.parametrize("alpha", [(0, 1), (1, 5)])
def test_pyramid_preset_layer_budgets(gpu_lib, alpha, n):
    """Pyramid (alpha = 0: SnapKV's even split inside each layer) and
    Ada-Pyramid (alpha = 1/5) with preset per-layer budgets that fall from the
    shallow layers to the deep ones, two sequences per layer: budgets,
    selections and offsets bit-exact against the oracle's Ada-KV allocation
    run per instance with its own budget, the flat cache exact, decode within
    tolerance.  The pages leave the schedule's hyper-parameters open; any
    caller-given schedule takes this path."""
    cfg = scaled(configs.LLAMA8B_MODEL, layers=4, batch=2, alpha=alpha, name=f"pyramid{alpha[0]}_{alpha[1]}")
    per_layer = [8 * 32 + p * n // 2500 for p in (1900, 1300, 700, 101)]   # decreasing with depth
    inst_budget = [per_layer[i // cfg.batch] for i in range(cfg.instances)]
    run_case(cfg, cfg.instances, n, 0, 2, 2, f"pyramid alpha {alpha}", inst_budget=inst_budget)


@pytest.mark.parametrize("sinks", [4, 0, 700])
def test_streaming_baseline(gpu_lib, sinks):
    cfg = scaled(configs.LLAMA8B_MODEL, layers=2, batch=2, alloc="streaming", stream_sinks=sinks,
                 name=f"streaming{sinks}")
    run_case(cfg, 4, 3000, 8 * 32 + 8 * 200 + 3, 2, 2, f"streaming sinks {sinks}")


@pytest.mark.parametrize("n", [600, 3001])
def test_ties_take_lower_index(gpu_lib, n):
    """Constant keys: every score of a head is identical, so the selection is
    decided by the index tie-break alone (n = 600: the one-workgroup instance
    path; n = 3001: the one-launch head top-k, rows of an odd length)."""
    cfg = scaled(configs.LLAMA8B_LAYER, name="ties", sinks=0, decode_steps=0)
    inst = synth.make_instance(cfg, 0, n_override=n)
    kconst = np.broadcast_to(inst["k"][:, :1, :], inst["k"].shape).copy()
    q = pipeline.to_device(inst["q_win"][None], "bf16")
    k = pipeline.to_device(kconst[None], "bf16")
    v = pipeline.to_device(inst["v"][None], "bf16")
    budget = 8 * 32 + 777
    ev = pipeline.Eviction(cfg, n_inst=1, n=n, budget=budget, reserve=0)
    ev.evict(q, k, v)
    torch.cuda.synchronize()
    s = ev.score.cpu().numpy()[0]
    assert np.all(s == s[:, :1])
    b, off, sel = ev.host_selection()
    r = allocation.ada_allocate(s.astype(np.float64), budget, cfg.w, cfg.alpha)
    check_selection(b[0], int(off[0]), sel[0], r["budgets"], r["sel"], "ties")


@pytest.mark.parametrize("n,frac,I", [(9001, 1.0, 1), (9001, 0.5, 1), (3001, 0.2, 32), (3001, 0.2, 33)])
def test_one_launch_head_topk(gpu_lib, n, frac, I):
    """Every head's top-B_g in one launch per row (calls of at most 256 rows):
    rows of 8969 scores (not a multiple of 4: scalar loads) with all of them
    kept (more than one 8192-index staging window) or half, and 256 against 264
    rows of one shape (either side of the one-launch path), every output
    against the oracle."""
    cfg = scaled(configs.LLAMA8B_LAYER, name=f"rowtopk_{n}_{I}", decode_steps=1, reserve=1)
    p = n - cfg.w
    run_case(cfg, I, n, cfg.w * cfg.hkv + int(frac * cfg.hkv * p), 1, 1, cfg.name)


def test_deterministic_repeat(gpu_lib):
    cfg = configs.LLAMA8B_LAYER
    n = 4096
    insts, st = _stack(cfg, 1, n)
    q, k, v = (pipeline.to_device(st[x], "bf16") for x in ("q_win", "k", "v"))
    outs = []
    for _ in range(2):
        ev = pipeline.Eviction(cfg, n_inst=1, n=n, budget=(20 * 8 * n) // 100, reserve=1)
        ev.evict(q, k, v)
        ev.run_decode(pipeline.to_device(np.ascontiguousarray(st["q_dec"][:, 0]), "bf16"))
        torch.cuda.synchronize()
        ss, sl = ev.seg_start.cpu(), ev.seg_len.cpu()
        used = torch.cat([torch.arange(int(ss[i]), int(ss[i]) + int(sl[i])) for i in range(sl.numel())])
        kf = ev.k_flat.view(torch.int16).cpu()[used]      # rows in use; reserve rows are never written
        vf = ev.v_flat.view(torch.int16).cpu()[used]
        outs.append([t.cpu().clone() for t in (ev.score, ev.budgets, ev.sel, ev.sel_off, ev.seg_start, ev.seg_len,
                                                ev.out)] + [kf, vf])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ full size, bench launch configuration
def _host64(t):
    """Device tensor -> float64 numpy, exactly (bf16 through its bit patterns)."""
    if t.dtype == torch.bfloat16:
        return synth.widen(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    return t.float().cpu().numpy().astype(np.float64)


def _bits(t):
    """Device bf16 tensor -> its uint16 bit patterns on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _pool_map(fn, items, workers=8):
    """Run the oracle over independent items on a few host threads (NumPy
    releases the interpreter lock in its kernels), BLAS limited to one thread
    per worker."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def test_llama_model_full(gpu_lib):
    """The 32-layer x batch-4 workload exactly as the benchmark launches it,
    every one of the 128 instances checked against the oracle: scores, budgets,
    selections and offsets, the flat segments after the 128 appends, and the
    decode output of the last step."""
    cfg = configs.LLAMA8B_MODEL
    log("drawing full Llama-3.1-8B model inputs on the device")
    data = synth.make_batch_torch(cfg, "cuda")
    ev = pipeline.Eviction(cfg)
    ev.evict(data["q_win"], data["k"], data["v"])
    steps = cfg.decode_steps
    for t in range(steps):
        ev.run_decode(data["q_dec"][t], data["k_new"][t], data["v_new"][t])
    torch.cuda.synchronize()
    log("full pass done; copying to the host")
    score = ev.score.cpu().numpy()
    b, off, sel = ev.host_selection()
    ss = ev.seg_start.cpu().numpy()
    sl = ev.seg_len.cpu().numpy()
    out = ev.out.cpu().numpy()
    kf_bits, vf_bits = _bits(ev.k_flat), _bits(ev.v_flat)
    q_bits, k_bits = _bits(data["q_win"]), _bits(data["k"])
    v_bits = _bits(data["v"])
    kn_bits, vn_bits = _bits(data["k_new"]), _bits(data["v_new"])
    qd_last = _host64(data["q_dec"][steps - 1])
    P = cfg.budget - cfg.w * cfg.hkv
    assert int(off[-1]) == cfg.instances * P
    assert np.all(sl == b.reshape(-1) + cfg.w)        # decode leaves seg_len as compaction wrote it
    del data
    torch.cuda.empty_cache()

    def check(i):
        q64 = synth.widen(q_bits[i], "bf16")
        k64 = synth.widen(k_bits[i], "bf16")
        ref, _ = oracle_scores("snapkv", q64, k64, None, None, cfg.pool, 0.0)
        worst = assert_scores_close(score[i], ref, f"model inst {i}")
        r = allocation.ada_allocate(score[i].astype(np.float64), cfg.budget, cfg.w, cfg.alpha)
        check_selection(b[i], int(off[i]), sel[i], r["budgets"], r["sel"], f"model inst {i}", off_ref=i * P)
        # the flat segments: selected rows, window rows, then the appended rows (bit patterns)
        for g in range(cfg.hkv):
            s_ = i * cfg.hkv + g
            st0, ln = int(ss[s_]), int(sl[s_])
            rows = np.concatenate([sel[i][g], np.arange(cfg.p, cfg.n)])
            assert ln == rows.size
            assert np.array_equal(kf_bits[st0:st0 + ln], k_bits[i, g, rows]), f"K segment {s_}"
            assert np.array_equal(vf_bits[st0:st0 + ln], v_bits[i, g, rows]), f"V segment {s_}"
            assert np.array_equal(kf_bits[st0 + ln:st0 + ln + steps], kn_bits[:, i, g]), f"K appends {s_}"
            assert np.array_equal(vf_bits[st0 + ln:st0 + ln + steps], vn_bits[:, i, g]), f"V appends {s_}"
        kh = [synth.widen(kf_bits[int(ss[i * cfg.hkv + g]):int(ss[i * cfg.hkv + g]) + int(sl[i * cfg.hkv + g]) + steps],
                          "bf16") for g in range(cfg.hkv)]
        vh = [synth.widen(vf_bits[int(ss[i * cfg.hkv + g]):int(ss[i * cfg.hkv + g]) + int(sl[i * cfg.hkv + g]) + steps],
                          "bf16") for g in range(cfg.hkv)]
        refo = cache.decode(qd_last[i], kh, vh)
        ma, rl = assert_decode_close(out[i], refo, f"model decode inst {i}")
        if i % 16 == 15:
            log(f"  instances up to {i} checked")
        return worst, ma, rl

    res = _pool_map(check, range(cfg.instances))
    worst = max(x[0] for x in res)
    log(f"  all {cfg.instances} instances: scores worst rel {worst:.2e}; budgets, selections and flat cache "
        f"exact after {steps} appends; decode worst max-abs {max(x[1] for x in res):.2e}, "
        f"rel-L2 {max(x[2] for x in res):.2e}")


def test_lava_full(gpu_lib):
    """The 32-layer Mistral-7B LAVa workload at n = 131072 exactly as the
    benchmark launches it: every layer's scores against the oracle, the layer
    budgets against the oracle's entropy split (a difference allowed only at a
    float64 near-tie of the split, and the selections then checked under the
    device's budgets), every layer's selection bit-exact, and every flat
    segment."""
    cfg = configs.MISTRAL7B_LAVA
    log("drawing full Mistral-7B LAVa inputs on the device")
    data = synth.make_batch_torch(cfg, "cuda")
    ev = pipeline.Eviction(cfg)
    ev.evict(data["q_win"], data["k"], data["v"])
    torch.cuda.synchronize()
    score = ev.score.cpu().numpy()
    b, off, sel = ev.host_selection()
    L, w, hkv = cfg.instances, cfg.w, cfg.hkv
    Bp = cfg.budget - L * w * hkv
    assert int(off[L]) == Bp
    r = allocation.lava_allocate(score.astype(np.float64), cfg.budget, w)
    lb = np.array([off[l + 1] - off[l] for l in range(L)])
    if not check_lava_layer_budgets(lb, r["layer_budgets"], r["entropy"], Bp, "lava full"):
        r = allocation.lava_allocate(score.astype(np.float64), cfg.budget, w, layer_budgets=lb)
    for l in range(L):
        check_selection(b[l], off[l], sel[l], r["budgets"][l], r["sel"][l], f"lava full layer {l}")
    log("  layer budgets and all 32 layers' selections exact")
    kf_bits, vf_bits = _bits(ev.k_flat), _bits(ev.v_flat)
    ss = ev.seg_start.cpu().numpy()
    sl = ev.seg_len.cpu().numpy()
    q_bits = _bits(data["q_win"])
    k_bits = _bits(data["k"])
    v_bits = _bits(data["v"])
    del data, ev
    torch.cuda.empty_cache()

    def check(l):
        q64 = synth.widen(q_bits[l], "bf16")
        k64 = synth.widen(k_bits[l], "bf16")
        v64 = synth.widen(v_bits[l], "bf16")
        ref, _ = oracle_scores("lava", q64, k64, v64, None, cfg.pool, 0.0)
        worst = assert_scores_close(score[l], ref, f"lava full layer {l}")
        for g in range(hkv):
            s_ = l * hkv + g
            st0, ln = int(ss[s_]), int(sl[s_])
            rows = np.concatenate([sel[l][g], np.arange(cfg.p, cfg.n)])
            assert ln == rows.size
            assert np.array_equal(kf_bits[st0:st0 + ln], k_bits[l, g, rows]), f"lava K segment {s_}"
            assert np.array_equal(vf_bits[st0:st0 + ln], v_bits[l, g, rows]), f"lava V segment {s_}"
        if l % 8 == 7:
            log(f"  layers up to {l} checked")
        return worst

    worst = max(_pool_map(check, range(L), workers=6))
    log(f"  all {L} layers: scores worst rel {worst:.2e}; flat segments exact")


def test_criticalkv_full(gpu_lib):
    """The Qwen2.5-32B CriticalKV layer at n = 65536, hidden 5120, as the
    benchmark launches it: the Ada-KV scores in full; the composite on every
    prefix key of every KV head (and, reported apart, on the keys within 1e-4
    relative of each head's stage-2 cut-off: the entries the second stage
    decides on); the two-stage selection bit-exact on the GPU's own fp32
    scores; the flat segments."""
    from oracle import scoring
    cfg = configs.QWEN32B_CK
    log("drawing full Qwen2.5-32B inputs on the device")
    data = synth.make_batch_torch(cfg, "cuda")
    ev = pipeline.Eviction(cfg)
    ev.evict(data["q_win"], data["k"], data["v"], data["w_o"])
    torch.cuda.synchronize()
    score = ev.score.cpu().numpy()[0]
    score2 = ev.score2.cpu().numpy()[0]
    b, off, sel = ev.host_selection()
    q64 = _host64(data["q_win"][0])
    k64 = _host64(data["k"][0])
    v64 = _host64(data["v"][0])
    wo64 = _host64(data["w_o"])                      # [hidden, hq*d], the nn.Linear layout
    kf = pipeline.to_host_f64(ev.k_flat)
    vf = pipeline.to_host_f64(ev.v_flat)
    ss, sl = ev.seg_start.cpu().numpy(), ev.seg_len.cpu().numpy()
    del data, ev
    torch.cuda.empty_cache()
    hq, hkv, p, d, G = cfg.hq, cfg.hkv, cfg.p, cfg.d, cfg.group
    a = scoring.snapkv_head_scores(q64, k64, cfg.pool)
    worst = assert_scores_close(score, scoring.group_mean(a, hkv), "criticalkv full attention score")
    r = allocation.criticalkv_allocate(score.astype(np.float64), score2.astype(np.float64), cfg.budget, cfg.w,
                                       cfg.alpha, cfg.ck)
    check_selection(b[0], int(off[0]), sel[0], r["budgets"], r["sel"], "criticalkv full", off_ref=0)
    wT = np.ascontiguousarray(wo64.T)                # the pages' W^O [hq*d, hidden]

    def comp_of(g, keys):
        """Oracle composite of KV head g at the given prefix keys."""
        nrm = scoring.projected_value_norms(v64[g:g + 1], wT[g * G * d:(g + 1) * G * d], G, keys)
        return ((a[g * G:(g + 1) * G][:, keys] + cfg.eps) * nrm).mean(axis=0)

    worst2 = 0.0
    for g in range(hkv):
        keys = np.arange(p)
        worst2 = max(worst2, assert_scores_close(score2[g], comp_of(g, keys), f"criticalkv composite head {g}"))
        log(f"  composite head {g}: every key within tolerance")
    near_total = 0
    for g in range(hkv):
        b1 = (int(r["budgets"][g]) * cfg.ck[0]) // cfg.ck[1]
        b2 = int(r["budgets"][g]) - b1
        rest = np.setdiff1d(np.arange(p), r["stage1"][g])
        if b2 == 0 or b2 >= rest.size:
            continue
        c_rest = np.sort(score2[g, rest].astype(np.float64))[::-1]
        cut = c_rest[b2 - 1]
        keys = rest[np.abs(score2[g, rest] - cut) <= 1e-4 * cut]
        ref = comp_of(g, keys)
        rel = np.abs(score2[g, keys] - ref) / np.abs(ref)
        assert (rel <= 1e-5).all(), f"criticalkv head {g}: composite near the stage-2 cut-off off by {rel.max():.2e}"
        worst2 = max(worst2, float(rel.max()))
        near_total += keys.size
    log(f"  composite at {near_total} keys near the stage-2 cut-offs within tolerance")
    check_flat(kf, vf, ss, sl, 0, hkv, k64, v64, sel[0], cfg.w, "criticalkv full")
    log(f"  scores worst rel {worst:.2e}, composite worst rel {worst2:.2e}; selection and flat segments exact")


def test_laprox_full_sampled(gpu_lib):
    """The 32-layer Mistral-7B LaProx workload at n = 32768, hidden 4096,
    exactly as the benchmark launches it (one scoring call per layer, one
    model-wide selection): the model-wide selection bit-exact against the
    oracle's run on the GPU's own fp32 scores; every layer's scores at 512
    sampled keys (the full V W^O in float64 would take minutes per layer) and
    every layer's flat segments against the oracle."""
    cfg = configs.MISTRAL7B_LAPROX
    log("drawing full Mistral-7B LaProx inputs on the device")
    data = synth.make_batch_torch(cfg, "cuda")
    ev = pipeline.Eviction(cfg)
    ev.evict(data["q_win"], data["k"], data["v"], data["w_o"])
    torch.cuda.synchronize()
    score = ev.score.cpu().numpy()
    b, off, sel = ev.host_selection()
    L, w, p = cfg.instances, cfg.w, cfg.p
    r = allocation.global_allocate(score.astype(np.float64), cfg.budget, w)
    assert int(off[L]) == r["Bp"]
    base = 0
    for l in range(L):
        check_selection(b[l], int(off[l]), sel[l], r["budgets"][l], r["sel"][l], f"laprox full layer {l}",
                        off_ref=base)
        base += int(r["budgets"][l].sum())
    log(f"  model-wide selection exact; layer budgets {r['layer_budgets'].min()}..{r['layer_budgets'].max()}")
    kf = pipeline.to_host_f64(ev.k_flat)
    vf = pipeline.to_host_f64(ev.v_flat)
    ss = ev.seg_start.cpu().numpy()
    sl = ev.seg_len.cpu().numpy()
    rng = np.random.default_rng(11)
    keys = np.unique(np.concatenate([[0, 1, p - 2, p - 1], rng.choice(p, 508, replace=False)]))
    worst_all = 0.0
    for l in range(L):
        q64 = pipeline.to_host_f64(data["q_win"][l])
        k64 = pipeline.to_host_f64(data["k"][l])
        v64 = pipeline.to_host_f64(data["v"][l])
        wo64 = pipeline.to_host_f64(data["w_o"][l])
        ref = scoring.laprox_scores(q64, k64, v64, wo64.T, keys=keys)
        worst = assert_scores_close(score[l][:, keys], ref, f"laprox full layer {l} (sampled keys)")
        check_flat(kf, vf, ss, sl, l, cfg.hkv, k64, v64, sel[l], w, f"laprox full layer {l}")
        worst_all = max(worst_all, worst)
    log(f"  all {L} layers: scores worst rel {worst_all:.2e} at {keys.size} keys each; flat segments exact")
    del data, ev
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ LAVa online prefill
def _same_step(a, b, l, I, what):
    """Two LavaOnline runs after the same step: budgets, offsets, selections
    and the flat cache identical."""
    ca, cb = a.current(), b.current()
    hkv = a.hkv
    for key, m in (("budgets", I * hkv), ("sel_off", I + 1), ("seg_start", I * hkv + 1), ("seg_len", I * hkv)):
        assert torch.equal(ca[key][:m], cb[key][:m]), f"{what} step {l}: {key} differs between the two routes"
    tot = int(ca["sel_off"][I].item())
    assert torch.equal(ca["sel"][:tot], cb["sel"][:tot]), f"{what} step {l}: sel differs between the two routes"
    rows = int(ca["seg_start"][I * hkv].item())
    for key in ("k_flat", "v_flat"):
        assert torch.equal(ca[key][:rows].view(torch.int16 if ca[key].element_size() == 2 else torch.int32),
                           cb[key][:rows].view(torch.int16 if cb[key].element_size() == 2 else torch.int32)), \
            f"{what} step {l}: {key} differs between the two routes"
    assert torch.equal(a.layer_ent[:I], b.layer_ent[:I]), f"{what} step {l}: cached entropies differ"


def run_online(cfg, n, total, label, twin=True):
    """Every step against the oracle's schedule; with twin, a second run that
    re-selects every layer from its full scores must give identical outputs."""
    log(f"case {label}: {cfg.name} L={cfg.layers} n={n} total={total}")
    L, w, hkv, dt = cfg.layers, cfg.w, cfg.hkv, cfg.dtype
    insts = [synth.make_instance(cfg, l, n_override=n) for l in range(L)]
    on = pipeline.LavaOnline(cfg, n=n, total=total)
    full = pipeline.LavaOnline(cfg, n=n, total=total) if twin else None
    k64 = [_w(x["k"], dt) for x in insts]
    v64 = [_w(x["v"], dt) for x in insts]
    prev_lb = np.zeros(0, dtype=np.int64)
    for l in range(L):
        q = pipeline.to_device(insts[l]["q_win"], dt)
        k = pipeline.to_device(insts[l]["k"], dt)
        v = pipeline.to_device(insts[l]["v"], dt)
        on.step(q, k, v)
        if full is not None:
            full.step(q, k, v, incremental=False)
        torch.cuda.synchronize()
        if full is not None:
            _same_step(on, full, l, l + 1, label)
        del q, k, v                                   # only the flat cache keeps this layer
        score = on.score[:l + 1].cpu().numpy().astype(np.float64)
        if l == 0:
            ref, _ = oracle_scores("lava", _w(insts[0]["q_win"], dt), k64[0], v64[0], None, cfg.pool, 0.0)
            assert_scores_close(score[0], ref, f"{label} layer 0 score")
        # the oracle's schedule over the GPU's own scores of the layers present
        # (step l depends on layers 0..l only; the caps are the device's
        # budgets of the previous step, themselves checked there)
        ref = allocation.lava_online_step(score, total, w, prev_lb)
        b, off, sel = on.host_selection()
        lb = np.array([off[j + 1] - off[j] for j in range(l + 1)])
        if not check_lava_layer_budgets(lb, ref["layer_budgets"], ref["entropy"], ref["Bp"], f"{label} step {l}",
                                        same_sum=False):
            assert (lb <= np.concatenate([prev_lb, [hkv * (n - w)]])).all(), f"{label} step {l}: a budget grew"
            rb, rsel = allocation.layer_top_select(score, lb)
            ref = {"budgets": rb, "sel": rsel}
        prev_lb = lb
        cur = on.current()
        kf = pipeline.to_host_f64(cur["k_flat"])
        vf = pipeline.to_host_f64(cur["v_flat"])
        ss = cur["seg_start"].cpu().numpy()
        sl = cur["seg_len"].cpu().numpy()
        for j in range(l + 1):
            check_selection(b[j], int(off[j]), sel[j], ref["budgets"][j], ref["sel"][j], f"{label} step {l} layer {j}")
            check_flat(kf, vf, ss, sl, j, hkv, k64[j], v64[j], sel[j], w, f"{label} step {l} layer {j}")
        log(f"  step {l}: layer budgets {lb.tolist()}; selections and flat cache exact")


def test_lava_online_prefill(gpu_lib):
    cfg = scaled(configs.MISTRAL7B_LAVA, layers=4, name="lava_online_L4")
    n = 3000
    run_online(cfg, n, 4 * 8 * 32 + 4 * 8 * 120, "lava online L4 n3000")


def test_lava_online_prefill_caps(gpu_lib):
    """A total larger than one layer's prefix: the first steps keep whole
    layers (the cap) and the budgets then fall step by step."""
    cfg = scaled(configs.MISTRAL7B_LAVA, layers=3, name="lava_online_caps")
    n = 700
    run_online(cfg, n, 3 * 8 * 32 + 3 * 8 * (n - 32) // 2, "lava online caps L3 n700")


def test_lava_online_route_switch(gpu_lib):
    """Both bounds of the incremental route: at step 1 the older layer's
    previous entries exceed 32768 in all (layer 0 keeps 32,944 after step 0),
    at steps 2 and 3 they fit but average more than 8192 per older layer, so
    every layer is re-selected from its full scores; from step 4 on they are
    re-selected from their previous entries."""
    cfg = scaled(configs.MISTRAL7B_LAVA, layers=6, name="lava_online_switch")
    n = 5032
    total = 33200            # B'(l) = 33200 - (l + 1) * 256 (hkv = 8, w = 32)
    bprev = lambda I: total - (I - 1) * 32 * 8          # noqa: E731
    assert bprev(2) > 32768
    assert all(bprev(I) > 8192 * (I - 1) for I in (3, 4))
    assert all(bprev(I) <= min(32768, 8192 * (I - 1)) for I in (5, 6))
    run_online(cfg, n, total, "lava online route switch L6 n5032")


def _online_alloc_direct(score_np, total, w, incremental):
    """Every step of the online allocation on given scores [L, hkv, p],
    through the C ABI alone (no scorer): per step budgets, sel_off, sel."""
    L, hkv, p = score_np.shape
    dev = "cuda"
    score = torch.from_numpy(score_np.astype(np.float32)).to(dev)
    lava = lib.AdakvAlloc(mode=lib.ADAKV_ALLOC_LAVA_LAYERS, alpha_num=0, alpha_den=1, ck_num=0, ck_den=1, sinks=0,
                          budget=L * w * hkv)
    shape = lambda I: lib.AdakvShape(n_inst=I, hq=hkv, hkv=hkv, d=128, n=p + w, w=w, pool=1,  # noqa: E731
                                     dtype=lib.ADAKV_BF16, scorer=lib.ADAKV_SCORE_LAVA, hidden=0, eps=0.0,
                                     reserved0=0)
    ws = torch.empty(lib.adakv_workspace_bytes(shape(L), lava, 0), dtype=torch.uint8, device=dev)
    ent = torch.zeros(L, dtype=torch.float64, device=dev)
    cap = max(total - w * hkv, 4)
    bufs = [{"budgets": torch.empty(L * hkv, dtype=torch.int32, device=dev),
             "sel": torch.empty(cap, dtype=torch.int32, device=dev),
             "sel_off": torch.empty(L + 1, dtype=torch.int64, device=dev)} for _ in range(2)]
    out = []
    for l in range(L):
        cur, prev = bufs[l % 2], bufs[(l + 1) % 2]
        inc = incremental and l > 0
        lib.adakv_lava_online_allocate(shape(l + 1), total, score[:l + 1], prev["sel_off"] if l else None,
                                       prev["budgets"] if inc else None, prev["sel"] if inc else None, ent,
                                       cur["budgets"], cur["sel"], cur["sel_off"], ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 0, "scores flagged as breaking the precondition"
        off = cur["sel_off"][:l + 2].cpu().numpy()
        out.append((cur["budgets"][:(l + 1) * hkv].cpu().numpy().reshape(l + 1, hkv), off,
                    cur["sel"][:int(off[-1])].cpu().numpy()))
    return out


@pytest.mark.parametrize("case", ["ties", "dominant_layer"])
def test_lava_online_allocate_given_scores(gpu_lib, case):
    """The online allocation alone on crafted scores, every step against the
    oracle and the two routes against each other: scores on a grid of 17
    values (ties across every threshold, zeros), and a layer whose mass sits
    on a few entries (low entropy: its budget falls to a handful)."""
    rng = np.random.default_rng(2024 if case == "ties" else 77)
    L, hkv, p, w = 6, 4, 1000, 32
    s = rng.integers(0, 17, size=(L, hkv, p)).astype(np.float64) / 16.0
    if case == "dominant_layer":
        s = rng.random((L, hkv, p))
        s[2] = 1e-6
        s[2, 1, 10:13] = 1.0
    s = s.astype(np.float32).astype(np.float64)
    total = L * w * hkv + 1500
    got_inc = _online_alloc_direct(s, total, w, True)
    got_full = _online_alloc_direct(s, total, w, False)
    prev_lb = np.zeros(0, dtype=np.int64)
    for l in range(L):
        (b, off, sel), (bf, offf, self_) = got_inc[l], got_full[l]
        assert np.array_equal(b, bf) and np.array_equal(off, offf) and np.array_equal(sel, self_), \
            f"{case} step {l}: the two routes differ"
        ref = allocation.lava_online_step(s[:l + 1], total, w, prev_lb)
        lb = np.diff(off)
        if not check_lava_layer_budgets(lb, ref["layer_budgets"], ref["entropy"], ref["Bp"], f"{case} step {l}",
                                        same_sum=False):
            rb, rsel = allocation.layer_top_select(s[:l + 1], lb)
            ref = {"budgets": rb, "sel": rsel}
        for j in range(l + 1):
            pos, heads = int(off[j]), []
            for g in range(hkv):
                heads.append(sel[pos:pos + int(b[j, g])])
                pos += int(b[j, g])
            check_selection(b[j], int(off[j]), heads, ref["budgets"][j], ref["sel"][j], f"{case} step {l} layer {j}")
        prev_lb = lb
        log(f"  {case} step {l}: layer budgets {lb.tolist()}; both routes and the oracle agree")


# ------------------------------------------------------------------ limits of the supported shapes
def test_widest_window_and_group(gpu_lib):
    """The largest window (64 rows: four N-blocks) and group (G = 8) the
    scorer builds, at bf16 d = 128 with 7-wide pooling, ragged prefix."""
    cfg = scaled(configs.LLAMA8B_LAYER, hq=64, hkv=8, w=64, name="max_window_group", decode_steps=1, reserve=1)
    n = 1100
    run_case(cfg, 2, n, (25 * 8 * n) // 100, 1, 1, "w64 G8 pool7")


@pytest.mark.parametrize("scorer", ["snapkv", "lava", "criticalkv", "laprox"])
def test_one_token_prefix(gpu_lib, scorer):
    """n = w + 1: a single evictable token per head (p = 1), and p = 5."""
    base = {"snapkv": configs.LLAMA8B_LAYER, "lava": scaled(configs.MISTRAL7B_LAVA, layers=2),
            "criticalkv": scaled(configs.QWEN32B_CK, hidden=128),
            "laprox": scaled(configs.MISTRAL7B_LAPROX, layers=2, hidden=128)}[scorer]
    cfg = scaled(base, name=f"tiny_prefix_{scorer}", decode_steps=0, reserve=0)
    I = 2 if scorer in ("lava", "laprox") else 1
    for p in (1, 5):
        n = cfg.w + p
        win = I * cfg.w * cfg.hkv
        budget = (win + I * cfg.hkv * p // 2) if scorer in ("lava", "laprox") else cfg.w * cfg.hkv + cfg.hkv * p // 2
        run_case(cfg, I, n, budget, 0, 0, f"{scorer} p={p}")


def test_many_kv_heads(gpu_lib):
    """256 KV heads (the most the ABI takes), MHA, fp32 d = 64."""
    cfg = scaled(configs.LLAMA8B_LAYER, hq=256, hkv=256, d=64, dtype="f32", w=16, pool=3, name="hkv256",
                 decode_steps=1, reserve=1)
    n = 300
    run_case(cfg, 1, n, 256 * 16 + 256 * 50 + 7, 1, 1, "hkv 256")


# ------------------------------------------------------------------ calling contract
def _eviction_outputs(ev):
    return [t.clone() for t in (ev.score, ev.budgets, ev.sel, ev.sel_off, ev.seg_start, ev.seg_len)]


def test_concurrent_streams_match_sequential(gpu_lib):
    """Calls are stateless: two evictions with their own workspaces on two
    streams at once give the same bytes as the same calls one after the other."""
    cfg = scaled(configs.LLAMA8B_MODEL, layers=1, batch=2, name="streams", decode_steps=0)
    n = 3000
    inputs = []
    for seed in (0, 1):
        insts = [synth.make_instance(cfg, 2 * seed + i, n_override=n) for i in range(2)]
        inputs.append({k: pipeline.to_device(np.stack([x[k] for x in insts]), "bf16") for k in ("q_win", "k", "v")})
    evs = [pipeline.Eviction(cfg, n_inst=2, n=n, budget=8 * 300, reserve=0) for _ in range(2)]
    ref = []
    for ev, x in zip(evs, inputs):
        ev.evict(x["q_win"], x["k"], x["v"])
        torch.cuda.synchronize()
        ref.append(_eviction_outputs(ev))
        for t in (ev.score, ev.sel, ev.budgets):
            t.zero_()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for ev, x, s in zip(evs, inputs, streams):
            with torch.cuda.stream(s):
                ev.evict(x["q_win"], x["k"], x["v"])
        torch.cuda.synchronize()
        for ev, r in zip(evs, ref):
            for a, b in zip(_eviction_outputs(ev), r):
                assert torch.equal(a, b), f"concurrent run {rep} differs"
    log("  two streams: every output identical to the sequential run, three times")


def test_graph_replay_matches_eager(gpu_lib):
    """The eviction calls launch on the caller's stream, need no host
    synchronisation and issue no memset, so they can be captured: every replay
    of the captured graph, with eager work between replays, matches the eager
    result."""
    cfg = scaled(configs.LLAMA8B_LAYER, name="graph", decode_steps=1, reserve=1)
    n = 2500
    inst = synth.make_instance(cfg, 0, n_override=n)
    q, k, v = (pipeline.to_device(inst[x][None], "bf16") for x in ("q_win", "k", "v"))
    qd = pipeline.to_device(inst["q_dec"][0][None], "bf16")
    ev = pipeline.Eviction(cfg, n_inst=1, n=n, budget=8 * 400, reserve=1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ev.evict(q, k, v)
        ev.run_decode(qd)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = _eviction_outputs(ev) + [ev.out.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ev.evict(q, k, v)
        ev.run_decode(qd)
    for rep in range(4):
        for t in (ev.score, ev.sel, ev.budgets, ev.out):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(_eviction_outputs(ev) + [ev.out], ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager run"
    log("  graph replays: four replays identical to the eager run")


@pytest.mark.parametrize("kind", ["ada", "floor", "global", "lava", "criticalkv"])
def test_score_precondition_flag(gpu_lib, kind):
    """The precondition word at the start of the allocation workspace: clear
    for valid scores (-0.0 included), set by a negative, NaN or infinite score
    in the first or the last chunk of the call, and the selection stays inside
    its buffers either way (budgets sum to the prefix budget, every index in
    [0, p))."""
    n = 700
    if kind == "ada":
        cfg, I, budget = scaled(configs.LLAMA8B_LAYER, name="flag_ada", decode_steps=0), 1, 8 * 32 + 8 * 100
    elif kind == "floor":
        cfg, I, budget = (scaled(configs.LLAMA8B_LAYER, name="flag_floor", alloc="floor", alpha=(1, 2),
                                 decode_steps=0), 1, 8 * 32 + 8 * 100)
    elif kind == "global":
        cfg, I, budget = scaled(configs.MISTRAL7B_LAPROX, layers=2, hidden=256, name="flag_global"), 2, 2 * 8 * 32 + 900
    elif kind == "lava":
        cfg, I, budget = scaled(configs.MISTRAL7B_LAVA, layers=3, name="flag_lava"), 3, 3 * 8 * 32 + 1500
    else:
        cfg, I, budget = scaled(configs.QWEN32B_CK, hidden=256, name="flag_ck", decode_steps=0), 1, 8 * 32 + 8 * 100
    log(f"case precondition flag: {kind} I={I} n={n} budget={budget}")
    insts, st = _stack(cfg, I, n)
    dt = cfg.dtype
    q, k, v = (pipeline.to_device(st[x], dt) for x in ("q_win", "k", "v"))
    w_o = None
    if kind == "criticalkv":
        w_o = pipeline.to_device(insts[0]["w_o"], dt)
    elif kind == "global":
        w_o = pipeline.to_device(np.stack([x["w_o"] for x in insts]), dt)
    ev = pipeline.Eviction(cfg, n_inst=I, n=n, budget=budget, reserve=0)
    ev.run_score(q, k, v if cfg.scorer != "snapkv" else None, w_o)
    ev.run_allocate()
    assert not ev.scores_invalid()
    p = n - cfg.w

    def in_bounds():
        b, off, sel = ev.host_selection()
        assert (b >= 0).all() and int(b.sum()) == ev.n_sel
        for heads in sel:
            for idx in heads:
                assert idx.size == 0 or (idx.min() >= 0 and idx.max() < p)

    targets = [ev.score] + ([ev.score2] if kind == "criticalkv" else [])
    for t in targets:
        good = t.clone()
        for pos in [(0, 1, 17), (I - 1, cfg.hkv - 1, p - 1)]:
            for val, bad in [(-1.0, True), (float("nan"), True), (float("inf"), True), (-float("inf"), True),
                             (-0.0, False), (0.0, False)]:
                t.copy_(good)
                t[pos] = val
                ev.run_allocate()
                assert ev.scores_invalid() == bad, (kind, pos, val)
                in_bounds()
        t.copy_(good)
    log(f"  {kind}: flag clear on valid scores, set on -1, NaN, +-inf; selection in bounds")


def test_decode_reserve_larger_than_compacted(gpu_lib):
    """The documented behaviour when decode is given a larger reserve than
    compaction used: an append that does not fit its segment is dropped (no
    row stored, none read past the segment), the call succeeds, and the output
    equals the attention over the rows already there (the same call without
    an append)."""
    from adaptive_head_budget_amd import lib
    cfg = scaled(configs.LLAMA8B_LAYER, name="reserve_mismatch", decode_steps=2, reserve=1)
    n = 2000
    insts, st = _stack(cfg, 1, n)
    q, k, v = (pipeline.to_device(st[x], "bf16") for x in ("q_win", "k", "v"))
    ev = pipeline.Eviction(cfg, n=n, budget=cfg.hkv * cfg.w + (cfg.hkv * (n - cfg.w)) // 5, reserve=1)
    ev.evict(q, k, v)
    qd = [pipeline.to_device(np.ascontiguousarray(st["q_dec"][:, t]), "bf16") for t in range(2)]
    kn = [pipeline.to_device(np.ascontiguousarray(st["k_new"][:, t]), "bf16") for t in range(2)]
    vn = [pipeline.to_device(np.ascontiguousarray(st["v_new"][:, t]), "bf16") for t in range(2)]
    # step 0 fills the one reserved row of every segment
    lib.adakv_decode_attn(ev.shape, ev.alloc, qd[0], kn[0], vn[0], ev.k_flat, ev.v_flat, ev.seg_start, ev.seg_len,
                          1, 0, ev.out, ev.ws)
    torch.cuda.synchronize()
    k_before, v_before = ev.k_flat.clone(), ev.v_flat.clone()
    # step 1 under a reserve of 3: passes the host check, does not fit on the device
    ws3 = torch.empty(lib.adakv_workspace_bytes(ev.shape, ev.alloc, 3), dtype=torch.uint8, device="cuda")
    out_app = torch.empty_like(ev.out)
    lib.adakv_decode_attn(ev.shape, ev.alloc, qd[1], kn[1], vn[1], ev.k_flat, ev.v_flat, ev.seg_start, ev.seg_len,
                          3, 1, out_app, ws3)
    torch.cuda.synchronize()
    assert torch.equal(ev.k_flat, k_before) and torch.equal(ev.v_flat, v_before), "a dropped append wrote rows"
    out_none = torch.empty_like(ev.out)
    lib.adakv_decode_attn(ev.shape, ev.alloc, qd[1], None, None, ev.k_flat, ev.v_flat, ev.seg_start, ev.seg_len,
                          1, 1, out_none, ws3)
    torch.cuda.synchronize()
    assert torch.isfinite(out_app).all()
    # the same rows attended (the two calls may split the rows differently, so
    # the sums can differ in rounding only)
    diff = (out_app - out_none).abs().max().item()
    assert diff <= 1e-5, f"a dropped append changed the output (max-abs {diff:.2e})"
    log("  reserve larger than compacted: the append is dropped, cache untouched, output = no-append output")


# ------------------------------------------------------------------ compaction against budgets that disagree with the offsets
def _rows_bf16(nrows, d, first_value):
    """Rows whose every element is one small integer (exact in bf16): row r holds first_value + r."""
    vals = torch.arange(first_value, first_value + nrows, dtype=torch.float32, device="cuda")
    return vals[:, None].expand(nrows, d).contiguous().to(torch.bfloat16)


def test_compact_budgets_past_offsets(gpu_lib):
    """adakv_compact given budgets that sum past the instance's span of sel
    (never an allocate output): the rows whose sel position lies past the span
    are left unwritten and nothing past the flat buffer's rows is touched.
    Every buffer is large enough that even unchecked reads would stay inside."""
    hkv, w, n, d = 2, 4, 40, 128
    p = n - w
    shape = lib.AdakvShape(n_inst=1, hq=hkv, hkv=hkv, d=d, n=n, w=w, pool=1, dtype=lib.ADAKV_BF16,
                           scorer=lib.ADAKV_SCORE_SNAPKV, hidden=0, eps=0.0, reserved0=0)
    alloc = lib.AdakvAlloc(mode=lib.ADAKV_ALLOC_ADA, alpha_num=1, alpha_den=5, ck_num=0, ck_den=1, sinks=0,
                           budget=8 + w * hkv, inst_budget=None)          # 8 selected rows, 16 retained
    k = _rows_bf16(hkv * n, d, 1).reshape(1, hkv, n, d)
    v = _rows_bf16(hkv * n, d, 101).reshape(1, hkv, n, d)       # all values below 256: exact in bf16
    budgets = torch.tensor([6, 6], dtype=torch.int32, device="cuda")        # 12 > the span of 8
    sel_off = torch.tensor([0, 8], dtype=torch.int64, device="cuda")
    sel = torch.tensor([1, 3, 5, 7, 9, 11, 2, 4, 6, 8, 10, 12] + [0] * 52, dtype=torch.int32, device="cuda")
    sentinel = -7.0
    kf = torch.full((64, d), sentinel, dtype=torch.bfloat16, device="cuda")
    vf = torch.full((64, d), sentinel, dtype=torch.bfloat16, device="cuda")
    seg_start = torch.empty(hkv + 1, dtype=torch.int64, device="cuda")
    seg_len = torch.empty(hkv, dtype=torch.int32, device="cuda")
    lib.adakv_compact(shape, alloc, k, v, budgets, sel, sel_off, 0, kf, vf, seg_start, seg_len)
    torch.cuda.synchronize()
    assert seg_start.tolist() == [0, 10, 20] and seg_len.tolist() == [10, 10]
    kv0 = kf[:, 0].float().cpu().numpy()
    tok_h0 = [1, 3, 5, 7, 9, 11, p, p + 1, p + 2, p + 3]
    want = [1 + t for t in tok_h0] + [1 + n + 2, 1 + n + 4] + [sentinel] * (64 - 12)
    assert kv0.tolist() == [float(x) for x in want], kv0[:20]
    assert (vf[:, 0].float().cpu().numpy()[:12] == np.array(want[:12]) + 100).all()
    log("  budgets past the offsets: rows past the span of sel unwritten, nothing past the flat buffer")


def test_online_compact_budgets_past_offsets(gpu_lib):
    """adakv_lava_online_compact given a layer whose budgets sum past its span
    of sel and a previous segment start past the previous cache's rows (never
    outputs of the library): those rows are left unwritten, every other row
    is the right one.  The previous cache has 64 rows, so even unchecked reads
    would stay inside it; max_rows is 24."""
    hkv, w, n, d = 2, 2, 20, 128
    p = n - w
    shape = lib.AdakvShape(n_inst=2, hq=hkv, hkv=hkv, d=d, n=n, w=w, pool=1, dtype=lib.ADAKV_BF16,
                           scorer=lib.ADAKV_SCORE_LAVA, hidden=0, eps=0.0, reserved0=0)
    dev = "cuda"
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=dev)   # noqa: E731
    i64 = lambda x: torch.tensor(x, dtype=torch.int64, device=dev)   # noqa: E731
    # every value below 256, so exact in bf16
    k_old, v_old = _rows_bf16(64, d, 1), _rows_bf16(64, d, 65)
    k_new = _rows_bf16(hkv * n, d, 129).reshape(hkv, n, d)
    v_new = _rows_bf16(hkv * n, d, 169).reshape(hkv, n, d)
    sel_old, sel_off_old = i32([1, 5, 9, 2, 4, 6] + [0] * 10), i64([0, 6])
    seg_start_old = i64([0, 5, 30])        # head 1's true end is 10
    budgets = i32([2, 3, 3, 3])             # layer 0 sums to 5 over a span of 4
    sel_off = i64([0, 4, 10])
    sel = i32([1, 9, 4, 6, 0, 3, 7, 1, 2, 8] + [0] * 6)
    sentinel = -7.0
    kf = torch.full((24, d), sentinel, dtype=torch.bfloat16, device=dev)
    vf = torch.full((24, d), sentinel, dtype=torch.bfloat16, device=dev)
    seg_start = torch.empty(2 * hkv + 1, dtype=torch.int64, device=dev)
    seg_len = torch.empty(2 * hkv, dtype=torch.int32, device=dev)
    lib.adakv_lava_online_compact(shape, k_new, v_new, k_old, v_old, seg_start_old, sel_old, sel_off_old, budgets,
                                  sel, sel_off, 24, kf, vf, seg_start, seg_len)
    torch.cuda.synchronize()
    assert seg_start.tolist() == [0, 4, 9, 14, 19]
    old_row = lambda r: 1 + r                        # noqa: E731
    new_row = lambda g, t: 129 + g * n + t           # noqa: E731
    want = ([old_row(r) for r in (0, 2, 3, 4)] + [old_row(6), old_row(7)] + [sentinel] * 3 +
            [new_row(0, t) for t in (0, 3, 7, p, p + 1)] + [new_row(1, t) for t in (1, 2, 8, p, p + 1)] +
            [sentinel] * 5)
    got = kf[:, 0].float().cpu().numpy()
    assert got.tolist() == [float(x) for x in want], got
    gv = vf[:, 0].float().cpu().numpy()
    for r, x in enumerate(want):
        if x != sentinel:
            assert gv[r] == x + (64 if x < 129 else 40), (r, gv[r], x)
    log("  online compact: a layer's budgets past its span and a previous segment past the previous cache skipped")


# ------------------------------------------------------------------ LAVa selection on given scores: head counts and ragged rows
def _lava_scores(rng, L, hkv, p, grid):
    """Scores on a grid of `grid` + 1 values in [0, 1] (ties across every
    threshold, zeros), one layer with its mass on a few entries."""
    s = rng.integers(0, grid + 1, size=(L, hkv, p)).astype(np.float64) / grid
    s[L // 2] = 1e-6
    s[L // 2, 0, 1:4] = 1.0
    return s.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("L,hkv,p", [(40, 1, 301), (5, 3, 1003), (3, 16, 257)])
def test_lava_allocate_given_scores(gpu_lib, L, hkv, p):
    """The offline LAVa allocation through the C ABI alone (no scorer) on
    crafted scores, against the oracle: one KV head, an odd head count and
    row length (scalar score loads), many heads per layer."""
    rng = np.random.default_rng(L * 1000 + hkv * 10 + p)
    w = 32
    s = _lava_scores(rng, L, hkv, p, 16)
    total = L * w * hkv + min(hkv * p, (L * hkv * p) // 7)
    shape = lib.AdakvShape(n_inst=L, hq=hkv, hkv=hkv, d=128, n=p + w, w=w, pool=1, dtype=lib.ADAKV_BF16,
                           scorer=lib.ADAKV_SCORE_LAVA, hidden=0, eps=0.0, reserved0=0)
    alloc = lib.AdakvAlloc(mode=lib.ADAKV_ALLOC_LAVA_LAYERS, alpha_num=0, alpha_den=1, ck_num=0, ck_den=1, sinks=0,
                           budget=total)
    score = torch.from_numpy(s.astype(np.float32)).cuda()
    ws = torch.empty(lib.adakv_workspace_bytes(shape, alloc, 0), dtype=torch.uint8, device="cuda")
    Bp = total - L * w * hkv
    budgets = torch.empty(L * hkv, dtype=torch.int32, device="cuda")
    sel = torch.empty(max(Bp, 4), dtype=torch.int32, device="cuda")
    sel_off = torch.empty(L + 1, dtype=torch.int64, device="cuda")
    lib.adakv_allocate(shape, alloc, score, None, budgets, sel, sel_off, ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0
    b = budgets.cpu().numpy().reshape(L, hkv)
    off = sel_off.cpu().numpy()
    hs = sel[:Bp].cpu().numpy()
    ref = allocation.lava_allocate(s, total, w)
    lb = np.diff(off)
    if not check_lava_layer_budgets(lb, ref["layer_budgets"], ref["entropy"], Bp, f"L{L} hkv{hkv} p{p}"):
        ref = allocation.lava_allocate(s, total, w, layer_budgets=lb)
    for l in range(L):
        pos, heads = int(off[l]), []
        for g in range(hkv):
            heads.append(hs[pos:pos + int(b[l, g])])
            pos += int(b[l, g])
        check_selection(b[l], int(off[l]), heads, ref["budgets"][l], ref["sel"][l], f"L{L} hkv{hkv} p{p} layer {l}")
    log(f"  LAVa L={L} hkv={hkv} p={p}: layer budgets {lb.tolist()[:8]}...; selections exact")


@pytest.mark.parametrize("L,hkv,p", [(40, 1, 301), (6, 3, 1003)])
def test_lava_online_allocate_head_counts(gpu_lib, L, hkv, p):
    """The online allocation on crafted scores with one KV head over 40 layers
    (small older sets, a low-entropy layer) and with three KV heads on odd
    rows: both routes identical at every step and equal to the oracle."""
    rng = np.random.default_rng(L * 7 + hkv + p)
    w = 32
    s = _lava_scores(rng, L, hkv, p, 16)
    total = L * w * hkv + min(hkv * p, 1500)
    got_inc = _online_alloc_direct(s, total, w, True)
    got_full = _online_alloc_direct(s, total, w, False)
    prev_lb = np.zeros(0, dtype=np.int64)
    for l in range(L):
        (b, off, sel), (bf, offf, self_) = got_inc[l], got_full[l]
        assert np.array_equal(b, bf) and np.array_equal(off, offf) and np.array_equal(sel, self_), \
            f"step {l}: the two routes differ"
        ref = allocation.lava_online_step(s[:l + 1], total, w, prev_lb)
        lb = np.diff(off)
        if not check_lava_layer_budgets(lb, ref["layer_budgets"], ref["entropy"], ref["Bp"], f"step {l}",
                                        same_sum=False):
            rb, rsel = allocation.layer_top_select(s[:l + 1], lb)
            ref = {"budgets": rb, "sel": rsel}
        for j in range(l + 1):
            pos, heads = int(off[j]), []
            for g in range(hkv):
                heads.append(sel[pos:pos + int(b[j, g])])
                pos += int(b[j, g])
            check_selection(b[j], int(off[j]), heads, ref["budgets"][j], ref["sel"][j], f"step {l} layer {j}")
        prev_lb = lb
    log(f"  online L={L} hkv={hkv} p={p}: {L} steps, both routes and the oracle agree")


@pytest.mark.parametrize("I,hkv,p,frac,alpha", [(4, 2, 3000, 0.3, (1, 5)), (3, 8, 5000, 0.2, (1, 5)),
                                                (2, 3, 20001, 0.1, (4, 5)), (1, 16, 40000, 0.05, (1, 5))])
def test_ada_allocate_given_scores(gpu_lib, I, hkv, p, frac, alpha):
    """The Ada-KV allocation through the C ABI alone on scores from a grid of
    17 values (ties at the layer threshold shared across heads in head order,
    ties inside each head), on each route: one workgroup per instance (4x2x3000),
    the one-launch head top-k (8x5000, 3x20001 with odd rows), and rows longer
    than 32768 on the chunked per-row passes (16x40000)."""
    rng = np.random.default_rng(I * 100003 + hkv * 101 + p)
    w = 32
    s = (rng.integers(0, 17, size=(I, hkv, p)).astype(np.float64) / 16.0).astype(np.float32)
    s[:, 0] *= np.float32(0.25)             # one sparse head per instance (the safeguard matters)
    P = int(frac * hkv * p)
    budget = w * hkv + P
    shape = lib.AdakvShape(n_inst=I, hq=hkv, hkv=hkv, d=128, n=p + w, w=w, pool=1, dtype=lib.ADAKV_BF16,
                           scorer=lib.ADAKV_SCORE_SNAPKV, hidden=0, eps=0.0, reserved0=0)
    alloc = lib.AdakvAlloc(mode=lib.ADAKV_ALLOC_ADA, alpha_num=alpha[0], alpha_den=alpha[1], ck_num=0, ck_den=1,
                           sinks=0, budget=budget)
    score = torch.from_numpy(s).cuda()
    ws = torch.empty(lib.adakv_workspace_bytes(shape, alloc, 0), dtype=torch.uint8, device="cuda")
    budgets = torch.empty(I * hkv, dtype=torch.int32, device="cuda")
    sel = torch.empty(I * P, dtype=torch.int32, device="cuda")
    sel_off = torch.empty(I + 1, dtype=torch.int64, device="cuda")
    lib.adakv_allocate(shape, alloc, score, None, budgets, sel, sel_off, ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0
    b = budgets.cpu().numpy().reshape(I, hkv)
    off = sel_off.cpu().numpy()
    hs = sel.cpu().numpy()
    assert off.tolist() == [i * P for i in range(I + 1)]
    for i in range(I):
        r = allocation.ada_allocate(s[i].astype(np.float64), budget, w, alpha)
        pos, heads = int(off[i]), []
        for g in range(hkv):
            heads.append(hs[pos:pos + int(b[i, g])])
            pos += int(b[i, g])
        check_selection(b[i], int(off[i]), heads, r["budgets"], r["sel"], f"ada {I}x{hkv}x{p} instance {i}")
    log(f"  Ada-KV {I}x{hkv}x{p} alpha {alpha}: budgets {b[0].tolist()[:8]}; selections exact")
