"""Cost model and policy search ("FlexGen 完全拆解", sections "用线性规划搜索
卸载策略", "从硬件画像得到每层时间", "为什么固定批量后能变成线性规划").

The oracle (oracle.cost) is pinned to figures the pages print; the product
(throughput_oriented_offloaded_amd.policy: the same model assembled as a
linear program) is held to the oracle: equal path times and peak memory for
arbitrary placements, and LP solutions that are feasible under the oracle's
own test, score what the LP claims, and are beaten by no grid placement and
no random feasible placement (the objective is convex in the shares)."""
import numpy as np
import pytest

from oracle import cost as oc

GIB = 2.0 ** 30
OPT175 = dict(l=96, h1=12288, h2=49152)


def _hw(**kw):
    base = dict(bw_c2g=12e9, bw_g2c=12e9, bw_d2c=2e9, bw_c2d=1e9, gemm_flops=50e12,
                prefill_flops=60e12, attn_bw=250e9, hbm_bw=300e9, cap_g=16e9, cap_c=208e9,
                cap_d=1.5e12)
    base.update(kw)
    return oc.Hardware(**base)


# ------------------------------------------------------------ oracle pins
def _pin_weights():
    """[P2] "FlexGen 统一调度权重、激活与 KV Cache": OPT-175B fp16 weights are
    about 325 GB (the figure is in binary units: 350e9 parameter bytes less
    the embeddings)."""
    m = oc.Model(s=512, n=32, **OPT175)
    total = m.l * oc.layer_weight_bytes(m)
    assert abs(total / GIB - 325) / 325 < 0.005
    return total


def _pin_kv_peak():
    """Same passage: at b = 512, s = 512, n = 32 the KV cache peaks near
    1.2 TB, 3.8 times the weights."""
    m = oc.Model(s=512, n=32, **OPT175)
    kv = m.l * oc.cache_bytes(m, 512, m.s + m.n)
    assert abs(kv / 2.0 ** 40 - 1.2) / 1.2 < 0.01
    assert abs(kv / _pin_weights() - 3.8) / 3.8 < 0.01


def test_pages_weight_bytes():
    _pin_weights()


def test_pages_kv_peak():
    _pin_kv_peak()


def test_pages_ssd_weight_read():
    """[P2] "SSD 不是更慢的显存": reading all 325 GB of fp16 weights from a
    2 GB/s SSD takes about 162.5 s per decode step: l disk -> CPU weight terms
    at the disk's rate."""
    m = oc.Model(s=512, n=32, **OPT175)
    hw = _hw(bw_d2c=2 * GIB)
    p = dict(wg=0, wc=0, wd=1, hg=1, hc=0, hd=0, cg=1, cc=0, cd=0)
    t = m.l * oc.path_times(m, hw, 144, p, "gen")["d2c"]
    assert abs(t - 162.5) / 162.5 < 0.005


def test_one_token_is_all_prefill():
    """T = l T_pre + l (n - 1) T_gen: with n = 1 the run is its prefill, and
    every further token adds the same l T_gen."""
    hw = _hw()
    p = dict(wg=0.3, wc=0.7, wd=0, hg=1, hc=0, hd=0, cg=0.2, cc=0.8, cd=0)
    m1 = oc.Model(l=4, h1=256, h2=1024, s=64, n=1)
    t_pre = max(oc.path_times(m1, hw, 32, p, "pre").values())
    assert oc.total_time(m1, hw, 32, p) == pytest.approx(4 * t_pre, rel=1e-12)
    # the mean decode cache length moves with n, so compare at the same n
    m9 = oc.Model(l=4, h1=256, h2=1024, s=64, n=9)
    t_gen = max(oc.path_times(m9, hw, 32, p, "gen").values())
    assert oc.total_time(m9, hw, 32, p) == pytest.approx(4 * t_pre + 4 * 8 * t_gen, rel=1e-12)


def test_slowest_path_sets_the_time():
    """With compute and all but one link made free, T_gen is that link's
    bytes over its bandwidth: moving a share of the weights from GPU to CPU
    adds exactly share x W / bandwidth to CPU -> GPU."""
    m = oc.Model(s=128, n=8, l=2, h1=512, h2=2048)
    fast = 1e30
    hw = _hw(bw_g2c=fast, bw_d2c=fast, bw_c2d=fast, gemm_flops=fast, prefill_flops=fast,
             attn_bw=fast, hbm_bw=fast)
    base = dict(wg=1, wc=0, wd=0, hg=1, hc=0, hd=0, cg=1, cc=0, cd=0)
    moved = dict(base, wg=0.75, wc=0.25)
    t0 = oc.path_times(m, hw, 16, base, "gen")
    t1 = oc.path_times(m, hw, 16, moved, "gen")
    assert t0["c2g"] == 0.0
    assert t1["c2g"] == pytest.approx(0.25 * oc.layer_weight_bytes(m) / hw.bw_c2g, rel=1e-12)
    assert max(t1.values()) == t1["c2g"]


def test_planted_cache_mistake_is_caught(monkeypatch):
    """A cache term that forgets V (2 bytes per element instead of 4 for K
    and V) fails the pages' KV-peak pin."""
    monkeypatch.setattr(oc, "cache_bytes", lambda m, bls, length: 2 * bls * length * m.h1 * m.c_ratio)
    with pytest.raises(AssertionError):
        _pin_kv_peak()


def _pin_decode_peak():
    """[P2] "FlexGen 的核心:计算图分块与张量生命周期": a tier that holds the
    current layer's weights w, the block's activations and the whole block's
    KV cache peaks at w + 2 h1 bls + 4 h1 bls l (s + n) bytes (fp16), which
    bounds the block by bls <= (M_C - w) / (2 h1 + 4 h1 l (s + n)).  In the
    oracle's terms that tier is the CPU with a weight share of one layer
    (1/l), the whole cache and the whole activation share."""
    m = oc.Model(s=512, n=32, **OPT175)
    w = oc.layer_weight_bytes(m)
    p = dict(wg=1 - 1 / m.l, wc=1 / m.l, wd=0, hg=0, hc=1, hd=0, cg=0, cc=1, cd=0)
    for bls in (1, 48, 144, 512):
        want = w + 2 * m.h1 * bls + 4 * m.h1 * bls * m.l * (m.s + m.n)
        got = oc.phase_memory(m, bls, 8, p, "gen")["c"]
        assert got == pytest.approx(want, rel=1e-12)
        # the decode step is the run's peak there (2 l n >= s - 1)
        assert oc.peak_memory(m, bls, 8, p)["c"] == pytest.approx(want, rel=1e-12)
    # the block-size bound: the largest bls whose placement fits M_C
    M_C = 208e9
    hw = _hw(cap_g=1e30, cap_c=M_C, cap_d=0.0)
    bound = int((M_C - w) // (2 * m.h1 + 4 * m.h1 * m.l * (m.s + m.n)))
    assert bound >= 1
    assert oc.feasible(m, hw, bound, 1, p)
    assert not oc.feasible(m, hw, bound + 1, 1, p)


def test_pages_decode_peak_and_block_bound():
    _pin_decode_peak()


@pytest.mark.parametrize("mistake", ["prompt_acts_in_decode", "cache_at_prompt_length", "no_layers"])
def test_planted_peak_mistakes_are_caught(monkeypatch, mistake):
    """Peak-memory terms that hold the prompt's activations during decode,
    count the cache at s instead of s + n positions, or drop the l layers of
    cache each fail the decode-peak pin."""
    real = oc.phase_memory
    if mistake == "prompt_acts_in_decode":
        monkeypatch.setattr(oc, "act_bytes", lambda m, bls, tokens: 2 * bls * m.s * m.h1)
    elif mistake == "cache_at_prompt_length":
        monkeypatch.setattr(oc, "phase_memory",
                            lambda m, bls, gbs, p, phase: real(m, bls, gbs, p, "pre" if phase == "gen" else phase))
    else:
        monkeypatch.setattr(oc, "cache_bytes", lambda m, bls, length: 4 * bls * length * m.h1 * m.c_ratio / m.l)
    with pytest.raises(AssertionError):
        _pin_decode_peak()


# ------------------------------------------------------ product vs oracle
@pytest.fixture(scope="module")
def pol():
    from throughput_oriented_offloaded_amd import policy
    return policy


def _pair(pol, wl_kw, hw_kw):
    m = oc.Model(**wl_kw)
    hw = _hw(**hw_kw)
    wl = pol.Workload(**wl_kw)
    mc = pol.Machine(**{k: getattr(hw, k) for k in pol.Machine.__dataclass_fields__})
    return m, hw, wl, mc


CASES = [
    (dict(l=48, h1=7168, h2=28672, s=512, n=32), {}),                                # 30B fp16, T4-like
    (dict(l=96, h1=12288, h2=49152, s=512, n=32, w_ratio=9 / 32, c_ratio=9 / 32),   # 175B 4-bit, MI355X-like
     dict(bw_c2g=55.9e9, bw_g2c=55.9e9, gemm_flops=961e12, prefill_flops=1.09e15, attn_bw=5.63e12,
          hbm_bw=5.6e12, cap_g=288e9, cap_c=1e12, cap_d=0.0, alpha_g=1.1)),
    (dict(l=24, h1=2048, h2=8192, s=256, n=64), dict(cap_g=2e9, cap_c=20e9, cap_d=0.0)),
]


@pytest.mark.parametrize("wl_kw,hw_kw", CASES)
def test_estimate_matches_oracle(pol, wl_kw, hw_kw):
    m, hw, wl, mc = _pair(pol, wl_kw, hw_kw)
    rng = np.random.default_rng(0)
    for _ in range(20):
        f = [rng.dirichlet(np.ones(3)) for _ in range(3)]
        p = dict(zip(pol.SHARES, np.concatenate(f).tolist()))
        bls, gbs = int(rng.integers(1, 64)) * 8, 8
        got = pol.estimate(wl, mc, bls, gbs, p)
        for ph in ("pre", "gen"):
            want = oc.path_times(m, hw, bls, p, ph)
            for k in oc.PATHS:
                assert got["paths_" + ph][k] == pytest.approx(want[k], rel=1e-12, abs=1e-18)
        pk = oc.peak_memory(m, bls, gbs, p)
        for t in "gcd":
            assert got["peak"][t] == pytest.approx(pk[t], rel=1e-12, abs=1e-3)
        assert got["T"] == pytest.approx(oc.total_time(m, hw, bls, p), rel=1e-12)


LP_CASES = [
    # 30B fp16 on a 16 GB GPU with 208 GB DRAM and a disk: weights and cache must leave the GPU
    (dict(l=48, h1=7168, h2=28672, s=512, n=32), {}, 144, 48, 0.1),
    # 1.3B-shape with tight GPU and host memory, no disk
    (dict(l=24, h1=2048, h2=8192, s=256, n=64), dict(cap_g=2e9, cap_c=20e9, cap_d=0.0), 256, 32, 0.05),
    # 175B 4-bit on MI355X-like constants at a block whose cache exceeds HBM
    (dict(l=96, h1=12288, h2=49152, s=512, n=32, w_ratio=9 / 32, c_ratio=9 / 32),
     dict(bw_c2g=55.9e9, bw_g2c=55.9e9, gemm_flops=961e12, prefill_flops=1.09e15, attn_bw=5.63e12,
          hbm_bw=5.6e12, cap_g=288e9, cap_c=1e12, cap_d=0.0, alpha_g=1.1), 512, 64, 0.05),
]


@pytest.mark.parametrize("wl_kw,hw_kw,bls,gbs,step", LP_CASES)
def test_lp_optimum_against_oracle_search(pol, wl_kw, hw_kw, bls, gbs, step):
    m, hw, wl, mc = _pair(pol, wl_kw, hw_kw)
    shares, v = pol.solve(wl, mc, bls, gbs)
    assert shares is not None
    assert oc.feasible(m, hw, bls, gbs, shares, tol=1e-7)
    assert oc.objective(m, hw, bls, shares) == pytest.approx(v, rel=1e-6)
    _, grid_v = oc.grid_search(m, hw, bls, gbs, step)
    assert v <= grid_v * (1 + 1e-9)
    rng = np.random.default_rng(1)
    no_disk = hw.cap_d == 0
    beaten = 0
    for _ in range(3000):
        f = [rng.dirichlet(np.ones(2 if no_disk else 3)) for _ in range(3)]
        if no_disk:
            f = [np.append(x, 0.0) for x in f]
        p = dict(zip(pol.SHARES, np.concatenate(f).tolist()))
        if oc.feasible(m, hw, bls, gbs, p):
            beaten += oc.objective(m, hw, bls, p) < v * (1 - 1e-9)
    assert beaten == 0


def test_lp_infeasible_block_reports_none(pol):
    """A block whose cache fits in no tier has no policy."""
    _, _, wl, mc = _pair(pol, dict(l=24, h1=2048, h2=8192, s=256, n=64),
                         dict(cap_g=2e9, cap_c=2e9, cap_d=0.0))
    shares, v = pol.solve(wl, mc, 4096, 64)
    assert shares is None and v == float("inf")


def test_search_cli_runs(pol, capsys):
    pol.main(["--model", "opt-30b", "--percent", "100", "0", "0", "100", "100", "0"])
    out = capsys.readouterr().out
    assert '"tokens_per_s"' in out


def test_search_picks_a_feasible_best_policy(pol):
    """The (gbs, nb) search on MI355X-like constants: the chosen policy is
    feasible under the oracle and no other grid point's LP optimum beats it;
    175B fp16 weights (348 GB) cannot all stay in 288 GB of HBM."""
    wl = pol.Workload(96, 12288, 49152, 512, 32)
    mc = pol.mi355x(1e12)
    best = pol.search(wl, mc, gbs_list=(16, 48), nb_max=8)
    assert best is not None
    m = oc.Model(l=96, h1=12288, h2=49152, s=512, n=32)
    hw = oc.Hardware(**{k: getattr(mc, k) for k in oc.Hardware.__dataclass_fields__})
    assert oc.feasible(m, hw, best["bls"], best["gbs"], best["shares"], tol=1e-7)
    assert best["shares"]["wg"] < 1.0
    for gbs in (16, 48):
        for nb in range(1, 9):
            _, v = pol.solve(wl, mc, gbs * nb, gbs)
            assert best["seconds_per_sequence"] <= v * (1 + 1e-9)


def test_executor_realization_rounds_up_and_stays_feasible(pol):
    """The LP under the executor's limits (activations on the GPU, at most
    half of an fp16 layer off it) and its realization: whole tiered layers
    and whole host-resident GPU batches, rounded up from the LP's shares, so
    the GPU holds no more than the LP placed there; the realized placement
    costs at least the LP optimum."""
    wl = pol.Workload(48, 7168, 28672, 512, 32, w_ratio=1.0, c_ratio=pol.Q4G64)
    base = pol.mi355x(32e9)
    mc = pol.Machine(**{**base.__dict__, "cap_g": 56e9})
    best = pol.search(wl, mc, gbs_list=(16, 32), nb_max=6, limits=pol.executor_limits(True))
    assert best is not None
    sh = best["shares"]
    assert sh["hg"] == pytest.approx(1.0) and sh["wc"] <= 0.5 + 1e-9 and sh["wd"] == pytest.approx(0.0)
    nb = best["num_gpu_batches"]
    r = pol.realize(wl, sh, nb)
    rs = r["shares"]
    assert rs["wc"] >= sh["wc"] - 1e-9 and rs["cc"] >= sh["cc"] - 1e-9
    assert r["n_tiered"] == len(r["tiered_layers"]) and rs["wc"] == r["n_tiered"] / (2 * wl.l)
    assert rs["cc"] == r["kv_host_batches"] / nb
    gaps = np.diff(r["tiered_layers"])
    assert len(gaps) == 0 or gaps.max() - gaps.min() <= 1          # evenly spaced
    est = pol.estimate(wl, mc, best["bls"], best["gbs"], rs)
    assert est["T"] / best["bls"] >= best["seconds_per_sequence"] * (1 - 1e-9)
    lp = pol.estimate(wl, mc, best["bls"], best["gbs"], sh)
    assert est["peak"]["g"] <= lp["peak"]["g"] + 1e-3
    # 4-bit weights never leave the GPU under the executor's limits
    wq = pol.Workload(48, 7168, 28672, 512, 32, w_ratio=pol.Q4G64, c_ratio=pol.Q4G64)
    bq = pol.search(wq, mc, gbs_list=(16,), nb_max=4, limits=pol.executor_limits(False))
    assert bq is not None and bq["shares"]["wc"] == pytest.approx(0.0)


# ------------------------------------------------- CPU attention (decode)
def _pin_cpu_attention_moves():
    """[P2] "为什么有时应该在 CPU 上算注意力": bringing a CPU-resident cache to
    the GPU for a one-query attention moves about 4 b s h1 bytes, while
    attending on the CPU moves only about 4 b h1, a factor of about s apart.
    With every link at 1 byte/s (times are bytes) and the whole cache on the
    host: without delegation CPU -> GPU carries 4 b L h1 (L the mean decode
    length standing for s); with it the two links together carry the new
    cache entries, which go back in either case, plus exactly 4 b h1 (the
    query going down and the attention row coming up)."""
    m = oc.Model(l=4, h1=512, h2=2048, s=300, n=20)
    hw = _hw(bw_c2g=1.0, bw_g2c=1.0, cpu_attn_bw=1e9)
    p = dict(wg=1, wc=0, wd=0, hg=1, hc=0, hd=0, cg=0, cc=1, cd=0)
    b, L = 24, m.s + m.n / 2
    off = oc.path_times(m, hw, b, p, "gen")
    on = oc.path_times(m, hw, b, p, "gen", cpu_attn=True)
    kv_move = 4 * b * L * m.h1
    act_move = 4 * b * m.h1
    new_entries = 4 * b * m.h1
    assert off["c2g"] == pytest.approx(kv_move, rel=1e-12)
    assert off["g2c"] == pytest.approx(new_entries, rel=1e-12)
    assert on["c2g"] + on["g2c"] - new_entries == pytest.approx(act_move, rel=1e-12)
    assert off["c2g"] / (on["c2g"] + on["g2c"] - new_entries) == pytest.approx(L, rel=1e-12)
    # the host reads the whole cache at its attention rate; the GPU none of it
    assert on["cpu"] == pytest.approx(kv_move / hw.cpu_attn_bw, rel=1e-12)
    free_attn = _hw(bw_c2g=1.0, bw_g2c=1.0, cpu_attn_bw=1e9, attn_bw=1e30)
    assert on["comp"] == pytest.approx(oc.path_times(m, free_attn, b, p, "gen")["comp"], rel=1e-12)


def test_pages_cpu_attention_moves():
    _pin_cpu_attention_moves()


def test_cpu_attention_without_a_host_share_changes_nothing():
    """Delegation only touches the host-resident cache share: with cc = 0
    every path time is the same either way and the CPU path is idle; the
    prompt phase is never delegated."""
    m = oc.Model(l=4, h1=512, h2=2048, s=128, n=16)
    hw = _hw(cpu_attn_bw=40e9)
    p = dict(wg=0.4, wc=0.5, wd=0.1, hg=0.7, hc=0.3, hd=0, cg=0.6, cc=0, cd=0.4)
    assert oc.path_times(m, hw, 32, p, "gen", True) == oc.path_times(m, hw, 32, p, "gen")
    q = dict(p, cg=0.2, cc=0.4)
    assert oc.path_times(m, hw, 32, q, "pre", True) == oc.path_times(m, hw, 32, q, "pre")
    assert oc.path_times(m, hw, 32, q, "gen")["cpu"] == 0.0


def test_cpu_attention_compressed_cache_rate(pol):
    """The pages' authors switch delegation off with a 4-bit cache (their
    CPU's dequantization eats the saving); here a compressed cache is
    delegated only at a rate of its own: without one both models refuse it
    and the search does not try it; with one, the host path reads the share's
    stored (compressed) bytes at that rate, and the links carry the same
    fp16 rows as for an fp16 cache."""
    kw = dict(l=4, h1=512, h2=2048, s=128, n=16, c_ratio=9 / 32)
    m = oc.Model(**kw)
    p = dict(wg=1, wc=0, wd=0, hg=1, hc=0, hd=0, cg=0, cc=1, cd=0)
    with pytest.raises(AssertionError):
        oc.path_times(m, _hw(cpu_attn_bw=40e9), 8, p, "gen", True)
    _, _, wl, mc = _pair(pol, kw, dict(cpu_attn_bw=40e9))
    with pytest.raises(ValueError):
        pol.estimate(wl, mc, 8, 8, p, cpu_attn=True)
    best = pol.search(wl, mc, gbs_list=(8,), nb_max=2)
    assert best is not None and best["cpu_attention"] is False
    hw = _hw(cpu_attn_bw=40e9, cpu_attn_bw_q4=7e9, bw_c2g=1.0, bw_g2c=1.0)
    b, L = 8, m.s + m.n / 2
    on = oc.path_times(m, hw, b, p, "gen", True)
    assert on["cpu"] == pytest.approx(4 * b * L * m.h1 * (9 / 32) / 7e9, rel=1e-12)
    assert on["c2g"] + on["g2c"] == pytest.approx(8 * b * m.h1, rel=1e-12)   # q, k, v down, the row up
    _, _, wl, mc = _pair(pol, kw, dict(cpu_attn_bw=40e9, cpu_attn_bw_q4=7e9, bw_c2g=1.0, bw_g2c=1.0))
    got = pol.estimate(wl, mc, b, 8, p, cpu_attn=True)
    for k in oc.PATHS:
        assert got["paths_gen"][k] == pytest.approx(on[k], rel=1e-12, abs=1e-18)


CPU_CASES = [
    # 30B fp16 on a 16 GB GPU: the cache lives on the host, PCIe-bound
    (dict(l=48, h1=7168, h2=28672, s=512, n=32), dict(cpu_attn_bw=50e9), 144, 48, 0.1),
    # 1.3B-shape, tight memories, a slow host
    (dict(l=24, h1=2048, h2=8192, s=256, n=64), dict(cap_g=2e9, cap_c=20e9, cap_d=0.0, cpu_attn_bw=5e9),
     256, 32, 0.05),
]


@pytest.mark.parametrize("wl_kw,hw_kw,bls,gbs,step", CPU_CASES)
def test_cpu_attention_estimate_and_lp_match_oracle(pol, wl_kw, hw_kw, bls, gbs, step):
    m, hw, wl, mc = _pair(pol, wl_kw, hw_kw)
    rng = np.random.default_rng(2)
    for _ in range(20):
        f = [rng.dirichlet(np.ones(3)) for _ in range(3)]
        p = dict(zip(pol.SHARES, np.concatenate(f).tolist()))
        got = pol.estimate(wl, mc, bls, gbs, p, cpu_attn=True)
        for ph in ("pre", "gen"):
            want = oc.path_times(m, hw, bls, p, ph, cpu_attn=True)
            for k in oc.PATHS:
                assert got["paths_" + ph][k] == pytest.approx(want[k], rel=1e-12, abs=1e-18)
        assert got["T"] == pytest.approx(oc.total_time(m, hw, bls, p, cpu_attn=True), rel=1e-12)
    shares, v = pol.solve(wl, mc, bls, gbs, cpu_attn=True)
    assert shares is not None
    assert oc.feasible(m, hw, bls, gbs, shares, tol=1e-7)
    assert oc.objective(m, hw, bls, shares, cpu_attn=True) == pytest.approx(v, rel=1e-6)
    _, grid_v = oc.grid_search(m, hw, bls, gbs, step, cpu_attn=True)
    assert v <= grid_v * (1 + 1e-9)


def test_search_delegates_only_when_it_pays(pol):
    """Where the host holds the cache and PCIe is the bottleneck, a host
    with spare bandwidth makes delegation the better policy; a host with
    almost none does not ("只在缓存本来就在 CPU、PCIe 搬运成为瓶颈、CPU 还有可用算力
    时成立")."""
    wl_kw = dict(l=48, h1=7168, h2=28672, s=512, n=32)
    _, _, wl, fast = _pair(pol, wl_kw, dict(cpu_attn_bw=50e9))
    _, _, _, slow = _pair(pol, wl_kw, dict(cpu_attn_bw=1e8))
    on = pol.search(wl, fast, gbs_list=(16, 48), nb_max=4)
    assert on["cpu_attention"] is True
    off = pol.search(wl, fast, gbs_list=(16, 48), nb_max=4, cpu_attn=False)
    assert on["seconds_per_sequence"] < off["seconds_per_sequence"]
    assert pol.search(wl, slow, gbs_list=(16, 48), nb_max=4)["cpu_attention"] is False


def test_realized_search_ranks_placements_as_realized(pol):
    """OPT-1.3B fp16 with all of HBM: the continuous LP prefers a sliver of
    host cache with CPU attention (the host attends in parallel with the
    GPU), but whole GPU batches are the executor's unit, and one whole batch
    on the host makes the CPU the slowest path; the realized search keeps
    every cache on the GPU.  Its choice fits the capacities under the
    oracle's own test and is no worse, as realized, than rounding either
    mode's LP optimum."""
    wl = pol.Workload(24, 2048, 8192, 512, 32)
    mc = pol.mi355x(64e9)
    lim = pol.executor_limits(True)
    kw = dict(gbs_list=(16, 32, 48, 64), nb_max=8, limits=lim)
    lp = pol.search(wl, mc, **kw)
    assert lp["cpu_attention"] is True and 0 < lp["shares"]["cc"] < 0.5
    best = pol.search_realized(wl, mc, **kw)
    assert best["cpu_attention"] is False and best["kv_host_batches"] == 0
    m = oc.Model(l=24, h1=2048, h2=8192, s=512, n=32)
    hw = oc.Hardware(**{k: getattr(mc, k) for k in oc.Hardware.__dataclass_fields__})
    assert oc.feasible(m, hw, best["bls"], best["gbs"], best["shares"], tol=1e-7)
    assert oc.objective(m, hw, best["bls"], best["shares"], best["cpu_attention"]) == \
        pytest.approx(best["seconds_per_sequence"], rel=1e-9)
    for ca in (False, True):
        b = pol.search(wl, mc, cpu_attn=ca, **kw)
        r = pol.realize(wl, b["shares"], b["num_gpu_batches"])
        v = oc.objective(m, hw, b["bls"], r["shares"], ca and r["kv_host_batches"] > 0)
        assert best["seconds_per_sequence"] <= v * (1 + 1e-9)
