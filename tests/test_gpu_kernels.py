"""Kernel-level parity of the HIP path against the oracle, through the C ABI.

  * projection kernel (RMSNorm prologue, store / residual / SwiGLU epilogues,
    fp32 and bf16 weights, every activation-tile size and ragged tails) vs the
    oracle's rms_norm / silu and a float64 matmul;
  * selection kernel: processed logits (penalty, min-new, suppress) bit-exact
    vs the oracle's processors; greedy ids bit-exact; given identical
    probabilities and noise the sampled id is bit-exact (top-p + race);
    Philox noise drawn on the device equals the oracle's Philox4x64-10;
    sampling from logits agrees with the oracle except near ties; a NaN row
    fails closed;
  * prompt-prefill attention (tiled matrix-core kernel and per-token kernel)
    vs the oracle's RMSNorm, rope and attention in float64.
"""
import numpy as np
import pytest

from codec_lm_autoregressive_amd import binding, synth
from oracle import model, philox, sampling

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _ref_linear(W, X, gain, eps, epi, Y0):
    x = X.astype(np.float64)
    if gain is not None:
        x = model.rms_norm(x, gain, eps, np.float64)
    y = x @ W.astype(np.float64).T
    if epi == 1:
        return Y0.astype(np.float64) + y
    if epi == 2:
        g, u = y[:, 0::2], y[:, 1::2]
        return model.silu(g) * u
    return y


@pytest.mark.parametrize("mc", [True, False])
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("N,K,M", [(4096, 1024, 1), (1024, 2048, 3), (6144, 1024, 8), (1024, 3072, 5),
                                   (3072, 512, 17), (200, 64, 2), (2048, 1024, 64), (96, 6144, 9),
                                   (1024, 3072, 16), (200, 96, 130), (6144, 1024, 257), (2048, 2048, 1024),
                                   (200, 1024, 12), (1000, 768, 30), (4096, 2048, 24), (1024, 3072, 128),
                                   (2052, 512, 100), (2048, 1024, 3), (3072, 2048, 16), (4096, 512, 7),
                                   (2048, 256, 4), (2056, 1536, 11), (6144, 1024, 32), (2048, 3072, 20),
                                   (6144, 1024, 64), (1024, 256, 40), (4096, 1024, 48),
                                   (3072, 1024, 8), (2048, 1024, 6), (1000, 2048, 4),
                                   (1024, 2048, 2100), (2056, 256, 4100), (4096, 1024, 2100),
                                   (4104, 512, 2050), (192, 512, 2100), (96, 256, 4100)])
@pytest.mark.parametrize("epi,norm", [(0, True), (1, False), (2, True)])
def test_linear_matches_oracle(mc, wdt, N, K, M, epi, norm):
    """mc: hand the library its row and split-K scratch, which routes bf16
    weights with 17..128 rows to the split-K MFMA GEMM and more rows to the
    split-activation MFMA GEMM; without it they take the LDS-tile FMA kernel.
    3..8 rows use the 8-row matrix-core GEMV (the 16-row one when its grid is
    a multiple of 256 blocks), 9..16 rows the register-operand matrix-core
    GEMV when N >= 2048 (also up to 32 rows) and the skinny MFMA kernel
    otherwise, either way. From 2048 rows without a gain the split GEMM reads
    fp32 activation tiles and splits them itself (2100 rows on 64 x 128
    tiles, 4100 rows on 128 x 128 tiles, both with ragged tails); from 4096
    columns and 2048 rows it runs 8 waves on 128 x 256 tiles (4096 and a
    ragged 4104 columns); 96 and 192 columns (the codec's late stages) pad
    their 128-wide tiles."""
    if not mc and (wdt != "bf16" or M < 16):
        pytest.skip("same kernel as the mc=True case")
    torch = _torch()
    g = np.random.default_rng(N * 7 + K + M)
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    if wdt == "bf16":
        W = synth.bf16_round(W)
    X = (g.standard_normal((M, K))).astype(np.float32)
    gain = (1 + 0.02 * g.standard_normal(K)).astype(np.float32) if norm else None
    Y0 = g.standard_normal((M, N // 2 if epi == 2 else N)).astype(np.float32)
    Wd = binding.to_device_weight(W, wdt)
    Xd = torch.from_numpy(X).cuda()
    Gd = torch.from_numpy(gain).cuda() if gain is not None else None
    Yd = torch.from_numpy(Y0.copy()).cuda()
    binding.debug_linear(Wd, Xd, Gd, 1e-6, epi, Yd, wdtype=wdt, matrix_cores=mc)
    torch.cuda.synchronize()
    got = Yd.cpu().numpy().astype(np.float64)
    ref = _ref_linear(W, X, gain, 1e-6, epi, Y0)
    scale = np.max(np.abs(ref)) + 1e-30
    assert np.max(np.abs(got - ref)) / scale < 2e-5, (np.max(np.abs(got - ref)), scale)


def test_linear_weight_copies_rotate():
    """qt_debug_linear's timing mode: launch i reads weight copy i % copies."""
    torch = _torch()
    g = np.random.default_rng(3)
    N, K, M = 512, 1024, 1
    W = [synth.bf16_round((g.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in range(2)]
    X = g.standard_normal((M, K)).astype(np.float32)
    Ws = torch.stack([binding.to_device_weight(w, "bf16") for w in W]).contiguous()
    Xd = torch.from_numpy(X).cuda()
    for reps, last in [(3, 0), (4, 1)]:
        Yd = binding.debug_linear(Ws, Xd, None, 1e-6, 0, reps=reps)
        torch.cuda.synchronize()
        ref = X.astype(np.float64) @ W[last].astype(np.float64).T
        assert np.max(np.abs(Yd.cpu().numpy() - ref)) < 1e-4 * np.max(np.abs(ref))


CFG = dict(eos_id=2150, suppress_begin=2048, suppress_end=3072)


def _seen_bits(seen_rows, V):
    W = (V + 31) // 32
    bits = np.zeros((len(seen_rows), W), dtype=np.uint32)
    for r, ids in enumerate(seen_rows):
        for i in ids:
            bits[r, i >> 5] |= np.uint32(1 << (i & 31))
    return bits


@pytest.mark.parametrize("sel_index", [0, 1, 2, 7])
def test_select_greedy_processors_bit_exact(sel_index):
    torch = _torch()
    B, V = 6, 3072
    g = np.random.default_rng(sel_index)
    L = (g.standard_normal((B, V)) * 2).astype(np.float32)
    L[0, 2150] = 50.0                       # EOS on top: masked while sel < 2
    L[1, 2500] = 60.0                       # suppressed control id
    L[2, [5, 9, 700]] = 30.0                # exact tie -> lowest index
    L[3, :] = 0.0                           # all-equal row: lowest allowed index
    seen = [list(g.integers(0, 2048, size=20)) for _ in range(B)]
    seen[4] = [int(np.argmax(L[4]))]        # penalised winner may lose its place
    samp = dict(synth.GREEDY)
    out, proc, st = binding.debug_select(torch.from_numpy(L).cuda(), samp,
                                         seen=torch.from_numpy(_seen_bits(seen, V).view(np.int32)).cuda(),
                                         processors=True, sel_index=sel_index, want_processed=True)
    proc = proc.cpu().numpy()
    for r in range(B):
        ref = sampling.talker_process(L[r], seen[r], sel_index, samp, CFG)
        np.testing.assert_array_equal(proc[r], ref)
        assert int(out[r]) == sampling.greedy(ref)
    assert int(st[0]) == 0


def test_select_probs_and_noise_bit_exact():
    torch = _torch()
    B, V = 16, 2048
    g = np.random.default_rng(5)
    P = np.zeros((B, V), dtype=np.float32)
    for r in range(B):
        ids = g.choice(V, size=int(g.integers(1, 60)), replace=False)
        w = g.integers(1, 64, size=ids.size).astype(np.float64)
        P[r, ids] = (w / 64.0 / w.sum() * 64.0).astype(np.float32)  # not necessarily dyadic
    E = g.exponential(size=(B, V)).astype(np.float32) + np.float32(1e-3)
    for tp in (0.8, 1.0, 0.3):
        samp = dict(synth.PRED_SAMPLING, top_p=tp)
        out, _, _ = binding.debug_select(torch.from_numpy(P).cuda(), samp, noise=torch.from_numpy(E).cuda(),
                                         probs=torch.from_numpy(P).cuda())
        for r in range(B):
            keep = sampling.top_p_keep(P[r], tp)
            ref, _ = sampling.race(P[r], keep, lambda i, r=r: E[r, i])
            assert int(out[r]) == ref, (r, tp)


@pytest.mark.parametrize("n_nonzero", [100, 600, 2048])
def test_select_many_survivors_bit_exact(n_nonzero):
    """More survivors than one wave holds: the block-wide orderings (ranks up to
    512 survivors, a bitonic sort beyond) feed the same top-p sum and race."""
    torch = _torch()
    B, V = 4, 2048
    g = np.random.default_rng(50 + n_nonzero)
    P = np.zeros((B, V), dtype=np.float32)
    for r in range(B):
        ids = g.choice(V, size=n_nonzero, replace=False)
        w = g.integers(1, 9, size=ids.size).astype(np.float64)   # many equal p: id order breaks the ties
        P[r, ids] = (w / w.sum()).astype(np.float32)
    E = g.exponential(size=(B, V)).astype(np.float32) + np.float32(1e-3)
    for tp in (0.8, 1.0, 0.3):
        samp = dict(synth.PRED_SAMPLING, top_p=tp, top_k=0)
        out, _, _ = binding.debug_select(torch.from_numpy(P).cuda(), samp, noise=torch.from_numpy(E).cuda(),
                                         probs=torch.from_numpy(P).cuda())
        for r in range(B):
            keep = sampling.top_p_keep(P[r], tp)
            ref, _ = sampling.race(P[r], keep, lambda i, r=r: E[r, i])
            assert int(out[r]) == ref, (n_nonzero, r, tp)


def test_device_philox_matches_oracle():
    """Same probabilities, noise drawn on the device vs the oracle's Philox."""
    torch = _torch()
    B, V = 32, 2048
    g = np.random.default_rng(6)
    P = np.zeros((B, V), dtype=np.float32)
    for r in range(B):
        ids = g.choice(V, size=40, replace=False)
        P[r, ids] = np.float32(1.0 / 40)    # equal p: the noise alone decides
    for seed, stream, idx in [(0, 0, 0), (12345, 3, 17), (2**63 + 5, 15, 1023)]:
        samp = dict(synth.PRED_SAMPLING, top_p=1.0)
        out, _, _ = binding.debug_select(torch.from_numpy(P).cuda(), samp, probs=torch.from_numpy(P).cuda(),
                                         seed=seed, stream_id=stream, sel_index=idx)
        for r in range(B):
            keep = sampling.top_p_keep(P[r], 1.0)
            ref, _ = sampling.race(P[r], keep, lambda i, r=r: philox.exp_noise(seed, r, stream, idx, i))
            assert int(out[r]) == ref, (seed, stream, idx, r)


def test_device_noise_bitwise_equals_oracle():
    """The selection kernel's Exp(1) noise against the oracle's independent
    Philox4x64-10 and -ln u, bit for bit: 120 000 counters (seeds up to 2^64 - 1,
    rows, streams 0..15, selection indices, vocabulary ids), and raw words at
    the ends of the uniform mapping (top 52 bits all zero or all one) plus
    random words."""
    torch = _torch()
    g = np.random.default_rng(12)
    n = 120_000
    ctr = np.stack([g.integers(0, 6144, n), g.integers(0, 16, n), g.integers(0, 1 << 20, n),
                    g.integers(0, 4096, n)], axis=1).astype(np.int64)
    for seed in (0, 7, 2**64 - 1):
        sl = slice(0, 40_000)
        dev = binding.debug_exp_noise(torch.from_numpy(ctr[sl]).cuda(), 0, seed).cpu().numpy()
        ref = np.array([philox.exp_noise(seed, int(c[3]), int(c[1]), int(c[2]), int(c[0])) for c in ctr[sl]],
                       dtype=np.float32)
        bad = np.nonzero(dev.view(np.uint32) != ref.view(np.uint32))[0]
        assert bad.size == 0, (seed, bad[:5], dev[bad[:5]], ref[bad[:5]])
        ctr = ctr[40_000:]
    edge = [0, 1, 4095, 4096, 8191, (1 << 64) - 1, (1 << 64) - 4096, (1 << 64) - 4097, 1 << 63, (1 << 63) - 1]
    words = edge + [int(x) for x in g.integers(0, 2**63 - 1, 20_000, dtype=np.int64)] \
        + [int(x) | (1 << 63) for x in g.integers(0, 2**63 - 1, 20_000, dtype=np.int64)]
    wt = torch.from_numpy(np.array(words, dtype=np.uint64).view(np.int64)).cuda()
    dev = binding.debug_exp_noise(wt, 1).cpu().numpy()
    ref = np.array([philox.noise_from_word(x) for x in words], dtype=np.float32)
    bad = np.nonzero(dev.view(np.uint32) != ref.view(np.uint32))[0]
    assert bad.size == 0, (bad[:5], [words[i] for i in bad[:5]], dev[bad[:5]], ref[bad[:5]])
    assert ref[0] == np.float32(-np.log(0.5 * 2.0 ** -52)) and ref[5] == np.float32(-np.log1p(-0.5 * 2.0 ** -52))


def test_select_sampling_from_logits_matches_oracle():
    torch = _torch()
    B, V = 48, 3072
    g = np.random.default_rng(8)
    L = (g.standard_normal((B, V)) * 1.5).astype(np.float32)
    seen = [list(g.integers(0, 2048, size=10)) for _ in range(B)]
    samp = dict(synth.SAMPLING)
    seed, idx = 99, 4
    out, _, st = binding.debug_select(torch.from_numpy(L).cuda(), samp,
                                      seen=torch.from_numpy(_seen_bits(seen, V).view(np.int32)).cuda(),
                                      processors=True, seed=seed, stream_id=0, sel_index=idx)
    agree, exempt = 0, 0
    for r in range(B):
        pl = sampling.talker_process(L[r], seen[r], idx, samp, CFG)
        ref, info = sampling.select(pl, samp, lambda i, r=r: philox.exp_noise(seed, r, 0, idx, i))
        if int(out[r]) == ref:
            agree += 1
        else:
            # identical logits: only float32 rounding of exp / sums can separate them
            assert sampling.flip_possible(pl, samp, lambda i, r=r: philox.exp_noise(seed, r, 0, idx, i), ref,
                                          int(out[r]), 1e-5), (r, info)
            exempt += 1
    assert agree >= B - 2
    assert int(st[0]) == 0


def test_select_topk_ties_kept():
    torch = _torch()
    V = 2048
    L = np.full((1, V), -5.0, dtype=np.float32)
    L[0, :8] = [3, 2, 2, 2, 2, 1, 0, 0]
    # top-k 2 with ties at the threshold keeps ids 0..4; equal noise -> highest p wins (id 0)
    samp = dict(synth.PRED_SAMPLING, top_k=2, top_p=1.0, temperature=1.0)
    E = np.ones((1, V), dtype=np.float32)
    out, _, _ = binding.debug_select(torch.from_numpy(L).cuda(), samp, noise=torch.from_numpy(E).cuda())
    assert int(out[0]) == 0
    # make id 4 the race winner: only possible if ties at the threshold survived
    E[0, :4] = 100.0
    out, _, _ = binding.debug_select(torch.from_numpy(L).cuda(), samp, noise=torch.from_numpy(E).cuda())
    assert int(out[0]) == 4
    E[0, :5] = 100.0     # 5 is outside top-k: the winner stays inside the kept set
    out, _, _ = binding.debug_select(torch.from_numpy(L).cuda(), samp, noise=torch.from_numpy(E).cuda())
    assert int(out[0]) in (0, 1, 2, 3, 4)


@pytest.mark.parametrize("case", ["normal", "outlier", "ties", "suppressed"])
def test_select_topk_cut_exact(case):
    """The sampled selection's top-k cut keeps exactly the values at or above
    the k-th largest, ties included. Per row one probe id (ranked around k)
    gets Exp(1) noise 1e-30 and every other id 1, so the probe wins the race
    if and only if it survived the cut; otherwise the row's largest value
    (lowest id on ties) wins. Rows of normal values, a wide range (one
    outlier far above the rest), integer values with hundreds of ties per
    value (crowded buckets: the kernel's radix fallback), and half the ids at
    -inf; k from 1 to V - 1 (many survivors take the block-wide path)."""
    torch = _torch()
    B, V = 64, 2048
    g = np.random.default_rng({"normal": 1, "outlier": 2, "ties": 3, "suppressed": 4}[case])
    if case == "ties":
        L = g.integers(-3, 4, size=(B, V)).astype(np.float32)
    else:
        L = (g.standard_normal((B, V)) * 2).astype(np.float32)
    if case == "outlier":
        L[:, 7] = 40.0
    if case == "suppressed":
        L[:, g.permutation(V)[:V // 2]] = -np.inf
    for k in (1, 2, 50, 300, V - 1):
        E = np.ones((B, V), dtype=np.float32)
        expect = np.empty(B, dtype=np.int64)
        probes = np.empty(B, dtype=np.int64)
        for r in range(B):
            order = np.argsort(-L[r], kind="stable")
            t = min(max(k - 1 + (r % 3) - 1, 0), V - 1)   # ranks k - 2, k - 1, k
            j = int(order[t])
            kth = L[r, order[k - 1]]
            kept = L[r, j] >= kth and np.isfinite(L[r, j])
            E[r, j] = 1e-30
            probes[r] = j
            expect[r] = j if kept else int(np.argmax(L[r]))
        samp = dict(synth.PRED_SAMPLING, top_k=k, top_p=1.0, temperature=1.0)
        print(f"top-k cut case={case} k={k}", flush=True)
        out, _, st = binding.debug_select(torch.from_numpy(L).cuda(), samp, noise=torch.from_numpy(E).cuda())
        got = out.cpu().numpy().astype(np.int64)
        assert int(st[0]) == 0
        bad = np.nonzero(got != expect)[0]
        assert bad.size == 0, (case, k, [(int(r), int(probes[r]), int(got[r]), int(expect[r])) for r in bad[:5]])


def test_select_nan_fails_closed():
    torch = _torch()
    L = np.zeros((3, 3072), dtype=np.float32)
    L[1, 17] = np.nan
    out, _, st = binding.debug_select(torch.from_numpy(L).cuda(), dict(synth.GREEDY), processors=True)
    assert int(st[0]) & 1
    L[1, 17] = np.inf
    out, _, st = binding.debug_select(torch.from_numpy(L).cuda(), dict(synth.GREEDY), processors=True)
    assert int(st[0]) & 1
    L[1, 17] = 0.0
    out, _, st = binding.debug_select(torch.from_numpy(L).cuda(), dict(synth.GREEDY), processors=True)
    assert int(st[0]) == 0


def _ref_prefill_attention(qkv, lens, q_gain, k_gain, cos, sin, nq, nkv, eps, kv):
    """Per row: the oracle's per-head RMSNorm and rope in float64, keys and
    values rounded to the cache type (through float32, as the kernel stores
    them), causal GQA attention in float64."""
    d = qkv.shape[1] // (nq + 2 * nkv)
    out, t0 = [], 0
    for L in lens:
        x = qkv[t0:t0 + L].astype(np.float64)
        q = x[:, :nq * d].reshape(L, nq, d)
        k = x[:, nq * d:(nq + nkv) * d].reshape(L, nkv, d)
        v = x[:, (nq + nkv) * d:].reshape(L, nkv, d)
        pos = np.arange(L)
        q = model.apply_rope(model.rms_norm(q, q_gain, eps, np.float64), pos, cos, sin, np.float64)
        k = model.apply_rope(model.rms_norm(k, k_gain, eps, np.float64), pos, cos, sin, np.float64)
        if kv == "f16":
            k = k.astype(np.float32).astype(np.float16).astype(np.float64)
            v = v.astype(np.float32).astype(np.float16).astype(np.float64)
        else:
            k = synth.bf16_round(k).astype(np.float64)
            v = synth.bf16_round(v).astype(np.float64)
        o = model.attention(q, k.transpose(1, 0, 2), v.transpose(1, 0, 2), pos, nkv, np.float64)
        out.append(o.reshape(L, nq * d))
        t0 += L
    return np.concatenate(out)


@pytest.mark.parametrize("kv", ["f16", "bf16"])
@pytest.mark.parametrize("lens,gain_scale", [([1, 45, 130], 1.0), ([33, 64, 65, 7, 96], 3.0), ([1500, 3], 2.0)])
def test_prefill_attention_tiled_matches_oracle(kv, lens, gain_scale):
    """The prompt prefill's attention at the talker's head shape (16 q / 8 kv
    heads, head_dim 128): runs of up to 32 tokens on the matrix cores
    (ragged last run, 64-key blocks with a ragged last block, a 1500-token
    row), against the oracle in float64 with the cache's rounding, and
    against the per-token kernel on the same cache.

    Tolerances. Oracle: the kernel stores keys rounded from its float32 rope,
    the oracle from float64 through float32, so a few stored key elements may
    differ by one unit of the cache type; one such unit moves a score by up
    to |q_i| ulp(k_i) / sqrt(d), which grows with both gains: 2e-3 for fp16,
    2e-3 g^2 for bf16 (8x coarser). Per-token kernel, same cache: the q and P
    operands are split into 16-bit hi + lo parts, 22 significant bits with
    fp16 (5e-5) and 16 with bf16 (5e-4)."""
    torch = _torch()
    nq, nkv, d, eps = 16, 8, 128, 1e-6
    lens = np.array(lens, dtype=np.int32)
    T, B, max_pos = int(lens.sum()), len(lens), 1536
    rng = np.random.default_rng(int(lens.sum()) + (7 if kv == "f16" else 8))
    qkv = rng.standard_normal((T, (nq + 2 * nkv) * d)).astype(np.float32)
    q_gain = (gain_scale * (1.0 + 0.1 * rng.standard_normal(d))).astype(np.float32)
    k_gain = (gain_scale * (1.0 + 0.1 * rng.standard_normal(d))).astype(np.float32)
    cos, sin = model.rope_tables(max_pos, d, 1.0e6)
    ref = _ref_prefill_attention(qkv, lens, q_gain, k_gain, cos, sin, nq, nkv, eps, kv)
    dev = [torch.from_numpy(a).cuda() for a in (qkv, q_gain, k_gain, cos, sin)]
    g2 = max(1.0, gain_scale) ** 2
    tol_oracle, tol_cross = (2e-3, 5e-5) if kv == "f16" else (2e-3 * g2, 5e-4)
    outs, errs = {}, {}
    for tiled in (True, False):
        kc = torch.zeros((B, nkv, max_pos, d), dtype=torch.float16 if kv == "f16" else torch.int16, device="cuda")
        vc = torch.zeros_like(kc)
        print(f"prefill attention kv={kv} lens={list(lens)} tiled={tiled}", flush=True)
        outs[tiled] = binding.debug_prefill_attention(dev[0], lens, dev[1], dev[2], dev[3], dev[4], kc, vc, nq, nkv,
                                                      eps, kv, tiled).cpu().numpy()
        errs[tiled] = float(np.max(np.abs(outs[tiled] - ref)))
        print(f"  max|out - oracle| {errs[tiled]:.3e} (tol {tol_oracle:.1e})", flush=True)
    cross = float(np.max(np.abs(outs[True] - outs[False])))
    print(f"  max|tiled - per-token| {cross:.3e} (tol {tol_cross:.1e})", flush=True)
    assert np.all(np.isfinite(outs[True])) and np.all(np.isfinite(outs[False]))
    assert cross <= tol_cross, cross
    assert errs[True] <= tol_oracle and errs[False] <= tol_oracle, errs


def _cache_round(x, kv):
    """Values as a cache of type kv holds them (rounded through float32)."""
    x = np.asarray(x, dtype=np.float32)
    if kv == "f16":
        return x.astype(np.float16).astype(np.float64)
    if kv == "bf16":
        return synth.bf16_round(x).astype(np.float64)
    return x.astype(np.float64)


def _ref_decode_attention(qkv, pos, kc, vc, q_gain, k_gain, cos, sin, nq, nkv, eps, kv):
    """Per row r: the oracle's per-head RMSNorm and rope of the new token at
    position pos[r] in float64, its key and value rounded to the cache type,
    GQA attention in float64 over cached positions 0 .. pos[r] - 1 (as
    stored) and the new one."""
    B, d = qkv.shape[0], qkv.shape[1] // (nq + 2 * nkv)
    out = np.empty((B, nq * d))
    for r in range(B):
        p = int(pos[r])
        x = qkv[r:r + 1].astype(np.float64)
        q = x[:, :nq * d].reshape(1, nq, d)
        k = x[:, nq * d:(nq + nkv) * d].reshape(1, nkv, d)
        v = x[:, (nq + nkv) * d:].reshape(1, nkv, d)
        q = model.apply_rope(model.rms_norm(q, q_gain, eps, np.float64), [p], cos, sin, np.float64)
        k = _cache_round(model.apply_rope(model.rms_norm(k, k_gain, eps, np.float64), [p], cos, sin, np.float64), kv)
        v = _cache_round(v, kv)
        K = np.concatenate([kc[r, :, :p], k.transpose(1, 0, 2)], axis=1)
        V = np.concatenate([vc[r, :, :p], v.transpose(1, 0, 2)], axis=1)
        out[r] = model.attention(q, K, V, [p], nkv, np.float64).reshape(nq * d)
    return out


@pytest.mark.parametrize("kv", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("pos,nkv,G,max_pos,splits", [
    ([0, 1, 15, 16, 17, 47, 48, 49, 63, 64, 65, 130], 8, 2, 256, (1, 2, 4, 8, 16)),
    ([1499, 700, 3], 8, 2, 1536, (1, 4, 16)),
    ([5, 33, 100], 4, 4, 128, (1, 2)),
    ([3, 9], 8, 2, 16, (1,)),
])
def test_decode_attention_matches_oracle(kv, pos, nkv, G, max_pos, splits):
    """One single-token decode step of the attention (the new token's
    QK-RMSNorm and rope, its K/V into the cache, GQA over positions 0 .. pos)
    for rows at ragged positions: empty caches, ragged tails of the 16- and
    64-key groups the kernels stream in, a 1500-token context, every key-range
    split, 4 q heads per kv head, and the predictor's 16-position cache;
    against the float64 oracle over the same cache contents. Tolerance as for
    the prefill attention: the kernel rounds its float32 rope result into the
    cache, the oracle its float64 one, so a few stored elements of the new key
    may sit one unit of the cache type apart (2e-3 at unit gains); split and
    unsplit runs on one cache agree to 1e-5 (ranges added in another order)."""
    torch = _torch()
    nq, d, eps = nkv * G, 128, 1e-6
    pos = np.array(pos, dtype=np.int32)
    B = len(pos)
    rng = np.random.default_rng(int(pos.sum()) + 11 * G + {"f16": 0, "bf16": 1, "f32": 2}[kv])
    qkv = rng.standard_normal((B, (nq + 2 * nkv) * d)).astype(np.float32)
    q_gain = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    k_gain = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    cos, sin = model.rope_tables(max_pos, d, 1.0e6)
    kc = _cache_round(rng.standard_normal((B, nkv, max_pos, d)), kv)
    vc = _cache_round(rng.standard_normal((B, nkv, max_pos, d)), kv)
    ref = _ref_decode_attention(qkv, pos, kc, vc, q_gain, k_gain, cos, sin, nq, nkv, eps, kv)

    def dev_cache(x):
        if kv == "f16":
            return torch.from_numpy(x.astype(np.float16)).cuda()
        if kv == "bf16":
            return torch.from_numpy(synth.bf16_bits(x.astype(np.float32)).view(np.int16)).cuda()
        return torch.from_numpy(x.astype(np.float32)).cuda()

    dev = [torch.from_numpy(a).cuda() for a in (qkv, q_gain, k_gain, cos, sin)]
    kcd, vcd = dev_cache(kc), dev_cache(vc)
    tol = 2e-3 if kv != "f32" else 1e-4
    outs = {}
    for S in splits:
        print(f"decode attention kv={kv} G={G} pos={list(pos)} kv_split={S}", flush=True)
        outs[S] = binding.debug_decode_attention(dev[0], pos, dev[1], dev[2], dev[3], dev[4], kcd, vcd, nq, nkv, eps,
                                                 kv, S).cpu().numpy()
        err = float(np.max(np.abs(outs[S] - ref)))
        print(f"  max|out - oracle| {err:.3e} (tol {tol:.1e})", flush=True)
        assert np.all(np.isfinite(outs[S])) and err <= tol, err
    for S in splits[1:]:
        cross = float(np.max(np.abs(outs[S] - outs[splits[0]])))
        assert cross <= 1e-5, (S, cross)


def _ref_decode_two_tokens(qkv, pos, kc, vc, q_gain, k_gain, cos, sin, nq, nkv, eps, kv):
    """Per row r: tokens 0 and 1 (qkv rows 2 r, 2 r + 1) at positions pos[r]
    and pos[r] + 1, each normed, roped and its key and value rounded to the
    cache type as in the one-token reference; token 0 attends over the cached
    positions and itself, token 1 also over token 0's key and value."""
    d = qkv.shape[1] // (nq + 2 * nkv)
    out = np.empty((qkv.shape[0], nq * d))
    for r in range(len(pos)):
        p = int(pos[r])
        K, V = kc[r, :, :p], vc[r, :, :p]
        for t in range(2):
            x = qkv[2 * r + t:2 * r + t + 1].astype(np.float64)
            q = x[:, :nq * d].reshape(1, nq, d)
            k = x[:, nq * d:(nq + nkv) * d].reshape(1, nkv, d)
            v = x[:, (nq + nkv) * d:].reshape(1, nkv, d)
            q = model.apply_rope(model.rms_norm(q, q_gain, eps, np.float64), [p + t], cos, sin, np.float64)
            k = _cache_round(model.apply_rope(model.rms_norm(k, k_gain, eps, np.float64), [p + t], cos, sin,
                                              np.float64), kv)
            K = np.concatenate([K, k.transpose(1, 0, 2)], axis=1)
            V = np.concatenate([V, _cache_round(v, kv).transpose(1, 0, 2)], axis=1)
            out[2 * r + t] = model.attention(q, K, V, [p + t], nkv, np.float64).reshape(nq * d)
    return out


@pytest.mark.parametrize("kv", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("pos,nkv,G,max_pos", [
    ([0, 0, 0, 0], 8, 2, 16),
    ([0], 8, 2, 16),
    ([3, 9, 14], 8, 2, 16),
    ([0, 40, 130], 8, 2, 160),
    ([5, 33], 4, 4, 64),
])
def test_decode_attention_two_tokens_matches_oracle(kv, pos, nkv, G, max_pos):
    """The code predictor's two-token pass as a decode step of two new
    tokens per row (positions pos and pos + 1; the second attends to the
    first's key and value): several rows at position 0 (the short kernel with
    both tokens in one block), one row, rows with cached keys up to the
    16-position limit, longer contexts and 4 q heads per kv head (the general
    kernel); against the float64 oracle, tolerance as for one token."""
    torch = _torch()
    nq, d, eps = nkv * G, 128, 1e-6
    pos = np.array(pos, dtype=np.int32)
    B = len(pos)
    rng = np.random.default_rng(int(pos.sum()) + 13 * G + 5 * B + {"f16": 0, "bf16": 1, "f32": 2}[kv])
    qkv = rng.standard_normal((2 * B, (nq + 2 * nkv) * d)).astype(np.float32)
    q_gain = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    k_gain = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    cos, sin = model.rope_tables(max_pos, d, 1.0e6)
    kc = _cache_round(rng.standard_normal((B, nkv, max_pos, d)), kv)
    vc = _cache_round(rng.standard_normal((B, nkv, max_pos, d)), kv)
    ref = _ref_decode_two_tokens(qkv, pos, kc, vc, q_gain, k_gain, cos, sin, nq, nkv, eps, kv)

    def dev_cache(x):
        if kv == "f16":
            return torch.from_numpy(x.astype(np.float16)).cuda()
        if kv == "bf16":
            return torch.from_numpy(synth.bf16_bits(x.astype(np.float32)).view(np.int16)).cuda()
        return torch.from_numpy(x.astype(np.float32)).cuda()

    dev = [torch.from_numpy(a).cuda() for a in (qkv, q_gain, k_gain, cos, sin)]
    print(f"two-token decode attention kv={kv} G={G} pos={list(pos)} max_pos={max_pos}", flush=True)
    out = binding.debug_decode_attention(dev[0], pos, dev[1], dev[2], dev[3], dev[4], dev_cache(kc), dev_cache(vc),
                                         nq, nkv, eps, kv, 1, ntok=2).cpu().numpy()
    err = float(np.max(np.abs(out - ref)))
    tol = 2e-3 if kv != "f32" else 1e-4
    print(f"  max|out - oracle| {err:.3e} (tol {tol:.1e})", flush=True)
    assert np.all(np.isfinite(out)) and err <= tol, err
