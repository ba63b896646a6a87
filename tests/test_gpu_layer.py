"""GPU parity of one spatten_layer_forward call against the oracle on the
same inputs: prefill (fp32 and bf16, bidirectional and causal, with and
without head pruning, ragged token counts) and decode (bf16 cache and
progressive-quantization planes)."""
import math

import numpy as np
import pytest
import torch

from gpu_util import PrefillWs, check_bf16_output, max_err_over_rms, to_dev, to_np
from oracle import spatten_ref as R

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    from cascade_token_head_amd import spatten
    spatten.load()
    return spatten


def _weights(rng, D, bf16):
    w = {}
    for k in ("wq", "wk", "wv", "wo"):
        v = (rng.standard_normal((D, D)) / math.sqrt(D)).astype(np.float32)
        w[k] = R.bf16_round(v).astype(np.float32) if bf16 else v
    return w


def _dev_w(w, dt):
    return {k: to_dev(v.T, dt) for k, v in w.items()}


PREFILL_CASES = [
    # (dtype, B, n, H, h_kept, dh, causal)
    ("f32", 1, 64, 4, 4, 32, False),
    ("f32", 2, 37, 4, 2, 32, False),
    ("f32", 2, 70, 4, 3, 32, True),
    ("bf16", 2, 200, 12, 12, 64, False),
    ("bf16", 2, 512, 12, 10, 64, False),
    ("bf16", 3, 279, 12, 10, 64, False),
    ("bf16", 2, 333, 6, 6, 64, True),
    ("bf16", 1, 300, 4, 3, 128, True),
    ("bf16", 2, 257, 4, 4, 128, False),
    # model dim 192 and 3 kept heads: odd k-tile counts in both projections
    ("bf16", 2, 300, 3, 3, 64, False),
    ("bf16", 1, 200, 5, 3, 64, True),
    # projections large enough for 256x256 GEMM tiles (all heads; kept heads
    # with a sequence length that is not a multiple of the tile)
    ("bf16", 4, 2048, 16, 16, 128, False),
    ("bf16", 3, 1900, 16, 12, 128, False),
    # degenerate shapes: one token, one kept head, tokens fewer than a tile
    ("bf16", 1, 1, 4, 1, 64, False),
    ("bf16", 2, 1, 4, 4, 128, True),
    ("bf16", 3, 17, 2, 1, 64, True),
    ("f32", 1, 1, 2, 2, 32, True),
]


@pytest.mark.parametrize("dt,B,n,H,hk,dh,causal", PREFILL_CASES)
def test_prefill_layer(S, dt, B, n, H, hk, dh, causal):
    print("prefill case", dt, B, n, H, hk, dh, causal, flush=True)
    bf16 = dt == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    rng = np.random.default_rng(B * 1000 + n + H)
    D = H * dh
    x = rng.standard_normal((B, n, D)).astype(np.float32)
    x[:, ::17] *= 3
    if bf16:
        x = R.bf16_round(x).astype(np.float32)
    w = _weights(rng, D, bf16)
    heads = np.stack([np.sort(rng.choice(H, hk, replace=False)) for _ in range(B)]).astype(np.int32)
    a0 = (rng.random((B, n)) * 10).astype(np.float32)
    g0 = (rng.random((B, H)) * 100).astype(np.float32)

    desc = S.make_desc(S.PREFILL, S.BF16 if bf16 else S.F32, causal, B, n, H, hk, dh)
    ws = torch.zeros(S.workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    xd = to_dev(x, tdt)
    wd = _dev_w(w, tdt)
    ad, gd = to_dev(a0, torch.float32), to_dev(g0, torch.float32)
    lse = torch.empty(B, hk, n, device="cuda")
    S.layer_forward(desc, xd, wd["wq"], wd["wk"], wd["wv"], wd["wo"], to_dev(heads, torch.int32),
                    ad, gd, ws, lse=lse)
    torch.cuda.synchronize()
    xo, ao, go, lo = to_np(xd), to_np(ad), to_np(gd), to_np(lse)
    lay = PrefillWs(B, n, hk, dh, 2 if bf16 else 4, bf16)
    es = 2 if bf16 else 4
    o_all = ws[lay.o: lay.o + B * n * hk * dh * es].view(tdt).view(B, n, hk, dh)
    o_all = to_np(o_all)
    # the Q and K the attention kernels read (bf16 rounding on the two sides
    # is independent, and at D in the thousands an occasional one-step
    # difference in q moves a row's scores: the row LSE is checked on the
    # GPU's own Q, K)
    q_all = to_np(ws[lay.q: lay.q + B * hk * lay.n_pad * dh * es].view(tdt)
                  .view(B, hk, lay.n_pad, dh))
    k_all = to_np(ws[lay.k: lay.k + B * hk * lay.n_pad * dh * es].view(tdt)
                  .view(B, hk, lay.n_pad, dh))
    for b in range(B):
        ex = {}
        xr, dcol, dg, lr = R.prefill_layer(x[b], w, heads[b], dh, causal, bf16, extras=ex)
        if bf16:
            e = check_bf16_output(xo[b], xr, what="x_out b=%d" % b)
            print("x_out b=%d nrmse %.3g max/rms %.3g" % (b, e[0], e[1]))
            for s, h in enumerate(heads[b]):
                check_bf16_output(o_all[b, :, s], ex[h]["o"], what="O b=%d h=%d" % (b, h))
        else:
            assert np.max(np.abs(xo[b] - xr)) <= 1e-4
            for s, h in enumerate(heads[b]):
                assert np.max(np.abs(o_all[b, :, s] - ex[h]["o"])) <= 1e-4
        da = ao[b] - a0[b]
        assert abs(da.sum() - hk * n) <= 1e-5 * hk * n
        # free running (the oracle's own Q, K): close in the RMS sense
        assert max_err_over_rms(da, dcol) <= (1e-3 if bf16 else 1e-5), max_err_over_rms(da, dcol)
        col_g = np.zeros(n)
        for s, h in enumerate(heads[b]):
            assert abs((go[b, h] - g0[b, h]) - dg[h]) <= (5e-3 if bf16 else 1e-5) * dg[h]
            Qg = q_all[b, s, :n].astype(np.float64)
            Kg = k_all[b, s, :n].astype(np.float64)
            _, cg, lg = R.head_attention(Qg, Kg, np.zeros((n, 1)), causal)
            col_g += cg
            np.testing.assert_allclose(lo[b, s], lg, rtol=5e-4 if bf16 else 1e-6,
                                       atol=1e-3 if bf16 else 2e-5)
        # on the GPU's own Q, K: fp32 column sums of h*n probabilities, the
        # stored a rounding at its own magnitude and ~1e-5 relative per sum
        tol = (2e-5 if bf16 else 2e-6) * np.max(np.abs(ao[b])) + 1e-5 * np.abs(col_g)
        assert np.all(np.abs(da - col_g) <= tol), np.max(np.abs(da - col_g) - tol)
        for h in set(range(H)) - set(heads[b].tolist()):
            assert go[b, h] == g0[b, h]


VPRUNE_PREFILL_CASES = [
    # (dtype, B, n, H, h_kept, dh, causal, tau)
    ("bf16", 2, 300, 12, 10, 64, False, 1e-3),
    ("bf16", 2, 333, 6, 6, 64, True, 2e-3),
    ("bf16", 1, 300, 4, 3, 128, True, 1e-3),
    ("bf16", 2, 257, 4, 4, 128, False, 5e-3),
    ("bf16", 1, 1, 4, 1, 64, False, 0.5),
    ("f32", 2, 70, 4, 3, 32, True, 1e-2),
    ("f32", 1, 64, 4, 4, 32, False, 0.05),
]


@pytest.mark.parametrize("dt,B,n,H,hk,dh,causal,tau", VPRUNE_PREFILL_CASES)
def test_prefill_layer_value_pruning(S, dt, B, n, H, hk, dh, causal, tau):
    """Local value pruning in prefill ("A. Cascade Token Pruning", bullet
    "Local Value Pruning"): on the GPU's own Q, K, V every head output must
    equal sum over P[i, j] >= tau of P[i, j] V[j] (fp64 P), up to the
    storage tolerance plus, per element, the weight of the V rows whose
    probability lies within 1e-4 (relative) of tau, where the fp32 and fp64
    decisions may differ; token importance still takes every probability,
    head importance the pruned output."""
    print("prefill vprune case", dt, B, n, H, hk, dh, causal, tau, flush=True)
    bf16 = dt == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    es = 2 if bf16 else 4
    rng = np.random.default_rng(B * 7000 + n + H)
    D = H * dh
    x = rng.standard_normal((B, n, D)).astype(np.float32)
    x[:, ::13] *= 3
    if bf16:
        x = R.bf16_round(x).astype(np.float32)
    w = _weights(rng, D, bf16)
    heads = np.stack([np.sort(rng.choice(H, hk, replace=False)) for _ in range(B)]).astype(np.int32)
    a0 = np.zeros((B, n), np.float32)
    g0 = np.zeros((B, H), np.float32)
    desc = S.make_desc(S.PREFILL, S.BF16 if bf16 else S.F32, causal, B, n, H, hk, dh,
                       v_threshold=tau)
    ws = torch.zeros(S.workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    xd, wd = to_dev(x, tdt), _dev_w(w, tdt)
    ad, gd = to_dev(a0, torch.float32), to_dev(g0, torch.float32)
    S.layer_forward(desc, xd, wd["wq"], wd["wk"], wd["wv"], wd["wo"], to_dev(heads, torch.int32),
                    ad, gd, ws)
    torch.cuda.synchronize()
    xo, ao, go = to_np(xd), to_np(ad), to_np(gd)
    lay = PrefillWs(B, n, hk, dh, es, bf16)
    npd = lay.n_pad
    o_all = to_np(ws[lay.o: lay.o + B * n * hk * dh * es].view(tdt).view(B, n, hk, dh))
    q_all = to_np(ws[lay.q: lay.q + B * hk * npd * dh * es].view(tdt).view(B, hk, npd, dh))
    k_all = to_np(ws[lay.k: lay.k + B * hk * npd * dh * es].view(tdt).view(B, hk, npd, dh))
    vt_all = to_np(ws[lay.vt: lay.vt + B * hk * npd * dh * es].view(tdt).view(B, hk, dh, npd))
    kept = total = 0
    for b in range(B):
        col = np.zeros(n)
        xr = x[b].astype(np.float64)
        delta = np.zeros((n, D))
        for s_, h in enumerate(heads[b]):
            Q, K = q_all[b, s_, :n], k_all[b, s_, :n]
            V = vt_all[b, s_, :, :n].T
            masked = causal & (np.arange(n)[None, :] > np.arange(n)[:, None])
            P = R.softmax_rows(np.where(masked, -np.inf, Q @ K.T / math.sqrt(dh)))
            keepm = P >= tau
            kept += int(keepm.sum())
            total += int((P > 0).sum())
            Oref = np.where(keepm, P, 0.0) @ V
            band = np.abs(P - tau) <= 1e-4 * tau
            allow = (np.where(band, P, 0.0) @ np.abs(V)) if band.any() else 0.0
            got = o_all[b, :, s_]
            stor = (np.abs(Oref) * 2.0 ** -8 + 1e-6) if bf16 else 1e-5
            err = np.abs(got - Oref) - allow - stor
            assert np.all(err <= 2e-2 * np.sqrt(np.mean(Oref ** 2)) + 1e-6), (
                "O b%d h%d: max excess %.3g" % (b, h, err.max()))
            col += P.sum(axis=0)
            gh = go[b, h] - g0[b, h]
            assert abs(gh - np.abs(got).sum()) <= 1e-3 * max(np.abs(got).sum(), 1e-6), (b, h)
            delta += (R.bf16_round(got) if bf16 else got) @ w["wo"][h * dh:(h + 1) * dh, :]
        np.testing.assert_allclose(ao[b] - a0[b], col, rtol=1e-4, atol=2e-5 * max(col.max(), 1))
        xref = R.bf16_round(xr + delta) if bf16 else xr + delta
        if bf16:
            check_bf16_output(xo[b], xref, what="x_out b=%d" % b)
        else:
            assert np.max(np.abs(xo[b] - xref)) <= 1e-4
    print("V entries kept %d of %d" % (kept, total), flush=True)
    if tau < 0.5:
        assert 0 < kept < total


def _decode_setup(rng, B, H, dh, L0, cap, quantized):
    D = H * dh
    K0 = R.bf16_round(rng.standard_normal((B, L0, D)) * rng.choice([1.0, 3.0], (B, L0, 1)))
    V0 = R.bf16_round(rng.standard_normal((B, L0, D)) * rng.choice([1.0, 3.0], (B, L0, 1)))
    return K0.astype(np.float32), V0.astype(np.float32)


DECODE_LAYER_CASES = [
    (3, 12, 100, False, 0.0), (2, 12, 1024, False, 0.0), (4, 16, 300, True, 0.1),
    (2, 16, 257, True, 0.0), (2, 16, 257, True, 1.01), (64, 12, 130, False, 0.0),
    # empty cache before the step (the new row is the only key)
    (1, 12, 0, False, 0.0), (2, 16, 0, True, 0.1),
    # the most heads the decode path takes, a new row opening a 32-row chunk
    (2, 32, 64, False, 0.0), (2, 32, 96, True, 0.1),
    # one head; an odd head count with a partial last wave
    (3, 1, 40, False, 0.0), (1, 5, 31, True, 0.05),
    # batches past the 64-row decode projection kernel (tiled GEMM fallback)
    (65, 12, 50, False, 0.0), (96, 16, 33, True, 0.1)]
# local value pruning: (B, H, L0, v_threshold). Threshold 0.5 keeps at most
# one V row per head, 1.01 keeps none (O = 0), and an empty cache's only row
# (p = 1) is kept.
VPRUNE_CASES = [(3, 12, 100, 1e-3), (2, 12, 1024, 1e-4), (64, 12, 130, 1e-2),
                (2, 32, 64, 2e-2), (3, 1, 40, 3e-2), (1, 5, 31, 5e-2), (65, 12, 50, 1e-2),
                (2, 12, 100, 0.5), (2, 12, 100, 1.01), (1, 12, 0, 0.5),
                # past the 4096 rows one workgroup holds: the split path
                (2, 12, 4200, 1e-4), (3, 5, 5000, 1e-3)]


# per-head importance (a is [B, H, cap]): (B, H, L0, v_threshold)
PERHEAD_CASES = [(3, 12, 100, 0.0), (2, 16, 257, 0.0), (64, 12, 130, 0.0), (1, 5, 31, 0.0),
                 (2, 12, 300, 1e-3), (2, 12, 4200, 1e-4)]


# per-head importance with quantized caches, whose scales are then per (head,
# slot): (B, H, L0, threshold)
PERHEAD_PQ_CASES = [(3, 16, 200, 0.1), (2, 12, 150, 1.01), (2, 16, 301, 0.0)]
# value pruning with quantized caches: (B, H, L0, threshold, v_threshold,
# per_head)
PQ_VPRUNE_CASES = [(3, 16, 200, 0.1, 1e-3, False), (2, 12, 300, 1.01, 2e-3, False),
                   (2, 16, 257, 0.0, 1e-2, False), (2, 16, 301, 0.1, 1e-3, True),
                   (1, 16, 4000, 0.1, 1e-4, False), (2, 16, 0, 0.1, 0.5, False)]


@pytest.mark.parametrize("B,H,L0,quantized,thr,vthr,per_head",
                         [c + (0.0, False) for c in DECODE_LAYER_CASES] +
                         [(B, H, L0, False, 0.0, v, False) for B, H, L0, v in VPRUNE_CASES] +
                         [(B, H, L0, False, 0.0, v, True) for B, H, L0, v in PERHEAD_CASES] +
                         [(B, H, L0, True, t, 0.0, True) for B, H, L0, t in PERHEAD_PQ_CASES] +
                         [(B, H, L0, True, t, v, ph) for B, H, L0, t, v, ph in PQ_VPRUNE_CASES])
def test_decode_layer(S, B, H, L0, quantized, thr, vthr, per_head):
    print("decode case", B, H, L0, quantized, thr, vthr, per_head, flush=True)
    dh = 64
    D = H * dh
    rng = np.random.default_rng(B * 10 + L0)
    cap = L0 + 5
    K0, V0 = _decode_setup(rng, B, H, dh, L0, cap, quantized)
    w = _weights(rng, D, True)
    x = R.bf16_round(rng.standard_normal((B, D))).astype(np.float32)
    a0 = np.zeros((B, H, cap) if per_head else (B, cap), np.float32)
    a0[..., :L0] = rng.random(a0[..., :L0].shape) * 5
    desc = S.make_desc(S.DECODE, S.BF16, False, B, 1, H, H, dh, L0, cap, quantized, thr, vthr,
                       per_head)
    ws = torch.zeros(S.workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    wd = _dev_w(w, torch.bfloat16)
    xd = to_dev(x.reshape(B, 1, D), torch.bfloat16)
    ad = to_dev(a0, torch.float32)
    gd = torch.zeros(B, H, device="cuda")
    hidx = torch.arange(H, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    rec = torch.full((B, H), -1, dtype=torch.int32, device="cuda")
    vk = torch.full((B, H), -1, dtype=torch.int32, device="cuda")
    kw = {}
    # per-head slots of a quantized cache: head h's slot r holds token
    # (r + h) mod L0, with that token's planes and scale, so each head reads
    # its own scale row
    ph_tok = (np.arange(L0)[:, None] + np.arange(H)[None, :]) % L0     # [slot, head]
    ph_cache = {}
    if quantized and per_head:
        for name, arr in (("k", K0), ("v", V0)):
            msb = np.zeros((B, H, cap, dh // 2), np.uint8)
            lsb = np.zeros_like(msb)
            sc = np.zeros((B, H, cap), np.float32)
            for b in range(B):
                m_, l_, s_ = R.quantize_kv(arr[b])
                m_ = m_.reshape(L0, H, dh // 2)[ph_tok, np.arange(H)[None, :]]   # [L0, H, dh/2]
                l_ = l_.reshape(L0, H, dh // 2)[ph_tok, np.arange(H)[None, :]]
                s_ = s_[ph_tok]                                                  # [L0, H]
                msb[b, :, :L0] = m_.transpose(1, 0, 2)
                lsb[b, :, :L0] = l_.transpose(1, 0, 2)
                sc[b, :, :L0] = s_.T
                ph_cache.setdefault(b, {}).update(
                    {name + "_msb": m_, name + "_lsb": l_, name + "_scale": s_})
            kw.update({name + "_msb": torch.from_numpy(msb).cuda(),
                       name + "_lsb": torch.from_numpy(lsb).cuda(),
                       name + "_scale": torch.from_numpy(sc).cuda()})
    elif quantized:
        for name, arr in (("k", K0), ("v", V0)):
            msb = torch.zeros(B, H, cap, dh // 2, dtype=torch.uint8, device="cuda")
            lsb = torch.zeros_like(msb)
            sc = torch.zeros(B, cap, device="cuda")
            S.quantize_kv(to_dev(arr, torch.bfloat16), msb, lsb, sc)
            kw.update({name + "_msb": msb, name + "_lsb": lsb, name + "_scale": sc})
    else:
        kc = torch.zeros(B, cap, D, dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        kc[:, :L0] = to_dev(K0, torch.bfloat16)
        vc[:, :L0] = to_dev(V0, torch.bfloat16)
        kw.update({"k_cache": kc, "v_cache": vc})
    S.layer_forward(desc, xd, wd["wq"], wd["wk"], wd["wv"], wd["wo"], hidx, ad, gd, ws,
                    recompute=rec, v_kept=vk, **kw)
    torch.cuda.synchronize()
    xo, ao, rc = to_np(xd).reshape(B, D), to_np(ad), rec.cpu().numpy()
    vkept = vk.cpu().numpy()
    assert float(gd.abs().sum()) == 0.0
    n_rec = 0
    for b in range(B):
        if quantized and per_head:
            cache = dict(ph_cache[b])
            # the new row's scale went to every head's slot L0
            for name in ("k_scale", "v_scale"):
                col = kw[name][b, :, L0].cpu().numpy()
                assert np.all(col == col[0]) and col[0] > 0, (name, b, col)
        elif quantized:
            cache = {}
            for name, arr in (("k", K0), ("v", V0)):
                m_, l_, s_ = R.quantize_kv(arr[b])
                cache.update({name + "_msb": m_, name + "_lsb": l_, name + "_scale": s_})
        else:
            cache = {"k": K0[b].reshape(L0, H, dh).astype(np.float64),
                     "v": V0[b].reshape(L0, H, dh).astype(np.float64)}
        xr, P, recr, cmax, kr = R.decode_layer(x[b], w, cache, H, dh, True, quantized, thr,
                                               v_threshold=vthr)
        # V rows kept: equal to the oracle's count but for probabilities
        # within 2% of the threshold, where the bf16 rounding of q and k on
        # the two sides may put a row on either side
        band = np.sum(np.abs(P - vthr) <= 2e-2 * vthr, axis=1) if vthr > 0 else 0
        assert np.all(np.abs(vkept[b] - kr) <= band), (b, vkept[b], kr)
        if quantized:
            for h in range(H):
                if abs(cmax[h] - thr) > 1e-5 * thr:
                    assert bool(rc[b, h]) == bool(recr[h]), (b, h, cmax[h])
                else:
                    pytest.skip("near-threshold row; decision adopted in stack tests")
            n_rec += int(recr.sum())
        else:
            assert np.all(rc[b] == 0)
        check_bf16_output(xo[b], xr, what="decode x_out b=%d" % b)
        if per_head:
            # each head's row of a takes that head's probabilities only
            da = ao[b, :, :L0 + 1] - a0[b, :, :L0 + 1]
            np.testing.assert_allclose(da, P, atol=2e-3 / (L0 + 1) + 1e-6, rtol=2e-2)
            np.testing.assert_allclose(da.sum(axis=1), 1.0, atol=1e-4)
            assert np.all(ao[b, :, L0 + 1:] == 0)
        else:
            da = ao[b, :L0 + 1] - a0[b, :L0 + 1]
            np.testing.assert_allclose(da, P.sum(axis=0), atol=2e-3 * H / (L0 + 1) + 1e-6,
                                       rtol=2e-2)
            assert abs(da.sum() - H) <= 1e-4 * H
            assert np.all(ao[b, L0 + 1:] == 0)
    if quantized and thr == 0.0:
        assert n_rec == 0
    if quantized and thr > 1:
        assert n_rec == B * H
