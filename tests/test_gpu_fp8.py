"""GPU parity of the FP8 forward (fa_fp8_quantize + fa_fwd_fp8; MI355X only).

Two layers, each against the oracle (``oracle.fp8``) on the same seeded
inputs and signs:

* Quantisation, bit-exact: the rotation runs in float32 in the same butterfly
  order on both sides and E4M3 rounding is to nearest even, so every code of
  rows < N and every block exponent must be identical; rows past N (the
  padding of the last 64-row block) must be zeros of either sign.  The V codes
  are compared after undoing the transposed tile layout the header documents.
* Attention: LSE within the stated LSE tolerance, plus the matrix-core term
  below, of the oracle's exact attention on the dequantised tensors (row sums
  are float32 on the GPU); O row by row within a bound derived from the
  roundings the oracle does not model.  First, the probabilities are rounded
  to E4M3 before the P V product.  A probability p (in units of the kernel's
  running reference, which lies within 8 binades below the row maximum)
  rounds with relative error at most 2^-4, or absolute error at most 2^-10
  where E4M3 is subnormal; in units of the normalised weights w that is
  |dw_i| <= 2^-4 w_i + 2^-10 w_max.  Treating the rounding errors as
  independent and zero-mean, the error vector of a row has norm about
  sigma = sqrt(sum_i (2^-4 w_i)^2 |v_i|^2 + (2^-10 w_max)^2 sum_i |v_i|^2)
  or below (v_i the dequantised rotated value rows; the rotation back is
  orthogonal and keeps norms).  The test allows 2 sigma plus the output
  dtype's rounding; an emulation of the kernel's rounding on the CPU stayed
  below 0.9 sigma on every row of comparable inputs.
* The FP8 matrix instruction does not sum its 64 products exactly: measured
  on the device, it aligns them to the largest and keeps about 13 to 15
  fraction bits (truncating toward -inf), while the accumulator input is
  added exactly -- errors up to 2^-12 of the largest product of one
  instruction were seen.  With EPS_ACC = 2^-11, a score of row i is off by at
  most dS_i = scale * EPS_ACC * (d / 64) * max|q_i| * max|k| (in rotated,
  dequantised units), which moves LSE by at most dS_i and O by at most
  2 dS_i sum_j w_j |v_j|; the P V instruction adds EPS_ACC sum_j w_j |v_j|.
  Both terms are added to the bounds above.

It also checks the pages' claim on the GPU result: on inputs with outlier
channels the method's error against exact attention is well below that of
per-tensor FP8 (computed by the oracle), and reports both."""

import numpy as np
import pytest
import torch

from io_aware_exact_fwd_amd import fa_fwd_fp8, fp8_quantize, fp8_workspace_views
from io_aware_exact_fwd_amd.workloads import (WORKLOADS, make_inputs, make_outlier_inputs,
                                              make_rising_inputs, make_signs)
from oracle import attention_forward
from oracle.attention import visibility
from oracle.fp8 import (E4M3_MAX, block_dequantize, block_quantize, e4m3_decode, e4m3_encode,
                        fp8_attention_forward, rotate_rows_f32)

from gpu_util import LSE_TOL, say, to_np

pytestmark = pytest.mark.gpu

OUT_EPS = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
EPS_ACC = 2.0 ** -11


def _kappa():
    """Key of byte p of a V codes tile row (the header's layout)."""
    p = np.arange(64)
    h, i = p // 32, p % 32
    return 32 * (i // 16) + 8 * ((i % 16) // 4) + 4 * h + i % 4


def _v_rowmajor(vc):
    """(heads, N64 / 64, d, 64) tile layout -> (heads, N64, d) row-major."""
    hk, nt, d, _ = vc.shape
    out = np.zeros((hk, nt, 64, d), dtype=vc.dtype)
    out[:, :, _kappa(), :] = vc.transpose(0, 1, 3, 2)
    return out.reshape(hk, nt * 64, d)


TINY = {"tiny": 2.0 ** -120, "small": 2.0 ** -95}  # magnitudes near float32 underflow


def _inputs(kind, B, H, hkv, N, d, dtype, qmul=1.0):
    gen = {"outlier": make_outlier_inputs, "rising": make_rising_inputs}.get(kind, make_inputs)
    q, k, v, _ = gen(B, H, N, d, dtype, hkv=hkv)
    if qmul != 1.0:
        q = (q.float() * qmul).to(q.dtype)
    if kind in TINY:
        q, k, v = ((x.float() * TINY[kind]).to(x.dtype) for x in (q, k, v))
    return q, k, v


def _check_codes(name, got_codes, got_exps, x, signs, N, vlayout=False, heads=None):
    """Codes of rows < N and all exponents bit-exact; padding codes zero."""
    xs = x.float().numpy()
    hs = x.shape[0] * x.shape[1]
    xs = xs.reshape(hs, N, -1)
    sel = range(hs) if heads is None else heads
    codes = got_codes if not vlayout else _v_rowmajor(got_codes)
    for h in sel:
        want_c, want_e = block_quantize(rotate_rows_f32(xs[h], signs))
        assert np.array_equal(got_exps[h], want_e), (name, h, "exponents")
        bad = np.argwhere(codes[h, :N] != want_c[:N])
        assert bad.size == 0, (name, h, "codes", bad[:5], codes[h, :N][tuple(bad[0])],
                               want_c[:N][tuple(bad[0])])
        assert np.all((codes[h, N:] & 0x7F) == 0), (name, h, "padding")


def _row_sigma(qd, kd, vd, rows, scale, causal, window, lse_ref):
    """sigma of the module docstring for the given rows of one head, and
    sum_j w_j |v_j| of the same rows."""
    n = kd.shape[0]
    s = (qd[rows] @ kd.T) * scale
    vis = visibility(rows, np.arange(n), causal, window=window)
    w = np.where(vis, np.exp(np.where(vis, s, 0.0) - lse_ref[rows, None]), 0.0)
    vn2 = (vd ** 2).sum(1)
    sig = np.sqrt(((2.0 ** -4 * w) ** 2) @ vn2 + (2.0 ** -10 * w.max(1)) ** 2 * vn2.sum())
    return sig, w @ np.sqrt(vn2)


def _check_attention(name, o_g, lse_g, o_ref, lse_ref, quant, dtype, scale, causal, window,
                     group, N, heads, rows=None):
    qc, qe = quant["q"]
    kc, ke = quant["k"]
    vc, ve = quant["v"]
    worst = {"lse": 0.0, "dlse": 0.0, "ratio": 0.0}
    for (b, h) in heads:
        hk = h // group
        qd = block_dequantize(qc[b, h], qe[b, h], N)
        kd = block_dequantize(kc[b, hk], ke[b, hk], N)
        vd = block_dequantize(vc[b, hk], ve[b, hk], N)
        r = np.arange(N) if rows is None else rows
        dl = np.abs(lse_g[b, h, r] - lse_ref[b, h, r])
        worst["dlse"] = max(worst["dlse"], float(dl.max()))
        sig, wv = _row_sigma(qd, kd, vd, r, scale, causal, window, lse_ref[b, h])
        ds = scale * EPS_ACC * (qd.shape[1] // 64) * np.abs(qd[r]).max(1) * np.abs(kd).max()
        lse_bound = LSE_TOL + ds
        worst["lse"] = max(worst["lse"], float((dl / lse_bound).max()))
        on = np.linalg.norm(o_ref[b, h, r], axis=1)
        err = np.linalg.norm(o_g[b, h, r] - o_ref[b, h, r], axis=1)
        bound = 2.0 * sig + (2.0 * ds + EPS_ACC) * wv + OUT_EPS[dtype] * on + 1e-4
        worst["ratio"] = max(worst["ratio"], float((err / bound).max()))
        bad = np.argmax(err / bound)
        assert err[bad] <= bound[bad], (name, (b, h), int(r[bad]), float(err[bad]),
                                        float(bound[bad]), float(sig[bad]))
    say(f"[case] {name}: max|dLSE| {worst['dlse']:.2e} (max ratio to its bound "
        f"{worst['lse']:.3f}), O: max err/bound {worst['ratio']:.3f}")
    assert worst["lse"] <= 1.0, (name, worst)


CASES = [
    # kind, dtype, d, B, H, hkv, N, causal, window, qmul
    ("normal", "f16", 64, 1, 2, 2, 1, True, 0, 1.0),          # one row, one key
    ("outlier", "bf16", 64, 2, 4, 2, 100, False, 0, 1.0),     # ragged single tile, grouped
    ("outlier", "f16", 128, 1, 3, 1, 257, True, 0, 1.0),      # ragged, multi-query, d = 128
    ("normal", "bf16", 128, 1, 2, 2, 1000, False, 0, 1.0),    # several tiles, non-causal
    ("normal", "f16", 64, 1, 2, 1, 130, True, 0, 1.0),        # a query wave wholly past N64
    ("outlier", "bf16", 64, 1, 4, 4, 1500, True, 300, 1.0),   # causal window
    ("normal", "f16", 128, 1, 2, 2, 700, False, 100, 1.0),    # two-sided window
    ("normal", "bf16", 64, 1, 2, 2, 1024, True, 0, 6.0),      # peaked rows: the lazy reference moves
    ("rising", "f16", 64, 1, 2, 2, 1000, True, 0, 1.0),       # the reference moves from a finite value
    ("rising", "bf16", 128, 1, 2, 1, 1000, False, 0, 1.0),
    ("normal", "f16", 128, 2, 2, 1, 640, False, 0, 4.0),
    ("tiny", "bf16", 128, 1, 2, 2, 200, True, 0, 1.0),      # block exponents at the -127 floor
    ("small", "bf16", 64, 1, 2, 2, 200, False, 0, 1.0),     # exponents near -100
]


@pytest.mark.parametrize("kind,dtype,d,B,H,hkv,N,causal,window,qmul", CASES)
def test_fp8_matches_oracle(kind, dtype, d, B, H, hkv, N, causal, window, qmul):
    name = f"{kind} {dtype} d={d} B={B} H={H} H_kv={hkv} N={N} causal={causal} window={window}"
    say(f"[case] {name}")
    q, k, v = _inputs(kind, B, H, hkv, N, d, dtype, qmul)
    signs = make_signs(d, seed=11 + d)
    scale = 1.0 / np.sqrt(d)
    dev = torch.device("cuda:0")
    qd, kd, vd, sd = (t.to(dev) for t in (q, k, v, signs))
    _, ws = fp8_quantize(qd, kd, vd, sd, causal, scale, window)
    o, lse = fa_fwd_fp8(qd, kd, vd, sd, causal, scale, window, workspace=ws)
    torch.cuda.synchronize()
    views = {nm: t.cpu().numpy() for nm, t in fp8_workspace_views(ws, B, H, hkv, N, d).items()}
    s_np = signs.numpy()
    _check_codes(name + " Q", views["qc"], views["qe"], q, s_np, N)
    _check_codes(name + " K", views["kc"], views["ke"], k, s_np, N)
    _check_codes(name + " V", views["vc"], views["ve"], v, s_np, N, vlayout=True)

    o_ref, lse_ref, quant = fp8_attention_forward(*(x.float().numpy() for x in (q, k, v)), scale,
                                                  s_np, causal, window)
    o_g, lse_g = to_np(o), to_np(lse)
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(lse_g)), name
    heads = [(b, h) for b in range(B) for h in range(H)]
    _check_attention(name, o_g, lse_g, o_ref, lse_ref, quant, dtype, scale, causal, window,
                     H // hkv, N, heads)


def _draw_fp8(i):
    """Seeded random FP8 problems: input kind, dtype, head dim, grouped heads,
    ragged lengths, causal or not, windows, peaked rows."""
    rng = np.random.default_rng(80000 + i)
    kind = str(rng.choice(["normal", "outlier", "rising"]))
    dtype = str(rng.choice(["f16", "bf16"]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2]))
    H = hkv * int(rng.choice([1, 2, 3]))
    N = int(rng.integers(1, 1600))
    causal = bool(rng.random() < 0.6)
    window = int(rng.choice([0, 0, int(rng.integers(1, 500))]))
    qmul = float(rng.choice([1.0, 1.0, 4.0]))
    return kind, dtype, d, 1, H, hkv, N, causal, window, qmul


@pytest.mark.parametrize("i", list(range(30)))
def test_fp8_random(i):
    test_fp8_matches_oracle(*_draw_fp8(i))

def test_fp8_repeatable():
    """Two calls on the same inputs give the same bits."""
    q, k, v = _inputs("normal", 1, 4, 2, 777, 128, "bf16")
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    sd = make_signs(128).to(dev)
    o1, l1 = fa_fwd_fp8(qd, kd, vd, sd, True)
    o2, l2 = fa_fwd_fp8(qd, kd, vd, sd, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_beats_per_tensor_fp8_on_outliers():
    """Error of the GPU result against exact attention vs that of per-tensor
    FP8 (one scale for the whole tensor, no rotation), on outlier inputs."""
    B, H, N, d = 1, 4, 1024, 64
    q, k, v = _inputs("outlier", B, H, H, N, d, "bf16")
    signs = make_signs(d, seed=3)
    scale = 1.0 / 8.0
    dev = torch.device("cuda:0")
    o, _ = fa_fwd_fp8(*(t.to(dev) for t in (q, k, v, signs)), causal=True, scale=scale)
    torch.cuda.synchronize()
    qn, kn, vn = (x.float().numpy() for x in (q, k, v))
    o_exact, _ = attention_forward(qn, kn, vn, scale, True)

    def per_tensor(x):
        sc = np.abs(x).max() / E4M3_MAX
        return e4m3_decode(e4m3_encode(x / sc)) * sc

    o_pt, _ = attention_forward(per_tensor(qn), per_tensor(kn), per_tensor(vn), scale, True)
    err_gpu = np.linalg.norm(to_np(o) - o_exact) / np.linalg.norm(o_exact)
    err_pt = np.linalg.norm(o_pt - o_exact) / np.linalg.norm(o_exact)
    say(f"[case] outliers: relative error, GPU FP8 with block scales + rotation {err_gpu:.4f}, "
        f"per-tensor FP8 {err_pt:.4f} (ratio {err_pt / err_gpu:.2f})")
    assert err_gpu * 1.5 < err_pt, (err_gpu, err_pt)


def test_fp8_full_size_sampled():
    """The FP8 workload at full size (B=2 H=16 N=8192 d=128 bf16, causal):
    codes of sampled heads bit-exact, LSE and O of sampled rows of two heads
    against the oracle."""
    w = WORKLOADS["long_wide_fp8"]
    B, H, hkv, N, d = w.B, w.H, w.H_kv, w.N, w.d
    name = f"{w.name} full size"
    say(f"[case] {name}")
    q, k, v, _ = make_inputs(B, H, N, d, w.dtype, hkv=hkv)
    signs = make_signs(d)
    dev = torch.device("cuda:0")
    qd, kd, vd, sd = (t.to(dev) for t in (q, k, v, signs))
    _, ws = fp8_quantize(qd, kd, vd, sd, w.causal, w.scale)
    o, lse = fa_fwd_fp8(qd, kd, vd, sd, w.causal, w.scale, workspace=ws)
    torch.cuda.synchronize()
    views = {nm: t.cpu().numpy() for nm, t in fp8_workspace_views(ws, B, H, hkv, N, d).items()}
    s_np = signs.numpy()
    heads = [0, B * H - 1]
    _check_codes(name + " Q", views["qc"], views["qe"], q, s_np, N, heads=heads)
    _check_codes(name + " K", views["kc"], views["ke"], k, s_np, N, heads=[0, B * hkv - 1])
    _check_codes(name + " V", views["vc"], views["ve"], v, s_np, N, vlayout=True,
                 heads=[0, B * hkv - 1])
    sample = [(0, 0), (B - 1, H - 1)]
    o_s, lse_s, quant = fp8_attention_forward(*(x.float().numpy() for x in (q, k, v)),
                                              w.scale, s_np, w.causal, heads=sample)
    o_ref = np.zeros((B, H, N, d))
    lse_ref = np.zeros((B, H, N))
    for i, (b, h) in enumerate(sample):  # the oracle stacks the selected heads
        o_ref[b, h], lse_ref[b, h] = o_s[i], lse_s[i]
    rows = np.unique(np.concatenate([np.arange(0, 130), np.arange(N - 130, N),
                                     np.random.default_rng(0).integers(0, N, 256)]))
    _check_attention(name, to_np(o), to_np(lse), o_ref, lse_ref, quant, w.dtype, w.scale,
                     w.causal, 0, H // hkv, N, sample, rows=rows)
