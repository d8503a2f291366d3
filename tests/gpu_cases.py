"""Shared helpers of the GPU parity tests: build the same cache on the GPU
(through the C ABI) and in the CPU oracle from the same seeded inputs, and
compare the two."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from bit_quantized_kv_amd import inputs, kvq

# Attention tolerance (one bar per path; see the derivations below).
# The oracle attends in fp64 over the exactly dequantized cache.
#  - fp32 output: |gpu - oracle| <= ATOL = 2e-3 everywhere.
#  - bf16 output (the reading of "max-abs-error 2e-3 with bf16 out"): the
#    output rounding alone is up to half a bf16 ulp (3.9e-3 for 1 <= |o| < 2),
#    so where |oracle| < 0.5 (half an ulp is below 1e-3 there) every element
#    must lie within 2e-3 of the oracle, and where |oracle| >= 0.5 within one
#    bf16 ulp of bf16_rne(oracle) and within 2e-3 plus half an ulp of the
#    oracle.  (Below 0.5 an output that results from cancellation can be a few
#    of its own tiny ulps away from the oracle at an absolute error of 1e-7,
#    so the ulp count is not the measure there.)
#  - paths that round each softmax weight to fp16 before the PV product (the
#    fused extend's steps wholly inside the cached prefix): each weight then
#    carries a relative error of at most 2^-11, which moves an output element
#    by at most 2^-11 * sum_t w_t |v_t,c| -- the softmax-weighted mean of |v|,
#    computed by the oracle -- so the bar there is ATOL + 2^-11 * that mean
#    (plus the bf16 output rounding for bf16 output).
# cosine to the oracle >= MIN_COS per (sequence, head); lse within LSE_ATOL.
ATOL = 2e-3
LSE_ATOL = 1e-3
MIN_COS = 0.9995
F16_WEIGHT_REL = 2.0 ** -11


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (nearest even, torch's cast) and widen back to fp64."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float64)).to(torch.bfloat16).double().numpy()


def check_values(out, ref, bf16=False, extra=None, label=""):
    """The element-wise bar above; extra (same shape as ref, or None) is the
    derived fp16-weight term.  Returns (max |gpu - oracle|, largest error / bar)."""
    out = np.asarray(out, np.float64)
    assert np.all(np.isfinite(out)), f"{label}: non-finite output"
    err = np.abs(out - ref)
    tol = np.full(ref.shape, ATOL)
    if extra is not None:
        tol = tol + extra
    if bf16:
        tol = tol + np.where(np.abs(ref) < 0.5, 0.0, bf16_half_ulp(ref))
        if extra is None:
            r = bf16_rne(ref)
            ulp = 2.0 * bf16_half_ulp(r)
            off = (np.abs(ref) >= 0.5) & (np.abs(out - r) > ulp)
            assert not off.any(), (f"{label}: {off.sum()} bf16 elements more than one ulp from bf16_rne(oracle), "
                                   f"first at {np.argwhere(off)[0].tolist()}")
    bad = err > tol
    assert not bad.any(), (f"{label}: {bad.sum()} elements out of tolerance, max err {err.max():.3g} "
                           f"at {np.unravel_index(err.argmax(), err.shape)} (bar there "
                           f"{tol.ravel()[err.argmax()]:.3g})")
    use = float((err / tol).max()) if err.size else 0.0
    print(f"  {label}: max |err| {err.max() if err.size else 0.0:.3g}, max |o| "
          f"{np.abs(ref).max() if ref.size else 0.0:.3g}, largest err / bar {use:.3f}", flush=True)
    return float(err.max()) if err.size else 0.0, use


def kv_rows(kind: str, seed: int, layer: int, n: int, H: int, D: int):
    if kind == "outliers":
        return inputs.kv_outlier_channels(seed, layer, n, H, D)
    if kind == "lognormal":
        return inputs.kv_lognormal_channels(seed, layer, n, H, D)
    if kind == "student_t":
        return inputs.kv_student_t(seed, layer, n, H, D)
    if kind in ("token_scaled", "token_scaled_o1"):
        # Student-t rows, each (token, head) row scaled by its own 2^u: u in
        # [-30, 12] (per-token scales over 42 binades), or u in [-30, 3] (33
        # binades with outputs of order 1 to 10, where an absolute bar is
        # meaningful)
        hi = 13 if kind == "token_scaled" else 4
        k, v = inputs.kv_student_t(seed, layer, n, H, D)
        rng = np.random.default_rng(seed * 1000 + layer)
        k = k * np.exp2(rng.integers(-30, hi, size=(n, H, 1))).astype(np.float32)
        v = v * np.exp2(rng.integers(-30, hi, size=(n, H, 1))).astype(np.float32)
        return k, v
    raise ValueError(kind)


class Case:
    """One layer cache with B sequences of lengths `lens`, stored on both sides."""

    def __init__(self, fmt, D, Hkv, G, P, lens, kind="outliers", in_dtype=torch.float32, gs=(1.0, 1.0),
                 shuffled=True, seed=1, poison=0xFF, extra_pages=3, drop_every=0):
        self.fmt, self.D, self.Hkv, self.G, self.P = fmt, D, Hkv, G, P
        self.lens = np.array(lens, np.int32)
        self.B = len(lens)
        self.Hq = Hkv * G
        self.max_len = int(self.lens.max()) if self.B else 0
        self.pages_per_seq = max(1, -(-self.max_len // P))
        self.num_pages = self.B * self.pages_per_seq + extra_pages
        self.bt = inputs.page_tables(seed, self.B, self.pages_per_seq, self.num_pages, shuffled=shuffled)
        ks, vs, slots = [], [], []
        for b in range(self.B):
            L = int(self.lens[b])
            k, v = kv_rows(kind, seed, b, L, Hkv, D)
            ks.append(k)
            vs.append(v)
            slots.append(inputs.slots_for(self.bt, P, b, 0, L))
        self.k = np.concatenate(ks) if ks else np.zeros((0, Hkv, D), np.float32)
        self.v = np.concatenate(vs) if vs else np.zeros((0, Hkv, D), np.float32)
        self.slots = np.concatenate(slots).astype(np.int32)
        if drop_every:
            self.slots[::drop_every] = -1  # skipped tokens keep the poison bytes
        self.in_dtype = in_dtype
        self.gs = gs
        # GPU side
        dev = torch.device("cuda")
        self.cache = kvq.Cache(fmt, self.num_pages, P, Hkv, D, device=dev, global_scale=gs)
        self.cache.pool.fill_(poison)
        self.k_dev = torch.from_numpy(self.k).to(dev).to(in_dtype)
        self.v_dev = torch.from_numpy(self.v).to(dev).to(in_dtype)
        self.slots_dev = torch.from_numpy(self.slots).to(dev)
        kvq.kvq_quantize_store(self.cache, self.k_dev, self.v_dev, self.slots_dev)
        # oracle side (bf16 inputs are handed over as their exact fp32 values)
        self.ref = oracle.Pool(fmt, self.num_pages, P, Hkv, D, global_scale=gs, fill=poison)
        k_in = self.k_dev.float().cpu().numpy()
        v_in = self.v_dev.float().cpu().numpy()
        self.ref.quantize_store(k_in, v_in, self.slots)
        self.q = inputs.query(seed, 99, self.B, self.Hq, D)
        self.q_dev = torch.from_numpy(self.q).to(dev).to(torch.bfloat16)
        self.bt_dev = torch.from_numpy(self.bt).to(dev)
        self.lens_dev = torch.from_numpy(self.lens).to(dev)

    def gpu_pool(self) -> np.ndarray:
        torch.cuda.synchronize()
        return self.cache.pool.cpu().numpy()

    def decode(self, out_dtype=torch.float32, num_splits=0, bt=None, want_lse=True):
        lse = torch.empty((self.B, self.Hq), dtype=torch.float32, device="cuda") if want_lse else None
        out = kvq.kvq_decode_attention(self.cache, self.q_dev, self.bt_dev if bt is None else bt, self.lens_dev,
                                       self.max_len, lse=lse, num_splits=num_splits, out_dtype=out_dtype)
        torch.cuda.synchronize()
        return out.float().cpu().numpy(), (lse.cpu().numpy() if want_lse else None)

    def oracle_decode(self):
        return self.ref.decode_attention(self.q, self.bt, self.lens)


def check_pool_bitexact(case: Case):
    got = case.gpu_pool()
    ref = case.ref.data
    if not np.array_equal(got, ref):
        diff = np.argwhere(got != ref)
        raise AssertionError(f"{len(diff)} pool bytes differ; first at {diff[:5].tolist()}: "
                             f"gpu {got[tuple(diff[0])]:#x} oracle {ref[tuple(diff[0])]:#x}")


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(np.dot(a.ravel(), b.ravel()) / (na * nb))


def check_attention(out, ref, lens, bf16=False, lse=None, ref_lse=None, label="", extra=None):
    """Element-wise bar (check_values), per-(sequence, head) cosine, lse."""
    err, _ = check_values(out, ref, bf16=bf16, extra=extra, label=label)
    for b in range(out.shape[0]):
        if lens[b] == 0:
            assert np.all(out[b] == 0), f"{label}: empty sequence must give zeros"
            continue
        for h in range(out.shape[1]):
            c = cosine(out[b, h], ref[b, h])
            assert c >= MIN_COS, f"{label}: cosine {c} at ({b},{h})"
    if lse is not None:
        for b in range(out.shape[0]):
            if lens[b] == 0:
                assert np.all(np.isneginf(lse[b])), f"{label}: lse of an empty sequence must be -inf"
            else:
                d = np.abs(lse[b] - ref_lse[b]).max()
                assert d <= LSE_ATOL, f"{label}: lse differs by {d}"
    return err


def check_dequant_prefix(case: Case, stride_extra: int = 0):
    for b in range(case.B):
        L = int(case.lens[b])
        stride = case.Hkv * case.D + stride_extra
        k_out = torch.full((max(L, 1), stride), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        v_out = torch.full((max(L, 1), stride), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        kvq.kvq_dequant_prefix(case.cache, case.bt_dev[b], L, k_out, v_out)
        torch.cuda.synchronize()
        if L == 0:
            continue
        rk, rv = case.ref.dequant_prefix(case.bt[b], L, out_token_stride=stride)
        for got, ref in ((k_out, rk), (v_out, rv)):
            g = got.view(torch.int16).cpu().numpy().view(np.uint16)[:L]
            used = np.zeros(stride, bool)
            used[: case.Hkv * case.D] = True
            assert np.array_equal(g[:, used], ref[:, used]), f"prefix dequant differs for sequence {b}"
            assert np.all(g[:, ~used] == 0x7FC0), "prefix dequant wrote outside its rows"
