"""Unit parity of the chunk-prep kernel (kda_prefill_varlen_prep): every
tensor it writes to the workspace against the fp64 chunked reference
(tests/chunk_ref.py, itself pinned to the oracle on the CPU).

"Kimi K3: The Manos, The Mythos, The Legendos", section "FlashKDA
algorithm": the first kernel prepares, per chunk, the cumulative decay, the
decayed K K^T and Q K^T blocks, the UT-transform inverse and the W / U
pseudo-value tensors.  The workspace holds, per (head, chunk slot),
  W = INV diag(beta) (k e^a), Q^ = q e^a, K-bar^T = (k e^{a_last - a})^T,
  U~^T = (INV diag(beta) v)^T, M (decayed Q K^T, lower incl. diagonal),
  gamma = e^{a_last}
(INV and A live in LDS only).  The layout is decoded here from its
definition (16 x 32 bf16 MFMA-operand fragments, stored lane by lane; U~^T
in 16 x 16 fragments of 8 bytes per lane).  Tolerances: 2e-2 relative per
(tensor, chunk, head) for the bf16 tensors (bf16 operands and storage, as
in the prefill bar), 1e-5 for the fp32 gamma.  M is a matrix of decayed dot
products of bf16 operands, whose rounding error is bounded componentwise by
a small multiple of the unit roundoff times sum_c |q_r[c]| e^{a_r[c] -
a_s[c]} |k_s[c]| (the standard bound for a floating-point dot product); its
error is measured against the largest of those sums (the same reference on
|q| and |k|) rather than against max |M|, which for random unit vectors is
several times smaller."""
import numpy as np
import pytest
import torch

import chunk_ref
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402


class Layout:
    """Byte offsets of one (head, slot) block of the workspace."""

    def __init__(self, C, Dk, Dv):
        self.C, self.Dk, self.Dv = C, Dk, Dv
        self.kst, self.cst, self.mt = (Dk + 31) // 32, (C + 31) // 32, C // 16
        o = 0
        self.W = o
        o += self.mt * self.kst * 1024
        self.Qh = o
        o += self.mt * self.kst * 1024
        self.KbT = o
        o += (Dk // 16) * self.cst * 1024
        self.UtT = o
        o += (Dv // 16) * self.mt * 512
        self.M = o
        o += self.mt * self.cst * 1024
        self.gamma = o
        o += Dk * 4
        self.block = (o + 255) // 256 * 256


def frag16(rows, cols, groups):
    """bf16 element index of (row, col) in a 16x32-fragment-major matrix."""
    r = rows[:, None]
    c = cols[None, :]
    f = (r >> 4) * groups + (c >> 5)
    lane = (r & 15) + 16 * ((c & 31) >> 3)
    return (f * 64 + lane) * 8 + (c & 7)


def frag_ut(js, rs, mt):
    j = js[:, None]
    r = rs[None, :]
    f = (j >> 4) * mt + (r >> 4)
    lane = (j & 15) + 16 * ((r & 15) >> 2)
    return (f * 64 + lane) * 4 + (r & 3)


def decode_block(blk, lay):
    """One workspace block (uint8 numpy) -> dict of float64 tensors."""
    def bf(off, n, idx):
        """bf16 elements idx of the n at byte offset off, as exact floats
        (slots outside idx are never written and not converted)."""
        bits = np.frombuffer(blk[off:off + 2 * n].tobytes(), np.uint16)[idx]
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(
            np.float64)
    C, Dk, Dv = lay.C, lay.Dk, lay.Dv
    rc, rk, rv = np.arange(C), np.arange(Dk), np.arange(Dv)
    nW = lay.mt * lay.kst * 512
    W = bf(lay.W, nW, frag16(rc, rk, lay.kst))
    Qh = bf(lay.Qh, nW, frag16(rc, rk, lay.kst))
    KbT = bf(lay.KbT, (Dk // 16) * lay.cst * 512, frag16(rk, rc, lay.cst))
    UtT = bf(lay.UtT, (Dv // 16) * lay.mt * 256, frag_ut(rv, rc, lay.mt))
    mi = frag16(rc, rc, lay.cst)
    # fragments (row tile m, column group cs) with 2 cs > m lie above the
    # diagonal: zero by definition, never written, never read
    above = (2 * (rc[None, :] >> 5)) > (rc[:, None] >> 4)
    M = bf(lay.M, lay.mt * lay.cst * 512, np.where(above, 0, mi))
    M[above] = 0.0
    gamma = np.frombuffer(blk[lay.gamma:lay.gamma + 4 * Dk].tobytes(),
                          np.float32)
    return dict(W=W, Qh=Qh, KbT=KbT, UtT=UtT, M=M, gamma=gamma)


def rel(x, ref):
    den = max(float(np.max(np.abs(ref))), 1e-30)
    return float(np.max(np.abs(np.asarray(x, np.float64) - ref))) / den


def check_prep(p, label):
    U.log("prep unit parity", label, "H=%d Dk=%d Dv=%d C=%d lengths=%s %s"
          % (p.H, p.K, p.V, p.C, p.seq_lengths.tolist(), p.dtype))
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(p.g), U.f32_dev(p.beta)
    cu = torch.from_numpy(p.cu_seqlens.astype(np.int32)).to(U.DEV)
    ws = kda.kda_prefill_varlen_prep(q, k, v, g, beta, cu,
                                     int(p.seq_lengths.max()),
                                     chunk_size=p.C)
    torch.cuda.synchronize()
    wsh = ws.cpu().numpy()
    lay = Layout(p.C, p.K, p.V)
    C, N = p.C, p.N
    nslots = p.tokens // C + N
    worst = {}
    for n in range(N):
        bos, eos = int(p.cu_seqlens[n]), int(p.cu_seqlens[n + 1])
        for t0 in range(bos, eos, C):
            L = min(C, eos - t0)
            slot = t0 // C + n

            def pad(x):
                out = np.zeros((C,) + x.shape[1:], np.float64)
                out[:L] = x[t0:t0 + L]
                return out
            for h in range(p.H):
                ref = chunk_ref.chunk_tensors(
                    pad(p.q[:, h]), pad(p.k[:, h]), pad(p.v[:, h]),
                    pad(p.g[:, h]), pad(p.beta[:, h]), tile=min(16, C))
                m_scale = np.max(chunk_ref.chunk_tensors(
                    np.abs(pad(p.q[:, h])), np.abs(pad(p.k[:, h])),
                    pad(p.v[:, h]), pad(p.g[:, h]), pad(p.beta[:, h]),
                    tile=min(16, C))["M"])
                off = (h * nslots + slot) * lay.block
                got = decode_block(wsh[off:off + lay.block], lay)
                pairs = (("W", got["W"], ref["W"]),
                         ("Qh", got["Qh"], ref["Qhat"]),
                         ("KbT", got["KbT"], ref["Kbar"].T),
                         ("UtT", got["UtT"], ref["Utilde"].T),
                         ("M", got["M"], ref["M"]),
                         ("gamma", got["gamma"], ref["gamma"]))
                for name, x, r in pairs:
                    e = (float(np.max(np.abs(x - r))) / max(m_scale, 1e-30)
                         if name == "M" else rel(x, r))
                    worst[name] = max(worst.get(name, 0.0), e)
    U.log("   " + "  ".join("%s %.2e" % kv for kv in sorted(worst.items())))
    for name, e in worst.items():
        assert e <= (1e-5 if name == "gamma" else U.PREFILL_TOL), (name, e)


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("C", [16, 32, 64])
def test_prep_tensors_ragged(D, C):
    p = inputs.make("varlen", seed=80 + D + C, H=2, K=D, V=D, C=C,
                    lengths=[2 * C + 7, 0, 1, C])
    check_prep(p, "ragged")


@pytest.mark.parametrize("case", ["g_min", "g_zero", "fp32"])
def test_prep_tensors_edge_values(case):
    kw = dict(g_min=dict(g_const=-5.0), g_zero=dict(g_const=0.0),
              fp32=dict(dtype="fp32"))[case]
    p = inputs.make("varlen", seed=81, H=3, lengths=[130, 64], **kw)
    check_prep(p, case)
