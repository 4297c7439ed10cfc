"""The library from a C++ program that uses only include/kda.h and the HIP
runtime (tests/c_consumer/kda_from_c, built by build()): no Python and no
torch in the process.  It runs an append-prefill of packed sequences from
initial states and then a decode step on the final states; its results must
match the fp64 oracle to the usual bars and the same calls made through the
Python binding bit for bit."""
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_consumer", "kda_from_c")


def _raw(x, dtype):
    """Bytes of x in the storage dtype (bf16 as its 16 high bits: the
    inputs are already bf16 values)."""
    x = np.ascontiguousarray(x, np.float32)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16).tobytes()
    return x.tobytes()


def _from_raw(b, shape, dtype):
    if dtype == "bf16":
        u = np.frombuffer(b, np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).reshape(shape)
    return np.frombuffer(b, np.float32).reshape(shape)


@pytest.mark.parametrize("dtype,D,C,H", [("bf16", 128, 64, 6),
                                         ("fp32", 64, 32, 3)])
def test_c_program_matches_oracle_and_binding(dtype, D, C, H, tmp_path):
    assert os.path.exists(EXE), "build() builds %s" % EXE
    lengths = [150, 0, 64, 33, 200]
    p = inputs.make("varlen", seed=91, H=H, K=D, V=D, C=C, dtype=dtype,
                    lengths=lengths)
    N, T = len(lengths), int(p.cu_seqlens[-1])
    d = inputs.make("decode", seed=92, B=N, H=H, K=D, V=D, dtype=dtype)
    scale = np.float32(D) ** np.float32(-0.5)
    hdr = struct.pack("<8q", N, T, H, D, C, 0 if dtype == "bf16" else 1, 1,
                      int(np.float32(scale).view(np.uint32)))
    blob = b"".join([hdr, p.cu_seqlens.astype(np.int32).tobytes(),
                     _raw(p.q, dtype), _raw(p.k, dtype), _raw(p.v, dtype),
                     _raw(p.g, "fp32"), _raw(p.beta, "fp32"),
                     _raw(p.initial_state, "fp32"),
                     _raw(d.q, dtype), _raw(d.k, dtype), _raw(d.v, dtype),
                     _raw(d.g, "fp32"), _raw(d.beta, "fp32")])
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    fin.write_bytes(blob)
    U.log("C program: %s D=%d C=%d H=%d lengths=%s" % (dtype, D, C, H,
                                                        lengths))
    r = subprocess.run([EXE, str(fin), str(fout)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = fout.read_bytes()
    es = 2 if dtype == "bf16" else 4
    sizes = [T * H * D * es, N * H * D * D * 4, N * H * D * es,
             N * H * D * D * 4]
    assert len(out) == sum(sizes)
    parts, off = [], 0
    for n in sizes:
        parts.append(out[off:off + n])
        off += n
    o = _from_raw(parts[0], (T, H, D), dtype)
    fs = _from_raw(parts[1], (N, H, D, D), "fp32")
    od = _from_raw(parts[2], (N, H, D), dtype)
    sd = _from_raw(parts[3], (N, H, D, D), "fp32")

    # against the oracle
    o_ref, s_ref = oracle.run_varlen(p.q, p.k, p.v, p.g, p.beta,
                                     p.cu_seqlens, p.initial_state,
                                     scale=float(scale))
    eo = max(U.prefill_o_rel(o, o_ref, p.cu_seqlens, C))
    efs = U.slice_rel(fs, s_ref, (0, 1))
    # the decode step against the oracle's step from the program's own
    # prefill states (the decode's bars), and the whole chain against the
    # oracle's chain (the prefill's error carries forward: its bar)
    od_ref, sd_ref = oracle.run_decode(d.q, d.k, d.v, d.g, d.beta,
                                       fs.astype(np.float64),
                                       scale=float(scale))
    eod = U.slice_rel(od, od_ref, (0, 1))
    esd = U.slice_rel(sd, sd_ref, (0, 1))
    oc_ref, sc_ref = oracle.run_decode(d.q, d.k, d.v, d.g, d.beta, s_ref,
                                       scale=float(scale))
    eoc = U.slice_rel(od, oc_ref, (0, 1))
    esc = U.slice_rel(sd, sc_ref, (0, 1))
    U.log("   prefill o %.3e state %.3e   decode o %.3e state %.3e   "
          "chain o %.3e state %.3e" % (eo, efs, eod, esd, eoc, esc))
    assert eo <= U.PREFILL_TOL and efs <= U.PREFILL_TOL
    assert eod <= U.DECODE_O_TOL[dtype] and esd <= U.DECODE_STATE_TOL
    assert eoc <= U.PREFILL_TOL and esc <= U.PREFILL_TOL

    # the same calls through the Python binding: bit for bit
    q, k, v = (U.to_dev(x, dtype) for x in (p.q, p.k, p.v))
    s0 = U.f32_dev(p.initial_state)
    ob, fsb = kda.kda_prefill_varlen(
        q, k, v, U.f32_dev(p.g), U.f32_dev(p.beta),
        torch.from_numpy(p.cu_seqlens).to(U.DEV), max(lengths), s0,
        chunk_size=C, scale=float(scale))
    dq, dk, dv = (U.to_dev(x, dtype) for x in (d.q, d.k, d.v))
    st = fsb.clone()
    odb = kda.kda_decode_step(dq, dk, dv, U.f32_dev(d.g), U.f32_dev(d.beta),
                              st, scale=float(scale))
    torch.cuda.synchronize()
    assert np.array_equal(U.host(ob), o)
    assert np.array_equal(fsb.cpu().numpy(), fs)
    assert np.array_equal(U.host(odb), od)
    assert np.array_equal(st.cpu().numpy(), sd)
