"""Untied directions (each direction its own layer: own x, dt, B, C, z, A, D, dt_bias; own gate and output)
against the fp64 oracle.

The paper's two directions are two independent Mamba layers (Section 3.2, eq. (4) with A_f, B_f, C_f and
eq. (5) with A_b, B_b, C_b) whose weights are not tied (Section 4.1, Table 8).
"""
import numpy as np
import pytest

import oracle
from bidirectional_mamba_selective_amd import inputs as I
from tests.gpu_util import Bar, check, say, to_host64, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bidirectional_mamba_selective_amd import load

    load()
    yield


def _set(batch, L, D, N, io, seed, a_jitter, param_seed):
    A, Dv, bias = I.make_params(D, N, seed=param_seed, a_jitter=a_jitter)
    act = I.make_activations(batch, L, D, N, io, seed=seed)
    act.update(A=A, D=Dv, dt_bias=bias)
    return act


def _run(f, r, io, flags=0):
    import torch

    from bidirectional_mamba_selective_amd import bimamba_scan_fwd_untied

    df, dr = upload(f, io), upload(r, io)
    if flags & 1:
        df["z"] = dr["z"] = None
    out_f, out_r = bimamba_scan_fwd_untied(df, dr, flags=flags)
    torch.cuda.synchronize()
    return to_host64(out_f), to_host64(out_r)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("L", [300, 2500])
def test_untied_two_sets(io, L):
    """Distinct sets (the forward one with geometric A, the reverse one with general A), batch 2, ragged
    lengths that span several chunks."""
    f = _set(2, L, 128, 16, io, seed=11, a_jitter=0.0, param_seed=0)
    r = _set(2, L, 128, 16, io, seed=12, a_jitter=0.2, param_seed=5)
    got_f, got_r = _run(f, r, io)
    want_f, want_r = oracle.scan_fwd_untied(f, r)
    check(got_f, want_f, io, f"untied {io} L={L} out_f")
    check(got_r, want_r, io, f"untied {io} L={L} out_r")


def test_untied_no_gate_and_small_states():
    f = _set(1, 777, 64, 5, "f32", seed=21, a_jitter=0.2, param_seed=1)
    r = _set(1, 777, 64, 5, "f32", seed=22, a_jitter=0.0, param_seed=2)
    got_f, got_r = _run(f, r, "f32", flags=1)
    want_f, want_r = oracle.scan_fwd_untied(f, r, gate=False)
    check(got_f, want_f, "f32", "untied no gate N=5 out_f")
    check(got_r, want_r, "f32", "untied no gate N=5 out_r")


def test_untied_equal_sets_sum_to_tied():
    """With both sets equal, out_f + out_r is the tied call's output (fp32 I/O)."""
    import torch

    from bidirectional_mamba_selective_amd import bimamba_scan_fwd

    s = _set(1, 1500, 128, 16, "f32", seed=31, a_jitter=0.0, param_seed=0)
    got_f, got_r = _run(s, s, "f32")
    d = upload(s, "f32")
    tied = to_host64(bimamba_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], d["dt_bias"]))
    torch.cuda.synchronize()
    # two fp32 computations of one result by different kernel paths: 1e-5 in every sense
    check(got_f + got_r, tied, Bar(1e-5, 1e-5, 1e-5, 1e-6), "untied equal sets vs tied")


def test_untied_long_full_width():
    """The benchmarked untied shape (L 65536, d_inner 4096, bf16; the forward set with geometric A, the
    reverse set with general A) over both whole outputs, against the oracle run on the host in channel shards."""
    from tests.gpu_util import oracle_sharded

    L, D, N = 65536, 4096, 16
    say("untied long full width: generating inputs")
    f = _set(1, L, D, N, "bf16", seed=13, a_jitter=0.0, param_seed=0)
    r = _set(1, L, D, N, "bf16", seed=14, a_jitter=0.2, param_seed=5)
    got_f, got_r = _run(f, r, "bf16")

    def both(sets, chan):
        sub = [{k: (c[k][:, :, chan] if k in ("x", "dt", "z") else (c[k][chan] if k in ("A", "D", "dt_bias")
                                                                     else c[k])) for k in c} for c in sets]
        return np.stack(oracle.scan_fwd_untied(sub[0], sub[1]))

    say("untied long full width: oracle on 4096 channels in host processes")
    want = oracle_sharded(both, (f, r), D, (2, 1, L, D))
    check(got_f, want[0], "bf16", "untied long out_f (all 65536 x 4096 outputs)")
    check(got_r, want[1], "bf16", "untied long out_r (all 65536 x 4096 outputs)")


def test_untied_layer_2k_subset():
    """The layer shape (batch 1, L 2048, d_inner 4096, d_state 16, bf16), both directions checked on a
    channel subset (each output channel depends only on its own channel and the shared B, C)."""
    f = _set(1, 2048, 4096, 16, "bf16", seed=41, a_jitter=0.0, param_seed=0)
    r = _set(1, 2048, 4096, 16, "bf16", seed=42, a_jitter=0.2, param_seed=3)
    got_f, got_r = _run(f, r, "bf16")
    chan = np.arange(3, 4096, 97)

    def sub(c):
        return {k: (c[k][:, :, chan] if k in ("x", "dt", "z") else (c[k][chan] if k in ("A", "D", "dt_bias")
                    else c[k])) for k in ("x", "dt", "z", "B", "C", "A", "D", "dt_bias")}

    want_f, want_r = oracle.scan_fwd_untied(sub(f), sub(r))
    check(got_f[:, :, chan], want_f, "bf16", "untied layer 2k subset out_f")
    check(got_r[:, :, chan], want_r, "bf16", "untied layer 2k subset out_r")


def test_untied_both_geometric_many_tiles():
    """Both sets with geometric A, fp32, batch 1, L 8192, d_inner 4096 (64 chunks of 8 tiles): both
    one-direction summaries in closed form, each over several tiles per chunk; both outputs on a channel
    subset.  The forward set has A[d,n] = -(n+1); the reverse set A[d,n] = (n+1) * A[d,0] with A[d,0] from
    -0.5 to -2.25 by channel (formed in fp32, so each row has the geometric form exactly)."""
    f = _set(1, 8192, 4096, 16, "f32", seed=51, a_jitter=0.0, param_seed=0)
    r = _set(1, 8192, 4096, 16, "f32", seed=52, a_jitter=0.0, param_seed=6)
    a0 = -(np.float32(0.5) + np.float32(0.25) * (np.arange(4096) % 8).astype(np.float32))
    r["A"] = (np.arange(1, 17, dtype=np.float32)[None, :] * a0[:, None]).astype(np.float32)
    assert np.array_equal(r["A"], np.float32(np.arange(1, 17))[None, :] * r["A"][:, :1])
    got_f, got_r = _run(f, r, "f32")
    chan = np.arange(5, 4096, 131)

    def sub(c):
        return {k: (c[k][:, :, chan] if k in ("x", "dt", "z") else (c[k][chan] if k in ("A", "D", "dt_bias")
                    else c[k])) for k in ("x", "dt", "z", "B", "C", "A", "D", "dt_bias")}

    want_f, want_r = oracle.scan_fwd_untied(sub(f), sub(r))
    check(got_f[:, :, chan], want_f, "f32", "untied both geometric out_f")
    check(got_r[:, :, chan], want_r, "f32", "untied both geometric out_r")


@pytest.mark.parametrize("G", [32, 200])
def test_untied_block_decoding_from_two_block_calls(G):
    """Block-cache decoding with untied directions is two block calls: the forward layer's set with
    FWD_ONLY and the cache, the reverse layer's set with REV_ONLY and no cache.  Over 4 chained blocks
    (32 tokens: single kernel; 200: chunked path), out_f, out_r and the cache against the oracle's block
    step of each set, and the chained forward outputs against the untied full-sequence forward output."""
    import torch

    from bidirectional_mamba_selective_amd import bimamba_scan_block
    from tests.gpu_util import f32_dev

    D, N, nblk = 128, 16, 4
    f = _set(1, G * nblk, D, N, "f32", seed=31, a_jitter=0.0, param_seed=3)
    r = _set(1, G * nblk, D, N, "f32", seed=32, a_jitter=0.2, param_seed=4)
    df, dr = upload(f, "f32"), upload(r, "f32")
    h = torch.zeros(1, D, N, device="cuda")
    h_host = None
    full_f, _ = oracle.scan_fwd_untied(f, r)
    for k in range(nblk):
        sl = slice(k * G, (k + 1) * G)
        bf = {key: df[key][:, sl].contiguous() for key in ("x", "dt", "z", "B", "C")}
        br = {key: dr[key][:, sl].contiguous() for key in ("x", "dt", "z", "B", "C")}
        out_f = bimamba_scan_block(bf["x"], bf["dt"], df["A"], bf["B"], bf["C"], df["D"], bf["z"], df["dt_bias"],
                                   h_in=h, h_out=h, flags=2)  # FWD_ONLY, committed in place
        out_r = bimamba_scan_block(br["x"], br["dt"], dr["A"], br["B"], br["C"], dr["D"], br["z"], dr["dt_bias"],
                                   flags=4)  # REV_ONLY
        torch.cuda.synchronize()
        hf = {key: f[key][:, sl] for key in ("x", "dt", "z", "B", "C")}
        hr = {key: r[key][:, sl] for key in ("x", "dt", "z", "B", "C")}
        want_f, want_h = oracle.scan_block(hf["x"], hf["dt"], f["A"], hf["B"], hf["C"], f["D"], hf["z"], f["dt_bias"],
                                           h_host, fwd=True, rev=False)
        want_r, _ = oracle.scan_block(hr["x"], hr["dt"], r["A"], hr["B"], hr["C"], r["D"], hr["z"], r["dt_bias"],
                                      None, fwd=False, rev=True)
        check(to_host64(out_f), want_f, "f32", f"untied block G={G} {k} out_f")
        check(to_host64(out_r), want_r, "f32", f"untied block G={G} {k} out_r")
        check(to_host64(h), want_h, "state", f"untied block G={G} {k} cache")
        check(to_host64(out_f), full_f[:, sl], "f32", f"untied block G={G} {k} out_f vs full forward")
        h_host = want_h
