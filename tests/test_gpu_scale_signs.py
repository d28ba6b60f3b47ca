"""Logit scales of any sign: decode and prefill against the oracle.

The softmax scale (and, for fp8 caches, the K dequantisation scale folded into
it) is an ordinary real number of the method: softmax(scale * q.K) is defined
for a negative scale and is the plain average of V for a zero one. A K head
whose values are all zero gets scale 0 from the max|x|/448 recipe. These tests
run every kernel family (decode on the vector path with 1 and 2 query heads
per KV head and on the matrix-core path with 4 and 8, the shared-prefix call,
and prefill) with negative and zero scales, per tensor and per KV head, against
oracle.attention.attend_one on the same (dequantised) K and V. Block 0 of the
pool is never in a table and holds NaN, so a finite output also shows that no
unused block was read.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oattn
from oracle import fp8 as ofp8
from paged_kv_cache_60_amd import ops
from tests.gpu_util import assert_close_to_oracle, log

pytestmark = pytest.mark.gpu
LENS = [1, 37, 300]  # one token, a ragged tile, many tiles and blocks


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _setup(seed, hkv, d, bs, kv, k_scales):
    """Cache [nb, hkv, bs, d] with the sequences' blocks at shuffled places
    (block 0 unused, NaN / 0x7F), tables [B, maxb] (-1 padded), and the
    dequantised K, V [B][L, hkv, d] float64."""
    g = np.random.default_rng(seed)
    nblk = [-(-L // bs) for L in LENS]
    nb = 1 + sum(nblk)
    perm = 1 + g.permutation(nb - 1)
    tables = np.full((len(LENS), max(nblk)), -1, dtype=np.int32)
    at = 0
    for i, n in enumerate(nblk):
        tables[i, :n] = perm[at:at + n]
        at += n
    kx = g.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vx = g.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    if kv == "f16":
        kc, vc = kx.astype(np.float16), vx.astype(np.float16)
        kc[0], vc[0] = np.nan, np.nan
        kd, vd = kc.astype(np.float64), vc.astype(np.float64)
    else:
        kc, vc = ofp8.quantize(kx, 1.0), ofp8.quantize(vx, 1.0)
        kc[0], vc[0] = 0x7F, 0x7F
        t = ofp8.decode_table("e4m3")
        ks = np.asarray(k_scales, dtype=np.float64).reshape(1, hkv, 1, 1)
        kd, vd = t[kc] * ks, t[vc]  # V at scale 1
    K = [np.stack([kd[tables[i, p // bs], :, p % bs, :] for p in range(L)]) for i, L in enumerate(LENS)]
    V = [np.stack([vd[tables[i, p // bs], :, p % bs, :] for p in range(L)]) for i, L in enumerate(LENS)]
    return kc, vc, tables, K, V


CASES = [  # hq, hkv, d, bs, kv, sm_scale sign, K scale(s) (fp8: a list is one per KV head)
    (8, 8, 64, 16, "f16", -1.0, None),
    (16, 8, 128, 16, "f16", 0.0, None),
    (32, 8, 128, 32, "f16", -1.0, None),
    (64, 8, 128, 64, "f16", 0.0, None),
    (16, 8, 128, 16, "fp8", 1.0, [0.0, -0.5, 1.0, 0.25, -1.0, 2.0, 0.0, 0.5]),
    (64, 8, 128, 64, "fp8", -1.0, [1.0, 0.0, -2.0, 0.5, 0.0, -0.25, 1.5, 1.0]),
    (32, 8, 64, 32, "fp8", 1.0, [0.0] * 8),
    (16, 8, 128, 16, "fp8", 1.0, -0.75),  # one negative K scale for the whole tensor
    (64, 8, 128, 64, "fp8", 1.0, 0.0),
    (8, 8, 128, 16, "fp8", -1.0, 0.5),
]


@pytest.mark.parametrize("hq,hkv,d,bs,kv,sign,ks", CASES)
def test_decode_and_prefill_with_signed_scales(hq, hkv, d, bs, kv, sign, ks):
    G = hq // hkv
    sm = sign * d ** -0.5
    per_head = isinstance(ks, list)
    k_scales = ks if per_head else [1.0 if ks is None else ks] * hkv
    kc, vc, tables, K, V = _setup(hq + d + bs, hkv, d, bs, kv, k_scales)
    g = np.random.default_rng(7 + hq)
    B = len(LENS)
    kscale_arg = _dev(np.asarray(k_scales, dtype=np.float32)) if per_head else k_scales[0]
    vscale_arg = _dev(np.ones(hkv, dtype=np.float32)) if per_head else 1.0
    kcd, vcd, td = _dev(kc), _dev(vc), _dev(tables)
    ctx = _dev(np.asarray(LENS, dtype=np.int32))

    # decode: one query per sequence at its last position
    q = g.standard_normal((B, hq, d), dtype=np.float32).astype(np.float16)
    ref = np.zeros((B, hq, d))
    for b in range(B):
        for h in range(hq):
            ref[b, h] = oattn.attend_one(q[b, h], K[b][:, h // G], V[b][:, h // G], sm)
    out = torch.full((B, hq, d), 3.0, dtype=torch.float16, device="cuda")
    log(f"decode hq={hq} hkv={hkv} d={d} bs={bs} {kv} sm={sm:+.3f} per_head={per_head}")
    ops.paged_attn_decode(out, _dev(q), kcd, vcd, td, ctx, sm, kv, kscale_arg, vscale_arg)
    torch.cuda.synchronize()
    assert_close_to_oracle(out.cpu().numpy(), ref, kv, "decode")

    # the shared-prefix call with no groups takes the same path
    out2 = torch.full_like(out, 3.0)
    groups = torch.zeros((3, 0), dtype=torch.int32, device="cuda")
    ops.paged_attn_decode_shared(out2, _dev(q), kcd, vcd, td, ctx, groups, sm, kv, kscale_arg, vscale_arg)
    torch.cuda.synchronize()
    assert_close_to_oracle(out2.cpu().numpy(), ref, kv, "decode (shared call)")

    # prefill: every position of every sequence is a query row
    n = sum(LENS)
    qp = g.standard_normal((n, hq, d), dtype=np.float32).astype(np.float16)
    q_start = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int32)
    refp = np.zeros((n, hq, d))
    for b in range(B):
        for p in range(LENS[b]):
            r = q_start[b] + p
            for h in range(hq):
                refp[r, h] = oattn.attend_one(qp[r, h], K[b][:p + 1, h // G], V[b][:p + 1, h // G], sm)
    outp = torch.full((n, hq, d), 3.0, dtype=torch.float16, device="cuda")
    log(f"prefill hq={hq} hkv={hkv} d={d} bs={bs} {kv} sm={sm:+.3f} per_head={per_head}")
    ops.paged_attn_prefill(outp, _dev(qp), kcd, vcd, td, ctx, _dev(q_start), sm, kv, kscale_arg, vscale_arg)
    torch.cuda.synchronize()
    assert_close_to_oracle(outp.cpu().numpy(), refp, kv, "prefill")


@pytest.mark.parametrize("hq,hkv,sign", [(16, 8, -1.0), (64, 8, 0.0), (64, 8, -1.0), (8, 8, 0.0)])
def test_shared_prefix_pass_with_signed_scales(hq, hkv, sign):
    """Two sequences whose tables start with the same 6 blocks (96 tokens),
    decoded by the shared-prefix call as one group."""
    d, bs, G = 128, 16, hq // hkv
    sm = sign * d ** -0.5
    g = np.random.default_rng(hq + 3)
    lens = [100, 120]
    nb = 1 + 6 + 1 + 2  # block 0 unused; 6 shared; the rest private
    tables = np.full((2, 8), -1, dtype=np.int32)
    tables[0, :7] = [3, 1, 4, 9, 2, 6, 5]
    tables[1, :8] = [3, 1, 4, 9, 2, 6, 7, 8]
    kc = g.standard_normal((nb, hkv, bs, d), dtype=np.float32).astype(np.float16)
    vc = g.standard_normal((nb, hkv, bs, d), dtype=np.float32).astype(np.float16)
    kc[0], vc[0] = np.nan, np.nan
    q = g.standard_normal((2, hq, d), dtype=np.float32).astype(np.float16)
    ref = np.zeros((2, hq, d))
    for b, L in enumerate(lens):
        K = np.stack([kc[tables[b, p // bs], :, p % bs, :] for p in range(L)]).astype(np.float64)
        V = np.stack([vc[tables[b, p // bs], :, p % bs, :] for p in range(L)]).astype(np.float64)
        for h in range(hq):
            ref[b, h] = oattn.attend_one(q[b, h], K[:, h // G], V[:, h // G], sm)
    out = torch.full((2, hq, d), 3.0, dtype=torch.float16, device="cuda")
    groups = _dev(np.asarray([[0], [2], [96]], dtype=np.int32))
    log(f"shared hq={hq} hkv={hkv} sm={sm:+.3f}")
    ops.paged_attn_decode_shared(out, _dev(q), _dev(kc), _dev(vc), _dev(tables), _dev(np.asarray(lens, np.int32)),
                                 groups, sm)
    torch.cuda.synchronize()
    assert_close_to_oracle(out.cpu().numpy(), ref, "f16", "shared-prefix decode")
