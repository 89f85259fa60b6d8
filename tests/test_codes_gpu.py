"""Every dequantization code through the GPU gather, bit for bit.

Page "feat(qsa): quantized KV pools with dequant-on-gather (fp8/int8/int4)",
part 4 registered tests: the fp8 gather is checked bit for bit against the
plain conversion of the pool.  Here the kernel's own conversions (the fp8
hardware conversion, the int8 byte path, the int4 nibble path, and the
tiered reader's choice between the int8 ring and the int4 pool) see every
code at every channel position, with unit scales:

  * V side: a list of one entry returns that entry's V row exactly (softmax
    of a single logit is 1), so out must equal the dequantized row bit for
    bit -- every code value is exact in bf16;
  * K side: with a one-hot query (q[h, d] = 1) the single logit is
    K[slot, g, d] / 16, so lse names the code at channel d; 22 rounds of 12
    channels per head group cover all 256 channels of every row.

Pool row r of KV head g holds, at byte i, (i + 37 r + 101 g) mod 256: over
the 256 rows every byte value appears at every byte position (fp8 keeps the
254 non-NaN codes: the two NaN codes are replaced by 0; int8 reads the byte
as a signed code, -128 included; u4x2 bytes carry every pair of nibbles).
Expected values come from the oracle (whose decoders are pinned
exhaustively on the CPU).
"""
import numpy as np
import pytest
import torch

import oracle
from qsa_testlib import say

import sparse_index_paged_amd as qsa

pytestmark = pytest.mark.gpu

ROWS = 256
HKV = 2
BS = 128


def code_bytes(width: int) -> np.ndarray:
    r = np.arange(ROWS)[:, None, None]
    g = np.arange(HKV)[None, :, None]
    i = np.arange(width)[None, None, :]
    return ((i + 37 * r + 101 * g) % 256).astype(np.uint8)


def pools_for(fmt: str):
    if fmt == "fp8":
        c = code_bytes(256)
        c[(c == 0x7F) | (c == 0xFF)] = 0
        return c, torch.from_numpy(c.copy())
    if fmt == "int8":
        c = code_bytes(256).view(np.int8)
        return c, torch.from_numpy(c.copy())
    c = code_bytes(128)
    return c, torch.from_numpy(c.copy())


def one_hot_q(t: int) -> torch.Tensor:
    """q[b, h, d] = 1 at d = 12 t + (h mod 12) (mod 256), else 0."""
    q = torch.zeros(BS, 12 * HKV, 256, dtype=torch.bfloat16)
    for h in range(12 * HKV):
        q[:, h, (12 * t + h % 12) % 256] = 1.0
    return q


def check_call(out, lse, o_ref, l_ref, label):
    o = out.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    bad = o != o_ref
    assert not bad.any(), (f"{label}: {int(bad.sum())} output values differ from the dequantized V "
                           f"rows, first at {np.argwhere(bad)[0].tolist()}")
    err = np.abs(lg - l_ref)
    tol = 5e-7 * np.abs(l_ref) + 1e-12
    assert np.all(err <= tol), (f"{label}: lse names the wrong K code at "
                                f"{np.argwhere(err > tol)[0].tolist()}")


def run_format(fmt, group, sdt, waves):
    host, dev = pools_for(fmt)
    kc = dev.cuda()
    vc = torch.from_numpy(np.ascontiguousarray(np.flip(host, axis=2)).copy()).cuda()
    v_host = vc.cpu().numpy()
    ns = 256 // group
    ones = np.ones((ROWS, HKV, ns), np.float32)
    ks = torch.from_numpy(ones).to(sdt).cuda()
    vs = ks.clone()
    cu = torch.arange(BS + 1, dtype=torch.int32)
    label = f"{fmt} g{group} {str(sdt).split('.')[-1]} waves={waves}"
    say(f"[gpu] codes {label}")
    qsa.set_option("waves_per_workgroup", waves)
    try:
        for sb in range(ROWS // BS):
            sel = torch.arange(sb * BS, (sb + 1) * BS, dtype=torch.int32)
            for t in range((256 + 11) // 12):
                q = one_hot_q(t)
                out, lse = qsa.decode(q.cuda(), kc, vc, sel.cuda(), cu.cuda(), kv_format=fmt,
                                      k_scale=ks, v_scale=vs, group_size=group)
                torch.cuda.synchronize()
                o_ref, l_ref = oracle.decode(q, host, v_host, sel.numpy(), cu.numpy(), fmt=fmt,
                                             group=group, k_scale=ones, v_scale=ones)
                check_call(out, lse, o_ref, l_ref, f"{label} rows {sb * BS}+ round {t}")
    finally:
        qsa.set_option("waves_per_workgroup", 0)


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("sdt", [torch.float32, torch.float16])
@pytest.mark.parametrize("fmt,group", [("fp8", 256), ("fp8", 64), ("fp8", 32), ("int8", 256),
                                       ("int8", 64), ("int8", 32), ("int4", 32), ("int4", 64)])
def test_every_code_exact(fmt, group, sdt, waves):
    run_format(fmt, group, sdt, waves)


@pytest.mark.parametrize("waves", [4, 8])
def test_every_code_exact_tiered(waves):
    """Tiered pool: ring rows (int8, 64-channel scales) for even slots below
    256, int4 rows (32-channel scales) for every other listed slot; both tiers
    hold every code at every position."""
    ring = code_bytes(256).view(np.int8)
    cold = np.concatenate([code_bytes(128), code_bytes(128)[::-1]], axis=0)  # 512 slots
    slots = cold.shape[0]
    owner = np.where(np.arange(ROWS) % 2 == 0, np.arange(ROWS), -1).astype(np.int32)
    rs = np.ones((ROWS, HKV, 4), np.float16)
    cs = np.ones((slots, HKV, 8), np.float16)
    dev = dict(ring_k=torch.from_numpy(ring.copy()).cuda(),
               ring_v=torch.from_numpy(np.ascontiguousarray(ring[:, :, ::-1])).cuda(),
               ring_k_scale=torch.from_numpy(rs).cuda(), ring_v_scale=torch.from_numpy(rs).cuda(),
               owner=torch.from_numpy(owner).cuda(),
               claim=torch.zeros(ROWS, dtype=torch.int32, device="cuda"),
               cold_k=torch.from_numpy(cold.copy()).cuda(),
               cold_v=torch.from_numpy(np.ascontiguousarray(cold[:, :, ::-1])).cuda(),
               cold_k_scale=torch.from_numpy(cs).cuda(), cold_v_scale=torch.from_numpy(cs).cuda())
    host = {k_: v_.cpu().numpy() for k_, v_ in dev.items()}
    cu = torch.arange(BS + 1, dtype=torch.int32)
    say(f"[gpu] codes tiered waves={waves}")
    qsa.set_option("waves_per_workgroup", waves)
    try:
        for sb in range(slots // BS):
            sel = torch.arange(sb * BS, (sb + 1) * BS, dtype=torch.int32)
            for t in range((256 + 11) // 12):
                q = one_hot_q(t)
                out, lse = qsa.decode_tiered(q.cuda(), dev, sel.cuda(), cu.cuda())
                torch.cuda.synchronize()
                o_ref, l_ref = oracle.decode_tiered(
                    q, host["owner"], host["ring_k"], host["ring_v"], host["ring_k_scale"],
                    host["ring_v_scale"], host["cold_k"], host["cold_v"], host["cold_k_scale"],
                    host["cold_v_scale"], sel.numpy(), cu.numpy())
                check_call(out, lse, o_ref, l_ref, f"tiered waves={waves} slots {sb * BS}+ round {t}")
    finally:
        qsa.set_option("waves_per_workgroup", 0)
