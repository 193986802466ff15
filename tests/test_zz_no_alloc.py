"""The allocation-free decode entry point (dsa_sparse_mla_decode_static)
against the workspace entry point it mirrors, through the C ABI.

Two calls in a row on one GPU share the library's static scratch: the
second, with a smaller batch, must not see anything of the first. Both must
equal dsa_sparse_mla_decode on the same inputs (same kernels, same split of
the selection lists) and sit within the attention tolerance of the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import Dev, check_attention, i32, log, to_np, torch_mod
from workloads import bf16_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_relu_amd as m

    m.load()
    return m


def _oracle_topk(wl, b):
    return oracle.indexer_topk(bf16_to_f64(b.q_idx), b.w.astype(np.float64),
                               wl.idx_cache.f64_view(), wl.page_table, wl.seq_lens, b.cu_q_lens,
                               wl.k)


def _case(dsa, wl, d, b, bt, tk, what):
    torch = torch_mod()
    log(f"static decode: {what}, T={b.T}, k={tk.shape[1]}")
    tkd = i32(tk, "cuda")
    ref_gpu = dsa.sparse_mla_decode(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens, bt["cu"],
                                    tkd, wl.sm_scale)
    got = dsa.sparse_mla_decode_static(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens,
                                       bt["cu"], tkd, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref_gpu.view(torch.int16)), \
        f"{what}: static-scratch result differs from the workspace entry point"
    ref = oracle.sparse_mla(bf16_to_f64(b.q_mla[0]), wl.kv_cache[0].f64_view(), wl.page_table,
                            wl.seq_lens, b.cu_q_lens, tk, wl.sm_scale, wl.Dv)
    check_attention(to_np(got), ref, what=f"static decode {what}")


def test_static_decode_two_calls_second_smaller(dsa):
    """Decode batch (8 x 8192, k 2048), then the tiny decode (2 rows,
    k 32) on the same static scratch."""
    wl2 = W.config(2)
    b2 = wl2.batches["decode"]
    d2 = Dev(wl2, layers=1)
    _case(dsa, wl2, d2, b2, d2.batch("decode"), _oracle_topk(wl2, b2), "decode batch 8x8192")
    wl1 = W.config(1)
    b1 = wl1.batches["decode"]
    d1 = Dev(wl1, layers=1)
    _case(dsa, wl1, d1, b1, d1.batch("decode"), _oracle_topk(wl1, b1), "tiny decode")


def test_static_decode_rejects_oversize(dsa):
    """A batch whose partials exceed the static scratch is refused on the
    host with DSA_ERR_UNSUPPORTED and nothing launched."""
    torch = torch_mod()
    T, H, k = 64, 64, 65536
    need = dsa.sparse_mla_decode_workspace(T, H, k)
    assert need > (32 << 20)
    q = torch.zeros((T, H, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 64, 576), dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    sl = torch.full((1,), 64, dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    tk = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DsaError) as e:
        dsa.sparse_mla_decode_static(q, kv, pt, sl, cu, tk, 0.1)
    assert e.value.status == 2 and "static scratch" in e.value.detail
