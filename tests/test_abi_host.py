"""C ABI on the host (no GPU): the library loads, exports every declared
symbol, and rejects bad arguments before it touches a device."""
import ctypes
import math

import numpy as np
import pytest

import paged_mla_decode_06_amd as mla


@pytest.fixture(scope="module")
def L():
    return mla.lib()


def good(**kw):
    base = dict(batch=2, q_len=1, num_heads=16, page_size=64, num_pages=16, block_table_stride=5,
                max_seq_len=257, kv_dtype=mla.MLA_KV_BF16, softmax_scale=1 / math.sqrt(192), k_scale=1.0,
                num_splits=0, min_work_units=0, num_cus=256)
    base.update(kw)
    return mla.make_params(**base)


def test_exports_every_declared_function(L):
    names = mla.header_functions()
    assert set(names) >= {"mla_abi_version", "mla_status_str", "mla_decode_workspace_size", "mla_decode",
                          "mla_gather_kv", "mla_plan_host", "mla_plan_device", "mla_check_inputs_host"}
    for n in names:
        assert hasattr(L, n), f"libmla.so does not export {n}"


def test_abi_version_and_status_strings(L):
    assert mla.mla_abi_version() == 3
    for code, name in [(0, "MLA_OK"), (1, "MLA_ERR_INVALID_VALUE"), (2, "MLA_ERR_NOT_SUPPORTED"),
                       (3, "MLA_ERR_WORKSPACE_TOO_SMALL"), (4, "MLA_ERR_HIP"), (99, "MLA_ERR_UNKNOWN")]:
        assert mla.status_name(code) == name


def test_params_struct_layout():
    # 10 int32, 2 float, 4 int32, no padding
    assert ctypes.sizeof(mla.mla_decode_params) == 16 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=16), mla.MLA_ERR_INVALID_VALUE),            # only 32 and 64
    (dict(page_size=128), mla.MLA_ERR_INVALID_VALUE),
    (dict(kv_lora_rank=256), mla.MLA_ERR_NOT_SUPPORTED),
    (dict(qk_rope_head_dim=32), mla.MLA_ERR_NOT_SUPPORTED),
    (dict(batch=-1), mla.MLA_ERR_INVALID_VALUE),
    (dict(q_len=0), mla.MLA_ERR_INVALID_VALUE),
    (dict(num_heads=0), mla.MLA_ERR_INVALID_VALUE),
    (dict(q_len=65), mla.MLA_ERR_NOT_SUPPORTED),
    (dict(num_heads=257), mla.MLA_ERR_NOT_SUPPORTED),
    (dict(q_len=64, num_heads=128), mla.MLA_ERR_NOT_SUPPORTED),   # q_len*H > 4096
    (dict(batch=8193), mla.MLA_ERR_NOT_SUPPORTED),
    (dict(num_pages=0), mla.MLA_ERR_INVALID_VALUE),
    (dict(max_seq_len=-1), mla.MLA_ERR_INVALID_VALUE),
    (dict(block_table_stride=4), mla.MLA_ERR_INVALID_VALUE),     # 4*64 < 257
    (dict(block_table_stride=0), mla.MLA_ERR_INVALID_VALUE),
    (dict(kv_dtype=7), mla.MLA_ERR_INVALID_VALUE),
    (dict(softmax_scale=0.0), mla.MLA_ERR_INVALID_VALUE),
    (dict(softmax_scale=float("nan")), mla.MLA_ERR_INVALID_VALUE),
    (dict(softmax_scale=float("inf")), mla.MLA_ERR_INVALID_VALUE),
    (dict(kv_dtype=mla.MLA_KV_FP8_E4M3FN, k_scale=0.0), mla.MLA_ERR_INVALID_VALUE),
    (dict(kv_dtype=mla.MLA_KV_FP8_E4M3FN, k_scale=float("nan")), mla.MLA_ERR_INVALID_VALUE),
    (dict(num_splits=-1), mla.MLA_ERR_INVALID_VALUE),
    (dict(num_splits=1025), mla.MLA_ERR_INVALID_VALUE),
    (dict(min_work_units=-3), mla.MLA_ERR_INVALID_VALUE),
    (dict(num_cus=-1), mla.MLA_ERR_INVALID_VALUE),
    (dict(quantize_q_fp8=1), mla.MLA_ERR_INVALID_VALUE),                             # bf16 pool
    (dict(kv_dtype=mla.MLA_KV_FP8_E4M3FN, quantize_q_fp8=2), mla.MLA_ERR_INVALID_VALUE),
    (dict(kv_dtype=mla.MLA_KV_FP8_E4M3FN, quantize_q_fp8=-1), mla.MLA_ERR_INVALID_VALUE),
])
def test_invalid_params_rejected(L, kw, status):
    p = good(**kw)
    n = ctypes.c_size_t(0)
    assert L.mla_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status
    fake = ctypes.c_void_p(0x1000)
    assert L.mla_decode(ctypes.byref(p), fake, fake, fake, fake, fake, None, ctypes.c_void_p(0x10000), 1 << 30,
                        None) == status


def test_bf16_pool_ignores_k_scale(L):
    p = good(k_scale=float("nan"))     # a bf16 pool never reads k_scale
    assert mla.mla_decode_workspace_size(p) > 0


def test_null_and_alignment_checks(L):
    p = good()
    fake = ctypes.c_void_p(0x100000)
    ws = ctypes.c_void_p(0x200000)
    big = 1 << 34
    assert L.mla_decode(ctypes.byref(p), None, fake, fake, fake, fake, None, ws, big, None) == mla.MLA_ERR_INVALID_VALUE
    assert L.mla_decode(ctypes.byref(p), fake, fake, fake, fake, fake, None, None, big, None) == \
        mla.MLA_ERR_INVALID_VALUE
    assert L.mla_decode(ctypes.byref(p), ctypes.c_void_p(0x100008), fake, fake, fake, fake, None, ws, big, None) == \
        mla.MLA_ERR_INVALID_VALUE     # q not 16-byte aligned
    assert L.mla_decode(ctypes.byref(p), fake, fake, fake, fake, fake, None, ctypes.c_void_p(0x200010), big,
                        None) == mla.MLA_ERR_INVALID_VALUE     # workspace not 256-byte aligned


def test_workspace_too_small_before_any_device_call(L):
    p = good()
    need = mla.mla_decode_workspace_size(p)
    fake = ctypes.c_void_p(0x100000)
    ws = ctypes.c_void_p(0x200000)
    assert L.mla_decode(ctypes.byref(p), fake, fake, fake, fake, fake, None, ws, need - 1, None) == \
        mla.MLA_ERR_WORKSPACE_TOO_SMALL


def test_empty_batch_is_a_noop(L):
    p = good(batch=0)
    assert L.mla_decode(ctypes.byref(p), None, None, None, None, None, None, None, 0, None) == mla.MLA_OK


def test_workspace_size_formula():
    # balanced: groups = min(whole groups the 8 XCDs of CUs/8 CUs hold, B*units(max));
    # slots = 2 * groups * nrb; per slot ROWS_PER_BLOCK rows x (512 bf16 + 1 fp32 lse);
    # the request offsets [B+1] and the 32-int class table first
    a256 = lambda x: (x + 255) // 256 * 256
    R = mla.ROWS_PER_BLOCK
    for heads, q_len in [(128, 1), (128, 4), (16, 1), (64, 3)]:
        p = good(batch=64, num_heads=heads, q_len=q_len, max_seq_len=4096, block_table_stride=64, num_cus=256)
        nrb = -(-q_len * heads // R)
        groups = min(8 * (32 // nrb), 64 * 128)
        slots = 2 * groups * nrb
        expect = a256((65 + 32) * 4) + a256(slots * R * 4) + slots * R * 512 * 2
        assert mla.mla_decode_workspace_size(p) == expect, (heads, q_len)
    # forced splits: groups = B*S, slots = groups * nrb
    p = good(batch=3, num_heads=128, q_len=2, num_splits=5, num_cus=0)
    slots = 3 * 5 * -(-2 * 128 // R)
    assert mla.mla_decode_workspace_size(p) == a256((4 + 32) * 4) + a256(slots * R * 4) + slots * R * 512 * 2


def test_check_inputs_host():
    from mla_synth import generate
    inp = generate("tiny")
    p = good()
    assert mla.mla_check_inputs_host(p, inp.block_table, inp.seq_lens) == mla.MLA_OK
    bt = inp.block_table.copy()
    bt[1, 4] = 16                      # read by tokens 256..257 of request 1
    assert mla.mla_check_inputs_host(p, bt, inp.seq_lens) == mla.MLA_ERR_INVALID_VALUE
    bt = inp.block_table.copy()
    bt[0, 2] = 99                      # past request 0's last page: never read
    assert mla.mla_check_inputs_host(p, bt, inp.seq_lens) == mla.MLA_OK
    sl = inp.seq_lens.copy()
    sl[0] = 258                        # above max_seq_len
    assert mla.mla_check_inputs_host(p, inp.block_table, sl) == mla.MLA_ERR_INVALID_VALUE
    sl[0] = -1
    assert mla.mla_check_inputs_host(p, inp.block_table, sl) == mla.MLA_ERR_INVALID_VALUE


def test_algorithmic_work_formula():
    nbytes, flops = mla.algorithmic_work(np.array([100, 257]), 1, 16, 64, 2)
    assert nbytes == 357 * 576 * 2 + 2 * 16 * (1152 + 1024 + 4) + 4 * (2 + 5) + 8
    assert flops == 2 * 16 * 1088 * 357
    _, f4 = mla.algorithmic_work(np.array([10]), 4, 1, 64, 2)
    assert f4 == 2 * 1088 * (7 + 8 + 9 + 10)


# ---- KV-cache append: argument checks before any device call
def test_append_params_struct_layout():
    # two int64 strides, 6 int32, 1 float, padded to 8 bytes
    assert ctypes.sizeof(mla.mla_kv_append_params) == 48
    assert "mla_kv_append" in mla.header_functions()


def good_append(**kw):
    base = dict(num_tokens=4, page_size=64, num_pages=8, kv_dtype=mla.MLA_KV_BF16, k_scale=1.0,
                nope_stride=576, rope_stride=576)
    base.update(kw)
    return mla.make_append_params(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=16), mla.MLA_ERR_INVALID_VALUE),
    (dict(num_tokens=-1), mla.MLA_ERR_INVALID_VALUE),
    (dict(num_pages=0), mla.MLA_ERR_INVALID_VALUE),
    (dict(kv_dtype=3), mla.MLA_ERR_INVALID_VALUE),
    (dict(kv_dtype=mla.MLA_KV_FP8_E4M3FN, k_scale=0.0), mla.MLA_ERR_INVALID_VALUE),
    (dict(kv_dtype=mla.MLA_KV_FP8_E4M3FN, k_scale=float("inf")), mla.MLA_ERR_INVALID_VALUE),
    (dict(nope_stride=511), mla.MLA_ERR_INVALID_VALUE),
    (dict(nope_stride=580), mla.MLA_ERR_INVALID_VALUE),       # rows must stay 16-byte aligned
    (dict(rope_stride=60), mla.MLA_ERR_INVALID_VALUE),
    (dict(kv_lora_rank=256), mla.MLA_ERR_NOT_SUPPORTED),
    (dict(qk_rope_head_dim=32), mla.MLA_ERR_NOT_SUPPORTED),
])
def test_append_invalid_params_rejected(L, kw, status):
    p = good_append(**kw)
    fake = ctypes.c_void_p(0x100000)
    assert L.mla_kv_append(ctypes.byref(p), fake, fake, fake, fake, None) == status


def test_append_null_and_alignment_checks(L):
    p = good_append()
    fake = ctypes.c_void_p(0x100000)
    assert L.mla_kv_append(ctypes.byref(p), None, fake, fake, fake, None) == mla.MLA_ERR_INVALID_VALUE
    assert L.mla_kv_append(ctypes.byref(p), fake, fake, fake, None, None) == mla.MLA_ERR_INVALID_VALUE
    assert L.mla_kv_append(ctypes.byref(p), ctypes.c_void_p(0x100008), fake, fake, fake, None) == \
        mla.MLA_ERR_INVALID_VALUE     # k_nope not 16-byte aligned
    assert L.mla_kv_append(ctypes.byref(p), fake, fake, ctypes.c_void_p(0x100004), fake, None) == \
        mla.MLA_ERR_INVALID_VALUE     # locations not 8-byte aligned
    assert L.mla_kv_append(None, fake, fake, fake, fake, None) == mla.MLA_ERR_INVALID_VALUE


def test_append_empty_is_a_noop(L):
    p = good_append(num_tokens=0)
    assert L.mla_kv_append(ctypes.byref(p), None, None, None, None, None) == mla.MLA_OK


def test_append_work_formula():
    assert mla.append_work(64, 2) == 64 * (1152 + 1152 + 8)
    assert mla.append_work(10, 1) == 10 * (1152 + 576 + 8)


# ---- query given as two parts: argument checks before any device call
@pytest.mark.parametrize("strides,status", [
    ((576 * 16, 576, 576 * 16, 576), None),               # the merged layout: gets past the checks
    ((512, 512 * 2, 64, 64 * 16), None),
    ((512 + 4, 512, 576, 576), mla.MLA_ERR_INVALID_VALUE),  # not a multiple of 8
    ((576, 576, 576, 60), mla.MLA_ERR_INVALID_VALUE),
    ((-576, 576, 576, 576), mla.MLA_ERR_INVALID_VALUE),
])
def test_qparts_stride_checks(L, strides, status):
    p = good()
    lay = mla.mla_query_layout(*strides)
    fake = ctypes.c_void_p(0x100000)
    ws = ctypes.c_void_p(0x200000)
    st = L.mla_decode_qparts(ctypes.byref(p), fake, ctypes.c_void_p(0x300000), ctypes.byref(lay), fake, fake, fake,
                             fake, None, ws, 1, None)
    if status is None:
        assert st == mla.MLA_ERR_WORKSPACE_TOO_SMALL      # every argument check passed
    else:
        assert st == status


def test_qparts_null_and_alignment(L):
    p = good()
    lay = mla.mla_query_layout(576 * 16, 576, 576 * 16, 576)
    fake = ctypes.c_void_p(0x100000)
    ws = ctypes.c_void_p(0x200000)
    big = 1 << 34
    assert L.mla_decode_qparts(ctypes.byref(p), fake, fake, None, fake, fake, fake, fake, None, ws, big, None) == \
        mla.MLA_ERR_INVALID_VALUE
    assert L.mla_decode_qparts(ctypes.byref(p), fake, None, ctypes.byref(lay), fake, fake, fake, fake, None, ws, big,
                               None) == mla.MLA_ERR_INVALID_VALUE
    assert L.mla_decode_qparts(ctypes.byref(p), fake, ctypes.c_void_p(0x100408), ctypes.byref(lay), fake, fake, fake,
                               fake, None, ws, big, None) == mla.MLA_ERR_INVALID_VALUE   # rope part misaligned


# ---- ragged batches: host checks
def test_qo_indptr_host_check():
    p = good(batch=3, q_len=4)
    assert mla.mla_check_qo_indptr_host(p, np.array([0, 2, 2, 6]), 6) == mla.MLA_OK
    assert mla.mla_check_qo_indptr_host(p, np.array([1, 2, 2, 6]), 6) == mla.MLA_ERR_INVALID_VALUE   # not from 0
    assert mla.mla_check_qo_indptr_host(p, np.array([0, 3, 2, 6]), 6) == mla.MLA_ERR_INVALID_VALUE   # backwards
    assert mla.mla_check_qo_indptr_host(p, np.array([0, 5, 6, 7]), 7) == mla.MLA_ERR_INVALID_VALUE   # q_b > q_len
    assert mla.mla_check_qo_indptr_host(p, np.array([0, 2, 2, 6]), 7) == mla.MLA_ERR_INVALID_VALUE   # total


def test_ragged_argument_checks(L):
    p = good()
    fake = ctypes.c_void_p(0x100000)
    ws = ctypes.c_void_p(0x200000)
    assert L.mla_decode_ragged(ctypes.byref(p), fake, None, 2, fake, fake, fake, fake, None, ws, 1 << 34,
                               None) == mla.MLA_ERR_INVALID_VALUE      # no offsets
    assert L.mla_decode_ragged(ctypes.byref(p), fake, fake, -1, fake, fake, fake, fake, None, ws, 1 << 34,
                               None) == mla.MLA_ERR_INVALID_VALUE      # negative token count
    assert L.mla_decode_ragged(ctypes.byref(p), fake, fake, 2, fake, fake, fake, fake, None, ws, 1,
                               None) == mla.MLA_ERR_WORKSPACE_TOO_SMALL  # every argument check passed
    # no query token at all: the parameters are checked, nothing is enqueued
    # and q, out, lse and the workspace may be null
    assert L.mla_decode_ragged(ctypes.byref(p), None, fake, 0, fake, fake, fake, None, None, None, 0,
                               None) == mla.MLA_OK
    bad = good(page_size=16)
    assert L.mla_decode_ragged(ctypes.byref(bad), None, fake, 0, fake, fake, fake, None, None, None, 0,
                               None) == mla.MLA_ERR_INVALID_VALUE


def test_ragged_algorithmic_work():
    nb, fl = mla.algorithmic_work_ragged(np.array([10, 20]), np.array([1, 3]), 2, 32, 2)
    nu, fu = mla.algorithmic_work(np.array([10]), 1, 2, 32, 2)
    assert fl == 2 * 2 * 1088 * (10 + 18 + 19 + 20)
    assert nb == 30 * 1152 + 4 * 2 * (1152 + 1024 + 4) + 4 * 2 + 8 + 12


# ---- rotary embedding: argument checks before any device call
@pytest.mark.parametrize("rope,ok", [
    ((0x100000, 0x200000, 4096, 1), True),
    ((0x100000, 0x200000, 4096, 0), True),
    ((0, 0x200000, 4096, 1), False),            # no positions
    ((0x100000, 0, 4096, 1), False),            # no cache
    ((0x100000, 0x200000, 0, 1), False),        # empty cache
    ((0x100000, 0x200000, 64, 2), False),       # is_neox must be 0 or 1
    ((0x100000, 0x200008, 64, 1), False),       # cache not 16-byte aligned
    ((0x100004, 0x200000, 64, 1), False),       # positions not 8-byte aligned
])
def test_rope_checks(L, rope, ok):
    r = mla.mla_rope(*rope)
    p = good()
    lay = mla.mla_query_layout(576 * 16, 576, 576 * 16, 576)
    fake = ctypes.c_void_p(0x100000)
    st = L.mla_decode_qparts_rope(ctypes.byref(p), fake, ctypes.c_void_p(0x300000), ctypes.byref(lay),
                                  ctypes.byref(r), fake, fake, fake, fake, None, ctypes.c_void_p(0x200000), 1, None)
    assert st == (mla.MLA_ERR_WORKSPACE_TOO_SMALL if ok else mla.MLA_ERR_INVALID_VALUE)
    pa = good_append(kv_dtype=mla.MLA_KV_FP8_E4M3FN, k_scale=0.0)   # invalid append params
    st = L.mla_kv_append_rope(ctypes.byref(pa), fake, fake, fake, ctypes.byref(r), fake, None)
    assert st == mla.MLA_ERR_INVALID_VALUE
    assert L.mla_kv_append_rope(ctypes.byref(good_append()), fake, fake, fake, None, fake, None) == \
        mla.MLA_ERR_INVALID_VALUE


def _decode_tensors(torch, B=3, ql=2, H=16, P=64, W=4):
    return dict(q=torch.zeros((B, ql, H, 576), dtype=torch.bfloat16),
                kv_pool=torch.zeros((10, P, 576), dtype=torch.bfloat16),
                block_table=torch.zeros((B, W), dtype=torch.int32),
                seq_lens=torch.zeros(B, dtype=torch.int32),
                out=torch.zeros((B, ql, H, 512), dtype=torch.bfloat16),
                lse=torch.zeros((B, ql, H), dtype=torch.float32))


def _shape_mistakes(torch, B=3, ql=2, H=16, P=64):
    # max_seq_len 200 needs ceil(200 / 64) = 4 block-table columns
    return [
        (dict(out=torch.zeros((B, ql, H, 256), dtype=torch.bfloat16)), "out must be"),
        (dict(out=torch.zeros((B, ql, H - 1, 512), dtype=torch.bfloat16)), "out must be"),
        (dict(lse=torch.zeros((B, ql), dtype=torch.float32)), "lse must be"),
        (dict(seq_lens=torch.zeros(B + 1, dtype=torch.int32)), "seq_lens must hold"),
        (dict(block_table=torch.zeros((B - 1, 4), dtype=torch.int32)), "block_table must be"),
        (dict(block_table=torch.zeros((B, 3), dtype=torch.int32)), "block_table must be"),
        (dict(kv_pool=torch.zeros((10, P, 576), dtype=torch.float32)), "kv_pool must be"),
        (dict(kv_pool=torch.zeros((10, P, 512), dtype=torch.bfloat16)), "kv_pool must be"),
    ]


def test_decode_binding_checks_shapes_before_any_device_work():
    """The library takes plain pointers, so the binding refuses tensors whose
    shapes disagree with the sizes the call implies (a smaller out, lse,
    seq_lens or block table would be accessed past its end)."""
    torch = pytest.importorskip("torch")
    kw = dict(max_seq_len=200, softmax_scale=0.07)
    t = _decode_tensors(torch)
    with pytest.raises(ValueError, match="GPU tensor"):   # well shaped: stops at the device check
        mla.mla_decode(**t, **kw)
    for change, msg in _shape_mistakes(torch):
        with pytest.raises(ValueError, match=msg):
            mla.mla_decode(**{**t, **change}, **kw)


def test_qparts_binding_checks_shapes():
    torch = pytest.importorskip("torch")
    kw = dict(max_seq_len=200, softmax_scale=0.07)
    t = _decode_tensors(torch)
    q = t.pop("q")
    t["q_nope"], t["q_rope"] = q[..., :512], q[..., 512:]
    with pytest.raises(ValueError, match="GPU tensor"):
        mla.mla_decode_qparts(**t, **kw)
    for change, msg in _shape_mistakes(torch):
        if msg == "out must be":
            msg = "(out|lse) must be"   # here out fixes B, q_len and H: another head count fails at lse
        with pytest.raises(ValueError, match=msg):
            mla.mla_decode_qparts(**{**t, **change}, **kw)


def test_ragged_binding_checks_shapes():
    torch = pytest.importorskip("torch")
    B, T, H = 3, 5, 16
    kw = dict(max_q_len=2, max_seq_len=200, softmax_scale=0.07)
    t = dict(q=torch.zeros((T, H, 576), dtype=torch.bfloat16), qo_indptr=torch.zeros(B + 1, dtype=torch.int32),
             kv_pool=torch.zeros((10, 64, 576), dtype=torch.bfloat16),
             block_table=torch.zeros((B, 4), dtype=torch.int32), seq_lens=torch.zeros(B, dtype=torch.int32),
             out=torch.zeros((T, H, 512), dtype=torch.bfloat16), lse=torch.zeros((T, H), dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU tensor"):
        mla.mla_decode_ragged(**t, **kw)
    for change, msg in [(dict(out=torch.zeros((T - 1, H, 512), dtype=torch.bfloat16)), "out must be"),
                        (dict(lse=torch.zeros((T, H + 1), dtype=torch.float32)), "lse must be"),
                        (dict(qo_indptr=torch.zeros(B, dtype=torch.int32)), "qo_indptr must hold"),
                        (dict(block_table=torch.zeros((B, 2), dtype=torch.int32)), "block_table must be"),
                        (dict(kv_pool=torch.zeros((10, 64, 576), dtype=torch.float16)), "kv_pool must be")]:
        with pytest.raises(ValueError, match=msg):
            mla.mla_decode_ragged(**{**t, **change}, **kw)
