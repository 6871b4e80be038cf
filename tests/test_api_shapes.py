"""Host-only checks of the Python binding: mis-shaped tensors raise ValueError before any
pointer reaches the library (a short tensor would otherwise be read past its end on the
device).  The tensors live on torch's meta device, so nothing is allocated or launched."""
import pytest
import torch

from decode_attention_kvq_amd import api

H, B, HQ, P = 2, 3, 8, 5
META = torch.device("meta")


def _t(*shape, dtype=torch.float32):
    return torch.empty(shape, dtype=dtype, device=META)


@pytest.fixture
def cache():
    c = api.KVCache.__new__(api.KVCache)      # skips the constructor's device checks
    c.num_pages, c.num_kv_heads, c.bits_k, c.bits_v = 4, H, 2, 2
    c.quant_k = c.quant_v = "percentile"
    c.p_lo, c.p_hi, c.alpha_k, c.alpha_v = 0.01, 0.99, 2.83, 2.83
    c.k_pages = _t(4, H, 2304, dtype=torch.uint8)
    c.v_pages = _t(4, H, 2304, dtype=torch.uint8)
    return c


@pytest.fixture
def win(cache):
    w = api.Window.__new__(api.Window)
    w.sink, w.keep, w.flush, w.num_rows, w.dtype = 2, 3, 4, B, torch.bfloat16
    w.k_win = _t(B, 9, H, 128, dtype=torch.bfloat16)
    w.v_win = _t(B, 9, H, 128, dtype=torch.bfloat16)
    return w


def _read_args():
    return dict(q=_t(B, HQ, 128), block_table=_t(B, P, dtype=torch.int32),
                seq_lens=_t(B, dtype=torch.int32), t_k_inv_t=_t(H, 128, 128), out=_t(B, HQ, 128))


def _raises_shape(fn, **kw):
    with pytest.raises(ValueError, match="shape|multiple"):
        fn(**kw)


def _well_shaped_reaches_device_check(fn, **kw):
    with pytest.raises(ValueError, match="device tensor"):
        fn(**kw)


def test_quantize_append(cache):
    good = dict(k=_t(7, H, 128), v=_t(7, H, 128), slot_mapping=_t(7, dtype=torch.int64),
                t_k=_t(H, 128, 128))
    f = lambda **kw: api.kvq_quantize_append(cache, **kw)
    _well_shaped_reaches_device_check(f, **good)
    for name, bad in [("k", _t(7, H + 1, 128)), ("k", _t(7, H, 64)), ("v", _t(6, H, 128)),
                      ("slot_mapping", _t(6, dtype=torch.int64)), ("t_k", _t(1, 128, 128)),
                      ("t_k", _t(H, 128, 127))]:
        _raises_shape(f, **{**good, name: bad})


@pytest.mark.parametrize("bad", [
    ("q", (B, HQ, 64)), ("q", (B, 3, 128)), ("block_table", (B - 1, P)), ("block_table", (B * P,)),
    ("seq_lens", (B - 1,)), ("t_k_inv_t", (H - 1, 128, 128)), ("t_k_inv_t", (H, 128, 64)),
    ("out", (B, HQ - 1, 128))])
def test_decode_attn(cache, bad):
    f = lambda **kw: api.kvq_decode_attn(cache, max_seq_len=64 * P, **kw)
    args = _read_args()
    _well_shaped_reaches_device_check(f, **args)
    name, shape = bad
    args[name] = _t(*shape, dtype=args[name].dtype)
    _raises_shape(f, **args)


@pytest.mark.parametrize("bad", [("k_new", (B, H, 100)), ("v_new", (B + 1, H, 128)),
                                 ("new_slots", (B + 1,)), ("t_k", (H, 64, 128)), ("seq_lens", (1,))])
def test_decode_step(cache, bad):
    f = lambda **kw: api.kvq_decode_step(cache, max_seq_len=64 * P, **kw)
    args = _read_args()
    args.update(k_new=_t(B, H, 128), v_new=_t(B, H, 128), new_slots=_t(B, dtype=torch.int64),
                t_k=_t(H, 128, 128))
    _well_shaped_reaches_device_check(f, **args)
    name, shape = bad
    args[name] = _t(*shape, dtype=args[name].dtype)
    _raises_shape(f, **args)


def test_dequant(cache):
    f = lambda **kw: api.kvq_dequant(cache, 0, **kw)
    _well_shaped_reaches_device_check(f, slots=_t(9, dtype=torch.int64), out=_t(9, H, 128))
    _raises_shape(f, slots=_t(9, 1, dtype=torch.int64))
    _raises_shape(f, slots=_t(9, dtype=torch.int64), out=_t(8, H, 128))


@pytest.mark.parametrize("bad", [("v", (10, H, 128)), ("cu_seqlens", (0,)), ("block_table", (B + 1, P)),
                                 ("win_rows", (B - 1,)), ("t_k", (H + 1, 128, 128))])
def test_window_prefill(cache, win, bad):
    f = lambda **kw: api.kvq_window_prefill(cache, win, **kw)
    args = dict(k=_t(11, H, 128, dtype=torch.bfloat16), v=_t(11, H, 128, dtype=torch.bfloat16),
                cu_seqlens=_t(B + 1, dtype=torch.int32), block_table=_t(B, P, dtype=torch.int32),
                win_rows=_t(B, dtype=torch.int32), t_k=_t(H, 128, 128, dtype=torch.bfloat16))
    _well_shaped_reaches_device_check(f, **args)
    name, shape = bad
    args[name] = _t(*shape, dtype=args[name].dtype)
    _raises_shape(f, **args)


@pytest.mark.parametrize("step", [False, True])
@pytest.mark.parametrize("bad", [("win_rows", (B + 2,)), ("block_table", (1, P)), ("k_new", (B, H, 127))])
def test_window_reads(cache, win, step, bad):
    args = _read_args()
    args["q"] = _t(B, HQ, 128, dtype=torch.bfloat16)
    args["win_rows"] = _t(B, dtype=torch.int32)
    if step:
        args.update(k_new=_t(B, H, 128, dtype=torch.bfloat16), v_new=_t(B, H, 128, dtype=torch.bfloat16))
        f = lambda **kw: api.kvq_window_decode_step(cache, win, max_seq_len=64 * P, **kw)
    else:
        f = lambda **kw: api.kvq_window_decode_attn(cache, win, max_seq_len=64 * P, **kw)
    _well_shaped_reaches_device_check(f, **args)
    name, shape = bad
    if name not in args:
        return
    args[name] = _t(*shape, dtype=args[name].dtype)
    _raises_shape(f, **args)
