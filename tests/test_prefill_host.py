"""Host-side checks of the chunked-prefill driver (no GPU): arguments are
refused before any library call is made."""
import pytest

torch = pytest.importorskip("torch")
cqb = pytest.importorskip("extreme_bit_kv_amd", reason="libcq.so not built")
from extreme_bit_kv_amd.prefill import ChunkedVisualQuantizer  # noqa: E402


def _caches(rows=1024):
    return torch.zeros((1, 2, rows, 128), dtype=torch.float16), torch.zeros((1, 2, rows, 128), dtype=torch.float16)


def test_segment_must_fit_the_cache():
    k, v = _caches(1024)
    with pytest.raises(ValueError):
        ChunkedVisualQuantizer(k, v, 1025)
    with pytest.raises(ValueError):
        ChunkedVisualQuantizer(k, v, 1000, row0=32)
    with pytest.raises(ValueError):
        ChunkedVisualQuantizer(k, v, 0)
    with pytest.raises(ValueError):
        ChunkedVisualQuantizer(k, torch.zeros((1, 2, 512, 128), dtype=torch.float16), 256)


def test_appends_must_stay_in_the_segment():
    k, v = _caches()
    q = ChunkedVisualQuantizer(k, v, 512)
    with pytest.raises(ValueError):
        q.append(513)
    with pytest.raises(ValueError):
        q.append(0)
    with pytest.raises(ValueError):
        q.finish()                       # nothing appended yet


def test_code_buffers_have_the_library_layout():
    k, v = _caches()
    q = ChunkedVisualQuantizer(k, v, 992, bits=2)
    kc, vc = q.out[cqb.CQ_LAYOUT_K][0], q.out[cqb.CQ_LAYOUT_V][0]
    assert tuple(kc.shape) == cqb.code_words_shape(1, 2, 992, 128, 2, cqb.CQ_LAYOUT_K) == (1, 2, 8, 992)
    assert tuple(vc.shape) == cqb.code_words_shape(1, 2, 992, 128, 2, cqb.CQ_LAYOUT_V) == (1, 2, 62, 128)


def test_row_window_of_the_binding():
    """The segment pointer is x's base plus row0 rows; windows past x are refused."""
    from extreme_bit_kv_amd._binding import _rows_ptr
    k, _ = _caches(256)
    assert _rows_ptr(k, 0, 0, 256).value == k.data_ptr()
    assert _rows_ptr(k, 32, 96, 128).value == k.data_ptr() + 32 * 128 * 2
    for row0, t0, m in ((200, 0, 64), (0, 224, 64), (-1, 0, 1), (0, -32, 32), (0, 0, -1)):
        with pytest.raises(ValueError):
            _rows_ptr(k, row0, t0, m)


def test_binding_refuses_host_tensors():
    k, _ = _caches(256)
    with pytest.raises(ValueError):
        cqb.cq_kv_range_update(k, 0, 64, reset=True)


def test_segment_so_far_needs_eager_codes_and_rows():
    k, v = _caches()
    with pytest.raises(ValueError):
        ChunkedVisualQuantizer(k, v, 512).current()            # deferred codes: nothing to decode between appends
    with pytest.raises(ValueError):
        ChunkedVisualQuantizer(k, v, 512, eager=True).current()    # nothing appended yet
    q = ChunkedVisualQuantizer(k, v, 1000, eager=True)
    q.t = 512                                                  # (as after appends of 512 rows)
    with pytest.raises(ValueError):
        q.current()                                            # capacity 1000 is no multiple of 32
    q = ChunkedVisualQuantizer(k, v, 992, eager=True)
    q.t = 512
    cur = q.current()
    assert (cur.n, cur.n_cap) == (512, 992)
