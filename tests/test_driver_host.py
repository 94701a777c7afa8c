"""Host logic of the sampling-loop driver: the dense/sparse schedule window.

The pages ("BSAI FastH3 Native VSA (recipe)", "The inputs that matter"; "ComfyUI Agrega
Nodo Central de Atencion Dispersa y Compilador Comfy", schedule and benchmark paragraphs)
keep short sequences, the steps outside the start/end window and the first transformer
layer dense.
"""
import pytest

from block_sparse_video_geometry_amd.driver import Schedule

LONG = 36096


def test_defaults_dense_first_layer_only():
    s = Schedule()
    assert not s.sparse(0, 4, 0, LONG)
    assert all(s.sparse(i, 4, layer, LONG) for i in range(4) for layer in (1, 2, 47))


def test_min_tokens_keeps_short_sequences_dense():
    s = Schedule(min_tokens=8192)
    assert not s.sparse(2, 4, 3, 8191)
    assert s.sparse(2, 4, 3, 8192)
    assert Schedule(min_tokens=0).sparse(0, 1, 1, 1)


def test_warmup_window():
    s = Schedule(start_percent=0.2, end_percent=1.0, dense_layers=())
    got = [s.sparse(i, 10, 5, LONG) for i in range(10)]
    assert got == [False, False] + [True] * 8
    # 19 steps: progress 3/19 = 0.158 < 0.2 stays dense, 4/19 = 0.21 is sparse
    got = [s.sparse(i, 19, 5, LONG) for i in range(19)]
    assert got == [False] * 4 + [True] * 15


def test_tail_window():
    s = Schedule(start_percent=0.0, end_percent=0.5, dense_layers=())
    assert [s.sparse(i, 10, 1, LONG) for i in range(10)] == [True] * 5 + [False] * 5
    s = Schedule(start_percent=0.3, end_percent=0.3, dense_layers=())
    assert not any(s.sparse(i, 10, 1, LONG) for i in range(10))


@pytest.mark.parametrize("kw", [dict(start_percent=-0.1), dict(end_percent=1.5),
                                dict(start_percent=0.6, end_percent=0.4), dict(min_tokens=-1)])
def test_bad_schedules(kw):
    with pytest.raises(ValueError):
        Schedule(**kw)


@pytest.mark.parametrize("step,n", [(-1, 4), (4, 4), (0, 0)])
def test_bad_steps(step, n):
    with pytest.raises(ValueError):
        Schedule().sparse(step, n, 1, LONG)
