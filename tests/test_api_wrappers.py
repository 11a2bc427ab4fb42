"""The user-level wrappers of the pages' interface (sequence_ring_attention_amd.api),
host side: the global-rank map of both grid numberings, and the options
attn refuses before anything runs."""
import pytest

from sequence_ring_attention_amd import api
from sequence_ring_attention_amd import binding as B


@pytest.mark.parametrize("rd,ud", [(4, 2), (2, 4), (3, 1), (1, 3), (4, 4)])
def test_rank_map_is_a_bijection_in_both_orders(rd, ud):
    for order in (api.ULYSSES_INNER, api.RING_INNER):
        cells = {api.rank_to_grid(g, rd * ud, rd, ud, order) for g in range(rd * ud)}
        assert cells == {(r, u) for r in range(rd) for u in range(ud)}


def test_rank_map_numbering():
    # Ulysses innermost: a Ulysses group is ud consecutive ranks
    assert [api.rank_to_grid(g, 8, 4, 2) for g in range(4)] == [(0, 0), (0, 1), (1, 0), (1, 1)]
    # the grid figure's numbering: GPU = 4 u + r on a 2 x 4 grid, a Ulysses group is {r, r + 4}
    assert api.rank_to_grid(5, 8, 4, 2, api.RING_INNER) == (1, 1)
    assert api.rank_to_grid(3, 8, 4, 2, api.RING_INNER) == (3, 0)


@pytest.mark.parametrize("args", [(8, 8, 4, 2), (-1, 8, 4, 2), (0, 6, 4, 2)])
def test_rank_map_rejects(args):
    with pytest.raises(ValueError):
        api.rank_to_grid(*args)
    with pytest.raises(ValueError):
        api.rank_to_grid(0, 8, 4, 2, order="diagonal")


@pytest.mark.parametrize("kw,what", [
    (dict(dropout_p=0.1), b"dropout"), (dict(window_size=(128, 0)), b"window"), (dict(softcap=30.0), b"softcap"),
    (dict(alibi_slopes=[0.5, 0.25]), b"ALiBi"),
])
def test_attn_refuses_unsupported_options_before_running(kw, what):
    # the refusal comes before any tensor is looked at
    with pytest.raises(B.UspError) as e:
        api.attn(None, None, None, 0, **kw)
    assert e.value.status == B.USP_ERR_UNSUPPORTED
    assert what.decode() in str(e.value)
