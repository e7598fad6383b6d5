"""Host-side logic of the host-pool decoder (no GPU): the buffer layout and the
order in which one step queues each layer's selection, transfer and attention."""
import pytest

from sparse_kv_retrieval_amd.host_pool import HostPoolDecoder, buffer_layout


def test_buffer_layout_per_layer():
    n, buf, shared = buffer_layout(32, 2, "per-layer")
    assert (n, shared) == (32, False)
    assert buf == list(range(32))


@pytest.mark.parametrize("lookahead, nbuf", [(1, 2), (2, 2), (3, 3), (5, 5)])
def test_buffer_layout_ping_pong(lookahead, nbuf):
    n, buf, shared = buffer_layout(32, lookahead, "ping-pong")
    assert (n, shared) == (nbuf, True)
    assert buf == [l % nbuf for l in range(32)]


def test_buffer_layout_few_layers_keep_residency():
    # no more layers than buffers: every layer owns its buffer
    assert buffer_layout(2, 2, "ping-pong") == (2, [0, 1], False)
    assert buffer_layout(1, 3, "ping-pong") == (1, [0], False)


@pytest.mark.parametrize("args", [(4, 2, "rings"), (0, 2, "ping-pong"), (4, 0, "per-layer")])
def test_buffer_layout_rejects(args):
    with pytest.raises(ValueError):
        buffer_layout(*args)


def step_order(layers, lookahead, mode):
    """The calls one step() queues, as (stage, layer), with the three stages stubbed."""
    calls = []
    dec = object.__new__(HostPoolDecoder)
    dec.layers, dec.lookahead, dec.mode = layers, lookahead, mode
    dec._select = lambda l, q, timer: calls.append(("select", l))
    dec._gather = lambda l, timer: calls.append(("gather", l))
    dec._attend = lambda l, q, timer: calls.append(("attend", l))
    dec.step([None] * layers)
    return calls


@pytest.mark.parametrize("mode", ["mapped", "copy"])
@pytest.mark.parametrize("lookahead", [1, 2, 3])
@pytest.mark.parametrize("buffers", ["per-layer", "ping-pong"])
def test_step_order_is_hazard_free(mode, lookahead, buffers):
    """Every layer is selected, transferred and attended once, in that order; and
    a shared buffer is refilled for layer l only after the attention of the layer
    that used it before (l - nbuf) is queued on the compute stream.  The copy
    stream waits for the selection's event, so queueing the selection after that
    attention orders the copy after it too."""
    layers = 7
    nbuf, buf, shared = buffer_layout(layers, lookahead, buffers)
    calls = step_order(layers, lookahead, mode)
    pos = {c: i for i, c in enumerate(calls)}
    assert len(calls) == 3 * layers and len(pos) == 3 * layers
    for l in range(layers):
        assert pos[("select", l)] < pos[("gather", l)] < pos[("attend", l)]
        prev = [p for p in range(l) if buf[p] == buf[l]]
        if prev:
            assert pos[("attend", prev[-1])] < pos[("select", l)], (l, prev[-1])
    if mode == "mapped":
        # the layer-aware schedule: layer l + lookahead is selected right after attend(l)
        for l in range(layers - lookahead):
            assert pos[("select", l + lookahead)] == pos[("attend", l)] + 1
