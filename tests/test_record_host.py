"""The compact routing record of the oracle (CPU): hand-worked values, round
trips, the record's size, and the rebuild from a record.

Reading of the page "IFM K2 Horizon Deep Dive: Inside Mixture-of-Value
Attention (MoVA) ...", section "The Two Architectural Caching Strategies for
MoVA", Option B (x_t kept with the top-4 expert ids and four fp16 weights): ids
packed at 6 bits each into one 32-bit word, weights as IEEE binary16.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "compact_record.json")


def cases():
    return json.load(open(GOLDEN))["cases"]


@pytest.mark.parametrize("case", range(4))
def test_hand_worked_records(case):
    c = cases()[case]
    ids, w16 = oracle.pack_routing_record([c["idx"]], [c["w"]])
    assert int(ids[0]) == c["ids"]
    assert w16.view(np.uint16)[0].tolist() == c["w16_bits"]
    idx, w = oracle.unpack_routing_record(ids, w16, len(c["idx"]))
    assert idx[0].tolist() == c["idx"]
    assert w[0].tolist() == [float(np.uint16(b).view(np.float16)) for b in c["w16_bits"]]


def test_round_trip_and_size():
    rng = np.random.default_rng(0)
    for k in range(1, 6):
        idx = rng.integers(0, 64, size=(300, k))
        w = rng.uniform(0, 2.5, size=(300, k))
        ids, w16 = oracle.pack_routing_record(idx, w)
        assert ids.dtype == np.uint32 and w16.dtype == np.float16
        i2, w2 = oracle.unpack_routing_record(ids, w16, k)
        np.testing.assert_array_equal(i2, idx)
        np.testing.assert_array_equal(w2, w.astype(np.float16).astype(np.float64))
        assert np.abs(w2 - w).max() <= 2.5 * 2.0 ** -11  # half an fp16 step at |w| <= 2.5
        assert ids.itemsize + k * w16.itemsize == 4 + 2 * k  # bytes per token (12 at k = 4)
    with pytest.raises(ValueError):
        oracle.pack_routing_record(np.zeros((1, 6), dtype=int), np.zeros((1, 6)))
    with pytest.raises(ValueError):
        oracle.pack_routing_record([[64]], [[1.0]])


def test_rebuild_from_record_matches_rebuild_and_forward():
    """The rebuild from a record is the rebuild from the unpacked routing, and
    within the fp16 weight rounding of the layer's own forward."""
    rng = np.random.default_rng(1)
    T, d, E, k, N = 9, 32, 6, 4, 16
    x = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d)) * 0.3
    W = rng.standard_normal((E, N, d)) / np.sqrt(d)
    r = oracle.route(x, Wr, None, k, 2.5)
    ids, w16 = oracle.pack_routing_record(r.idx, r.w)
    got = oracle.rebuild_from_record(x, W, ids, w16, k)
    want = oracle.rebuild_values(x, W, r.idx, r.w.astype(np.float16).astype(np.float64))
    np.testing.assert_array_equal(got, want)
    full = oracle.value_forward(x, Wr, None, W, k, 2.5, 1, N)[0].reshape(T, N)
    silu_max = np.abs(oracle.silu(np.einsum("end,td->ten", W, x))).max()
    assert np.abs(got - full).max() <= k * 2.5 * 2.0 ** -11 * silu_max
    # An id at or beyond E marks an unused slot (possible when E < 64).
    ids2, _ = oracle.pack_routing_record(np.where(np.arange(k) == 3, 63, r.idx), r.w)
    got2 = oracle.rebuild_from_record(x, W, ids2, w16, k)
    want2 = oracle.rebuild_values(x, W, np.where(np.arange(k) == 3, -1, r.idx),
                                  r.w.astype(np.float16).astype(np.float64))
    np.testing.assert_array_equal(got2, want2)


def _golden_ok(pack, unpack):
    for c in cases():
        try:
            ids, w16 = pack([c["idx"]], [c["w"]])
        except ValueError:
            return False
        if int(ids[0]) != c["ids"] or w16.view(np.uint16)[0].tolist() != c["w16_bits"]:
            return False
        idx, _ = unpack(ids, w16, len(c["idx"]))
        if idx[0].tolist() != c["idx"]:
            return False
    return True


def test_planted_record_mistakes_fail_the_pins(monkeypatch):
    """Each plausible mistake in the record's packing fails a hand-worked case."""
    assert _golden_ok(oracle.pack_routing_record, oracle.unpack_routing_record)
    m = oracle.mova_oracle
    monkeypatch.setattr(m, "RECORD_ID_BITS", 5)  # narrower id fields
    assert not _golden_ok(m.pack_routing_record, m.unpack_routing_record)
    monkeypatch.undo()

    def reversed_slots(idx, w):  # slot 0 in the top field
        idx = np.asarray(idx)[:, ::-1]
        ids, _ = oracle.pack_routing_record(idx, w)
        return ids, np.asarray(w, dtype=np.float64).astype(np.float16)
    assert not _golden_ok(reversed_slots, oracle.unpack_routing_record)

    def truncating(idx, w):  # fp16 by truncation instead of nearest even
        ids, _ = oracle.pack_routing_record(idx, w)
        f32 = np.asarray(w, dtype=np.float32)
        bits = (f32.view(np.uint32) >> 13) & 0x3FF
        exp = ((f32.view(np.uint32) >> 23) & 0xFF).astype(np.int64) - 127 + 15
        h = np.where(f32 == 0, 0, (exp << 10) | bits).astype(np.uint16)
        return ids, h.view(np.float16)
    assert not _golden_ok(truncating, oracle.unpack_routing_record)
