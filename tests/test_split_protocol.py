"""The tail split's counter protocol, run on the host with the library's own protocol code
(split_protocol.h over host atomics, through muon_debug_split_protocol): exactly one piece
completes a tile, it sees every other piece's partial sums, the counters are left at zero
for the next launch, and a wait that runs out sets the status word, keeps the counters and
leaves no later piece a stale count to act on."""

import pytest

import newton_schulz_02_amd as nm


@pytest.mark.parametrize("pieces", [2, 3, 5, 8])
def test_threads_one_last_piece_sees_every_slot(pieces):
    for _ in range(20):
        lasts, ok, c0, c1, status, seen, _, _ = nm.split_protocol(pieces, 0, 1 << 22)
        assert (lasts, ok, c0, c1, status, seen) == (1, 1, 0, 0, 0, pieces)


@pytest.mark.parametrize("pieces", [2, 4, 8])
def test_in_order_completes_without_waiting(pieces):
    assert nm.split_protocol(pieces, 2, 0) == [1, 1, 0, 0, 0, pieces, -1, -1]


@pytest.mark.parametrize("pieces", [2, 3, 8])
@pytest.mark.parametrize("spins", [-1, 0, 10])
def test_timeout_sets_status_and_keeps_counters(pieces, spins):
    lasts, ok, c0, c1, status, seen, c1_late, later_lasts = nm.split_protocol(pieces, 1, spins)
    assert lasts == 1 and ok == 0 and status == 1 and seen == 0
    assert c0 == pieces and c1 == pieces - 2       # nothing was cleared
    assert c1_late == pieces - 1                   # the late publish lands on the kept pair
    assert later_lasts == 0                        # no later piece takes a stale count


def test_protocol_argument_errors():
    for args in ((1, 0, 10), (9, 0, 10), (4, 3, 10), (4, 1, -2)):
        with pytest.raises(nm.MuonError):
            nm.split_protocol(*args)
    with pytest.raises(nm.MuonError):
        nm.split_spins(-3)
