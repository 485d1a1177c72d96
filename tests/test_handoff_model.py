"""CPU model of the route handoff inside the small-batch grouped GEMM (MOE_FWD_FUSED_ROUTE).

The kernel's protocol, restated as a discrete simulation of workgroups on a limited number of
CU slots with in-order dispatch:
  - token t is routed by wave t // G of workgroup t % G, before that wave waits for anything;
    each route is published as one word kRouteTag | expert (a word carries its own validity);
  - every workgroup with weight slices waits until the route words it reads carry the tag, for
    at most a bounded number of polls; a wait that gives up sets the status word and the
    workgroup skips its work;
  - the combine clears the route words after the step.
The model checks that the protocol finishes whenever the routing workgroups fit on the chip at
once, that it ends with the status set (never hangs) when they do not, and that words left by
an earlier step or old bytes never pass for fresh routes.  It runs on the host only and does
not execute the kernel."""
import numpy as np
import pytest

TAG = 0x7FBA0000


def simulate(M, k, G, slots, slices_of, max_polls, words, route_of):
    """Workgroups 0..G-1 dispatched in order onto `slots` CU slots; one simulated tick = one
    poll round or one unit of routing work.  Returns (ids seen per workgroup, status, ticks)."""
    R = M * k
    status = 0
    pending = list(range(G))
    running = {}                        # wg -> state dict
    seen = {}
    tick = 0
    while pending or running:
        while pending and len(running) < slots:
            wg = pending.pop(0)
            tokens = [t for t in range(M) if t % G == wg]
            running[wg] = {"route": tokens, "polls": 0}
        tick += 1
        for wg in list(running):
            st = running[wg]
            if st["route"]:              # routing waves publish first, waiting for nothing
                for t in st["route"]:
                    for j in range(k):
                        words[t * k + j] = TAG | route_of(t, j)
                st["route"] = []
                continue
            if slices_of(wg) == 0:       # no weight slices: done after routing
                del running[wg]
                continue
            ready = all((words[r] & 0xFFFF0000) == TAG for r in range(R))
            if ready:
                seen[wg] = [words[r] & 0xFFFF for r in range(R)]
                del running[wg]
            else:
                st["polls"] += 1
                if st["polls"] >= max_polls:
                    status = 1
                    del running[wg]
        assert tick < 10 ** 6
    return seen, status, tick


def route_of(t, j):
    return (7 * t + 3 * j) % 256


@pytest.mark.parametrize("M,k,G,slots", [(128, 8, 256, 256), (128, 8, 256, 130),
                                         (300, 4, 256, 256), (1, 1, 256, 1)])
def test_handoff_finishes_when_routing_workgroups_are_resident(M, k, G, slots):
    words = np.zeros(M * k, np.uint32)
    seen, status, _ = simulate(M, k, G, slots, lambda wg: 32, 1000, words, route_of)
    assert status == 0
    want = [route_of(r // k, r % k) for r in range(M * k)]
    assert len(seen) == G and all(v == want for v in seen.values())


def test_handoff_gives_up_instead_of_hanging():
    # 300 tokens need all 256 workgroups resident (waves 0 and 1 route); with 200 slots the
    # resident ones wait for routes whose workgroups are never dispatched: every wait ends at
    # its bound with the status set, the slots free up, and the rest run
    words = np.zeros(300 * 4, np.uint32)
    seen, status, ticks = simulate(300, 4, 256, 200, lambda wg: 32, 50, words, route_of)
    assert status == 1 and ticks < 10 ** 6


@pytest.mark.parametrize("old", ["previous_step_cleared", "bytes_0xA5", "zeros", "slot_ids"])
def test_old_words_never_pass_for_routes(old):
    # what the route words can hold at launch: cleared words (the combine zeroes them), old
    # bytes, or route slots of a staged step in the same workspace part; none carries the tag
    R = 128 * 8
    if old == "previous_step_cleared":
        words = np.zeros(R, np.uint32)
    elif old == "bytes_0xA5":
        words = np.full(R, 0xA5A5A5A5, np.uint32)
    elif old == "zeros":
        words = np.zeros(R, np.uint32)
    else:
        words = np.arange(R, dtype=np.uint32)
    assert not ((words & 0xFFFF0000) == TAG).any()
    # a workgroup that polls before any routing wave ran sees no route
    assert not all((words[r] & 0xFFFF0000) == TAG for r in range(R))


def test_tag_is_no_value_the_library_stores():
    # the tag's high half 0x7FBA as the top of a float is a signalling NaN (computed NaNs are
    # the default quiet one, 0x7FC00000) and holds the byte 0x7F, which the E4M3 encoder never
    # writes (it saturates to 0x7E); ids, counts and slots are far below 2^16 << 16
    f = np.array([TAG | 0x1234], np.uint32).view(np.float32)[0]
    assert np.isnan(f)
    assert (TAG >> 22) & 1 == 0                                  # quiet bit clear
    assert 0x7F in np.array([TAG], np.uint32).view(np.uint8)
    assert TAG > 2 ** 16 * 1024
