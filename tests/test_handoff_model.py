"""CPU model of the route handoff inside the small-batch grouped GEMM (the two-kernel step).

The kernel's protocol, restated as a discrete simulation of workgroups on a limited number of
CU slots with in-order dispatch:
  - token t is routed by wave t // G of workgroup t % G, before that wave waits for anything;
    each route is published as one word TAG_BASE | epoch << 8 | expert, which carries its own
    validity;
  - every workgroup with weight slices polls the route words it reads until they carry this
    call's tag, for at most max_polls rounds; words still missing after that are routed by
    the waiting workgroup itself (the same selection, so the same experts), which sets the
    status word;
  - the combine clears the route words after the step.
The model checks three things:
  - the protocol ends with every workgroup holding the right routes, whether or not the
    routing workgroups fit on the chip at once;
  - it sets the status only when a workgroup had to route for itself;
  - words left by an earlier call, and old bytes, never pass for fresh routes.
It runs on the host only and does not execute the kernel."""
import numpy as np
import pytest

TAG_BASE = 0x7FA00000
TAG_MASK = 0xFFFFFF00


def tag_of(epoch):
    return TAG_BASE | ((epoch & 0xFFF) << 8)


def simulate(M, k, G, slots, slices_of, max_polls, words, route_of, epoch=5):
    """Workgroups 0..G-1 dispatched in order onto `slots` CU slots.  One simulated tick is
    one poll round, or one unit of routing work.  Returns (ids seen per workgroup, status,
    ticks)."""
    R = M * k
    tag = tag_of(epoch)
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
                        words[t * k + j] = tag | route_of(t, j)
                st["route"] = []
                continue
            if slices_of(wg) == 0:       # no weight slices: done after routing
                del running[wg]
                continue
            have = [(int(words[r]) & TAG_MASK) == tag for r in range(R)]
            if all(have):
                seen[wg] = [int(words[r]) & 0xFF for r in range(R)]
                del running[wg]
            elif st["polls"] >= max_polls:
                # route the missing tokens itself: the same selection gives the same experts
                status = 1
                seen[wg] = [int(words[r]) & 0xFF if have[r] else route_of(r // k, r % k)
                            for r in range(R)]
                del running[wg]
            else:
                st["polls"] += 1
        assert tick < 10 ** 6
    return seen, status, tick


def route_of(t, j):
    return (7 * t + 3 * j) % 256


def want(M, k):
    return [route_of(r // k, r % k) for r in range(M * k)]


@pytest.mark.parametrize("M,k,G,slots", [(128, 8, 256, 256), (128, 8, 256, 130),
                                         (300, 4, 256, 256), (1, 1, 256, 1)])
def test_handoff_finishes_when_routing_workgroups_are_resident(M, k, G, slots):
    words = np.zeros(M * k, np.uint32)
    seen, status, _ = simulate(M, k, G, slots, lambda wg: 32, 1000, words, route_of)
    assert status == 0
    assert len(seen) == G and all(v == want(M, k) for v in seen.values())


def test_late_routing_workgroups_are_covered_by_the_waiting_ones():
    # 300 tokens need all 256 workgroups resident (waves 0 and 1 route); with 200 slots the
    # resident ones wait for routes whose workgroups are not dispatched yet: each wait ends
    # at its bound, the waiting workgroup routes the missing tokens itself (status set), the
    # slots free up, and the rest run; every workgroup ends with the right routes
    words = np.zeros(300 * 4, np.uint32)
    seen, status, ticks = simulate(300, 4, 256, 200, lambda wg: 32, 50, words, route_of)
    assert status == 1 and ticks < 10 ** 6
    assert len(seen) == 256 and all(v == want(300, 4) for v in seen.values())


def test_no_handoff_routes_everything_locally():
    # max_polls = 0 (the self-routing flag): no wait at all, the same routes everywhere
    words = np.zeros(128 * 8, np.uint32)
    seen, status, _ = simulate(128, 8, 256, 256, lambda wg: 32, 0, words, route_of)
    assert all(v == want(128, 8) for v in seen.values())


@pytest.mark.parametrize("old", ["cleared", "bytes_0xA5", "slot_ids", "previous_call",
                                 "floats", "e4m3_codes"])
def test_old_words_never_pass_for_routes(old):
    # what the route words can hold at launch: cleared words (the combine zeroes them), old
    # bytes, route slots of a staged step in the same workspace part, the previous call's
    # words (an older epoch), or float data and E4M3 codes of other tensors; none carries
    # this call's tag
    R = 128 * 8
    epoch = 77
    rng = np.random.default_rng(0)
    if old == "cleared":
        words = np.zeros(R, np.uint32)
    elif old == "bytes_0xA5":
        words = np.full(R, 0xA5A5A5A5, np.uint32)
    elif old == "slot_ids":
        words = np.arange(R, dtype=np.uint32)
    elif old == "previous_call":
        words = np.array([tag_of(epoch - 1) | route_of(r // 8, r % 8) for r in range(R)],
                         np.uint32)
    elif old == "floats":
        f = np.concatenate([rng.standard_normal(R - 6).astype(np.float32) * 1e30,
                            np.array([np.inf, -np.inf, np.nan, -np.nan, 3.4e38, -0.0],
                                     np.float32)])
        words = f.view(np.uint32)
    else:
        codes = rng.integers(0, 256, 4 * R, dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x7E          # the encoder saturates, never 0x7F
        words = codes.view(np.uint32)
    assert not ((words & TAG_MASK) == tag_of(epoch)).any()


def test_every_tag_is_a_signalling_nan_with_a_0x7F_byte():
    # as a float every route word is a NaN with the quiet bit clear (computed NaNs are the
    # quiet default 0x7FC00000, infinities 0x7F800000 / 0xFF800000), and its top byte is 0x7F,
    # a code the E4M3 encoder never writes
    for epoch in (0, 1, 0xFFF, 0x1000, 123456):
        for e in (0, 1, 255):
            w = np.array([tag_of(epoch) | e], np.uint32)
            f = w.view(np.float32)[0]
            assert np.isnan(f)
            assert (int(w[0]) >> 22) & 1 == 0                     # quiet bit clear
            assert int(w[0]) >> 24 == 0x7F
            assert int(w[0]) != 0x7F800000
