"""CPU model of lce_tile's K-loop ordering of LDS buffer accesses (no GPU needed).

Every wave of a workgroup runs the same sequence: the DMA of a stage into one of two
LDS buffers (global_load_lds), a wait for its own outstanding DMA (s_waitcnt vmcnt(0)),
barriers, and the fragment reads of each K16 step, two steps ahead.  Between two
barriers the waves run at their own pace, so two accesses to one buffer conflict when
they fall in the same barrier epoch and one of them is a write, or when a read of a
stage falls before that stage's DMA has been waited for and published by a barrier.

The schedule below is the kernel's loop written as events; the checks are that
(1) every fragment read of stage s reads the buffer holding stage s after the barrier
that follows the wait for stage s's DMA, and (2) no DMA write (from issue to the
barrier after its wait) shares an epoch with a read of the same buffer.
"""

import pytest


def schedule(nk, grad=False):
    """Per-wave events: ('dma', stage, buf), ('wait',), ('barrier',), ('read', stage, step, buf).

    With grad, the gradient tiles' transposing reads of the W rows (step 'wt') are added
    where the kernel makes them: a stage's, after the wait that lands the next stage and
    before the barrier that frees the stage's buffer; the last stage's, after the final
    wait."""
    ev = [("dma", 0, 0), ("wait",), ("barrier",)]
    if nk > 1:
        ev.append(("dma", 1, 1))
    ev += [("read", 0, 0, 0), ("read", 0, 1, 0)]
    for kt in range(nk - 1):
        cur = kt & 1
        ev += [("read", kt, 2, cur), ("read", kt, 3, cur), ("wait",)]
        if grad:
            ev.append(("read", kt, "wt", cur))
        ev.append(("barrier",))
        # the last iteration re-loads stage nk - 1 into the free buffer (never read)
        ev.append(("dma", min(kt + 2, nk - 1), cur))
        ev += [("read", kt + 1, 0, cur ^ 1), ("read", kt + 1, 1, cur ^ 1)]
    cur = (nk - 1) & 1
    ev += [("read", nk - 1, 2, cur), ("read", nk - 1, 3, cur), ("wait",)]
    if grad:
        ev.append(("read", nk - 1, "wt", cur))
    return ev


def check(nk, grad=False):
    ev = schedule(nk, grad)
    epoch = 0
    pending = []          # DMAs issued and not yet waited for: (stage, buf, issue epoch)
    writes = []           # (buf, first epoch, last epoch) of each DMA's write window
    published = {}        # stage -> (buf, epoch from which its data may be read)
    landed = []           # DMAs waited for, published at the next barrier
    reads = []            # (buf, epoch)
    for e in ev:
        if e[0] == "dma":
            pending.append((e[1], e[2], epoch))
        elif e[0] == "wait":
            landed += pending
            pending = []
        elif e[0] == "barrier":
            for stage, buf, e0 in landed:
                writes.append((buf, e0, epoch))
                published.setdefault(stage, (buf, epoch + 1))
            landed = []
            epoch += 1
        else:
            _, stage, step, buf = e
            assert stage in published, f"nk={nk}: stage {stage} read before its DMA was published"
            pbuf, pe = published[stage]
            assert pbuf == buf and epoch >= pe, f"nk={nk}: stage {stage} step {step} read too early"
            reads.append((buf, epoch))
    # writes still in flight at the end run to the kernel's final wait
    for stage, buf, e0 in landed + pending:
        writes.append((buf, e0, epoch))
    for buf, e0, e1 in writes:
        for rbuf, re in reads:
            if rbuf == buf and e0 <= re <= e1:
                # a read in the window is only allowed of the data this DMA brings,
                # which would have to be published after e1: impossible inside it
                raise AssertionError(f"nk={nk}: buffer {buf} written in epochs {e0}..{e1}, read in {re}")


@pytest.mark.parametrize("nk", [1, 2, 3, 4, 5, 64, 65])
@pytest.mark.parametrize("grad", [False, True])
def test_two_ahead_pipeline_has_no_lds_race(nk, grad):
    check(nk, grad)


def test_model_catches_transposing_reads_after_the_barrier():
    """Reading a stage's W rows after its buffer is freed (past the barrier) is a race."""
    real = schedule

    def late(nk, grad=False):
        ev = [e for e in real(nk) if e[0] != "read" or e[2] != "wt"]
        k = [i for i, e in enumerate(ev) if e[0] == "barrier"][2]
        return ev[:k + 2] + [("read", 1, "wt", 1)] + ev[k + 2:]

    globals()["schedule"] = late
    try:
        with pytest.raises(AssertionError):
            check(4)
    finally:
        globals()["schedule"] = real


def test_model_catches_a_missing_barrier():
    """The checker itself: dropping the stage barrier must be reported."""
    real = schedule

    def no_barrier(nk, grad=False):
        ev = real(nk, grad)
        i = [k for k, e in enumerate(ev) if e[0] == "barrier"][1]
        return ev[:i] + ev[i + 1:]

    globals()["schedule"] = no_barrier
    try:
        with pytest.raises(AssertionError):
            check(4)
    finally:
        globals()["schedule"] = real


def test_model_catches_reads_three_ahead_with_this_barrier():
    """Reading a third step ahead (stage kt + 1 step 2 before the barrier) is a race."""
    real = schedule

    def too_far(nk, grad=False):
        ev = real(nk, grad)
        k = [i for i, e in enumerate(ev) if e[0] == "wait"][1]
        return ev[:k] + [("read", 1, 2, 1)] + ev[k:]

    globals()["schedule"] = too_far
    try:
        with pytest.raises(AssertionError):
            check(4)
    finally:
        globals()["schedule"] = real
