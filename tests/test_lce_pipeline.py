"""CPU model of lce_tile's K-loop ordering of LDS buffer accesses (no GPU needed).

Every wave of a workgroup runs the same sequence: the DMA of a stage's A rows into one
of two A buffers and of its B rows into one of three B buffers (buffer_load ... lds),
waits for its own outstanding DMA (s_waitcnt vmcnt(n): all but the last n loads, which
retire in order), barriers, and the fragment reads of each K16 step, two steps ahead.
Between two barriers the waves run at their own pace, so two accesses to one buffer
conflict when they fall in the same barrier epoch and one of them is a write, or when a
read of a stage falls before that stage's DMA has been waited for and published by a
barrier.

The schedule below is the kernel's loop written as events; the checks are that
(1) every fragment read of stage s reads, for each operand, the buffer holding stage s
after the barrier that follows the wait for that DMA, and (2) no DMA write (from issue
to the barrier after its wait) shares an epoch with a read of the same buffer.
"""

import pytest


def schedule(nk, grad=False):
    """Per-wave events: ('dma', op, stage, buf) with op 'A' or 'B'; ('wait', keep): every
    DMA but the last `keep` issued has landed; ('barrier',); ('read', stage, step,
    abuf, bbuf), where step 'wt' (the gradient tiles' transposing reads of the W rows,
    a stage's after the wait that lands the next stage and before the barrier that
    frees its buffer, the last stage's after the final wait) reads only the B buffer."""
    ev = [("dma", "A", 0, 0), ("dma", "B", 0, 0), ("wait", 0), ("barrier",)]
    if nk > 1:
        ev += [("dma", "B", 1, 1), ("dma", "A", 1, 1)]
    ev += [("read", 0, 0, 0, 0), ("read", 0, 1, 0, 0)]
    cb = 0
    for kt in range(nk - 1):
        ca = kt & 1
        b_next = (cb + 1) % 3
        b_load = (b_next + 1) % 3
        # the last iteration re-loads stage nk - 1 into free buffers (never read)
        kl = min(kt + 2, nk - 1)
        # steps 0 and 1: stage kt's steps 2 and 3 read, the B rows of stage kt + 2 loaded
        ev += [("read", kt, 2, ca, cb), ("dma", "B", kl, b_load), ("read", kt, 3, ca, cb)]
        ev.append(("wait", 1))
        if grad:
            ev.append(("read", kt, "wt", None, cb))
        ev.append(("barrier",))
        # steps 2 and 3: the A rows of stage kt + 2 loaded, stage kt + 1's steps 0, 1 read
        ev += [("dma", "A", kl, ca), ("read", kt + 1, 0, ca ^ 1, b_next), ("read", kt + 1, 1, ca ^ 1, b_next)]
        cb = b_next
    ca = (nk - 1) & 1
    ev += [("read", nk - 1, 2, ca, cb), ("read", nk - 1, 3, ca, cb), ("wait", 0)]
    if grad:
        ev.append(("read", nk - 1, "wt", None, cb))
    return ev


def check(nk, grad=False, sched=None):
    ev = (sched or schedule)(nk, grad)
    epoch = 0
    pending = []          # DMAs issued and not yet waited for: (op, stage, buf, issue epoch)
    writes = []           # (op, buf, first epoch, last epoch) of each DMA's write window
    published = {}        # (op, stage) -> (buf, epoch from which its data may be read)
    landed = []           # DMAs waited for, published at the next barrier
    reads = []            # (op, buf, epoch)
    for e in ev:
        if e[0] == "dma":
            pending.append((e[1], e[2], e[3], epoch))
        elif e[0] == "wait":
            keep = e[1]
            cut = len(pending) - keep
            landed += pending[:cut]
            pending = pending[cut:]
        elif e[0] == "barrier":
            for op, stage, buf, e0 in landed:
                writes.append((op, buf, e0, epoch))
                published.setdefault((op, stage), (buf, epoch + 1))
            landed = []
            epoch += 1
        else:
            _, stage, step, abuf, bbuf = e
            for op, buf in (("A", abuf), ("B", bbuf)):
                if buf is None:
                    continue
                assert (op, stage) in published, f"nk={nk}: stage {stage} {op} read before its DMA was published"
                pbuf, pe = published[(op, stage)]
                assert pbuf == buf and epoch >= pe, f"nk={nk}: stage {stage} step {step} {op} read too early"
                reads.append((op, buf, epoch))
    # writes still in flight at the end run to the kernel's final wait
    for op, stage, buf, e0 in landed + pending:
        writes.append((op, buf, e0, epoch))
    for op, buf, e0, e1 in writes:
        for rop, rbuf, re in reads:
            if rop == op and rbuf == buf and e0 <= re <= e1:
                # a read in the window is only allowed of the data this DMA brings,
                # which would have to be published after e1: impossible inside it
                raise AssertionError(f"nk={nk}: {op} buffer {buf} written in epochs {e0}..{e1}, read in {re}")


@pytest.mark.parametrize("nk", [1, 2, 3, 4, 5, 6, 7, 64, 65])
@pytest.mark.parametrize("grad", [False, True])
def test_two_ahead_pipeline_has_no_lds_race(nk, grad):
    check(nk, grad)


def mutated(fn):
    def sched(nk, grad=False):
        return fn(schedule(nk, grad))
    return sched


def test_model_catches_transposing_reads_after_the_barrier():
    """Reading a stage's W rows after its buffer is freed (past the barrier) is a race."""
    def late(ev):
        ev = [e for e in ev if e[0] != "read" or e[2] != "wt"]
        k = [i for i, e in enumerate(ev) if e[0] == "barrier"][2]
        return ev[:k + 2] + [("read", 1, "wt", None, 1)] + ev[k + 2:]
    with pytest.raises(AssertionError):
        check(5, sched=mutated(late))


def test_model_catches_a_missing_barrier():
    """The checker itself: dropping the stage barrier must be reported."""
    def no_barrier(ev):
        i = [k for k, e in enumerate(ev) if e[0] == "barrier"][1]
        return ev[:i] + ev[i + 1:]
    with pytest.raises(AssertionError):
        check(4, sched=mutated(no_barrier))


def test_model_catches_reads_three_ahead_with_this_barrier():
    """Reading a third step ahead (stage kt + 1 step 2 before the barrier) is a race."""
    def too_far(ev):
        k = [i for i, e in enumerate(ev) if e[0] == "wait"][1]
        return ev[:k] + [("read", 1, 2, 1, 1)] + ev[k:]
    with pytest.raises(AssertionError):
        check(4, sched=mutated(too_far))


def test_model_catches_b_rows_loaded_into_a_buffer_in_use():
    """With two B buffers (the B rows of stage kt + 2 into stage kt's), the early B load
    would overwrite rows that steps 0 and 1 are still reading."""
    def two_b(ev):
        out = []
        for e in ev:
            if e[0] == "dma" and e[1] == "B":
                e = ("dma", "B", e[2], e[2] % 2)
            elif e[0] == "read" and e[4] is not None:
                e = e[:4] + (e[1] % 2,)
            out.append(e)
        return out
    with pytest.raises(AssertionError, match="written in epochs"):
        check(6, sched=mutated(two_b))


def test_model_catches_a_wait_that_leaves_the_next_stage_pending():
    """Keeping two loads groups in flight at the barrier (vmcnt(16)) would publish stage
    kt + 1's A rows before they land."""
    def lax(ev):
        return [("wait", 2) if e == ("wait", 1) else e for e in ev]
    with pytest.raises(AssertionError):
        check(4, sched=mutated(lax))
