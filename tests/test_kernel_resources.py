"""Register and scratch budgets of the compiled kernels (from the compiler's
resource figures that the build records).

* No kernel spills to scratch memory.
* Every kernel that waits for AllGather chunk flags (the dense AllGather
  modes and every MoE layer-0 form) leaves room on each SIMD for one wave of
  the chunk-push kernel.  A consumer launch may fill every compute unit while
  it waits; a push kernel on another stream that is dispatched after it must
  still find registers beside it, or the consumer only ever ends by its spin
  limit."""
import json
import re

import pytest

pytestmark = pytest.mark.usefixtures("built_library")

REGS_PER_SIMD = 512      # unified VGPR + AGPR file per SIMD lane (gfx950)


def _kernels():
    from tile_gemm_communication_amd import build
    return json.load(open(build.RESOURCES))


def _alloc(k):
    """Registers one wave is given: VGPRs rounded to 4, then AGPRs, in 8s."""
    v = -(-k.get("vgpr", 0) // 4) * 4
    return -(-(v + k.get("agpr", 0)) // 8) * 8


def _template_ints(name):
    return [int(x) for x in re.findall(r"Li(\d+)E", name)]


def test_every_kernel_is_listed_and_none_spills():
    ks = _kernels()
    names = [k["name"] for k in ks]
    assert any("push_kernel" in n for n in names)
    assert sum("dense_kernel" in n for n in names) > 20
    assert sum("moe_kernel" in n for n in names) > 20
    spill = [k["name"] for k in ks if k.get("scratch", 0) != 0]
    assert not spill, spill


def test_chunk_consumers_leave_room_for_their_producers():
    """The AllGather consumers against the kernels that publish their flags
    from another stream: the chunk push for the gathered-buffer forms (dense
    mode AG, MoE layer 0 with or without flags), the paced signal for the pull
    forms (dense mode AGP, MoE layer 0 pull).  The in-launch producer forms
    share one launch and need no room."""
    ks = _kernels()
    need = {}
    for key, pat in (("push", "push_kernel"), ("paced", "paced_kernel")):
        found = [k for k in ks if pat in k["name"]]
        assert len(found) == 1, pat
        need[key] = _alloc(found[0])
    checked = 0
    for k in ks:
        n = k["name"]
        if "dense_kernel" in n:
            # dense_kernel<E, BM, BN, NW, Mode, ...>
            mode = int(re.search(r"ModeE(\d+)E", n).group(1))
            if mode not in (1, 4):
                continue
            producer = "paced" if mode == 4 else "push"
        elif "moe_kernel" in n:
            # moe_kernel<E, BM, BN, NW, SCATTER, KTAIL, PULL, ACT>
            scatter, _, pull = re.findall(r"Lb([01])E", n)[:3]
            if scatter == "1":
                continue
            producer = "paced" if pull == "1" else "push"
        else:
            continue
        nw = _template_ints(n)[2]
        free = REGS_PER_SIMD - (nw // 4) * _alloc(k)
        assert free >= need[producer], (n, k, free, producer, need[producer])
        checked += 1
    assert checked > 20
