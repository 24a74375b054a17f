"""The early-release ring protocol of gemm_early, checked on the host: the
kernel's own step tables (csrc/ring_plan.hpp) replayed by tests/ring_model.cpp
for the four waves of a workgroup, for every format and for persistent runs of
several tiles ("B200 TMA Pipeline Designer", section E step 8: validate that
each stage's ready and free have a unique producer and consumer; section B:
consuming right after the load is issued, or reusing a buffer before the
readers are done, are the failure modes).  The mutation cases move a load
into phase A, drop a barrier or a wait, or weaken a wait count, and the
model must report each."""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matrix_core_engineering_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "ring_model.cpp")

OPS = {0: "bf16 32x32x16", 1: "bf16 16x16x32", 2: "MX E4M3", 3: "MX E4M3 scale groups",
       4: "MX E5M2", 5: "MX E5M2 scale groups", 6: "MX E2M1",
       7: "level 9 bf16 32x32x16", 8: "level 9 bf16 16x16x32", 9: "level 9 MX E4M3",
       10: "level 9 MX E5M2"}


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    so = tmp_path_factory.mktemp("ringmodel") / "libringmodel.so"
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", f"-I{CSRC}", SRC, "-o", str(so)],
                   check=True)
    lib = ctypes.CDLL(str(so))
    ip = ctypes.POINTER(ctypes.c_int)
    lib.ring_model.argtypes = [ctypes.c_int, ip, ctypes.c_int, ip, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, ctypes.c_char_p, ctypes.c_int]
    lib.ring_step_id.argtypes = [ctypes.c_char_p]
    return lib


def tables(lib):
    buf = (ctypes.c_int * 64)()
    n = lib.ring_prologue_steps(buf)
    pro = list(buf[:n])
    n = lib.ring_loop_steps(buf)
    return pro, list(buf[:n])


def check(lib, op, pro, loop, tiles, nk, wait_delta=0):
    msg = ctypes.create_string_buffer(512)
    a = (ctypes.c_int * len(pro))(*pro)
    b = (ctypes.c_int * len(loop))(*loop)
    n = lib.ring_model(op, a, len(pro), b, len(loop), tiles, nk, wait_delta, msg, 512)
    assert n >= 0
    return n, msg.value.decode()


def sid(lib, name):
    i = lib.ring_step_id(name.encode())
    assert i >= 0, name
    return i


def shapes(lib, op):
    """Persistent runs with ragged tails: workgroups with 0, 1, 2, 3 or 5
    tiles, each of nk K tiles (a whole number of scale groups)."""
    u = lib.ring_unroll(op)
    nks = sorted({max(2, u), 2 * max(2, u), 4 * u if u > 1 else 3, 16 if u > 1 else 5})
    return [(t, nk) for t in (0, 1, 2, 3, 5) for nk in nks if nk % u == 0]


@pytest.mark.parametrize("op", list(OPS), ids=list(OPS.values()))
def test_kernel_tables_are_race_free(model, op):
    pro, loop = tables(model)
    for tiles, nk in shapes(model, op):
        n, msg = check(model, op, pro, loop, tiles, nk)
        assert n == 0, f"{OPS[op]} tiles={tiles} nk={nk}: {msg}"


def move(seq, item, before):
    s = list(seq)
    s.remove(item)
    s.insert(s.index(before), item)
    return s


def drop_nth(seq, item, nth):
    s = list(seq)
    idx = [i for i, x in enumerate(s) if x == item][nth]
    del s[idx]
    return s


MUTATIONS = ["load into phase A", "drop barrier 1", "drop barrier 2", "drop vm wait",
             "drop lgkm wait", "head read before ready", "weaker vm wait", "drop pending loads",
             "drop prologue wait", "drop prologue barrier", "tail read after free"]


@pytest.mark.parametrize("op", list(OPS), ids=list(OPS.values()))
@pytest.mark.parametrize("mutation", MUTATIONS)
def test_protocol_mutations_are_caught(model, op, mutation):
    pro, loop = tables(model)
    s = lambda n: sid(model, n)
    delta = 0
    if mutation == "load into phase A":
        loop = move(loop, s("ISSUE_X"), s("WAIT_LGKM"))
    elif mutation == "drop barrier 1":
        loop = drop_nth(loop, s("BARRIER"), 0)
    elif mutation == "drop barrier 2":
        loop = drop_nth(loop, s("BARRIER"), 1)
    elif mutation == "drop vm wait":
        loop = drop_nth(loop, s("WAIT_VM"), 0)
    elif mutation == "drop lgkm wait":
        loop = drop_nth(loop, s("WAIT_LGKM"), 0)
    elif mutation == "head read before ready":
        loop = move(loop, s("READ_HEAD"), s("WAIT_VM"))
    elif mutation == "weaker vm wait":
        delta = 1
    elif mutation == "drop pending loads":
        loop = drop_nth(loop, s("ISSUE_PENDING"), 0)
    elif mutation == "drop prologue wait":
        pro = drop_nth(pro, s("WAIT_VM_PRO"), 0)
    elif mutation == "drop prologue barrier":
        pro = drop_nth(pro, s("BARRIER"), 0)
    elif mutation == "tail read after free":
        loop = move(loop, s("READ_TAIL"), s("ISSUE_X"))
    caught = [check(model, op, pro, loop, t, nk, delta)[0] for t, nk in shapes(model, op) if t > 0]
    if mutation == "drop pending loads" and model.ring_pending_loads(op) == 0:
        # formats whose K tiles leave no loads for phase A lose nothing:
        # the step issues an empty range there
        assert not any(caught)
        return
    assert all(c > 0 for c in caught), f"{mutation} not caught for {OPS[op]}: {caught}"
