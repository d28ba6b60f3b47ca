"""Drives fixture operation lists against any block-manager implementation.

The adapter protocol (implemented by the oracle model and by the C++ block
manager's Python binding): allocate, append, fork, share_prefix, free_seq,
block_table, num_tokens, refcount, free_list, available_blocks, state.
Errors surface as exceptions carrying a ``code`` attribute.
"""
from __future__ import annotations

import json
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

ERR_CODES = {"INVALID": -1, "OOM": -2, "NO_SEQ": -3, "EXISTS": -4}


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def run_unit_case(make, case, block_size):
    """make(num_blocks, block_size, free_order) -> manager."""
    m = make(case["num_blocks"], block_size, None)
    for op in case["ops"]:
        kind = op[0]
        if kind == "allocate":
            m.allocate(op[1], op[2])
        elif kind == "available":
            assert m.available_blocks() == op[1], (case["name"], op)
        elif kind == "free":
            m.free_seq(op[1])
        elif kind == "append_n_times":
            for _ in range(op[2]):
                m.append(op[1], 1)
        elif kind == "share_prefix":
            m.share_prefix(op[1], op[2], op[3])
        elif kind == "allocate_fails":
            before = (m.free_list(), [m.refcount(b) for b in range(case["num_blocks"])])
            try:
                m.allocate(op[1], op[2])
            except Exception as e:  # noqa: BLE001
                assert e.code == ERR_CODES[op[3]]
            else:
                raise AssertionError("allocation should have failed")
            assert (m.free_list(), [m.refcount(b) for b in range(case["num_blocks"])]) == before
        else:
            raise ValueError(kind)
    return m


def run_walkthrough(make):
    fx = load("refcount_walkthrough.json")
    ids = {"A": 0, "B": 1}
    m = make(fx["num_blocks"], fx["block_size"], fx["initial_free_order"])
    cow = None
    for op in fx["ops"]:
        if op[0] == "allocate":
            m.allocate(ids[op[1]], op[2])
        elif op[0] == "fork":
            m.fork(ids[op[1]], ids[op[2]])
        elif op[0] == "append":
            r = m.append(ids[op[1]], op[2])
            cow = [r.cow_src, r.cow_dst]
    for name, table in fx["expected_tables"].items():
        assert m.block_table(ids[name]) == table
    for label, rc in fx["expected_refcounts"].items():
        assert m.refcount(int(label[1:]) - 1) == rc, label
    assert cow == fx["expected_cow_pair"]
    m.free_seq(ids["B"])
    for label, rc in fx["after_free_B"]["expected_refcounts"].items():
        assert m.refcount(int(label[1:]) - 1) == rc, label
    for b in fx["after_free_B"]["reclaimed"]:
        assert b in m.free_list()
    assert m.block_table(ids["A"]) == fx["expected_tables"]["A"]
    return m


def run_rag_simulation(make):
    fx = load("rag_simulation.json")
    m = make(fx["num_blocks"], fx["block_size"], None)
    reqs = fx["requests"]

    def check(stage):
        exp = fx[stage]
        if "tables" in exp:
            for r, t in exp["tables"].items():
                assert m.block_table(int(r)) == t, (stage, r)
        assert m.available_blocks() == exp["free_blocks"], stage
        used = fx["num_blocks"] - m.available_blocks()
        assert round(100.0 * used / fx["num_blocks"], 2) == exp["utilization_pct"], stage

    for r in reqs:
        m.allocate(r, 200)
    check("after_allocate")
    for _ in range(50):
        for r in reqs:
            m.append(r, 1)
    for r in reqs:
        assert m.num_tokens(r) == fx["after_appends"]["tokens"]
    check("after_appends")
    for r in reqs:
        m.free_seq(r)
    check("after_release")
    tail = fx["after_release"]["free_list_tail"]
    fl = m.free_list()
    assert fl[:len(fl) - len(tail)] == list(range(24, 200))
    assert fl[len(fl) - len(tail):] == tail
    return m
