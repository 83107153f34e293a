"""Pins of the oracle's counter-based generator (CPU only).

Published vectors pin the two mixing functions; closed forms and chi-square
tests pin the uniform / Gumbel maps and the independence of the streams.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import rng

GOLD = os.path.join(os.path.dirname(__file__), "golden", "rng_vectors.json")


def test_splitmix64_published_sequence():
    g = json.load(open(GOLD))
    s = g["splitmix64_seed"]
    outs = []
    for _ in range(len(g["splitmix64_outputs"])):
        s, o = oracle.splitmix64_next(s)
        outs.append(o)
    assert outs == g["splitmix64_outputs"]


def test_fmix32_murmur3_empty_vectors():
    g = json.load(open(GOLD))
    for seed, h in g["murmur3_x86_32_empty"]:
        assert oracle.fmix32(seed) == h
        assert int(oracle.fmix32(np.array([seed], dtype=np.uint32))[0]) == h


def test_uniforms_exact_in_fp32_and_open_interval():
    key = oracle.row_key(5, 17, 3, oracle.DRAFT)
    u = oracle.uniforms(key, 1 << 16)
    assert np.all(u > 0) and np.all(u < 1)
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    # odd multiples of 2^-24
    m = u * 2.0 ** 24
    assert np.all(m == np.round(m)) and np.all(np.round(m) % 2 == 1)
    # the scalar path agrees with the array path
    for v in (0, 1, 2, 1000, 65535):
        assert oracle.uniform_at(key, v) == u[v]


def test_row_hash_is_a_bijection_in_v():
    key = oracle.row_key(1, 2, 3, 4)
    v = np.arange(1 << 20, dtype=np.uint32)
    h = rng._hash_elements(key, v)
    assert np.unique(h).size == v.size


@pytest.mark.parametrize("purpose", [oracle.DRAFT, oracle.RESID])
def test_uniform_chi_square(purpose):
    key = oracle.row_key(123, 456, 2, purpose)
    u = oracle.uniforms(key, 1 << 20)
    counts, _ = np.histogram(u, bins=256, range=(0, 1))
    p = stats.chisquare(counts).pvalue
    assert p > 1e-4


def test_serial_pairs_chi_square():
    key = oracle.row_key(9, 9, 1, oracle.DRAFT)
    u = oracle.uniforms(key, 1 << 20)
    a = np.minimum((u[:-1] * 16).astype(int), 15)
    b = np.minimum((u[1:] * 16).astype(int), 15)
    counts = np.bincount(a * 16 + b, minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-4


def test_streams_are_independent_across_keys():
    # element v of neighbouring (request, position, purpose) rows: joint cells uniform
    n = 1 << 16
    base = oracle.uniforms(oracle.row_key(3, 10, 1, oracle.DRAFT), n)
    for other in (oracle.row_key(3, 11, 1, oracle.DRAFT), oracle.row_key(3, 10, 2, oracle.DRAFT),
                  oracle.row_key(3, 10, 1, oracle.RESID), oracle.row_key(4, 10, 1, oracle.DRAFT)):
        o = oracle.uniforms(other, n)
        assert not np.array_equal(o, base)
        a = np.minimum((base * 8).astype(int), 7)
        b = np.minimum((o * 8).astype(int), 7)
        counts = np.bincount(a * 8 + b, minlength=64)
        assert stats.chisquare(counts).pvalue > 1e-4
        assert abs(np.corrcoef(base, o)[0, 1]) < 4.0 / math.sqrt(n)


def test_accept_uniforms_across_requests_uniform():
    us = np.array([oracle.uniform_at(oracle.row_key(77, req, 1, oracle.ACCEPT), 0)
                   for req in range(20000)])
    counts, _ = np.histogram(us, bins=50, range=(0, 1))
    assert stats.chisquare(counts).pvalue > 1e-4


def test_gumbel_moments_closed_form():
    g = oracle.gumbels(oracle.row_key(1, 1, 1, oracle.DRAFT), 1 << 20)
    n = g.size
    euler_gamma = 0.5772156649015329
    var = math.pi ** 2 / 6
    assert abs(g.mean() - euler_gamma) < 5 * math.sqrt(var / n)
    assert abs(g.var() - var) < 0.02 * var
    # CDF exp(-exp(-x)) at a few points
    for x in (-1.0, 0.0, 1.0, 3.0):
        emp = np.mean(g <= x)
        assert abs(emp - math.exp(-math.exp(-x))) < 5e-3
