"""CPU unit test of the balanced persistent schedule's planner
(selective_state_space_mssm_amd/csrc/balanced_plan.h, the integer arithmetic
the forward kernel and the backward pre-pass use to cut their work).

The header is compiled alone with g++ (its __host__ __device__ markers
defined away) into a small driver that walks every worker's segments for
many (channel blocks, tiles per block, workers) triples and checks:

* every (block, tile) unit is run exactly once, by the worker whose
  contiguous range [U w / workers, U (w + 1) / workers) holds it;
* every worker has at least one segment, and a block is split between at
  most two workers;
* a segment that starts inside a block waits for a published state, is its
  worker's last segment and starts exactly where a lower-numbered worker's
  published piece ends; that piece starts at the block's first tile from h0
  (it depends on nobody) and is its worker's first segment (it publishes
  before that worker waits on anyone) -- so every wait ends;
* every published state is waited for (no orphan hand-over), and pieces that
  finish a block end at its last tile.

And that the host's guard is needed: with fewer blocks than workers some
range lies inside one block, which this cut cannot run.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_mssm_amd", "csrc")

DRIVER = r"""
#include "balanced_plan.h"
#include <cstdio>
#include <vector>
using namespace mssm;

static int fail(const char* what, long nblk, long T, long workers, long w) {
    std::printf("FAIL %s nblk=%ld T=%ld workers=%ld w=%ld\n", what, nblk, T, workers, w);
    return 1;
}

static int check(long nblk, long T, long workers) {
    const long U = nblk * T;
    std::vector<int> owner(U, -1);
    std::vector<int> pub_w(nblk, -1), wait_w(nblk, -1);
    std::vector<long> pub_end(nblk, -1), wait_begin(nblk, -1);
    std::vector<int> nowners(nblk, 0), last_owner(nblk, -1);
    for (long w = 0; w < workers; ++w) {
        const BalancedRange r = balanced_range(nblk, T, workers, w);
        const long u0 = U * w / workers, u1 = U * (w + 1) / workers;
        if (r.nseg < 1) return fail("no segment", nblk, T, workers, w);
        long units = 0;
        for (int sg = 0; sg < r.nseg; ++sg) {
            const BalancedSegment s = balanced_segment(r, T, sg);
            if (s.blk < 0 || s.blk >= nblk) return fail("block out of range", nblk, T, workers, w);
            if (s.tile_begin < 0 || s.tile_begin >= s.tile_end || s.tile_end > T)
                return fail("tile range", nblk, T, workers, w);
            for (long t = s.tile_begin; t < s.tile_end; ++t) {
                const long u = (long)s.blk * T + t;
                if (u < u0 || u >= u1) return fail("unit outside the worker's range", nblk, T, workers, w);
                if (owner[u] != -1) return fail("unit run twice", nblk, T, workers, w);
                owner[u] = (int)w;
                ++units;
            }
            if (last_owner[s.blk] != (int)w) { last_owner[s.blk] = (int)w; ++nowners[s.blk]; }
            if (s.from == kFromH0 && s.tile_begin != 0) return fail("h0 piece not at the block start", nblk, T, workers, w);
            if (s.to == kFinal && s.tile_end != T) return fail("final piece not at the block end", nblk, T, workers, w);
            if (s.to == kPublish) {
                if (sg != 0) return fail("publishing piece is not the first segment", nblk, T, workers, w);
                if (s.from != kFromH0 || s.tile_end >= T) return fail("publishing piece shape", nblk, T, workers, w);
                if (pub_w[s.blk] != -1) return fail("block published twice", nblk, T, workers, w);
                pub_w[s.blk] = (int)w; pub_end[s.blk] = s.tile_end;
            }
            if (s.from == kFromPublished) {
                if (sg != r.nseg - 1) return fail("waiting piece is not the last segment", nblk, T, workers, w);
                if (s.tile_begin == 0 || s.to != kFinal) return fail("waiting piece shape", nblk, T, workers, w);
                if (wait_w[s.blk] != -1) return fail("block waited for twice", nblk, T, workers, w);
                wait_w[s.blk] = (int)w; wait_begin[s.blk] = s.tile_begin;
            }
            if (s.from == kFromChunkCarry || s.to == kKeep) return fail("chunk-schedule role", nblk, T, workers, w);
        }
        if (units != u1 - u0) return fail("worker's units != its range", nblk, T, workers, w);
    }
    for (long u = 0; u < U; ++u)
        if (owner[u] == -1) return fail("unit never run", nblk, T, workers, -1);
    for (long b = 0; b < nblk; ++b) {
        if (nowners[b] > 2) return fail("block split over more than two workers", nblk, T, workers, b);
        if ((pub_w[b] == -1) != (wait_w[b] == -1)) return fail("hand-over without both ends", nblk, T, workers, b);
        if (wait_w[b] != -1) {
            if (pub_w[b] >= wait_w[b]) return fail("wait on a later worker", nblk, T, workers, b);
            if (pub_end[b] != wait_begin[b]) return fail("hand-over at the wrong tile", nblk, T, workers, b);
        }
    }
    return 0;
}

int main() {
    const long Ts[] = {1, 2, 3, 7, 16, 63, 64, 256, 1000, 65536};
    const long Ws[] = {1, 2, 3, 5, 7, 64, 80, 104, 120, 128, 240, 255, 256, 304, 512};
    long cases = 0, bad = 0, unsafe = 0;
    for (long T : Ts)
        for (long workers : Ws)
            for (long nblk = 1; nblk <= 1200; nblk += (nblk < 300 ? 1 : 7)) {
                if (!balanced_plan_ok(nblk, workers)) {
                    // the guard is needed: some range then lies inside one block
                    bool inside = false;
                    for (long w = 0; w < workers && !inside; ++w)
                        inside = balanced_range(nblk, T, workers, w).nseg < 1;
                    if (inside) ++unsafe;
                    continue;
                }
                if ((long)nblk * T > 4000000) continue;
                ++cases;
                bad += check(nblk, T, workers);
                if (bad > 20) { std::printf("too many failures\n"); return 1; }
            }
    std::printf("cases %ld failures %ld unsafe_without_guard %ld\n", cases, bad, unsafe);
    return bad ? 1 : 0;
}
"""


def test_balanced_planner_invariants(tmp_path):
    src = tmp_path / "planner_check.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "planner_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-D__host__=", "-D__device__=", "-I", CSRC, str(src), "-o",
                    str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
    import re
    fields = {k: int(v) for k, v in re.findall(r"(\w+) (\d+)", res.stdout.strip().splitlines()[-1])}
    assert int(fields["cases"]) > 10000
    assert int(fields["failures"]) == 0
    assert int(fields["unsafe_without_guard"]) > 0   # the host guard (nblk >= workers) matters


def test_kernel_uses_the_planner():
    """The forward kernel takes its segments from this header (the code tested
    above), and the host launches the balanced schedule only under its guard."""
    src = open(os.path.join(CSRC, "scan_fwd_kernels.h")).read()
    assert '#include "balanced_plan.h"' in src
    assert "balanced_range(a.nblk, T_, a.workers, blockIdx.x)" in src
    assert "balanced_segment(rg, T_, sg)" in src
    assert "balanced_plan_ok(a.nblk, ncu)" in src
