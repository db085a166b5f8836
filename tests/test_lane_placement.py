"""Block placement (csrc/sv_lanes.h), checked exhaustively on the host.

The kernels' waits are safe only if every item a block waits for sits in an earlier
block of the same XCD lane.  This test compiles the placement header itself with g++
(it is plain C++) and enumerates every block of many grids: each (phase, unit, item)
must be placed exactly once, in its own lane, padding blocks must report no work, and
the orders the kernels rely on must hold.
"""
import subprocess
from pathlib import Path

import pytest

CSRC = Path(__file__).resolve().parents[1] / "rejection_sampling_verify_02_amd" / "csrc"

HARNESS = r"""
#include <cstdio>
#include <vector>
#include "sv_lanes.h"
using namespace sv;

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { if (fails++ < 10) { std::printf("FAIL " __VA_ARGS__); std::printf("\n"); } } } while (0)

// lane_decode: items are unit*per + index; the unit's last first-phase item (its
// finisher) comes after its other first-phase items, and its second phase after all of them.
static void plain(int units, int per1, int per2) {
  const long grid = (long)LANES * ((units + LANES - 1) / LANES) * (per1 + per2);
  std::vector<long> at1((long)units * per1, -1), at2((long)units * per2, -1);
  for (long p = 0; p < grid; ++p) {
    int phase = 0, item = -1;
    if (!lane_decode((int)p, units, per1, per2, phase, item)) continue;
    const int per = phase == 1 ? per1 : per2;
    const int unit = item / per;
    CHECK(unit >= 0 && unit < units, "plain unit %d of %d", unit, units);
    CHECK(unit % LANES == p % LANES, "plain lane: block %ld unit %d", p, unit);
    std::vector<long> &at = phase == 1 ? at1 : at2;
    CHECK(at[item] == -1, "plain item %d placed twice", item);
    at[item] = p;
  }
  for (int u = 0; u < units; ++u) {
    long last1 = -1, first2 = -1;
    for (int s = 0; s < per1; ++s) {
      const long p = at1[(long)u * per1 + s];
      CHECK(p >= 0, "plain unit %d item %d missing", u, s);
      if (s < per1 - 1) CHECK(p < at1[(long)u * per1 + per1 - 1], "plain finisher order unit %d", u);
      last1 = p > last1 ? p : last1;
    }
    for (int s = 0; s < per2; ++s) {
      const long p = at2[(long)u * per2 + s];
      CHECK(p >= 0, "plain unit %d second item %d missing", u, s);
      if (first2 < 0 || p < first2) first2 = p;
      if (s < per2 - 1) CHECK(p < at2[(long)u * per2 + per2 - 1], "plain combiner order unit %d", u);
    }
    if (per2) CHECK(first2 > last1, "plain: second phase of unit %d before its first", u);
  }
}

// lane_decode_lag: every second-phase item of a unit after all its first-phase items,
// the unit's last second-phase item after the others.
static void lagged(int units, int per1, int per2, int lag) {
  const long grid = (long)LANES * ((units + LANES - 1) / LANES) * (per1 + per2);
  std::vector<long> at1((long)units * per1, -1), at2((long)units * per2, -1);
  for (long p = 0; p < grid; ++p) {
    int phase = 0, unit = -1, sub = -1;
    if (!lane_decode_lag((int)p, units, per1, per2, lag, phase, unit, sub)) continue;
    CHECK(unit >= 0 && unit < units, "lag unit %d of %d", unit, units);
    CHECK(unit % LANES == p % LANES, "lag lane: block %ld unit %d", p, unit);
    const int per = phase == 1 ? per1 : per2;
    CHECK(sub >= 0 && sub < per, "lag sub %d of %d", sub, per);
    std::vector<long> &at = phase == 1 ? at1 : at2;
    CHECK(at[(long)unit * per + sub] == -1, "lag item placed twice");
    at[(long)unit * per + sub] = p;
  }
  for (int u = 0; u < units; ++u) {
    long last1 = -1;
    for (int s = 0; s < per1; ++s) {
      const long p = at1[(long)u * per1 + s];
      CHECK(p >= 0, "lag unit %d first item %d missing", u, s);
      last1 = p > last1 ? p : last1;
    }
    for (int s = 0; s < per2; ++s) {
      const long p = at2[(long)u * per2 + s];
      CHECK(p >= 0, "lag unit %d second item %d missing", u, s);
      CHECK(p > last1, "lag: second item %d of unit %d (block %ld) before first phase (%ld)", s, u, p, last1);
      if (s < per2 - 1) CHECK(p < at2[(long)u * per2 + per2 - 1], "lag combiner order unit %d", u);
    }
  }
}

int main() {
  const int units[] = {1, 2, 7, 8, 9, 15, 16, 17, 63, 64, 65, 111, 256, 513};
  const int pers[][2] = {{1, 0}, {8, 0}, {9, 4}, {72, 32}, {1, 1}, {16, 8}, {2, 1}, {38, 19}};
  for (int U : units)
    for (auto &pp : pers) {
      plain(U, pp[0], pp[1]);
      if (pp[1] > 0)
        for (int lag = 1; lag <= 4; ++lag) lagged(U, pp[0], pp[1], lag);
    }
  std::printf(fails ? "FAILED %d\n" : "OK\n", fails);
  return fails ? 1 : 0;
}
"""


def test_placement_exhaustive(tmp_path):
    src = tmp_path / "lanes.cpp"
    src.write_text(HARNESS)
    exe = tmp_path / "lanes"
    subprocess.run(["g++", "-O1", "-std=c++17", "-Wall", "-I", str(CSRC), "-o", str(exe), str(src)],
                   check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout
