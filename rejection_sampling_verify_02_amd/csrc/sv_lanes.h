// sv_lanes.h -- placement of work items on the grid's blocks, XCD by XCD.  Plain C++
// (host and device), so the host can check the placement exhaustively.
//
// The device hands workgroups to its XCDs round-robin (blockIdx % 8), each XCD in
// blockIdx order.  Work comes in UNITS (a row, a sequence, or a target/draft pair) of
// per1 first-phase items and per2 second-phase items, and some items of a unit wait for
// other items of the same unit.  Block p runs item q = p / LANES of lane k = p % LANES,
// and lane k owns units k, k + LANES, ...  So each XCD streams whole units, the waiting
// items (a unit's last ones) are spread over every XCD instead of all landing on one,
// and every wait is for an earlier item of the same lane, i.e. a smaller blockIdx: the
// grid cannot stall, wherever the blocks run.  Padding blocks of short lanes get false.
#pragma once

#if defined(__HIPCC__)
#define SV_HD __host__ __device__ inline
#else
#define SV_HD inline
#endif

namespace sv {

constexpr int LANES = 8;

// Lane k runs all first-phase items of its units, unit after unit, then all their
// second-phase items.  item = unit * per (of that phase) + index within the unit.
SV_HD bool lane_decode(int p, int units, int per1, int per2, int &phase, int &item) {
  const int k = p % LANES, q = p / LANES;
  const int nu = (units > k) ? (units - k + LANES - 1) / LANES : 0;
  if (q < nu * per1) {
    const int s = q / per1;
    item = (k + LANES * s) * per1 + (q - s * per1);
    phase = 1;
    return true;
  }
  const int q2 = q - nu * per1;
  if (q2 < nu * per2) {
    const int s = q2 / per2;
    item = (k + LANES * s) * per2 + (q2 - s * per2);
    phase = 2;
    return true;
  }
  return false;
}

// Lane k runs the first-phase items of its n-th unit followed by the second-phase items
// of its (n - lag)-th unit, so a unit's second phase comes soon after its first (lag >= 1:
// the second phase always follows every first-phase item of its unit).
SV_HD bool lane_decode_lag(int p, int units, int per1, int per2, int lag, int &phase, int &unit,
                           int &sub) {
  const int k = p % LANES;
  int q = p / LANES;
  const int nu = (units > k) ? (units - k + LANES - 1) / LANES : 0;
  const int n1 = lag < nu ? lag : nu;  // leading units with no second phase beside them
  const int nm = nu - n1;              // groups: first phase of unit n1+g, second of unit g
  const int gs = per1 + per2;
  int lu;
  if (q < n1 * per1) {
    lu = q / per1;
    sub = q - lu * per1;
    phase = 1;
  } else if ((q -= n1 * per1) < nm * gs) {
    const int g = q / gs, s = q - g * gs;
    if (s < per1) {
      lu = n1 + g;
      sub = s;
      phase = 1;
    } else {
      lu = g;
      sub = s - per1;
      phase = 2;
    }
  } else if ((q -= nm * gs) < n1 * per2) {
    lu = nm + q / per2;
    sub = q - (q / per2) * per2;
    phase = 2;
  } else {
    return false;
  }
  unit = k + LANES * lu;
  return true;
}

}  // namespace sv
