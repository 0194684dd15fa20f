// Staging plan of the windowed forward kernel: one record per tile of WIN_TILE
// sorted voxels, computed during the map build.
//
//   [0]      rows to stage R, or -1 when they exceed the capacity (direct gathers)
//   [1]      number of ranges nr (<= 9)
//   [2..10]  first sorted position of range r
//   [11..19] first slot of range r (slot 0 for range 0, increasing)
//   [20..28] per (dz, dy) row d: slot = sorted position + delta[d]
//
// A tile's neighbours in one (dz, dy) row lie in a window of sorted positions (the
// union of its groups' windows); the 9 windows merge into a few ranges, staged one
// after the other.
#pragma once

#include "common.h"

namespace sc {

constexpr int PLAN_INTS = 32;
constexpr int WIN_TILE = 128;    // voxels per tile (4 groups of 32)
constexpr int WIN_SLOTS = 1024;  // row slots per buffer; the last one always holds zeros
constexpr int WIN_CAP = WIN_SLOTS - 1;

// 16-lane inclusive scans (shuffles of width 16 stay inside a team)
__device__ __forceinline__ int32_t team_scan_add(int32_t x, int q)
{
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        const int32_t y = __shfl_up(x, off, 16);
        x += q >= off ? y : 0;
    }
    return x;
}
__device__ __forceinline__ int32_t team_scan_max(int32_t x, int q)
{
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        const int32_t y = __shfl_up(x, off, 16);
        x = q >= off && y > x ? y : x;
    }
    return x;
}

// One tile's record from a team of 16 lanes (q = lane within the team): lane q < 9
// brings row q's window [lo, hi] (lo = GWIN_NONE when the row is empty).  The rows
// are ranked by window start (ties by row, empty rows last), each lane takes the row
// of its rank, and the merge into ranges is a set of team scans: sorted element i
// starts a range when its start exceeds by more than one the largest end before it
// (the end of the current range, since ranges end in increasing order).  Writes the
// PLAN_INTS ints of `rec` (any memory).  All 16 lanes of the team must call it.
__device__ __forceinline__ void plan_tile_team(int32_t lo, int32_t hi, int q, int cap, int32_t *rec)
{
    int rank = q;
    if (q < 9) {
        rank = 0;
#pragma unroll
        for (int e = 0; e < 9; ++e) {
            const int32_t le = __shfl(lo, e, 16);
            rank += (le < lo || (le == lo && e < q)) ? 1 : 0;
        }
    }
    int src = q;
#pragma unroll
    for (int e = 0; e < 9; ++e) {
        const int re = __shfl(rank, e, 16);
        src = (q < 9 && re == q) ? e : src;
    }
    const int32_t slo = __shfl(lo, src, 16), shi = __shfl(hi, src, 16);
    const bool ne = q < 9 && slo != GWIN_NONE;        // a non-empty row (they come first)

    // ranges: starts, the start of each element's range, ends, lengths, slot bases
    const int32_t incl_max = team_scan_max(ne ? shi : INT32_MIN, q);
    const int32_t prev_max = __shfl_up(incl_max, 1, 16);
    const bool start = ne && (q == 0 || slo > prev_max + 1);
    const int32_t rlo = team_scan_max(start ? slo : INT32_MIN, q);   // the range's first position
    const bool next_ne = q < 15 && __shfl_down(ne ? 1 : 0, 1, 16) != 0;
    const bool next_start = q < 15 && __shfl_down(start ? 1 : 0, 1, 16) != 0;
    const bool end = ne && (!next_ne || next_start);
    const int32_t len = end ? incl_max - rlo + 1 : 0;
    const int32_t incl_len = team_scan_add(len, q);
    const int32_t base = incl_len - len;                            // slot of the range's first row
    const int32_t total = __shfl(incl_len, 15, 16);
    const int32_t rid = team_scan_add(start ? 1 : 0, q) - 1;        // range index (at a start)
    const int32_t nr = __shfl(rid, 15, 16) + 1;

    if (q < 9) {
        if (start) {
            rec[2 + rid] = slo;
            rec[11 + rid] = base;
        }
        if (q >= nr) {
            rec[2 + q] = 0;
            rec[11 + q] = total;
        }
        rec[20 + src] = ne ? base - rlo : 0;  // slot = sorted position + delta
    } else if (q == 9) {
        rec[0] = total <= cap ? total : -1;
        rec[1] = nr;
    } else if (q < 13) {
        rec[29 + (q - 10)] = 0;
    }
}

}  // namespace sc
