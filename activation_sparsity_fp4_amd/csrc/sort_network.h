// Comparator network that sorts 8 keys (19 compare-exchanges, depth 6).
// Used to find the 8th-largest key of a 16-entry group for 8:16 selection:
// both halves are sorted, then a bitonic half-cleaner pairs entry i of one half
// with entry 7 - i of the other; the 8 larger entries of those pairs are the
// top 8 of the group and their minimum is the selection threshold.
// Plain C++ (no HIP types) so that a host test can check the network on every
// 0/1 input (the 0-1 principle).
#pragma once

namespace sharq {

constexpr int kSort8Size = 19;
// (i, j) with i < j: after the exchange a[i] >= a[j] (descending order).
constexpr int kSort8[kSort8Size][2] = {
    {0, 2}, {1, 3}, {4, 6}, {5, 7},
    {0, 4}, {1, 5}, {2, 6}, {3, 7},
    {0, 1}, {2, 3}, {4, 5}, {6, 7},
    {2, 4}, {3, 5},
    {1, 4}, {3, 6},
    {1, 2}, {3, 4}, {5, 6},
};

}  // namespace sharq
