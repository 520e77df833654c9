// kl_replay.cpp -- host replay of the workgroup order of the masked-dense
// MHA distillation-loss kernel (csrc/kl.hip, mha_kl_dense_kernel).
//
// The kernel takes its (batch, key split, query block) from kl::work_of and
// its launch size from kl::per_xcd (csrc/kl_schedule.h); this program calls
// the same functions for every workgroup id of a launch and checks that
//   * every (batch, split, block) pair is taken by exactly one workgroup and
//     no workgroup takes anything outside the launch's pairs;
//   * a workgroup's split belongs to its XCD (id mod 8);
//   * within each XCD and batch, in id order, every pair inside the causal
//     area comes before every pair past it, the causal pairs of one split
//     form one run, longest block first;
//   * the XCDs' causal shares differ by at most an eighth of a split's
//     blocks per batch (square launches where every XCD has the same number
//     of splits);
//   * the merge (which reads every split of a row) reads only written states.
// Usage: kl_replay -> runs the built-in shapes, one line each, exits 0 when
// every check holds.
#define __host__
#define __device__
#include "kl_schedule.h"

#include <cstdio>
#include <map>
#include <tuple>
#include <vector>

using namespace dsa::kl;

namespace {

int failures = 0;

void fail(const char *what, int B, int T, int S) {
    if (failures < 20) std::printf("  FAIL %s (B=%d T=%d S=%d)\n", what, B, T, S);
    ++failures;
}

bool causal(int s, int qb, int T, int S) {
    const int last_row = (qb * kQ + kQ - 1 < T - 1) ? qb * kQ + kQ - 1 : T - 1;
    return s * kSplitTiles * kKeys <= S - T + last_row;
}

void replay(int B, int T, int S) {
    const int before = failures;
    const int nqb = blocks_of(T), nsplit = splits_of(S), per = per_xcd(nqb, nsplit);
    const long long grid = (long long)kXcds * B * per;
    std::map<std::tuple<int, int, int>, long long> taken;
    // per (xcd, batch): the order of (split, block, causal) in id order
    std::vector<std::vector<std::vector<std::tuple<int, int, bool>>>> queue(
        kXcds, std::vector<std::vector<std::tuple<int, int, bool>>>(B));
    for (long long id = 0; id < grid; ++id) {
        const Work w = work_of((int)id, T, S, nqb, nsplit, per);
        if (w.split < 0) continue;
        if (w.b < 0 || w.b >= B || w.split >= nsplit || w.qb < 0 || w.qb >= nqb) {
            fail("work outside the launch", B, T, S);
            continue;
        }
        const int x = (int)(id % kXcds);
        bool mine = false;
        for (int k = 0; k < slots_of(nsplit); ++k) mine |= split_of_slot(x, k) == w.split;
        if (!mine) fail("split of another XCD", B, T, S);
        const auto key = std::make_tuple(w.b, w.split, w.qb);
        if (taken.count(key)) fail("pair taken twice", B, T, S);
        taken[key] = id;
        queue[x][w.b].emplace_back(w.split, w.qb, causal(w.split, w.qb, T, S));
    }
    for (int b = 0; b < B; ++b)
        for (int s = 0; s < nsplit; ++s)
            for (int qb = 0; qb < nqb; ++qb)
                if (!taken.count(std::make_tuple(b, s, qb))) fail("pair never taken", B, T, S);
    // merge: every split of every row, all written above
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t)
            for (int s = 0; s < nsplit; ++s)
                if (!taken.count(std::make_tuple(b, s, t / kQ))) fail("merge reads an unwritten state", B, T, S);
    int share_min = 1 << 30, share_max = 0;
    bool equal_slots = true;
    for (int x = 0; x < kXcds; ++x) {
        int nsl = 0;
        for (int k = 0; k < slots_of(nsplit); ++k) nsl += split_of_slot(x, k) < nsplit;
        equal_slots &= nsl == slots_of(nsplit);
        int share = 0;
        for (int b = 0; b < B; ++b) {
            const auto &q = queue[x][b];
            bool seen_past = false;
            int prev_split = -1, prev_qb = 0;
            std::map<int, bool> closed;  // causal runs already finished
            for (const auto &e : q) {
                const int s = std::get<0>(e), qb = std::get<1>(e);
                const bool c = std::get<2>(e);
                if (c) {
                    ++share;
                    if (seen_past) fail("causal pair after a pair past the causal area", B, T, S);
                    if (s != prev_split) {
                        if (closed.count(s)) fail("causal run of a split split in two", B, T, S);
                        if (prev_split >= 0) closed[prev_split] = true;
                    } else if (qb >= prev_qb) {
                        fail("causal run not longest block first", B, T, S);
                    }
                    prev_split = s;
                    prev_qb = qb;
                } else {
                    seen_past = true;
                }
            }
        }
        share_min = share < share_min ? share : share_min;
        share_max = share > share_max ? share : share_max;
    }
    if (equal_slots && nsplit % 16 == 0 && S == T && share_max - share_min > B * nqb / 8)
        fail("XCD shares of the causal triangle unequal", B, T, S);
    std::printf("B=%d T=%d S=%d: %lld workgroups, %d splits x %d blocks, causal share per XCD "
                "%d..%d%s\n", B, T, S, grid, nsplit, nqb, share_min, share_max,
                failures == before ? "" : "  <-- failed");
}

}  // namespace

int main() {
    const int shapes[][3] = {{1, 4096, 4096},  {2, 1000, 4096}, {1, 100, 100},  {1, 1, 5000},
                             {3, 777, 9000},   {1, 4096, 65536}, {1, 2048, 2048}, {2, 33, 33},
                             {2, 300, 5000},   {2, 1500, 1500}, {1, 8192, 8192}, {4, 64, 65536},
                             {1, 4095, 4096},  {2, 999, 1032}};  // rows 1 and 33 short of the cache
    for (const auto &sh : shapes) replay(sh[0], sh[1], sh[2]);
    std::printf("%s: %d failed checks\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
