// kl_schedule.h -- workgroup order and launch size of the masked-dense MHA
// distillation-loss kernel (kl.hip, mha_kl_dense_kernel) and the splits its
// merge reads.
//
// The kernel takes its (batch, key split, query block) from kl::work_of and
// the launch is sized by kl::per_xcd, so a host program can replay every
// workgroup id of a launch and check that each (batch, split, block) pair is
// taken exactly once.  The includer provides __host__ / __device__ (the HIP
// runtime header on the device side; empty definitions in a host-only build).
#pragma once

namespace dsa {
namespace kl {

constexpr int kQ = 32;          // query rows per block (one workgroup)
constexpr int kKeys = 32;       // keys per tile
constexpr int kSplitTiles = 8;  // tiles per key split (256 keys)
constexpr int kXcds = 8;        // workgroup id mod 8 picks the XCD

__host__ __device__ inline int splits_of(int S) {
    return (S + kSplitTiles * kKeys - 1) / (kSplitTiles * kKeys);
}
__host__ __device__ inline int blocks_of(int T) { return (T + kQ - 1) / kQ; }
__host__ __device__ inline int slots_of(int nsplit) { return (nsplit + kXcds - 1) / kXcds; }

// Split taken by XCD x in its slot k: 16 m + x and 16 m + 15 - x for
// m = 0, 1, ... (a short and a long column of the causal triangle), which
// may lie past the last split.
__host__ __device__ inline int split_of_slot(int x, int k) {
    return kXcds * k + ((k & 1) ? kXcds - 1 - x : x);
}

// First query block whose last row reaches split s (keys 256 s ..), with row
// t at position off + t; every later block reaches it.  nqb when none does.
__host__ __device__ inline int first_block(int s, int off, int nqb) {
    const int q = s * kSplitTiles * kKeys - off - (kQ - 1);
    const int qb = q <= 0 ? 0 : (q + kQ - 1) / kQ;
    return qb < nqb ? qb : nqb;
}

// Workgroups per XCD and batch: all (split, block) pairs of the XCD with
// the most splits.  The launch has kXcds * B * per_xcd(...) workgroups.
__host__ __device__ inline int per_xcd(int nqb, int nsplit) {
    int most = 0;
    for (int x = 0; x < kXcds; ++x) {
        int n = 0;
        for (int k = 0; k < slots_of(nsplit); ++k)
            if (split_of_slot(x, k) < nsplit) n += nqb;
        most = n > most ? n : most;
    }
    return most;
}

struct Work {
    int b;      // batch
    int split;  // key split; -1: past this XCD's share (the workgroup ends)
    int qb;     // query block
};

// Workgroup id -> work.  XCD x = id mod 8 takes its splits (split_of_slot)
// for every batch; its queue holds first the (split, block) pairs inside the
// causal area, one run per split, the longest blocks first, then the pairs
// past it (work only for a selection of later positions).  Consecutive
// workgroups of an XCD go to its shader engines in turn, so work and no-work
// workgroups come in runs, never alternating.
__host__ __device__ inline Work work_of(int id, int T, int S, int nqb, int nsplit, int per) {
    const int x = id % kXcds;
    const int jx = id / kXcds;
    Work w;
    w.b = jx / per;
    w.split = -1;
    w.qb = 0;
    int rem = jx % per;
    for (int pass = 0; pass < 2 && w.split < 0; ++pass) {
        for (int k = 0; k < slots_of(nsplit); ++k) {
            const int sp = split_of_slot(x, k);
            if (sp >= nsplit) continue;
            const int first = first_block(sp, S - T, nqb);
            const int n = pass == 0 ? nqb - first : first;
            if (rem < n) {
                w.split = sp;
                w.qb = pass == 0 ? nqb - 1 - rem : rem;
                break;
            }
            rem -= n;
        }
    }
    return w;
}

}  // namespace kl
}  // namespace dsa
