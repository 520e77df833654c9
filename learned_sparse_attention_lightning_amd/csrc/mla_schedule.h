// mla_schedule.h -- tile schedule and memory addressing of the MLA attention
// kernel and its split merge (attention_mla.hip).
//
// Every global address the two kernels form, every workgroup-to-work mapping
// and every ring slot they use comes from the functions here, so a host
// program can replay them over all workgroups, waves and steps of a launch
// and check each address against its buffer and each LDS ring slot against
// the barrier schedule.  The includer provides __host__ / __device__ (the HIP
// runtime header on the device side; empty definitions in a host-only build).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace dsa {
namespace mla {

constexpr int kDqk = 576;                  // latent row: 512 value dims + 64 rope dims
constexpr int kDv = 512;
constexpr int kHg = 64;                    // heads per workgroup
constexpr int kKt = 32;                    // selected entries per tile
constexpr int kRing = 4;                   // latent tiles resident in LDS
constexpr int kSelRing = 8;                // tiles of the selection kept in LDS
constexpr int kLatRowBytes = kDqk * 2;     // 1152: a latent row in memory
constexpr int kVRowBytes = kDv * 2;        // 1024: its value dims
constexpr int kStageRows = kKt / 4;        // rows of a tile each of the 4 PV waves gathers
constexpr int kRopeSteps = (kDqk - kDv) / 16;  // 16-dim k-steps of rope (4)
constexpr int kHalfSteps = kDqk / 16 / 2;  // k-steps of one S wave's half of the dims (18)
// LDS: a tile row holds the value dims plus one spare 16-byte slot (a bank
// shift of 4 dwords a row); after the last step each PV wave stages its
// output block [32 heads][kOutPitch floats] in the tile ring.
constexpr int kRowPitch = kVRowBytes + 16;  // 1040
constexpr int kTileBytes = kKt * kRowPitch;  // 33280
constexpr int kOutPitch = 136;               // floats per head row of the output staging block
static_assert(4 * 32 * kOutPitch * 4 <= kRing * kTileBytes, "output staging fits the tile ring");

// Tiles handled in step `it` (one workgroup barrier per step), as offsets
// from it.  Steps run it = 0 .. ntiles for the PV waves (PV of tile it-1)
// and it = 0 .. ntiles-1 for the S waves.
constexpr int kSelAhead = 5;     // wave 0 writes the selection ring entry of tile it+5
constexpr int kSelPrologue = 5;  // ... and tiles 0..4 before the first barrier
constexpr int kGatherAhead = 4;  // PV waves load the rows of tile it+4 into registers
constexpr int kParkAhead = 2;    // ... and park tile it+2 (loaded two steps earlier) in LDS
constexpr int kRopeAhead = 2;    // kh = 1 S waves load the rope dims of tile it+2
constexpr int kSAhead = 1;       // S products (and the mask) of tile it+1; softmax of tile it
constexpr int kPvBehind = 1;     // PV products of tile it-1
// Tile X: its selection entry is written in step X - kSelAhead and read in
// steps X - kGatherAhead (gather), X - kRopeAhead (rope) and X - kSAhead
// (mask), then overwritten in step X + kSelRing - kSelAhead.  Its latent
// rows are parked in step X - kParkAhead, read in steps X - kSAhead (S) and
// X + kPvBehind (PV), then overwritten in step X + kRing - kParkAhead.
static_assert(kSelAhead > kGatherAhead, "a ring entry is written a step before its gather");
static_assert(kSelRing - kSelAhead > -kSAhead, "a ring entry outlives its last reader");
static_assert(kRing - kParkAhead > kPvBehind, "a tile is parked over one the PV waves are done with");

// ---- launch plan ----
// Entry splits of one launch of n query rows (x B sequences x H/64 head
// groups): enough workgroups to cover the 256 CUs, at least four tiles a
// split so the gather pipeline has work to overlap.  per_split entries each
// (a multiple of the tile), `splits` of them used.
struct Plan {
    int splits;
    int per_split;
};
__host__ __device__ inline Plan launch_plan(int B, int n, int H, int k) {
    const long long wgs = (long long)B * n * (H / kHg);
    const int max_splits = (k + 4 * kKt - 1) / (4 * kKt);
    long long s = (256 + wgs - 1) / wgs;
    if (s > max_splits) s = max_splits;
    if (s < 1) s = 1;
    const int per = (k + (int)s - 1) / (int)s;
    Plan p;
    p.per_split = (per + kKt - 1) / kKt * kKt;
    p.splits = (k + p.per_split - 1) / p.per_split;
    return p;
}
// Workspace of one launch with split partials in an output type of
// `out_bytes` bytes: o_part, then lse_part (fp32) right after it.
__host__ __device__ inline size_t part_elems(int B, int n, int splits, int H) {
    return (size_t)B * n * splits * H * kDv;
}
__host__ __device__ inline size_t launch_workspace_bytes(int B, int n, int splits, int H,
                                                         int out_bytes) {
    return splits > 1 ? part_elems(B, n, splits, H) * out_bytes + (size_t)B * n * splits * H * 4
                      : 0;
}

__host__ __device__ constexpr int sel_slot(int tile) { return tile % kSelRing; }
__host__ __device__ constexpr int ring_slot(int tile) { return tile % kRing; }

// What one workgroup of the attention launch computes.
struct Work {
    int hg;       // head group: heads hg*64 .. hg*64+63
    int split;    // entry split of the query row
    int qidx;     // query row of the launch, b * rows + r
    int r, b;     // row within the launch chunk, sequence
};

// Workgroup id -> work.  With a multiple of 8 query rows, XCD x (= id mod 8)
// takes the rows qidx = x mod 8 with all their head groups and splits, so
// the gathers, the query block and the split partials of a row stay in one
// XCD's L2; else, with a multiple of 8 (row, split) units, the head groups of
// one unit sit 8 ids apart (same XCD); else plain order.
__host__ __device__ inline Work work_of(int id, int rows, int B, int hgs, int splits) {
    Work w;
    if ((rows * B) % 8 == 0) {
        const int x = id & 7, j = id >> 3;
        const int per = hgs * splits;
        const int qg = j / per, rem = j - qg * per;
        w.hg = rem % hgs;
        w.split = rem / hgs;
        w.qidx = 8 * qg + x;
    } else if ((rows * B * splits) % 8 == 0) {
        const int slot = id >> 3;
        w.hg = slot % hgs;
        const int unit = (slot / hgs) * 8 + (id & 7);
        w.qidx = unit / splits;
        w.split = unit % splits;
    } else {
        w.hg = id % hgs;
        w.split = (id / hgs) % splits;
        w.qidx = id / (hgs * splits);
    }
    w.r = w.qidx % rows;
    w.b = w.qidx / rows;
    return w;
}

// Entries of the split [e_begin, e_begin + len).  causal_tail: the row's
// selection is min(k, t+1) positions then -1 only, so entries past that count
// are not visited (t = the row's position, already clamped to S-1).
__host__ __device__ inline int split_len(int split, int per_split, int k, bool causal_tail, int t) {
    const int e_begin = split * per_split;
    int len = (k < e_begin + per_split ? k : e_begin + per_split) - e_begin;
    if (causal_tail) {
        const int nvalid = t < 0 ? 0 : (k < t + 1 ? k : t + 1);
        const int lim = nvalid - e_begin;
        len = len < lim ? len : lim;
        len = len > 0 ? len : 0;
    }
    return len;
}

// Tiles walked: at least one (a split without entries runs one masked tile).
__host__ __device__ inline int split_tiles(int len) {
    const int n = (len + kKt - 1) / kKt;
    return n > 1 ? n : 1;
}

// ---- global addresses (byte offsets into the latent rows of sequence b,
// element offsets into q, out, the split partials and lse) ----

// Row s of the latent table: masked entries (s < 0) read row 0 (their
// probability is forced to 0).  Entries past the cache (s > last = S - 1) are
// outside the selection's contract; their loads are kept inside the
// sequence's rows (row `last`), so a bad selection cannot read past the table.
__host__ __device__ inline uint64_t latent_row_offset(int32_t s, int32_t last) {
    const int32_t r = s > 0 ? (s < last ? s : last) : 0;
    return (uint64_t)(uint32_t)r * (uint64_t)kLatRowBytes;
}
// 16-byte piece `lane` (0..63) of a row's value dims, gathered by a PV wave.
__host__ __device__ inline uint64_t gather_offset(int32_t s, int32_t last, int lane) {
    return latent_row_offset(s, last) + 16ull * (uint64_t)lane;
}
// Rope piece j (0..3) of lane half `half` (kh = 1 S waves).
__host__ __device__ inline uint64_t rope_offset(int32_t s, int32_t last, int half, int j) {
    return latent_row_offset(s, last) + (uint64_t)kVRowBytes + 16ull * (uint64_t)half +
           32ull * (uint64_t)j;
}
// First element of the 8 query dims of k-step ks for (head tile ht, lane
// l32/half, dim half kh); q is [B*T rows][H][576].
__host__ __device__ inline size_t q_offset(size_t rowq, int H, int head0, int ht, int l32,
                                           int half, int kh, int ks) {
    return (rowq * H + head0 + ht * 32 + l32) * kDqk + 8 * half + 16 * kHalfSteps * kh + 16 * ks;
}
// Output (single split) and split partial of head `head` (0..H-1), 4 dims
// from dim d: out is [B*T rows][H][512], o_part [launch rows][splits][H][512],
// lse_part [launch rows][splits][H].  A PV wave writes heads head + 2m
// (m = 0..15) from one base: kHeadPairStride elements apart.
constexpr size_t kHeadPairStride = 2 * (size_t)kDv;
__host__ __device__ inline size_t out_offset(size_t rowq, int H, int head, int d) {
    return (rowq * H + head) * kDv + d;
}
__host__ __device__ inline size_t part_split_stride(int H) { return (size_t)H * kDv; }
__host__ __device__ inline size_t lse_split_stride(int H) { return (size_t)H; }
__host__ __device__ inline size_t part_offset(size_t prow, int splits, int split, int H,
                                              int head, int d) {
    return (prow * splits * H + head) * kDv + d + (size_t)split * part_split_stride(H);
}
__host__ __device__ inline size_t lse_part_offset(size_t prow, int splits, int split, int H,
                                                  int head) {
    return prow * splits * H + head + (size_t)split * lse_split_stride(H);
}

// ---- split merge ----
constexpr int kCombineBatch = 16;  // splits whose loads are issued together

struct CombineWork {
    int hp;    // head pair
    int qidx;  // query row of the launch
};
__host__ __device__ inline CombineWork combine_work_of(int id, int rows, int B, int H) {
    const int hps = H / 2;
    CombineWork c;
    if ((rows * B) % 8 == 0) {
        const int x = id & 7, j = id >> 3;
        c.hp = j % hps;
        c.qidx = 8 * (j / hps) + x;
    } else {
        c.hp = id % hps;
        c.qidx = id / hps;
    }
    return c;
}
// Split read by batch slot j of the batch starting at s0 (clamped: slots past
// the last split re-read it with weight 0).
__host__ __device__ inline int combine_split(int s0, int j, int splits) {
    return s0 + j < splits - 1 ? s0 + j : splits - 1;
}

}  // namespace mla
}  // namespace dsa
