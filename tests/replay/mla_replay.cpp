// mla_replay.cpp -- host replay of the MLA attention kernel and its split
// merge (learned_sparse_attention_lightning_amd/csrc/attention_mla.hip) over
// every workgroup, wave and step of a launch.
//
// The kernel takes its workgroup mapping, split plan, ring slots, tile
// schedule and every global address from mla_schedule.h; this program calls
// the same functions.  For each launch it
//   * walks each of the 8 waves of each workgroup through the kernel's
//     phases (barrier to barrier), recording the LDS ring slots it reads and
//     writes: a slot written by one wave and touched by another in the same
//     phase is a race; a read must find the tile it expects, completely
//     written in an earlier phase;
//   * checks every global address the waves form -- selection reads, latent
//     gathers, rope loads, query loads, output, split partial and lse stores,
//     and the merge's reads and writes -- against the size of its buffer;
//   * checks that every output element of the launch is written exactly once
//     and every split partial is written once and read by the merge.
// A second model replays the kernel as committed at 07:13 on the day of the
// fault report (a three-tile ring, two barriers a step, the split's
// selection copied whole into LDS), transcribed from that commit.
//
// Usage: mla_replay  -> runs the built-in launch list, prints one line per
// launch, exits 0 when every check holds.
#define __host__
#define __device__
#include "mla_schedule.h"

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <string>
#include <vector>

using namespace dsa::mla;

namespace {

long long g_fail = 0;
std::string g_where;

void fail(const char *what, long long a = 0, long long b = 0) {
    if (g_fail < 20) std::printf("  FAIL %s: %s (%lld, %lld)\n", g_where.c_str(), what, a, b);
    ++g_fail;
}

// [lo, hi) inside [0, size)
void in_bounds(const char *what, long long lo, long long hi, long long size) {
    if (lo < 0 || hi > size || lo > hi) fail(what, lo, size);
}

struct Launch {
    std::string name;
    int B, T, S, H, k;
    int row0, rows;       // the launch's rows of each sequence
    bool causal_tail;
    int out_bytes;        // 2 (bf16) or 4 (fp32)
    std::vector<int> qpos;  // [B*T] or empty (t = S - T + i)
    std::string sel;        // "causal" | "max" | "holes" | "wild"
};

int row_pos(const Launch &L, int b, int i) {
    int t = L.qpos.empty() ? L.S - L.T + i : L.qpos[(size_t)b * L.T + i];
    return t >= L.S ? L.S - 1 : t;  // positions past the cache are the last one
}

// Selection [B*T][k]: what the kernel reads from idx.
std::vector<int32_t> make_selection(const Launch &L, uint64_t seed) {
    std::vector<int32_t> idx((size_t)L.B * L.T * L.k, -1);
    std::mt19937_64 rng(seed);
    for (int b = 0; b < L.B; ++b)
        for (int i = 0; i < L.T; ++i) {
            int32_t *row = &idx[((size_t)b * L.T + i) * L.k];
            const int t = row_pos(L, b, i);
            if (L.sel == "max") {
                for (int e = 0; e < L.k; ++e) row[e] = L.S - 1;
            } else if (L.sel == "wild") {
                // outside the contract: entries at and far past the cache's end
                for (int e = 0; e < L.k; ++e)
                    row[e] = (e % 3 == 0) ? L.S + (int32_t)(rng() % 1000000u)
                                          : (e % 3 == 1) ? INT32_MAX - (int32_t)(rng() % 7u) : L.S;
            } else if (L.sel == "holes") {
                for (int e = 0; e < L.k; ++e)
                    row[e] = (rng() % 5 == 0) ? -1 : (int32_t)(rng() % (uint64_t)L.S);
            } else {  // causal: min(k, t+1) ascending positions of 0..t, then -1
                if (t < 0) continue;
                const int n = std::min(L.k, t + 1);
                if (n == t + 1) {
                    for (int e = 0; e < n; ++e) row[e] = e;
                } else {
                    // n distinct positions of 0..t: a sorted random sample,
                    // always including 0 and t (the ends of the range)
                    std::vector<int32_t> pick;
                    pick.reserve(n);
                    pick.push_back(0);
                    pick.push_back(t);
                    const int stride = std::max(1, (t + 1) / n);
                    for (int s = 1; (int)pick.size() < n && s < t; s += stride) pick.push_back(s);
                    for (int s = 1; (int)pick.size() < n; ++s)
                        if (std::find(pick.begin(), pick.end(), s) == pick.end()) pick.push_back(s);
                    std::sort(pick.begin(), pick.end());
                    for (int e = 0; e < n; ++e) row[e] = pick[e];
                }
            }
        }
    return idx;
}

// ------------------------------------------------------------ LDS model --
// Objects of the kernel's LDS, each a set of slots; a slot holds one tile's
// data and is written in `parts` pieces (one per writing wave).
enum Obj { SEL, KV, P, PART, CORR, RESC, FINL, STAGE, NOBJ };
const char *obj_name[NOBJ] = {"sel ring", "latent ring", "P", "S half", "rescale factors",
                              "rescale flags", "1/l", "output staging"};

struct Access {
    int obj, slot, part;  // part: which writer's piece (-1 = every piece, reads)
    bool write;
    int tile;             // tile written, or tile expected by a read
    int wave;
};

struct SlotState {
    int tile = -1000;     // tile held (-1000: never written)
    unsigned parts = 0;   // pieces written for that tile
};

// Pieces a slot of each object is written in.
int parts_of(int obj) { return obj == KV ? 4 : 1; }

class Lds {
  public:
    Lds() : state_(NOBJ) {
        const int slots[NOBJ] = {kSelRing, kRing, 4, 4, 4, 4, 2, 4};
        for (int o = 0; o < NOBJ; ++o) state_[o].resize(slots[o]);
    }
    // one barrier-to-barrier phase, all waves' accesses
    void phase(const std::vector<Access> &acc) {
        // races: a slot written by one wave and touched by another
        std::map<std::pair<int, int>, std::vector<const Access *>> by_slot;
        for (const Access &a : acc) by_slot[{a.obj, a.slot}].push_back(&a);
        for (auto &kv : by_slot) {
            for (const Access *w : kv.second) {
                if (!w->write) continue;
                for (const Access *o : kv.second)
                    if (o->wave != w->wave && (o->write ? o->part == w->part || o->part < 0 ||
                                                              w->part < 0
                                                        : true))
                        fail((std::string("LDS race on ") + obj_name[w->obj]).c_str(), w->slot,
                             o->wave);
            }
        }
        // the output staging blocks live in the latent ring: no ring access
        // may share their phase
        bool staging = false, ring = false;
        for (const Access &a : acc) {
            staging |= a.obj == STAGE;
            ring |= a.obj == KV;
        }
        if (staging && ring) fail("output staging overlaps latent ring use", 0, 0);
        // reads see the state left by earlier phases
        for (const Access &a : acc) {
            if (a.write) continue;
            const SlotState &s = state_[a.obj][a.slot];
            const unsigned full = (1u << parts_of(a.obj)) - 1u;
            if (s.tile != a.tile || s.parts != full)
                fail((std::string("stale or partial ") + obj_name[a.obj]).c_str(), a.tile, s.tile);
        }
        for (const Access &a : acc) {
            if (!a.write) continue;
            SlotState &s = state_[a.obj][a.slot];
            if (s.tile != a.tile) {
                s.tile = a.tile;
                s.parts = 0;
            }
            s.parts |= a.part < 0 ? ((1u << parts_of(a.obj)) - 1u) : (1u << a.part);
        }
    }
    const SlotState &at(int obj, int slot) const { return state_[obj][slot]; }

  private:
    std::vector<std::vector<SlotState>> state_;
};

// ---------------------------------------------------- the current kernel --
struct Buffers {
    long long idx_elems, lat_bytes, q_elems, out_elems, lse_elems;
    long long part_elems, lse_part_elems, ws_bytes;
};

// Per wave: list of phases, each a list of LDS accesses.
typedef std::vector<std::vector<Access>> WavePhases;

struct Ctx {
    const Launch *L;
    const std::vector<int32_t> *idx;
    Buffers buf;
    int splits, per_split;
    std::vector<uint8_t> out_written, part_written, part_read;
};

void replay_workgroup(Ctx &C, int id) {
    const Launch &L = *C.L;
    const int hgs = L.H / kHg;
    const Work wk = work_of(id, L.rows, L.B, hgs, C.splits);
    if (wk.b < 0 || wk.b >= L.B || wk.r < 0 || wk.r >= L.rows || wk.hg >= hgs ||
        wk.split >= C.splits)
        fail("workgroup maps outside the launch", id, wk.qidx);
    const int i = L.row0 + wk.r;
    const int head0 = wk.hg * kHg;
    const int e_begin = wk.split * C.per_split;
    const int len = split_len(wk.split, C.per_split, L.k, L.causal_tail, row_pos(L, wk.b, i));
    const int ntiles = split_tiles(len);
    const size_t rowq = (size_t)wk.b * L.T + i;
    const size_t prow = (size_t)wk.qidx;
    const long long lat_b = (long long)wk.b * L.S * kLatRowBytes;
    const size_t sel_base = rowq * L.k + e_begin;
    auto sel_of = [&](int e) -> int32_t {
        if (e < len) {
            in_bounds("selection read", (long long)(sel_base + e), (long long)(sel_base + e + 1),
                      C.buf.idx_elems);
            return (*C.idx)[sel_base + e];
        }
        return -1;
    };
    auto gather = [&](int32_t s) {  // one wave load of a row's value dims, lanes 0..63
        in_bounds("latent gather", lat_b + (long long)gather_offset(s, L.S - 1, 0),
                  lat_b + (long long)gather_offset(s, L.S - 1, 63) + 16, C.buf.lat_bytes);
    };
    auto rope = [&](int32_t s) {
        for (int half = 0; half < 2; ++half)
            for (int j = 0; j < kRopeSteps; ++j)
                in_bounds("rope load", lat_b + (long long)rope_offset(s, L.S - 1, half, j),
                          lat_b + (long long)rope_offset(s, L.S - 1, half, j) + 16, C.buf.lat_bytes);
    };

    // ---- the 8 waves, phase by phase (a phase ends at a workgroup barrier)
    std::vector<WavePhases> waves(8);
    for (int wave = 0; wave < 8; ++wave) {
        WavePhases &ph = waves[wave];
        ph.emplace_back();
        auto acc = [&](int obj, int slot, int part, bool w, int tile) {
            ph.back().push_back({obj, slot, part, w, tile, wave});
        };
        auto barrier = [&]() { ph.emplace_back(); };
        // contents of the selection ring as wave 0 left it (for addresses)
        if (wave < 4) {
            const int ht = wave & 1, kh = wave >> 1;
            for (int l32 = 0; l32 < 32; ++l32)
                for (int half = 0; half < 2; ++half)
                    for (int ks = 0; ks < kHalfSteps; ++ks) {
                        const size_t o = q_offset(rowq, L.H, head0, ht, l32, half, kh, ks);
                        in_bounds("query load", (long long)o, (long long)o + 8, C.buf.q_elems);
                    }
            // P0: wave 0 writes the selection of tiles 0..4
            if (wave == 0) {
                for (int t = 0; t < kSelPrologue; ++t) {
                    for (int l = 0; l < kKt; ++l) sel_of(t * kKt + l);
                    acc(SEL, sel_slot(t), -1, true, t);
                }
                for (int l = 0; l < kKt; ++l) sel_of(kSelAhead * kKt + l);
            }
            barrier();
            // P1: rope of tiles 0 and 1
            if (kh == 1)
                for (int t = 0; t < 2; ++t) {
                    acc(SEL, sel_slot(t), -1, false, t);
                    for (int l = 0; l < kKt; ++l) rope(sel_of(t * kKt + l));
                }
            barrier();  // B0
            // P2: S of tile 0
            acc(KV, ring_slot(0), -1, false, 0);
            if (kh == 1) acc(PART, 0 * 2 + ht, -1, true, 0);
            if (kh == 0) acc(SEL, sel_slot(0), -1, false, 0);
            barrier();  // B1
            for (int it = 0; it < ntiles; ++it) {
                const bool more = it + kSAhead < ntiles;
                if (wave == 0) {
                    acc(SEL, sel_slot(it + kSelAhead), -1, true, it + kSelAhead);
                    for (int l = 0; l < kKt; ++l) sel_of((it + kSelAhead + 1) * kKt + l);
                }
                if (kh == 0) {
                    if (more) acc(KV, ring_slot(it + kSAhead), -1, false, it + kSAhead);
                    // softmax of tile it: partner's half in, P and factors out
                    acc(PART, (it & 1) * 2 + ht, -1, false, it);
                    acc(P, (it & 1) * 2 + ht, -1, true, it);
                    acc(CORR, (it & 1) * 2 + ht, -1, true, it);
                    acc(RESC, (it & 1) * 2 + ht, -1, true, it);
                    if (more) acc(SEL, sel_slot(it + kSAhead), -1, false, it + kSAhead);
                } else {
                    if (more) {
                        acc(KV, ring_slot(it + kSAhead), -1, false, it + kSAhead);
                        acc(PART, ((it + kSAhead) & 1) * 2 + ht, -1, true, it + kSAhead);
                    }
                    if (it + kRopeAhead < ntiles) {
                        acc(SEL, sel_slot(it + kRopeAhead), -1, false, it + kRopeAhead);
                        for (int l = 0; l < kKt; ++l) rope(sel_of((it + kRopeAhead) * kKt + l));
                    }
                }
                barrier();
            }
            barrier();  // matches the PV waves' last step
            if (kh == 0) acc(FINL, ht, -1, true, 0);
            barrier();  // E1
            if (kh == 0) {
                for (int hl = ht * 32; hl < ht * 32 + 32; ++hl) {
                    if (C.splits == 1) {
                        in_bounds("lse store", (long long)(rowq * L.H + head0 + hl),
                                  (long long)(rowq * L.H + head0 + hl + 1), C.buf.lse_elems);
                    } else {
                        const size_t o = lse_part_offset(prow, C.splits, wk.split, L.H, head0 + hl);
                        in_bounds("lse partial store", (long long)o, (long long)o + 1,
                                  C.buf.lse_part_elems);
                    }
                }
            }
        } else {
            const int d = wave - 4;
            const int dv0 = d * 128;
            auto stage_load = [&](int t, bool from_ring) {
                if (from_ring) acc(SEL, sel_slot(t), -1, false, t);
                for (int m = 0; m < kStageRows; ++m) gather(sel_of(t * kKt + kStageRows * d + m));
            };
            stage_load(0, false);
            stage_load(1, false);
            barrier();
            acc(KV, ring_slot(0), d, true, 0);
            acc(KV, ring_slot(1), d, true, 1);
            stage_load(2, true);
            stage_load(3, true);
            barrier();  // B0
            barrier();  // B1
            for (int it = 0; it <= ntiles; ++it) {
                const int tp = it - kPvBehind;
                if (tp >= 0) {
                    acc(RESC, (tp & 1) * 2 + 0, -1, false, tp);
                    acc(RESC, (tp & 1) * 2 + 1, -1, false, tp);
                    acc(KV, ring_slot(tp), -1, false, tp);
                    acc(P, (tp & 1) * 2 + 0, -1, false, tp);
                    acc(P, (tp & 1) * 2 + 1, -1, false, tp);
                    acc(CORR, (tp & 1) * 2 + 0, -1, false, tp);
                    acc(CORR, (tp & 1) * 2 + 1, -1, false, tp);
                }
                acc(KV, ring_slot(it + kParkAhead), d, true, it + kParkAhead);
                stage_load(it + kGatherAhead, true);
                barrier();
            }
            barrier();  // E1
            acc(FINL, 0, -1, false, 0);
            acc(FINL, 1, -1, false, 0);
            // output staging: this wave's block in the (now free) tile ring
            const long long blk0 = (long long)d * 32 * kOutPitch * 4;
            in_bounds("output staging in LDS", blk0, blk0 + 32LL * kOutPitch * 4,
                      (long long)kRing * kTileBytes);
            acc(STAGE, d, -1, true, 0);
            for (int a = 0; a < 2; ++a)
                for (int half = 0; half < 2; ++half)
                    for (int l32 = 0; l32 < 32; ++l32) {
                        const int dd = dv0 + 4 * l32;
                        for (int m = 0; m < 16; ++m) {
                            const int head = head0 + a * 32 + half + 2 * m;
                            if (C.splits == 1) {
                                const size_t o = out_offset(rowq, L.H, head0 + a * 32 + half, dd) +
                                                 m * kHeadPairStride;
                                if (o != out_offset(rowq, L.H, head, dd))
                                    fail("output address is not head + 2m", head, m);
                                in_bounds("output store", (long long)o, (long long)o + 4,
                                          C.buf.out_elems);
                                if (o + 4 <= (size_t)C.buf.out_elems) C.out_written[o / 4]++;
                            } else {
                                const size_t o = part_offset(prow, C.splits, wk.split, L.H,
                                                             head0 + a * 32 + half, dd) +
                                                 m * kHeadPairStride;
                                if (o != part_offset(prow, C.splits, wk.split, L.H, head, dd))
                                    fail("partial address is not head + 2m", head, m);
                                in_bounds("partial store", (long long)o, (long long)o + 4,
                                          C.buf.part_elems);
                                if (o + 4 <= (size_t)C.buf.part_elems) C.part_written[o / 4]++;
                            }
                        }
                    }
        }
    }
    // ---- the phases must line up (same barrier count on every wave)
    const size_t nph = waves[0].size();
    for (int w = 1; w < 8; ++w)
        if (waves[w].size() != nph) fail("waves disagree on the number of barriers", w,
                                         (long long)waves[w].size());
    Lds lds;
    for (size_t p = 0; p < nph; ++p) {
        std::vector<Access> all;
        for (int w = 0; w < 8; ++w)
            if (p < waves[w].size()) all.insert(all.end(), waves[w][p].begin(), waves[w][p].end());
        lds.phase(all);
    }
}

void replay_combine(Ctx &C) {
    const Launch &L = *C.L;
    const int n = L.rows;
    const long long ncg = (long long)(L.H / 2) * n * L.B;
    for (long long id = 0; id < ncg; ++id) {
        const CombineWork cw = combine_work_of((int)id, n, L.B, L.H);
        const int r = cw.qidx % n, b = cw.qidx / n;
        if (b >= L.B || cw.hp >= L.H / 2) fail("merge workgroup outside the launch", id, cw.qidx);
        const size_t rowq = (size_t)b * L.T + L.row0 + r;
        const size_t prow = (size_t)b * n + r;
        for (int tid = 0; tid < 256; ++tid) {
            const int h = cw.hp * 2 + (tid >> 7);
            const int d = (tid & 127) * 4;
            const size_t lp = lse_part_offset(prow, C.splits, 0, L.H, h);
            const size_t op = part_offset(prow, C.splits, 0, L.H, h, d);
            for (int s0 = 0; s0 < C.splits; s0 += kCombineBatch)
                for (int j = 0; j < kCombineBatch; ++j) {
                    const size_t sc = (size_t)combine_split(s0, j, C.splits);
                    const size_t lo = lp + sc * lse_split_stride(L.H);
                    const size_t oo = op + sc * part_split_stride(L.H);
                    if (lo != lse_part_offset(prow, C.splits, (int)sc, L.H, h) ||
                        oo != part_offset(prow, C.splits, (int)sc, L.H, h, d))
                        fail("merge address is not the partial's", (long long)sc, h);
                    in_bounds("merge lse read", (long long)lo, (long long)lo + 1,
                              C.buf.lse_part_elems);
                    in_bounds("merge partial read", (long long)oo, (long long)oo + 4,
                              C.buf.part_elems);
                    if (s0 + j < C.splits && oo + 4 <= (size_t)C.buf.part_elems)
                        C.part_read[oo / 4]++;
                }
            const size_t o = out_offset(rowq, L.H, h, d);
            in_bounds("merge output store", (long long)o, (long long)o + 4, C.buf.out_elems);
            if (o + 4 <= (size_t)C.buf.out_elems) C.out_written[o / 4]++;
        }
    }
}

void replay_launch(const Launch &L, uint64_t seed) {
    g_where = L.name;
    const long long f0 = g_fail;
    const std::vector<int32_t> idx = make_selection(L, seed);
    Ctx C;
    C.L = &L;
    C.idx = &idx;
    const Plan p = launch_plan(L.B, L.rows, L.H, L.k);
    C.splits = p.splits;
    C.per_split = p.per_split;
    if ((long long)C.splits * C.per_split < L.k || (long long)(C.splits - 1) * C.per_split >= L.k)
        fail("split plan does not tile the budget", C.splits, C.per_split);
    Buffers &bf = C.buf;
    bf.idx_elems = (long long)L.B * L.T * L.k;
    bf.lat_bytes = (long long)L.B * L.S * kLatRowBytes;
    bf.q_elems = (long long)L.B * L.T * L.H * kDqk;
    bf.out_elems = (long long)L.B * L.T * L.H * kDv;
    bf.lse_elems = (long long)L.B * L.T * L.H;
    bf.part_elems = (long long)part_elems(L.B, L.rows, C.splits, L.H);
    bf.lse_part_elems = (long long)L.B * L.rows * C.splits * L.H;
    bf.ws_bytes = (long long)launch_workspace_bytes(L.B, L.rows, C.splits, L.H, L.out_bytes);
    if (C.splits > 1 && bf.part_elems * L.out_bytes + bf.lse_part_elems * 4 > bf.ws_bytes)
        fail("workspace smaller than the partials", bf.ws_bytes, bf.part_elems);
    C.out_written.assign((size_t)bf.out_elems / 4, 0);
    if (C.splits > 1) {
        C.part_written.assign((size_t)bf.part_elems / 4, 0);
        C.part_read.assign((size_t)bf.part_elems / 4, 0);
    }
    const long long nwg = (long long)(L.H / kHg) * C.splits * L.rows * L.B;
    for (long long id = 0; id < nwg; ++id) replay_workgroup(C, (int)id);
    if (C.splits > 1) {
        for (size_t j = 0; j < C.part_written.size(); ++j)
            if (C.part_written[j] != 1) {
                fail("partial piece not written exactly once", (long long)j, C.part_written[j]);
                break;
            }
        replay_combine(C);
        for (size_t j = 0; j < C.part_read.size(); ++j)
            if (C.part_read[j] != 1) {
                fail("partial piece not read exactly once by the merge", (long long)j,
                     C.part_read[j]);
                break;
            }
    }
    // output pieces of the launch's rows written once, the others untouched
    for (int b = 0; b < L.B; ++b)
        for (int i = 0; i < L.T; ++i) {
            const bool mine = i >= L.row0 && i < L.row0 + L.rows;
            const size_t base = ((size_t)b * L.T + i) * L.H * kDv / 4;
            for (size_t j = 0; j < (size_t)L.H * kDv / 4; ++j)
                if (C.out_written[base + j] != (mine ? 1 : 0)) {
                    fail("output piece not written exactly once", i, C.out_written[base + j]);
                    b = L.B;
                    break;
                }
            if (b == L.B) break;
        }
    std::printf("%-44s B=%d T=%d S=%d H=%d k=%d rows=%d+%d splits=%d x %d  wgs=%lld  %s\n",
                L.name.c_str(), L.B, L.T, L.S, L.H, L.k, L.row0, L.rows, C.splits, C.per_split,
                nwg, g_fail == f0 ? "ok" : "FAILED");
}

// ------------------------------------------- the kernel as of 07:13 ----
// Transcribed from that commit's attention_mla.hip: 8 waves; three-tile LDS
// ring; the split's selection copied into LDS (sm.idx, 4096 entries) before
// the first barrier; every wave stages 16-byte pieces of tiles it+4 (q =
// 512 m + 64 wave + lane, 72 pieces a 1152-byte row; S waves m < 5, PV waves
// m < 4) and parks tile it+2; S of tile it+1 (waves 0-3), PV of tile it
// (waves 4-7); two barriers a step; fp32 partials; merge grid (H/2, n, B).
namespace v0713 {
constexpr int kRing3 = 3, kSlotsRow = 72, kMaxSplit = 4096, kRowPitch3 = 1168;

struct Counts {
    long long gathers = 0;
};

void replay(const Launch &L, uint64_t seed) {
    g_where = L.name + " [07:13 kernel]";
    const long long f0 = g_fail;
    const std::vector<int32_t> idx = make_selection(L, seed);
    const int hgs = L.H / kHg;
    const int n = L.rows;
    // mla_splits of that commit (plus its selection-table bound)
    const long long wgs = (long long)L.B * n * hgs;
    const int max_splits = (L.k + 4 * kKt - 1) / (4 * kKt);
    long long s = (256 + wgs - 1) / wgs;
    if (s > max_splits) s = max_splits;
    if (s < (L.k + kMaxSplit - 1) / kMaxSplit) s = (L.k + kMaxSplit - 1) / kMaxSplit;
    if (s < 1) s = 1;
    const int splits = (int)s;
    const int per_split = ((L.k + splits - 1) / splits + kKt - 1) / kKt * kKt;
    const int used = (L.k + per_split - 1) / per_split;
    const long long lat_bytes = (long long)L.B * L.S * kLatRowBytes;
    const long long part_elems = (long long)L.B * n * used * L.H * kDv;
    const long long lse_part_elems = (long long)L.B * n * used * L.H;
    const long long ws_floats = (long long)L.B * n * splits * L.H * (kDv + 1) + 64;
    if (used > 1 && part_elems + lse_part_elems > ws_floats)
        fail("workspace smaller than the partials", ws_floats, part_elems);
    std::vector<uint8_t> part_written(used > 1 ? (size_t)part_elems : 0, 0);
    const long long nwg = (long long)hgs * used * n * L.B;
    for (long long id = 0; id < nwg; ++id) {
        int hg, split, qidx;
        if ((n * L.B * used) % 8 == 0) {
            const int slot = (int)(id >> 3);
            hg = slot % hgs;
            const int unit = (slot / hgs) * 8 + (int)(id & 7);
            qidx = unit / used;
            split = unit % used;
        } else {
            hg = (int)(id % hgs);
            split = (int)((id / hgs) % used);
            qidx = (int)(id / (hgs * used));
        }
        const int r = qidx % n, b = qidx / n;
        if (b >= L.B) fail("workgroup maps outside the launch", id, qidx);
        const int i = L.row0 + r;
        const int head0 = hg * kHg;
        const int e_begin = split * per_split;
        const int len = std::min(L.k, e_begin + per_split) - e_begin;
        const int ntiles = (len + kKt - 1) / kKt;
        if (len < 1) fail("split without entries (its last-row reload reads idx[-1])", split, len);
        if (ntiles * kKt > kMaxSplit) fail("selection table overflows its LDS array", ntiles, 0);
        const size_t rowq = (size_t)b * L.T + i;
        const size_t sel_base = rowq * L.k + e_begin;
        // the selection table (filled for e < ntiles*32, -1 past len)
        std::vector<int32_t> table(kMaxSplit, INT32_MIN);  // INT32_MIN: never written
        for (int e = 0; e < ntiles * kKt; ++e) {
            if (e < len) in_bounds("selection read", (long long)(sel_base + e),
                                   (long long)(sel_base + e + 1), (long long)idx.size());
            table[e] = e < len ? idx[sel_base + e] : -1;
        }
        const long long lat_b = (long long)b * L.S * kLatRowBytes;
        // stage loads of tile t by wave w: m < 5 (S waves) or m < 4 (PV waves)
        auto stage = [&](int t, int wave) {
            const int nl = wave < 4 ? 5 : 4;
            for (int m = 0; m < nl; ++m)
                for (int lane = 0; lane < 64; lane += 63) {
                    const int q = 512 * m + 64 * wave + lane;
                    const int row = q / kSlotsRow;
                    const int c = q - row * kSlotsRow;
                    if (row >= kKt) fail("staged piece outside the tile", q, row);
                    const int e = t * kKt + row;
                    const int ee = std::min(e, len - 1);
                    if (ee < 0 || ee >= kMaxSplit) {
                        fail("selection table index out of range", ee, e);
                        continue;
                    }
                    const int32_t sel = table[ee];
                    if (sel == INT32_MIN) fail("selection table entry never written", ee, t);
                    const uint64_t src_row = (uint32_t)std::max(sel, 0);
                    in_bounds("latent gather", lat_b + (long long)(src_row * kLatRowBytes + c * 16),
                              lat_b + (long long)(src_row * kLatRowBytes + c * 16) + 16,
                              lat_bytes);
                    // the LDS piece it parks into
                    const long long lds = (long long)row * kRowPitch3 + c * 16;
                    in_bounds("parked piece in the tile", lds, lds + 16, (long long)kKt * kRowPitch3);
                }
        };
        for (int wave = 0; wave < 8; ++wave) {
            stage(0, wave);
            stage(1, wave);
            stage(2, wave);
            stage(3, wave);
            for (int it = 0; it < ntiles; ++it) stage(it + 4, wave);
        }
        // ring: step it parks tile it+2 into slot (it+2)%3, S reads tile it+1,
        // PV reads tile it; every slot written in a step holds tile it-1,
        // which the PV waves finished in step it-1
        for (int it = 0; it < ntiles; ++it) {
            const int wslot = (it + 2) % kRing3;
            if (wslot == (it + 1) % kRing3 || wslot == it % kRing3)
                fail("parked over a tile in use", it, wslot);
        }
        // query block, outputs
        for (int w = 0; w < 4; ++w) {
            const int ht = w & 1, kh = w >> 1;
            for (int l32 = 0; l32 < 32; l32 += 31)
                for (int half = 0; half < 2; ++half) {
                    const size_t qp = (rowq * L.H + head0 + ht * 32 + l32) * kDqk + 8 * half +
                                      16 * 18 * kh;
                    in_bounds("query load", (long long)qp, (long long)(qp + 17 * 16 + 8),
                              (long long)L.B * L.T * L.H * kDqk);
                }
        }
        for (int d = 0; d < 4; ++d)
            for (int a = 0; a < 2; ++a)
                for (int m = 0; m < 16; ++m)
                    for (int half = 0; half < 2; ++half)
                        for (int l32 = 0; l32 < 32; ++l32) {
                            const int hl = a * 32 + 2 * m + half;
                            const int dd = d * 128 + 4 * l32;
                            if (used == 1) {
                                const size_t o = (rowq * L.H + head0 + hl) * kDv + dd;
                                in_bounds("output store", (long long)o, (long long)o + 4,
                                          (long long)L.B * L.T * L.H * kDv);
                            } else {
                                const size_t o =
                                    (((size_t)qidx * used + split) * L.H + head0 + hl) * kDv + dd;
                                in_bounds("partial store", (long long)o, (long long)o + 4,
                                          part_elems);
                                if (o + 4 <= (size_t)part_elems)
                                    for (int e = 0; e < 4; ++e) part_written[o + e]++;
                            }
                        }
        if (used > 1)
            for (int hl = 0; hl < kHg; ++hl) {
                const size_t o = ((size_t)qidx * used + split) * L.H + head0 + hl;
                in_bounds("lse partial store", (long long)o, (long long)o + 1, lse_part_elems);
            }
    }
    if (used > 1) {
        for (size_t j = 0; j < part_written.size(); ++j)
            if (part_written[j] != 1) {
                fail("partial not written exactly once", (long long)j, part_written[j]);
                break;
            }
        // merge: grid (H/2, n, B), 256 threads
        for (int bz = 0; bz < L.B; ++bz)
            for (int r = 0; r < n; ++r)
                for (int bx = 0; bx < L.H / 2; ++bx)
                    for (int tid = 0; tid < 256; tid += 127) {
                        const int h = bx * 2 + (tid >> 7);
                        const int d = (tid & 127) * 4;
                        const size_t prow = (size_t)bz * n + r;
                        for (int sc = 0; sc < used; ++sc) {
                            const size_t lp = prow * used * L.H + h + (size_t)sc * L.H;
                            const size_t op = (prow * used * L.H + h) * kDv + d +
                                              (size_t)sc * L.H * kDv;
                            in_bounds("merge lse read", (long long)lp, (long long)lp + 1,
                                      lse_part_elems);
                            in_bounds("merge partial read", (long long)op, (long long)op + 4,
                                      part_elems);
                        }
                        const size_t o = (((size_t)bz * L.T + L.row0 + r) * L.H + h) * kDv + d;
                        in_bounds("merge output store", (long long)o, (long long)o + 4,
                                  (long long)L.B * L.T * L.H * kDv);
                    }
    }
    std::printf("%-44s B=%d T=%d S=%d H=%d k=%d rows=%d+%d splits=%d x %d  wgs=%lld  %s\n",
                g_where.c_str(), L.B, L.T, L.S, L.H, L.k, L.row0, L.rows, used, per_split, nwg,
                g_fail == f0 ? "ok" : "FAILED");
}
}  // namespace v0713

Launch mk(const char *name, int B, int T, int S, int H, int k, int row0, int rows, bool tail,
          int out_bytes, const char *sel, std::vector<int> qpos = {}) {
    Launch L;
    L.name = name;
    L.B = B, L.T = T, L.S = S, L.H = H, L.k = k, L.row0 = row0, L.rows = rows;
    L.causal_tail = tail, L.out_bytes = out_bytes, L.qpos = qpos, L.sel = sel;
    return L;
}

}  // namespace

int main(int argc, char **argv) {
    // --quick: no 2048-row prefill chunks; --mini: the 128K decode launches
    // and the small shapes only (the mutation test)
    const std::string mode = argc > 1 ? argv[1] : "";
    const bool quick = mode == "--quick" || mode == "--mini";
    const bool mini = mode == "--mini";
    std::vector<Launch> launches = {
        // the 128K decode step: 8 sequences x 131072, one query row each
        mk("128K decode (forward: causal tail)", 8, 1, 131072, 128, 2048, 0, 1, true, 2, "causal"),
        mk("128K decode, every entry = S-1", 8, 1, 131072, 128, 2048, 0, 1, false, 2, "max"),
        mk("128K decode, entries past the cache (outside the contract)", 8, 1, 131072, 128, 2048,
           0, 1, false, 2, "wild"),
        mk("128K decode, holes and -1 anywhere", 8, 1, 131072, 128, 2048, 0, 1, false, 2,
           "holes"),
        mk("128K decode, positions t < k (empty splits)", 8, 1, 131072, 128, 2048, 0, 1, true, 2,
           "causal", {0, 1, 31, 32, 100, 2047, 2048, 131071}),
        mk("128K decode, positions past the cache", 8, 1, 131072, 128, 2048, 0, 1, true, 2,
           "causal", {131072, 140000, 131071, 5, 0, -1, 2049, 65536}),
        // the 32K x 64 decode step
        mk("32K x 64 decode (forward)", 64, 1, 32768, 128, 2048, 0, 1, true, 2, "causal"),
        // unit tests' shapes
        mk("prefill rows 40 of 3000", 1, 40, 3000, 128, 2048, 0, 40, false, 2, "holes"),
        mk("decode 2 x 5000 fp32 out", 2, 1, 5000, 128, 2048, 0, 1, false, 4, "holes"),
        mk("ragged budget 3 x 7 of 700, k=100", 3, 7, 700, 128, 100, 0, 7, false, 2, "holes"),
        mk("one step 1 x 64, k=64", 1, 1, 64, 128, 64, 0, 1, false, 4, "causal"),
        mk("dense limit n = k = 2048 (causal tail)", 1, 2048, 2048, 128, 2048, 0, 2048, true, 2,
           "causal"),
        mk("chunked forward: last chunk of 3 rows", 1, 1027, 65536, 128, 2048, 1024, 3, true, 2,
           "causal"),
        mk("decode 4 x 3000 causal tail, t < k", 4, 1, 3000, 128, 2048, 0, 1, true, 2, "causal",
           {2999, 100, 2047, 0}),
        mk("256 heads, 5 rows", 1, 5, 4000, 256, 2048, 0, 5, true, 2, "causal"),
    };
    if (!quick) {
        // a 32K prefill chunk as the forward pass launches it (2048 rows)
        launches.push_back(mk("32K prefill chunk (rows 30720..32767)", 1, 32768, 32768, 128, 2048,
                              30720, 2048, true, 2, "causal"));
        launches.push_back(mk("32K prefill first chunk (rows 0..2047)", 1, 32768, 32768, 128,
                              2048, 0, 2048, true, 2, "causal"));
    }
    uint64_t seed = 1;
    for (const Launch &L : launches) {
        if (mini && L.rows * L.B > 512) continue;
        replay_launch(L, seed++);
    }
    // the 07:13 kernel at the launches of the fault report and its neighbours
    std::vector<Launch> old = {
        mk("128K decode, sorted distinct entries", 8, 1, 131072, 128, 2048, 0, 1, false, 2,
           "causal"),
        mk("128K decode, every entry = S-1", 8, 1, 131072, 128, 2048, 0, 1, false, 2, "max"),
        mk("128K decode, holes", 8, 1, 131072, 128, 2048, 0, 1, false, 2, "holes"),
        mk("decode 2 x 5000", 2, 1, 5000, 128, 2048, 0, 1, false, 4, "holes"),
        mk("ragged budget 3 x 7 of 700, k=100", 3, 7, 700, 128, 100, 0, 7, false, 2, "holes"),
    };
    for (const Launch &L : old) v0713::replay(L, seed++);
    std::printf("%s: %lld failed checks\n", g_fail ? "FAILED" : "ok", g_fail);
    return g_fail ? 1 : 0;
}
