// attention_mla.hip -- MLA-latent sparse attention on gfx950 matrix cores.
//
// Attention over the selected latent rows in the MQA mode of MLA: one latent
// row c_s (576 = 512 latent + 64 rope dims, bf16) per position is both the key
// (all 576 dims) and the value (first 512 dims) of every head, and one
// selected set per query serves all heads ("DeepSeek Sparse Attention:
// Learned Token Selection from Scratch", sections 3.3 and 4.1-4.2; "DeepSeek
// NSA and DSA", section 3.1).  Because every gathered row is shared by all
// heads, the heads form the M dimension of dense MFMA tiles.
//
// Workgroup = 8 waves = one query row x 64 heads x one range of selected
// entries, walked 32 entries at a time, one workgroup barrier a tile
// (details at the kernel):
//   gather  the latent dims (0..511) of the selected rows are loaded into
//           registers two tiles ahead and parked in a four-tile LDS ring; the
//           row pitch carries one spare 16-byte slot against bank conflicts;
//           masked entries load a valid row whose probability is then forced
//           to 0; the rope dims (512..575) go from memory straight into the
//           registers of the waves that multiply them;
//   S       4 waves compute S^T = C(32 keys) . Q^T(32 heads), each over half
//           of the 576 dims (v_mfma_f32_32x32x16_bf16), the query block held
//           in registers as the B operand; the halves meet in LDS;
//   softmax online, fp32, on the S waves, one tile behind their products and
//           interleaved with them; probabilities written to LDS as bf16
//           [head][key];
//   PV      4 waves accumulate O[64 heads, 128 dims each] += P . V one tile
//           behind the softmax, V read straight from the row-major tile with
//           the LDS transpose read (ds_read_b64_tr_b16) as the B operand.
// Decode rows split their entries over several workgroups; each writes a
// normalised partial output and its log-sum-exp, merged by a second kernel.
#include "dsa_internal.h"
#include "mla_schedule.h"

namespace dsa {
namespace {

using namespace mla;  // shapes, tile schedule and addressing (mla_schedule.h)

constexpr float kRescaleLog2 = 8.0f;  // reference-max slack, base-2 units

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 lds_b128(const uint8_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i%4 of the 4-element vectors addressed by lanes
// 4e + i/4 (e = 0..3): pointing lane j at row r0 + j/4, column c0 + 4*(j%4)
// of a row-major bf16 tile hands lane i the column c0 + i of rows r0..r0+3.
__device__ __forceinline__ bf16x4 lds_tr16(const uint8_t *p) {
    typedef __attribute__((address_space(3))) bf16x4 *lds_v4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4)(p));
}

// 4 consecutive outputs (16-byte aligned as fp32, 8-byte as bf16)
template <typename Tout>
__device__ __forceinline__ void store_out4(Tout *p, f32x4 v);
template <>
__device__ __forceinline__ void store_out4<float>(float *p, f32x4 v) {
    *reinterpret_cast<f32x4 *>(p) = v;
}
template <>
__device__ __forceinline__ void store_out4<uint16_t>(uint16_t *p, f32x4 v) {
    const bf16x4 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *reinterpret_cast<bf16x4 *>(p) = b;
}

template <typename Tout>
__device__ __forceinline__ void store_out(Tout *p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t *p, float v) {
    *p = (uint16_t)f32_to_bf16_bits(v);
}

// ---------------------------------------------------------------------------
// The kernel: 8 waves = 2 per SIMD, 32-entry tiles.  Iteration it:
//   waves 0-3 ("S" waves): wave (ht = w&1, kh = w>>1) holds the query block of
//       32 heads over half of the 576 dims (18 k-steps, 72 registers) and
//       computes that half of S^T for tile it+1; the kh = 1 half goes through
//       LDS to its kh = 0 partner.  Between those products the kh = 0 wave
//       runs the online softmax of tile it: its own half of S(it), kept in
//       registers since the previous iteration, plus the partner's half; it
//       writes P(it) (bf16) and the rescale factors.  The 32-entry tile max
//       is in-wave (16 registers and one cross-half swap).
//   waves 4-7 ("PV" waves): wave 4+d owns O[64 heads, dims 128d..128d+127]
//       and adds P(it-1) . V(it-1); it also gathers the latent dims of rows
//       8d..8d+7 of tile it+4 into registers and parks those of tile it+2.
// The rows of each tile sit in an LDS ring of selections, kept filled by
// wave 0 five tiles ahead.
// One workgroup barrier ends each iteration.  Tiles it-1 (PV), it (PV next),
// it+1 (S) and it+2 (parked now) fill the four ring slots; P, the rescale
// factors and the S halves alternate between two buffers by tile parity.
// The S and PV waves share each SIMD, so one role's latencies are covered by
// the other's matrix work.  The kh = 1 waves read the rope dims of tile it+1
// from registers loaded one iteration earlier.
constexpr int kPPitch = kKt * 2 + 16;            // 80 bytes per head row of P
constexpr int kLdsSteps1 = kHalfSteps - kRopeSteps;  // 14 k-steps of kh = 1 read from LDS
constexpr int kThreads = 512;

// LDS row of entry m of a tile: within each block of 16 entries, entry
// 4a + b sits in row 4b + a.  A row is 1040 bytes (16 bytes past a multiple
// of 256), so rows 16 bytes apart in bank order; the S reads (16 consecutive
// entries, one 16-byte piece each) still hit 16 distinct bank groups, and the
// transposed V reads (4 consecutive entries x 64 bytes) now land 64 bytes
// apart instead of overlapping.
__device__ __forceinline__ int tile_row(int m) {
    return (m & ~15) | ((m & 3) << 2) | ((m >> 2) & 3);
}

struct __align__(16) MlaSmem {
    uint8_t kv[kRing][kTileBytes];    // 4 x 33280
    uint8_t p[2][kHg * kPPitch];      // 2 x 5120
    f32x4 part[2][2][4][64];          // kh = 1 halves of S: [tile parity][head tile][j][lane]
                                      // = registers 4j..4j+3 of lane l
    float corr[2][kHg];
    float fin_l[kHg];                   // 1 / softmax denominator per head
    int32_t sel[kSelRing][kKt];         // rows of tile t at [t % kSelRing]; -1: none
    int32_t resc[2][2];                 // per tile parity and head tile: any corr != 1
};
static_assert(offsetof(MlaSmem, corr) % 16 == 0, "corr is read in 16-byte pieces");
static_assert(sizeof(MlaSmem) <= 160 * 1024, "fits the LDS of a CU");

template <typename Tout>
__global__ __launch_bounds__(kThreads, 1) void mla_attention_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ lat,
    const int32_t *__restrict__ idx, int T, int S, int H, int k, float scale, int row0,
    int rows, int B, int splits, int per_split, Tout *__restrict__ out, float *__restrict__ lse,
    Tout *__restrict__ o_part, float *__restrict__ lse_part, const int32_t *__restrict__ q_pos,
    int causal_tail) {
    __shared__ MlaSmem sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int hgs = H / kHg;
    const int id = blockIdx.x;
    // XCD-aware order: the two head groups of a query row share the gathered
    // rows and the query block in one XCD's L2, and the split partials are
    // written where the merge reads them
    const Work wk = work_of(id, rows, B, hgs, splits);
    const int hg = wk.hg, split = wk.split, qidx = wk.qidx, r = wk.r, b = wk.b;
    const int i = row0 + r;
    const int head0 = hg * kHg;
    const int e_begin = split * per_split;
    // entries of this split; with causal_tail the tiles past the row's
    // min(k, t+1) selected positions are empty and not visited
    const int len = split_len(split, per_split, k, causal_tail != 0,
                              causal_tail ? query_pos(q_pos, b, i, T, S) : 0);
    const int ntiles = split_tiles(len);
    const int32_t *sel_row = idx + ((size_t)b * T + i) * k + e_begin;
    const uint8_t *lat_b = reinterpret_cast<const uint8_t *>(lat) + (size_t)b * S * kLatRowBytes;
    const int32_t s_last = S - 1;  // gathers stay inside the sequence's rows
    const size_t rowq = (size_t)b * T + i;
    const size_t prow = (size_t)qidx;  // row of this launch's split partials
    // selected row of entry e of the split (-1: masked or past the split)
    auto sel_of = [&](int e) -> int32_t { return e < len ? sel_row[e] : -1; };

    const float sl2 = scale * 1.4426950408889634f;
    if (wave < 4) {
        // ======================= S waves =======================
        const int ht = wave & 1, kh = wave >> 1;
        bf16x8 qb[kHalfSteps];
        {
#pragma unroll
            for (int ks = 0; ks < kHalfSteps; ++ks)
                qb[ks] = *reinterpret_cast<const bf16x8 *>(
                    q + q_offset(rowq, H, head0, ht, l32, half, kh, ks));
        }
        // rope fragments (kh = 1) of tile t: k-steps 14..17 of this half
        auto rope_load = [&](int t, bf16x8 (&rp)[kRopeSteps]) {
            const int32_t s = sm.sel[sel_slot(t)][l32];
#pragma unroll
            for (int j = 0; j < kRopeSteps; ++j)
                rp[j] = *reinterpret_cast<const bf16x8 *>(lat_b + rope_offset(s, s_last, half, j));
        };
        // this wave's half of S^T(t): K fragments from the LDS ring (and, for
        // kh = 1, the rope registers)
        auto s_read = [&](int t, bf16x8 (&af)[kHalfSteps], const bf16x8 (&rp)[kRopeSteps]) {
            const uint8_t *arow =
                sm.kv[ring_slot(t)] + tile_row(l32) * kRowPitch + 16 * half + 576 * kh;
            if (kh == 0) {
#pragma unroll
                for (int ks = 0; ks < kHalfSteps; ++ks) af[ks] = lds_b128(arow + ks * 32);
            } else {
#pragma unroll
                for (int ks = 0; ks < kLdsSteps1; ++ks) af[ks] = lds_b128(arow + ks * 32);
#pragma unroll
                for (int j = 0; j < kRopeSteps; ++j) af[kLdsSteps1 + j] = rp[j];
            }
        };
        auto put_part = [&](int t, const f32x16 &acc) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm.part[t & 1][ht][j][lane] = f32x4{acc[4 * j], acc[4 * j + 1], acc[4 * j + 2],
                                                    acc[4 * j + 3]};
        };
        float m_run = -INFINITY, l_run = 0.0f;
        // Masked entries of tile t (kh = 0): its own half of S set to -inf, so
        // the sum with the partner's half is -inf too.  Whole tiles are the
        // rule; the branch is uniform.
        auto mask_tile = [&](int t, f32x16 &acc) {
            // an entry counts when it is a cached position: -1 (unused) and
            // entries past the cache (outside the contract) are masked
            const uint32_t vmask =
                (uint32_t)__ballot((uint32_t)sm.sel[sel_slot(t)][l32] < (uint32_t)S);
            if (vmask != 0xffffffffu) {
                const uint32_t mh = vmask >> (4 * half);
#pragma unroll
                for (int rg = 0; rg < 16; ++rg)
                    if (!((mh >> (8 * (rg >> 2) + (rg & 3))) & 1u)) acc[rg] = -INFINITY;
            }
        };
        // Online softmax of tile t (kh = 0): own half `acc` (masked entries
        // -inf) plus the partner's half from LDS.  Branch-free, so it
        // schedules between the products; the scale is applied to the max and
        // inside the exponent (fma), since scale > 0 keeps the order.
        auto softmax = [&](int t, f32x16 acc) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 o = sm.part[t & 1][ht][j][lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[4 * j + e] += o[e];
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) tmax = fmaxf(tmax, acc[rg]);
            tmax = max_halves(tmax) * sl2;
            const bool grow = tmax > m_run + kRescaleLog2;
            const float corr = grow ? (m_run == -INFINITY ? 0.0f
                                                          : __builtin_amdgcn_exp2f(m_run - tmax))
                                    : 1.0f;
            m_run = grow ? tmax : m_run;
            // no selected entry so far: every entry is -inf and exp2 gives 0
            const float m_ref = m_run == -INFINITY ? 0.0f : m_run;
            float ps0 = 0.0f, ps1 = 0.0f;
            uint8_t *prow = sm.p[t & 1] + (ht * 32 + l32) * kPPitch;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float pv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pv[j] = __builtin_amdgcn_exp2f(fmaf(acc[4 * g + j], sl2, -m_ref));
                ps0 += pv[0] + pv[1];
                ps1 += pv[2] + pv[3];
                const bf16x4 pk = {(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3]};
                *reinterpret_cast<bf16x4 *>(prow + (8 * g + 4 * half) * 2) = pk;
            }
            l_run = l_run * corr + (ps0 + ps1);
            sm.corr[t & 1][ht * 32 + l32] = corr;  // both halves write the same value
            sm.resc[t & 1][ht] = __ballot(corr != 1.0f) != 0;
        };
        // Ask the scheduler to spread the LDS reads over the products (the
        // first few ahead of them) and to put vector work between the
        // products: right after a barrier every wave wants LDS at once, and
        // reading a whole K half before the first product would hold the
        // matrix pipe until the slowest read.
        auto interleave = [&](auto valu_per_product) {
            constexpr int kValu = decltype(valu_per_product)::value;
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // 6 LDS reads
#pragma unroll
            for (int j = 0; j < kHalfSteps; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                if constexpr (kValu > 0) __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
            }
        };

        // Wave 0 keeps the selection ring filled: the rows of tile it+5 are
        // written at iteration it from a load issued one iteration earlier
        // (the wave has no other memory loads, so that wait is free), ahead of
        // every reader: the gathering waves (tile it+4), the rope loads (tile
        // it+2) and the mask (tile it+1).
        int32_t sel_next = 0;
        if (wave == 0) {
            int32_t sv[kSelPrologue];
#pragma unroll
            for (int t = 0; t < kSelPrologue; ++t) sv[t] = sel_of(t * kKt + l32);
            sel_next = sel_of(kSelAhead * kKt + l32);
#pragma unroll
            for (int t = 0; t < kSelPrologue; ++t)
                if (half == 0) sm.sel[sel_slot(t)][l32] = sv[t];
        }
        lds_barrier();  // selection of tiles 0..4
        bf16x8 rp[2][kRopeSteps];  // kh = 1: rope of tiles it+1 (in use) and it+2
        if (kh == 1) {  // in flight together with the first gathers
            rope_load(0, rp[0]);
            rope_load(1, rp[1]);
        }
        lds_barrier();  // B0: tiles 0 and 1
        f32x16 s_cur;  // kh = 0: own half of S of the tile the softmax takes next
        {
            bf16x8 af[kHalfSteps];
            s_read(0, af, rp[0]);
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < kHalfSteps; ++ks)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], qb[ks], acc, 0, 0, 0);
            if (kh == 1) put_part(0, acc);
            if (kh == 0) mask_tile(0, acc);
            s_cur = acc;
        }
        lds_barrier();  // B1: S(0) halves
        // iteration it: products of tile it+1, softmax of tile it; rope of
        // tile it+1 in rp[c], loads of tile it+2 into rp[c ^ 1]
        auto s_step = [&](const int it, bf16x8 (&rcur)[kRopeSteps],
                          bf16x8 (&rnext)[kRopeSteps]) {
            const bool more = it + kSAhead < ntiles;
            if (wave == 0) {
                if (half == 0) sm.sel[sel_slot(it + kSelAhead)][l32] = sel_next;
                sel_next = sel_of((it + kSelAhead + 1) * kKt + l32);
            }
            if (kh == 0) {
                if (more) {
                    bf16x8 af[kHalfSteps];
                    s_read(it + kSAhead, af, rcur);
                    f32x16 nx = {};
#pragma unroll
                    for (int ks = 0; ks < kHalfSteps; ++ks)
                        nx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], qb[ks], nx, 0, 0, 0);
                    softmax(it, s_cur);
                    interleave(std::integral_constant<int, 5>{});
                    mask_tile(it + kSAhead, nx);
                    s_cur = nx;
                } else {
                    softmax(it, s_cur);
                }
            } else {
                if (more) {
                    bf16x8 af[kHalfSteps];
                    s_read(it + kSAhead, af, rcur);
                    f32x16 nx = {};
#pragma unroll
                    for (int ks = 0; ks < kHalfSteps; ++ks)
                        nx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], qb[ks], nx, 0, 0, 0);
                    interleave(std::integral_constant<int, 0>{});
                    put_part(it + kSAhead, nx);
                }
                if (it + kRopeAhead < ntiles) rope_load(it + kRopeAhead, rnext);
            }
            lds_barrier();
        };
        // Pairs of steps, so that the rope registers alternate statically.
        int it = 0;
        for (; it + 1 < ntiles; it += 2) {
            s_step(it, rp[1], rp[0]);
            s_step(it + 1, rp[0], rp[1]);
        }
        if (it < ntiles) s_step(it, rp[1], rp[0]);
        lds_barrier();  // matches the PV waves' last step
        float l_all = 0.0f;
        if (kh == 0) {
            l_all = sum_halves(l_run);  // both key halves
            if (half == 0) sm.fin_l[ht * 32 + l32] = l_all > 0.0f ? 1.0f / l_all : 0.0f;
        }
        lds_barrier();  // E1: 1/l for the output
        if (kh == 0 && half == 0) {
            const int hl = ht * 32 + l32;
            const float ls = l_all > 0.0f ? (m_run + log2f(l_all)) * 0.6931471805599453f : -INFINITY;
            if (splits == 1) {
                if (lse) lse[rowq * H + head0 + hl] = ls;
            } else {
                lse_part[lse_part_offset(prow, splits, split, H, head0 + hl)] = ls;
            }
        }
    } else {
        // ======================= PV waves =======================
        const int d = wave - 4;
        const int dv0 = d * 128;
        // gather: rows 8d..8d+7 of tile t, one row a load (lane = 16-byte
        // piece); the rows come from the selection ring
        auto stage_load = [&](int t, u32x4 (&st)[kStageRows]) {
            const int32_t *sr = sm.sel[sel_slot(t)] + kStageRows * d;
            int32_t rowv[kStageRows];
#pragma unroll
            for (int m = 0; m < kStageRows; ++m) rowv[m] = sr[m];
#pragma unroll
            for (int m = 0; m < kStageRows; ++m) {
                const int32_t s = __builtin_amdgcn_readfirstlane(rowv[m]);
                st[m] = *reinterpret_cast<const u32x4 *>(lat_b + gather_offset(s, s_last, lane));
            }
        };
        auto stage_store = [&](int t, const u32x4 (&st)[kStageRows]) {
            uint8_t *dst = sm.kv[ring_slot(t)] + 16 * lane;
#pragma unroll
            for (int m = 0; m < kStageRows; ++m)
                *reinterpret_cast<u32x4 *>(dst + tile_row(kStageRows * d + m) * kRowPitch) = st[m];
        };
        // the first tiles take their rows straight from the selection in memory
        // (uniform loads), so their gathers start before the ring is filled
        auto stage_load_first = [&](int t, u32x4 (&st)[kStageRows]) {
#pragma unroll
            for (int m = 0; m < kStageRows; ++m) {
                const int32_t s =
                    __builtin_amdgcn_readfirstlane(sel_of(t * kKt + kStageRows * d + m));
                st[m] = *reinterpret_cast<const u32x4 *>(lat_b + gather_offset(s, s_last, lane));
            }
        };
        u32x4 stg[2][kStageRows];
        stage_load_first(0, stg[0]);
        stage_load_first(1, stg[1]);
        lds_barrier();  // selection of tiles 0..4 (matches the S waves')
        stage_store(0, stg[0]);
        stage_store(1, stg[1]);
        stage_load(2, stg[0]);
        __builtin_amdgcn_sched_barrier(0);
        stage_load(3, stg[1]);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 o[2][4];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c) o[a][c] = f32x16{};
        lds_barrier();  // B0 (matches the S waves')
        lds_barrier();  // B1
        const int trj = lane & 15, trg = lane >> 4;
        const int vrow = 8 * (trg >> 1) + (trj >> 2);
        const int vrow_lo = tile_row(vrow), vrow_hi = tile_row(vrow + 4);
        const int vcol = (dv0 + 16 * (trg & 1) + 4 * (trj & 3)) * 2;
        // Operands of one 16-entry k-step of tile `tile`: P (A, 32 heads x 16
        // entries per head tile) and V (B, 16 entries x 32 dims per column tile).
        auto pv_read = [&](int tile, int ks, bf16x8 (&pa)[2], bf16x8 (&vb)[4]) {
            const uint8_t *kvt = sm.kv[ring_slot(tile)];
            const uint8_t *pt = sm.p[tile & 1];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                pa[a] = lds_b128(pt + (a * 32 + l32) * kPPitch + (16 * ks + 8 * half) * 2);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint8_t *vp = kvt + 16 * ks * kRowPitch + vcol + 64 * c;
                const bf16x4 lo = lds_tr16(vp + vrow_lo * kRowPitch);
                const bf16x4 hi = lds_tr16(vp + vrow_hi * kRowPitch);
                vb[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        };
        auto pv_mfma = [&](const bf16x8 (&pa)[2], const bf16x8 (&vb)[4]) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int a = 0; a < 2; ++a)
                    o[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[a], vb[c], o[a][c], 0,
                                                                      0, 0);
        };
        // Iteration it: P(it-1) . V(it-1); park tile it+2 (loaded two
        // iterations ago) and gather tile it+4.  The first k-step's reads are
        // issued before the parking, so their latency overlaps it; the gathers
        // and the second k-step's reads follow the first k-step's products.
        auto o_step = [&](const int it, u32x4 (&st)[kStageRows]) {
            const int tp = it - kPvBehind;
            const bool pv = tp >= 0;
            int32_t f0 = 0, f1 = 0;
            bf16x8 pa[2], vb[4];
            if (pv) {
                f0 = sm.resc[tp & 1][0];
                f1 = sm.resc[tp & 1][1];
                pv_read(tp, 0, pa, vb);
            }
            __builtin_amdgcn_sched_barrier(0);
            stage_store(it + kParkAhead, st);
            __builtin_amdgcn_sched_barrier(0);
            if (pv) {
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    if (__builtin_amdgcn_readfirstlane(a == 0 ? f0 : f1)) {
                        f32x4 cr[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            cr[j] = *reinterpret_cast<const f32x4 *>(
                                &sm.corr[tp & 1][a * 32 + 8 * j + 4 * half]);
#pragma unroll
                        for (int c = 0; c < 4; ++c)
#pragma unroll
                            for (int rg = 0; rg < 16; ++rg) o[a][c][rg] *= cr[rg >> 2][rg & 3];
                    }
                }
                pv_mfma(pa, vb);
            }
            __builtin_amdgcn_sched_barrier(0);
            stage_load(it + kGatherAhead, st);
            __builtin_amdgcn_sched_barrier(0);
            if (pv) {
                pv_read(tp, 1, pa, vb);
                pv_mfma(pa, vb);
            }
            lds_barrier();
        };
        // ntiles + 1 steps, in pairs so that at the top of the loop the stg[1]
        // loads are always the newer ones and parking stg[0] waits for its own
        // loads only.
        int it = 0;
        for (; it + 1 <= ntiles; it += 2) {
            o_step(it, stg[0]);
            o_step(it + 1, stg[1]);
        }
        if (it <= ntiles) o_step(it, stg[0]);
        lds_barrier();  // E1: 1/l from the S waves
        // Output through LDS (the tile ring is free now): the accumulator
        // layout gives a lane one dim of 16 heads, memory wants rows of dims;
        // each 32-head half goes to a [head][dim] block (pitch 136 floats, so
        // the two lane halves write disjoint banks) and leaves in 16-byte
        // pieces, 4 consecutive dims a lane.
        float *blk = reinterpret_cast<float *>(sm.kv[0]) + d * (32 * kOutPitch);
        float inv[2][16];  // 1/l per head, all read before any block write
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                inv[a][rg] = sm.fin_l[a * 32 + 8 * (rg >> 2) + 4 * half + (rg & 3)];
            }
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const int hr = 8 * (rg >> 2) + 4 * half + (rg & 3);  // head within the half
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    blk[hr * kOutPitch + 32 * c + l32] = o[a][c][rg] * inv[a][rg];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            f32x4 v[16];  // 32 heads x 128 dims = 16 rounds of 64 x 4, all read first
#pragma unroll
            for (int m = 0; m < 16; ++m)
                v[m] = *reinterpret_cast<const f32x4 *>(blk + (2 * m + half) * kOutPitch + 4 * l32);
            const int dd = dv0 + 4 * l32;
            // heads head0 + a*32 + half + 2m
            Tout *ob = splits == 1
                           ? out + out_offset(rowq, H, head0 + a * 32 + half, dd)
                           : o_part + part_offset(prow, splits, split, H, head0 + a * 32 + half, dd);
#pragma unroll
            for (int m = 0; m < 16; ++m) store_out4(ob + m * kHeadPairStride, v[m]);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();  // block reused by the second half
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
}

// 4 consecutive partial outputs as fp32
template <typename Tout>
__device__ __forceinline__ f32x4 load_out4(const Tout *p);
template <>
__device__ __forceinline__ f32x4 load_out4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
template <>
__device__ __forceinline__ f32x4 load_out4<uint16_t>(const uint16_t *p) {
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}

// Merge split partials: out = sum_s exp(lse_s - lse) o_s, lse = log sum exp lse_s.
// The partials are normalised outputs kept in the output type (bf16 partials
// halve the bytes written and read back; their rounding is that of the output).
// Two heads per workgroup, 4 dims per thread; the splits are read in batches
// of 16 whose loads are all issued before any is used (clamped indices, zero
// weight past the last split), merged online across batches, so a row costs
// one memory latency per 16 splits.
template <typename Tout>
__global__ __launch_bounds__(256) void mla_combine_kernel(
    const Tout *__restrict__ o_part, const float *__restrict__ lse_part, int T, int H,
    int row0, int rows, int B, int splits, Tout *__restrict__ out, float *__restrict__ lse) {
    // workgroup = (query row, head pair); with a multiple of 8 rows the rows
    // map to XCDs as in the attention kernel, so the partials come from L2
    const CombineWork cw = combine_work_of(blockIdx.x, rows, B, H);
    const int hp = cw.hp, qidx = cw.qidx;
    const int h = hp * 2 + (threadIdx.x >> 7);
    const int d = (threadIdx.x & 127) * 4;
    const int r = qidx % rows;
    const int b = qidx / rows;
    const size_t rowq = (size_t)b * T + row0 + r;
    const size_t prow = (size_t)b * rows + r;  // row of the launch's split partials
    // split s at lp[s * lse_split_stride] and op[s * part_split_stride]
    const float *lp = lse_part + lse_part_offset(prow, splits, 0, H, h);
    const Tout *op = o_part + part_offset(prow, splits, 0, H, h, d);
    float mx = -INFINITY, wsum = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < splits; s0 += kCombineBatch) {
        float ls[kCombineBatch];
        f32x4 ov[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {
            const size_t sc = (size_t)combine_split(s0, j, splits);
            ls[j] = lp[sc * lse_split_stride(H)];
            ov[j] = load_out4(op + sc * part_split_stride(H));
        }
        float bmx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j)
            if (s0 + j < splits) bmx = fmaxf(bmx, ls[j]);
        const float nmx = fmaxf(mx, bmx);
        if (nmx == -INFINITY) continue;  // nothing selected so far
        const float rs = mx == -INFINITY ? 0.0f : __expf(mx - nmx);
        wsum *= rs;
        acc *= rs;
        mx = nmx;
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {
            const float wgt = s0 + j < splits ? __expf(ls[j] - mx) : 0.0f;
            wsum += wgt;
            acc += wgt * ov[j];
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    Tout *o = out + out_offset(rowq, H, h, d);
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out(o + e, acc[e] * inv);
    if (lse && d == 0) lse[rowq * H + h] = wsum > 0.0f ? mx + __logf(wsum) : -INFINITY;
}

}  // namespace

bool mla_fast_path(const dsa_attn_desc_t &d) {
    return d.form == DSA_MLA && d.dtype == DSA_BF16 && d.d_qk == kDqk && d.d_v == kDv &&
           d.num_heads % kHg == 0;
}

size_t mla_workspace_bytes(const dsa_attn_desc_t &d, int B, int T, int k) {
    // A launch covers at most kMaxGridY rows; any row count up to that bound
    // (a short last chunk included) may need split partials, and only counts
    // with fewer than 256 workgroups split at all.
    size_t total = 0;
    const int hgs = d.num_heads / kHg;
    const int top = min(T, kMaxGridY);
    for (int n = 1; n <= top; ++n) {
        if ((long long)B * n * hgs >= 256) break;
        const Plan p = launch_plan(B, n, d.num_heads, k);
        const size_t need = launch_workspace_bytes(B, n, p.splits, d.num_heads, 4) + 256;
        if (p.splits > 1) total = need > total ? need : total;
    }
    return total;
}

hipError_t launch_mla(const dsa_attn_desc_t &d, const void *q, const void *kv,
                      const int32_t *idx, int B, int T, int S, int row0, int rows, int k,
                      void *out, float *lse, void *workspace, hipStream_t stream,
                      const int32_t *q_pos, bool causal_tail) {
    const int H = d.num_heads;
    for (int r0 = 0; r0 < rows; r0 += kMaxGridY) {
        const int n = min(kMaxGridY, rows - r0);
        const Plan p = launch_plan(B, n, H, k);
        const int used_splits = p.splits, per_split = p.per_split;
        const size_t pe = part_elems(B, n, used_splits, H);
        const long long nwg = (long long)(H / kHg) * used_splits * n * B;
        dim3 grid((unsigned)nwg);
        if (d.out_dtype == DSA_BF16)
            hipLaunchKernelGGL(mla_attention_kernel<uint16_t>, grid, dim3(kThreads), 0, stream,
                               static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv),
                               idx, T, S, H, k, d.scale, row0 + r0, n, B, used_splits, per_split,
                               static_cast<uint16_t *>(out), lse,
                               static_cast<uint16_t *>(workspace),
                               reinterpret_cast<float *>(static_cast<uint16_t *>(workspace) + pe),
                               q_pos, causal_tail ? 1 : 0);
        else
            hipLaunchKernelGGL(mla_attention_kernel<float>, grid, dim3(kThreads), 0, stream,
                               static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv),
                               idx, T, S, H, k, d.scale, row0 + r0, n, B, used_splits, per_split,
                               static_cast<float *>(out), lse, static_cast<float *>(workspace),
                               static_cast<float *>(workspace) + pe, q_pos,
                               causal_tail ? 1 : 0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (used_splits > 1) {
            const dim3 cg((unsigned)((long long)(H / 2) * n * B));
            if (d.out_dtype == DSA_BF16)
                hipLaunchKernelGGL(mla_combine_kernel<uint16_t>, cg, dim3(256), 0, stream,
                                   static_cast<const uint16_t *>(workspace),
                                   reinterpret_cast<const float *>(
                                       static_cast<const uint16_t *>(workspace) + pe),
                                   T, H, row0 + r0, n, B, used_splits,
                                   static_cast<uint16_t *>(out), lse);
            else
                hipLaunchKernelGGL(mla_combine_kernel<float>, cg, dim3(256), 0, stream,
                                   static_cast<const float *>(workspace),
                                   static_cast<const float *>(workspace) + pe, T, H,
                                   row0 + r0, n, B, used_splits,
                                   static_cast<float *>(out), lse);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace dsa
