// attention_mha.hip -- MHA-form sparse attention on gfx950 matrix cores, for
// dense selections (prefill, k a large share of the causal prefix).
//
//   out[t,h] = sum_{s in S_t} softmax_s( scale * q[t,h] . K[s,h] ) V[s,h]
// ("DeepSeek Sparse Attention: Learned Token Selection from Scratch",
// sections 3.3 and 10.1; per-head K and V rows, one selected set S_t per query
// shared by every head).  When k is a large fraction of the t+1 candidates
// the page notes that the masked-dense form does little extra work
// (section 9.3): here every (query block, 64-key tile) of the causal area up
// to the block's last selected key is computed with MFMA and the
// probabilities of unselected keys are forced to 0, which gives exactly the
// softmax over S_t.
//
//   mha_bitmap_kernel  idx -> one bit per (row, key) and the row's largest
//                      selected position
//   mha_fa_kernel      one workgroup = 128 query rows x one head, two groups
//       of 4 waves (32 queries each) over the same rows: group 0 takes the
//       even 64-key tiles, group 1 the odd ones, so the longest rows' chain
//       of tiles is halved, and the two partial softmax states are merged
//       through LDS at the end.  Each tile of K and V is brought into LDS
//       once for its group's 4 waves by buffer loads straight to LDS
//       (double-buffered per group, the group's next tile in flight during
//       the current one).  Per wave and
//       tile: S^T = K(64 keys) . Q^T(32 queries) (v_mfma_f32_32x32x16_bf16,
//       the query block in registers as the B operand), bitmap mask, online
//       softmax in fp32; the probabilities stay in registers: in the S^T
//       layout a lane holds one query's keys, and one swap of lane halves
//       per 16-key step turns them into the B operand of
//       O^T(d x 32 queries) += V^T(d x 16 keys) . P^T, with V^T read from
//       the row-major tile by the LDS transpose read.  O^T keeps one query
//       per lane too, so the rescale of the online softmax is lane-local.
#include <type_traits>

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kFaQ = 128;          // query rows per workgroup
constexpr int kFaWaves = kFaQ / 32;  // waves of a group (one per 32 queries)
constexpr int kFaGroups = 2;       // groups over alternate key tiles
constexpr int kFaThreads = 64 * kFaWaves * kFaGroups;
constexpr int kFaKeys = 64;        // keys per tile
// s_waitcnt immediate: vmcnt 0, expcnt and lgkmcnt at their maxima (no wait)
constexpr int kWaitVm0 = 0x0F70;
constexpr int kMaxS = 65536;       // bitmap row of a row kept in LDS by the bitmap kernel (8 KB)
constexpr float kRescaleLog2 = 8.0f;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// LDS tile of 64 rows (keys) x D bf16 with a 16-byte pad per row (pitch
// 272 bytes for D = 128, 144 for D = 64), so that rows start 16 bytes apart
// in bank order: the operand reads of S (16 consecutive rows, the same
// 16-byte piece) hit distinct banks.  Within each block of 16 rows, key
// 4a + b sits in row 4b + a, so the 4 consecutive keys of a transposed V read
// are 4 rows (64 bytes) apart and do not overlap either.  Every read is a
// lane base plus an immediate offset.  Loads fill the tile in 16-byte slots
// (17 or 9 a row, the last one the pad, read from past the buffer as zeros).
template <int D>
struct FaTile {
    static constexpr int row_bytes = D * 2;
    static constexpr int pitch = row_bytes + 16;                   // 272 / 144
    static constexpr int slots = pitch / 16;                       // 17 / 9
    static constexpr int bytes = kFaKeys * pitch;                  // 17408 / 9216
    static constexpr int wave_loads = kFaKeys * slots / 64;        // 17 / 9 (1024 bytes each)
    static constexpr int max_loads = (wave_loads + kFaWaves - 1) / kFaWaves;  // per wave: 5 / 3
    static_assert(wave_loads * 64 == kFaKeys * slots, "wave loads cover the tile exactly");
};

// LDS row of key m of a tile (an involution within blocks of 16 keys)
__device__ __forceinline__ int fa_row(int m) {
    return (m & ~15) | ((m & 3) << 2) | ((m >> 2) & 3);
}

// One wave per row (4 rows a workgroup): the wave zeroes its own bitmap row
// in LDS, ORs in the selected positions (eight loads of the selection in
// flight per lane), and writes the row out with its largest position.  The
// wave is alone with its row, so no workgroup barrier is needed.
constexpr int kBmRows = 4;
// grid: x = group of 4 rows among the nr rows of this launch, y = batch;
// rows = the row stride of bits and row_hi per batch
__global__ __launch_bounds__(kBmRows * 64) void mha_bitmap_kernel(const int32_t *__restrict__ idx,
                                                                  int T, int S, int row0, int nr,
                                                                  int rows, int k,
                                                                  uint32_t *__restrict__ bits,
                                                                  int32_t *__restrict__ row_hi) {
    __shared__ uint32_t w[kBmRows][kMaxS / 32];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = blockIdx.x * kBmRows + wave, b = blockIdx.y;
    if (r >= nr) return;  // the whole wave
    const int words = (S + 31) / 32;
    uint32_t *wr = w[wave];
    for (int j = lane; j < words; j += 64) wr[j] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int32_t *sel = idx + ((size_t)b * T + row0 + r) * k;
    int hi = -1;
    for (int e0 = lane; e0 < k; e0 += 8 * 64) {
        int sv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) sv[u] = e0 + 64 * u < k ? sel[e0 + 64 * u] : -1;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            // the 64 lanes hold consecutive entries: within each row of 16
            // lanes, runs of lanes with the same bitmap word (the rule for a
            // top-k row, which is ascending) are merged with DPP row shifts
            // first, and only the first lane of each run ORs into LDS -- the
            // LDS atomics are the slow part; any order stays exact, only with
            // more of them
            const int s = sv[u];
            const bool valid = s >= 0 && s < S;
            const int wd = valid ? s >> 5 : -1 - lane;  // a word of its own when unused
            uint32_t acc = valid ? 1u << (s & 31) : 0u;
            hi = valid ? max(hi, s) : hi;
            const int lr = lane & 15;
            // row_shl:n -- lane i reads lane i + n of its row
#define DSA_MERGE_STEP(n, ctrl)                                                             \
    {                                                                                       \
        const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)acc, ctrl, 0xf, 0xf, false); \
        const int ow = __builtin_amdgcn_mov_dpp(wd, ctrl, 0xf, 0xf, false);                \
        if (lr + n < 16 && ow == wd) acc |= o;                                              \
    }
            DSA_MERGE_STEP(1, 0x101)
            DSA_MERGE_STEP(2, 0x102)
            DSA_MERGE_STEP(4, 0x104)
            DSA_MERGE_STEP(8, 0x108)
#undef DSA_MERGE_STEP
            // row_shr:1 -- lane i reads lane i - 1 of its row
            const int pw = __builtin_amdgcn_mov_dpp(wd, 0x111, 0xf, 0xf, false);
            if (valid && (lr == 0 || pw != wd)) atomicOr(&wr[wd], acc);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) hi = max(hi, __shfl_xor(hi, off, 64));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t *out = bits + ((size_t)b * rows + r) * words;
    for (int j = lane; j < words; j += 64) out[j] = wr[j];
    if (lane == 0) row_hi[(size_t)b * rows + r] = hi;
}

// 4 consecutive outputs (8-byte aligned as bf16, 16-byte as fp32)
template <typename Tout>
__device__ __forceinline__ void mha_store4(Tout *p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void mha_store4<float>(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{a, b, c, d};
}
template <>
__device__ __forceinline__ void mha_store4<uint16_t>(uint16_t *p, float a, float b, float c,
                                                     float d) {
    *reinterpret_cast<bf16x4 *>(p) = bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t fa_buffer(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Loads of one 64-key tile of K and V straight to LDS: this wave's loads m,
// LDS bytes [1024 (wave + 4 m), +1024) of each tile (wave + 4 m < the tile's
// wave loads); pad slots and rows past the cache read as zeros.
template <int D>
__device__ __forceinline__ void fa_issue(uint8_t *kdst, uint8_t *vdst, const uint16_t *kb,
                                         const uint16_t *vb, int key0, int S, int H, int wave,
                                         const uint32_t *koff, const uint32_t *voff) {
    typedef FaTile<D> Ft;
    typedef __attribute__((address_space(3))) void *lds_ptr;
    const uint32_t rowstride = (uint32_t)H * D * 2;
    const uint32_t nb = (uint32_t)min(kFaKeys, S - key0) * rowstride;
    const __amdgpu_buffer_rsrc_t rk = fa_buffer(kb + (size_t)key0 * H * D, nb);
    const __amdgpu_buffer_rsrc_t rv = fa_buffer(vb + (size_t)key0 * H * D, nb);
#pragma unroll
    for (int m = 0; m < Ft::max_loads; ++m) {
        if (wave + kFaWaves * m < Ft::wave_loads) {  // uniform per wave
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (lds_ptr)(kdst + 1024 * (wave + kFaWaves * m)), 16, koff[m], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (lds_ptr)(vdst + 1024 * (wave + kFaWaves * m)), 16, voff[m], 0, 0, 0);
        }
    }
}

// grid: 1-D over (batch, query block, head); the longest query blocks (the
// last rows: the causal area grows with the row) go first, and with a
// multiple of 8 (batch, head) pairs each head stays on one XCD (its K and V
// are read by every query block of the head).
template <int D, typename Tout>
__global__ __launch_bounds__(kFaThreads, 1) void mha_fa_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const uint32_t *__restrict__ bits,
    const int32_t *__restrict__ row_hi, int T, int S, int H, float scale, int row0, int rows,
    int B, Tout *__restrict__ out, float *__restrict__ lse) {
    typedef FaTile<D> Ft;
    constexpr int KS = D / 16;   // k-steps of S
    constexpr int DT = D / 32;   // 32-dim tiles of O
    // K and V tiles per (group, buffer), each a separate LDS object: the
    // compiler then sees that the loads into one buffer do not alias the
    // reads of the other and waits only for a tile's own loads (with one
    // array indexed at run time it waited for every load before every read).
    // After the last tile, K tile i holds wave i's part of group 1's state.
    __shared__ __align__(16) uint8_t k00[Ft::bytes], k01[Ft::bytes], k10[Ft::bytes],
        k11[Ft::bytes];
    __shared__ __align__(16) uint8_t v00[Ft::bytes], v01[Ft::bytes], v10[Ft::bytes],
        v11[Ft::bytes];
    __shared__ float ml_s[kFaWaves][2][64];
    __shared__ int hi_w[kFaWaves];
    static_assert((D / 32) * 16 * 64 * 4 <= Ft::bytes, "a wave's O^T fits a K tile");

    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wv / kFaWaves;    // 0: even tiles, 1: odd tiles
    const int wave = wv % kFaWaves;   // query sub-block of 32 rows
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int nqb = (rows + kFaQ - 1) / kFaQ;
    const int id = blockIdx.x;
    const int BH = B * H;
    int g, qbi;
    if (BH % 8 == 0) {
        const int x = id & 7, j = id >> 3, per = BH / 8;
        qbi = j / per;
        g = (j - qbi * per) * 8 + x;
    } else {
        qbi = id / BH;
        g = id - qbi * BH;
    }
    const int b = g / H, h = g - (g / H) * H;
    const int qb = nqb - 1 - qbi;

    const int words = (S + 31) / 32;
    const int my_r = qb * kFaQ + wave * 32 + l32;    // this lane's query row (in the launch)
    const bool my_live = my_r < rows;
    const int rr = my_live ? my_r : rows - 1;
    const uint32_t *my_bits = bits + ((size_t)b * rows + rr) * words;
    int hi = my_live ? row_hi[(size_t)b * rows + rr] : -1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) hi = max(hi, __shfl_xor(hi, off, 64));
    if (lane == 0 && grp == 0) hi_w[wave] = hi;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kFaWaves; ++w) hi = max(hi, hi_w[w]);
    const int ntiles = hi < 0 ? 0 : hi / kFaKeys + 1;  // uniform over the workgroup

    // query block (B operand of S): lane (query l32, half) holds dims 16 ks + 8 half .. +8
    bf16x8 qf[KS];
    {
        const uint16_t *qp = q + (((size_t)b * T + row0 + rr) * H + h) * D + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
    }

    // tile loads: slot lane of wave load m (LDS bytes 1024 (wave + 4 m) + 16
    // lane) is piece q mod slots of LDS row q / slots, q = 64 (wave + 4 m) +
    // lane; K row r holds key r, V row r holds key fa_row(r); pads and rows
    // past the tile read from an offset past every buffer
    constexpr uint32_t kDrop = 0x7ffffff0u;
    const uint32_t rowstride = (uint32_t)H * D * 2;
    uint32_t koff[Ft::max_loads], voff[Ft::max_loads];
#pragma unroll
    for (int m = 0; m < Ft::max_loads; ++m) {
        const int q = 64 * (wave + kFaWaves * m) + lane;
        const int r = q / Ft::slots, pc = q % Ft::slots;
        const bool real = r < kFaKeys && pc < Ft::slots - 1;
        koff[m] = real ? (uint32_t)r * rowstride + (uint32_t)(pc << 4) : kDrop;
        voff[m] = real ? (uint32_t)fa_row(r) * rowstride + (uint32_t)(pc << 4) : kDrop;
    }
    const uint16_t *kb = kc + ((size_t)b * S * H + h) * D;
    const uint16_t *vb = vc + ((size_t)b * S * H + h) * D;
    typedef std::integral_constant<int, 0> I0;
    typedef std::integral_constant<int, 1> I1;
    auto ktile_of = [&](auto G, auto BUF) -> uint8_t * {
        if constexpr (decltype(G)::value == 0) return decltype(BUF)::value == 0 ? k00 : k01;
        else return decltype(BUF)::value == 0 ? k10 : k11;
    };
    auto vtile_of = [&](auto G, auto BUF) -> uint8_t * {
        if constexpr (decltype(G)::value == 0) return decltype(BUF)::value == 0 ? v00 : v01;
        else return decltype(BUF)::value == 0 ? v10 : v11;
    };
    // selection bits of this lane's query for the keys of tile j (2 words;
    // the second word of a tile that ends past the row is taken as 0 when it
    // is used, so that nothing here waits for the loads)
    auto mask_words = [&](int j, uint32_t &w0, uint32_t &w1) {
        const int i0 = 2 * j, i1 = min(2 * j + 1, words - 1);
        w0 = my_bits[i0];
        w1 = my_bits[i1];
    };
    auto mask_valid = [&](int j) { return 2 * j + 1 < words; };

    f32x16 o[DT];
#pragma unroll
    for (int c = 0; c < DT; ++c) o[c] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;
    const float sl2 = scale * 1.4426950408889634f;

    // transpose-read lane address (see the MLA kernel): key 16 ks + j/4
    // (+ 4 for the upper keys), dims 32 c + c0 + 4 (j%4) within each group of
    // 16 lanes
    const int trj = lane & 15, trg = lane >> 4;
    const int vkey = 8 * (trg >> 1) + (trj >> 2);
    const int vcol = (16 * (trg & 1) + 4 * (trj & 3)) * 2;
    const int vlo = fa_row(vkey) * Ft::pitch + vcol, vhi = fa_row(vkey + 4) * Ft::pitch + vcol;

    uint32_t mw0 = 0u, mw1 = 0u, nw0 = 0u, nw1 = 0u;
    // step i: group G takes tile 2 i + G into buffer i mod 2 (both groups
    // meet at every barrier); the next tile of the group goes into the other
    // buffer, freed by the barrier
    auto step = [&](auto G, auto BUF, const int i) __attribute__((always_inline)) {
        constexpr int g = decltype(G)::value, nbuf = 1 - decltype(BUF)::value;
        const int j = 2 * i + g;
        // tile j in LDS: this wave's loads have landed (the wait is explicit:
        // the barrier's fence does not reliably wait for direct-to-LDS
        // loads); after the barrier every wave's have, and every wave is past
        // step i-1
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
        mw0 = nw0;
        mw1 = nw1;
        if (j + 2 < ntiles) {
            fa_issue<D>(ktile_of(G, std::integral_constant<int, nbuf>{}),
                        vtile_of(G, std::integral_constant<int, nbuf>{}), kb, vb,
                        (j + 2) * kFaKeys, S, H, wave, koff, voff);
            mask_words(j + 2, nw0, nw1);
        }
        if (j >= ntiles) return;  // group 1 when the count of tiles is odd
        if (!my_live) mw0 = mw1 = 0u;
        if (!mask_valid(j)) mw1 = 0u;
        const uint8_t *ktile = ktile_of(G, BUF);
        const uint8_t *vtile = vtile_of(G, BUF);
        // ---- S^T for two 32-key subtiles: register rg holds key
        // 32 u + 8 (rg/4) + 4 half + rg%4 of query l32
        f32x16 s[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r = 32 * u + l32;
            bf16x8 af[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                af[ks] = *reinterpret_cast<const bf16x8 *>(ktile + r * Ft::pitch +
                                                           (16 * ks + 8 * half) * 2);
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], qf[ks], acc, 0, 0, 0);
            s[u] = acc;
        }
        // ---- mask, online softmax (lane-local query, partner half holds the
        // other keys of the same query)
        float tmax = -INFINITY;
        if (__ballot((mw0 & mw1) != 0xffffffffu)) {  // some key of the tile not selected
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t mw = (u == 0 ? mw0 : mw1) >> (4 * half);
#pragma unroll
                for (int rg = 0; rg < 16; ++rg) {
                    // all ones when key rg is selected, else zero
                    const uint32_t keep =
                        (uint32_t)__builtin_amdgcn_sbfe((int)mw, 8 * (rg >> 2) + (rg & 3), 1);
                    s[u][rg] = __uint_as_float((__float_as_uint(s[u][rg]) & keep) |
                                               (0xff800000u & ~keep));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) tmax = fmaxf(tmax, s[u][rg]);
        tmax = max_halves(tmax) * sl2;
        const bool grow = tmax > m_run + kRescaleLog2;
        const float corr =
            grow ? (m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - tmax)) : 1.0f;
        m_run = grow ? tmax : m_run;
        const float m_ref = m_run == -INFINITY ? 0.0f : m_run;
        // probabilities as bf16 pairs: pk[u][g][0..1] = keys 8 g + 4 half + 0..3
        uint32_t pk[2][4][2];
        float ps = 0.0f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pv[e] = __builtin_amdgcn_exp2f(fmaf(s[u][4 * gq + e], sl2, -m_ref));
                ps += (pv[0] + pv[1]) + (pv[2] + pv[3]);
                pk[u][gq][0] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)pv[0], (__bf16)pv[1]});
                pk[u][gq][1] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)pv[2], (__bf16)pv[3]});
            }
        l_run = l_run * corr + ps;
        if (__ballot(corr != 1.0f)) {
#pragma unroll
            for (int c = 0; c < DT; ++c) o[c] *= corr;
        }
        // ---- O^T += V^T . P^T over 4 k-steps of 16 keys
#pragma unroll
        for (int ks = 0; ks < kFaKeys / 16; ++ks) {
            const int u = ks >> 1, g0 = 2 * (ks & 1);
            // lanes of half 0 take keys 16 ks' + 0..7, half 1 keys + 8..15: the
            // upper lanes' first group and the lower lanes' second group trade
            const auto x0 = __builtin_amdgcn_permlane32_swap(pk[u][g0][0], pk[u][g0 + 1][0],
                                                             false, false);
            const auto x1 = __builtin_amdgcn_permlane32_swap(pk[u][g0][1], pk[u][g0 + 1][1],
                                                             false, false);
            typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
            const u32x4v pw = {x0[0], x1[0], x0[1], x1[1]};
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
            for (int c = 0; c < DT; ++c) {
                const uint8_t *vp = vtile + 16 * ks * Ft::pitch + 64 * c;
                typedef __attribute__((address_space(3))) bf16x4 *lds_v4;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4)(vp + vlo));
                const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4)(vp + vhi));
                const bf16x8 va = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[c], 0, 0, 0);
            }
        }
    };
    const int nsteps = (ntiles + 1) / 2;
    // the query block must have arrived before the loop: left in flight, the
    // compiler's wait for it inside the loop would count the tile loads
    // issued there and stall on them
    __builtin_amdgcn_s_waitcnt(0);
    auto run = [&](auto G) __attribute__((always_inline)) {
        if (decltype(G)::value < ntiles) {
            fa_issue<D>(ktile_of(G, I0{}), vtile_of(G, I0{}), kb, vb,
                        decltype(G)::value * kFaKeys, S, H, wave, koff, voff);
            mask_words(decltype(G)::value, nw0, nw1);
        }
        for (int i = 0; i < nsteps; i += 2) {
            step(G, I0{}, i);
            if (i + 1 < nsteps) step(G, I1{}, i + 1);
        }
    };
    if (grp == 0) run(I0{});
    else run(I1{});

    // merge the odd tiles' state (group 1) into group 0's: both hold
    // sum exp2(x - m) and sum exp2(x - m) v against their own reference m
    __syncthreads();  // every wave is done with the tiles
    float *xs = reinterpret_cast<float *>(wave == 0 ? k00 : wave == 1 ? k01 : wave == 2 ? k10
                                                                                        : k11) +
                lane;
    if (grp == 1) {
#pragma unroll
        for (int c = 0; c < DT; ++c)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) xs[(16 * c + rg) * 64] = o[c][rg];
        ml_s[wave][0][lane] = m_run;
        ml_s[wave][1][lane] = l_run;
    }
    __syncthreads();
    if (grp == 1) return;
    {
        const float m1 = ml_s[wave][0][lane], l1 = ml_s[wave][1][lane];
        const float mm = fmaxf(m_run, m1);
        const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mm);
        const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
        for (int c = 0; c < DT; ++c)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) o[c][rg] = a0 * o[c][rg] + a1 * xs[(16 * c + rg) * 64];
        l_run = a0 * l_run + a1 * l1;
        m_run = mm;
    }

    // normalise: l of query l32 = both key halves; O^T register rg of tile c
    // holds dim 32 c + 8 (rg/4) + 4 half + rg%4 of this lane's query
    const float l_all = sum_halves(l_run);
    const float inv = l_all > 0.0f ? 1.0f / l_all : 0.0f;
    if (my_live) {
        Tout *op = out + (((size_t)b * T + row0 + my_r) * H + h) * D + 4 * half;
#pragma unroll
        for (int c = 0; c < DT; ++c)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
                mha_store4(op + 32 * c + 8 * gq, o[c][4 * gq] * inv, o[c][4 * gq + 1] * inv,
                           o[c][4 * gq + 2] * inv, o[c][4 * gq + 3] * inv);
        if (lse && half == 0)
            lse[((size_t)b * T + row0 + my_r) * H + h] =
                l_all > 0.0f ? (m_run + log2f(l_all)) * 0.6931471805599453f : -INFINITY;
    }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// Masked-dense MFMA form: bf16 in, d_qk = d_v in {64, 128}, at least one full
// query block of rows, and a selection covering at least a quarter of the
// keys (then the dense area is at most ~4x the selected work).
bool mha_dense_path(const dsa_attn_desc_t &d, int rows, int S, int k) {
    return d.form == DSA_MHA && d.dtype == DSA_BF16 && d.d_qk == d.d_v &&
           (d.d_qk == 64 || d.d_qk == 128) && rows >= 32 && S <= kMaxS &&
           4LL * k >= (long long)S;
}

size_t mha_workspace_bytes(int B, int rows, int S) {
    const size_t words = (size_t)(S + 31) / 32;
    return align256((size_t)B * rows * words * 4) + align256((size_t)B * rows * 4);
}

hipError_t launch_selection_bitmap(const int32_t *idx, int B, int T, int S, int row0, int rows,
                                   int k, uint32_t *bits, int32_t *row_hi, hipStream_t stream) {
    if (S > kMaxS) return hipErrorInvalidValue;
    const size_t words = (size_t)(S + 31) / 32;
    for (int r0 = 0; r0 < rows; r0 += kMaxGridY) {
        const int n = min(kMaxGridY, rows - r0);
        hipLaunchKernelGGL(mha_bitmap_kernel, dim3((n + kBmRows - 1) / kBmRows, B),
                           dim3(kBmRows * 64), 0, stream, idx, T, S, row0 + r0, n, rows, k,
                           bits + (size_t)r0 * words, row_hi + r0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

void mha_bitmap_of(void *workspace, int B, int rows, int S, uint32_t **bits, int32_t **row_hi) {
    const size_t words = (size_t)(S + 31) / 32;
    *bits = static_cast<uint32_t *>(workspace);
    *row_hi = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                          align256((size_t)B * rows * words * 4));
}

hipError_t launch_mha_dense(const dsa_attn_desc_t &d, const void *q, const void *kv,
                            const void *v, const int32_t *idx, int B, int T, int S, int row0,
                            int rows, int k, void *out, float *lse, void *workspace,
                            hipStream_t stream, bool bitmap_ready) {
    uint32_t *bits;
    int32_t *row_hi;
    mha_bitmap_of(workspace, B, rows, S, &bits, &row_hi);
    if (!bitmap_ready) {
        const hipError_t e =
            launch_selection_bitmap(idx, B, T, S, row0, rows, k, bits, row_hi, stream);
        if (e != hipSuccess) return e;
    }
    const int nqb = (rows + kFaQ - 1) / kFaQ;
    const long long units = (long long)B * nqb * d.num_heads;
    const dim3 grid((unsigned)units);
    const uint16_t *qp = static_cast<const uint16_t *>(q);
    const uint16_t *kp = static_cast<const uint16_t *>(kv);
    const uint16_t *vp = static_cast<const uint16_t *>(v);
    if (d.d_qk == 128) {
        if (d.out_dtype == DSA_BF16)
            hipLaunchKernelGGL((mha_fa_kernel<128, uint16_t>), grid, dim3(kFaThreads), 0, stream, qp, kp,
                               vp, bits, row_hi, T, S, d.num_heads, d.scale, row0, rows, B,
                               static_cast<uint16_t *>(out), lse);
        else
            hipLaunchKernelGGL((mha_fa_kernel<128, float>), grid, dim3(kFaThreads), 0, stream, qp, kp,
                               vp, bits, row_hi, T, S, d.num_heads, d.scale, row0, rows, B,
                               static_cast<float *>(out), lse);
    } else {
        if (d.out_dtype == DSA_BF16)
            hipLaunchKernelGGL((mha_fa_kernel<64, uint16_t>), grid, dim3(kFaThreads), 0, stream, qp, kp,
                               vp, bits, row_hi, T, S, d.num_heads, d.scale, row0, rows, B,
                               static_cast<uint16_t *>(out), lse);
        else
            hipLaunchKernelGGL((mha_fa_kernel<64, float>), grid, dim3(kFaThreads), 0, stream, qp, kp,
                               vp, bits, row_hi, T, S, d.num_heads, d.scale, row0, rows, B,
                               static_cast<float *>(out), lse);
    }
    return hipGetLastError();
}

}  // namespace dsa
