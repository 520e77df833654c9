// indexer.hip -- lightning-indexer scores on gfx950.
//
//   I[t,s] = sum_j w[t,j] * ReLU( q_I[t,j] . k_I[s] ),  0 <= s <= t
// ("DeepSeek Sparse Attention: Learned Token Selection from Scratch", section
// 2.1; "DeepSeek NSA and DSA", section 3.2).  One key per position serves all
// index heads, so for one query the H_I head vectors form the rows of an
// M = H_I matrix and the keys the columns: a dense contraction over d_I that
// maps onto MFMA, followed by an elementwise ReLU and a w-weighted reduction
// over the rows (the heads) kept in fp32.
//
// Two kernels:
//  * indexer_mfma_kernel<Fp8>: H_I = 64, d_I = 128 in bf16 (v_mfma 32x32x16)
//    or OCP fp8 e4m3 (v_mfma 32x32x64 f8f6f4).  One wave owns one query row
//    and a chunk of key positions; its 64x128 query block stays in registers
//    as the A operand, each 32-key tile of keys is the B operand.
//  * indexer_generic_kernel: any H_I*d_I <= 16384 and any index dtype, plain
//    fp32 FMA (small shapes such as the n=16 running example).
#include <type_traits>

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;
constexpr int kKeyTile = 32;
constexpr int kStreamMaxChunk = 2048;  // keys per wave in the decode key stream

// ---------------------------------------------------------------- MFMA ----
// Register layouts (32x32 MFMA, wave of 64 lanes, h = lane / 32):
//   A (query heads x dims): lane holds head (lane % 32) of a 32-head tile and
//     the dims of k-step ks given by dim_base(ks, h) -- the same dims that the
//     B operand of the same lane half holds for its key, so the k-sum covers
//     every dim exactly once.
//   B (dims x keys): lane holds key (lane % 32) of the tile.
//   D (heads x keys): register r holds head 8*(r/4) + 4*h + r%4 of the tile,
//     key lane % 32.
// bf16: 8 dims per lane per k-step, 8 k-steps; half h reads dims
//   [64h + 8ks, 64h + 8ks + 8), i.e. one contiguous 128-byte half row.
// fp8:  32 dims per lane per k-step, 2 k-steps; half h reads dims
//   [64h + 32ks, 64h + 32ks + 32), one contiguous 64-byte half row.
template <bool Fp8>
struct IdxTraits;

template <>
struct IdxTraits<false> {
    typedef bf16x8 operand;
    static constexpr int ksteps = 8;
    static constexpr int elem_bytes = 2;
    static constexpr int dims_per_step = 8;
    __device__ static operand load(const uint8_t *p) {
        return *reinterpret_cast<const operand *>(p);
    }
    __device__ static operand zero() { return operand{}; }
    __device__ static f32x16 mma(operand a, operand b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct IdxTraits<true> {
    typedef i32x8 operand;
    static constexpr int ksteps = 2;
    static constexpr int elem_bytes = 1;
    static constexpr int dims_per_step = 32;
    __device__ static operand load(const uint8_t *p) {
        return *reinterpret_cast<const operand *>(p);
    }
    __device__ static operand zero() { return operand{}; }
    __device__ static f32x16 mma(operand a, operand b, f32x16 c) {
        // format 0 = fp8 e4m3 for both operands; E8M0 scale 127 = 1.0
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    }
};

// ReLU as an integer max on the bit pattern: every negative float (and -0)
// has its sign bit set, i.e. is a negative int32, so max(bits, 0) maps it to
// +0 and leaves non-negative values alone -- one VALU op, no NaN quieting.
__device__ __forceinline__ float relu_bits(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// This lane's share of sum_h w[h] ReLU(S[h, key]) over the 32 heads it holds
// (16 of each 32-head tile); four independent accumulators keep the FMA
// chain short.  The other 32 heads of the key sit in the partner lane half.
__device__ __forceinline__ float weighted_relu_sum(const f32x16 &acc0, const f32x16 &acc1,
                                                   const float (&wr)[2][16]) {
    float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f, p3 = 0.0f;
#pragma unroll
    for (int rg = 0; rg < 16; rg += 2) {
        p0 = fmaf(wr[0][rg], relu_bits(acc0[rg]), p0);
        p1 = fmaf(wr[0][rg + 1], relu_bits(acc0[rg + 1]), p1);
        p2 = fmaf(wr[1][rg], relu_bits(acc1[rg]), p2);
        p3 = fmaf(wr[1][rg + 1], relu_bits(acc1[rg + 1]), p3);
    }
    return (p0 + p1) + (p2 + p3);
}

template <bool Fp8>
__global__ __launch_bounds__(256) void indexer_mfma_kernel(
    const uint8_t *__restrict__ q_idx, const uint8_t *__restrict__ k_idx,
    const float *__restrict__ w, const int32_t *__restrict__ q_pos, int B, int T, int S,
    int row0, int rows, int chunk, int nchunks, float *__restrict__ scores,
    size_t batch_stride, int write_masked, uint32_t *__restrict__ clear, size_t clear_words) {
    typedef IdxTraits<Fp8> Tr;
    if (clear_words) {  // zero the next kernel's counters, spread over the grid
        const size_t nthreads = (size_t)gridDim.x * blockDim.x;
        for (size_t j = (size_t)blockIdx.x * blockDim.x + threadIdx.x; j < clear_words; j += nthreads)
            clear[j] = 0u;
    }
    typedef typename Tr::operand Op;
    constexpr int EB = Tr::elem_bytes;
    constexpr int KS = Tr::ksteps;
    constexpr int DPS = Tr::dims_per_step;

    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int col = lane & 31;
    const long long wave_id = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const long long total = (long long)B * rows * nchunks;
    if (wave_id >= total) return;
    // longest rows first: the causal row length grows with the row index
    const int c = (int)(wave_id % nchunks);
    const int rr = (int)((wave_id / nchunks) % rows);
    const int b = (int)(wave_id / ((long long)nchunks * rows));
    const int r = rows - 1 - rr;
    const int i = row0 + r;
    const int t = query_pos(q_pos, b, i, T, S);

    const int s_begin = c * chunk;
    const int s_end = min(s_begin + chunk, S);
    const int s_hi = min(s_end, t + 1);  // causal end of this chunk
    float *out = scores + (size_t)b * batch_stride + (size_t)r * S;

    if (write_masked) {
        for (int s = max(s_begin, s_hi) + lane; s < s_end; s += 64) out[s] = -INFINITY;
    }
    if (s_begin >= s_hi) return;

    // query block (A operand) and head weights
    const size_t qrow = ((size_t)b * T + i) * kIdxHeads;
    Op qa[2][KS];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
        const uint8_t *qp = q_idx + ((qrow + tile * 32 + col) * kIdxDim + 64 * half) * EB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[tile][ks] = Tr::load(qp + ks * DPS * EB);
    }
    float wr[2][16];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
        for (int rg = 0; rg < 16; ++rg)
            wr[tile][rg] = w[qrow + tile * 32 + 8 * (rg >> 2) + 4 * half + (rg & 3)];

    const uint8_t *kbase = k_idx + ((size_t)b * S * kIdxDim + 64 * half) * EB;
    Op kb[KS], kn[KS];
    {
        const int key = s_begin + col;
        const uint8_t *kp = kbase + (size_t)key * kIdxDim * EB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kb[ks] = key < s_hi ? Tr::load(kp + ks * DPS * EB) : Tr::zero();
    }
    for (int s0 = s_begin; s0 < s_hi; s0 += kKeyTile) {
        // prefetch the next tile while this one is multiplied
        const int nkey = s0 + kKeyTile + col;
        const uint8_t *np = kbase + (size_t)nkey * kIdxDim * EB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kn[ks] = nkey < s_hi ? Tr::load(np + ks * DPS * EB) : Tr::zero();

        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            acc0 = Tr::mma(qa[0][ks], kb[ks], acc0);
            acc1 = Tr::mma(qa[1][ks], kb[ks], acc1);
        }
        const float all = sum_halves(weighted_relu_sum(acc0, acc1, wr));
        const int key = s0 + col;
        if (half == 0 && key < s_hi) out[key] = all;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kb[ks] = kn[ks];
    }
}

// --------------------------------------------------------- key stream ----
// Decode variant: every key is read by exactly one query row, so the cache is
// streamed.  The `nwaves` waves of one (sequence, row) take the 32-key tiles
// round-robin (wave c owns tiles c, c + nwaves, ...), so at any moment they
// sweep one contiguous stretch of the cache together -- a long run of adjacent
// DRAM pages -- instead of nwaves separate streams.  Each tile is pulled with
// fully coalesced nontemporal 16-byte loads (lane l takes bytes 16(l + 64j)),
// parked in a wave-private LDS tile with a padded row pitch (conflict-free
// operand reads), and multiplied with the B operands of the MFMA layout
// above.  Depth tiles are in flight per wave.  The scores wait in LDS and
// leave in one pass at the end, so the loop issues no global store.
template <bool Fp8>
struct StreamTile {
    static constexpr int row_bytes = kIdxDim * IdxTraits<Fp8>::elem_bytes;  // 128 / 256
    static constexpr int pitch = row_bytes + 16;                             // 144 / 272
    static constexpr int pieces = row_bytes / 16;                            // 8 / 16
    static constexpr int loads = kKeyTile * row_bytes / 1024;                // 4 / 8
    static constexpr int bytes = kKeyTile * pitch;
};

template <bool Fp8>
__global__ __launch_bounds__(256) void indexer_stream_kernel(
    const uint8_t *__restrict__ q_idx, const uint8_t *__restrict__ k_idx,
    const float *__restrict__ w, const int32_t *__restrict__ q_pos, int B, int T, int S,
    int row0, int rows, int nwaves, float *__restrict__ scores, size_t batch_stride,
    int write_masked, uint32_t *__restrict__ clear, size_t clear_words) {
    typedef IdxTraits<Fp8> Tr;
    typedef StreamTile<Fp8> St;
    __shared__ __align__(16) uint8_t tiles[4][St::bytes];
    __shared__ float staged[4][kStreamMaxChunk];  // a wave's scores until its last tile
    if (clear_words) {  // zero the next kernel's counters, spread over the grid
        const size_t nthreads = (size_t)gridDim.x * blockDim.x;
        for (size_t j = (size_t)blockIdx.x * blockDim.x + threadIdx.x; j < clear_words; j += nthreads)
            clear[j] = 0u;
    }
    typedef typename Tr::operand Op;
    constexpr int EB = Tr::elem_bytes;
    constexpr int KS = Tr::ksteps;
    constexpr int DPS = Tr::dims_per_step;

    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int col = lane & 31;
    uint8_t *tile = tiles[threadIdx.x >> 6];
    float *stage = staged[threadIdx.x >> 6];
    const long long wave_id = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const long long total = (long long)B * rows * nwaves;
    if (wave_id >= total) return;
    const int c = (int)(wave_id % nwaves);
    const int r = (int)((wave_id / nwaves) % rows);
    const int b = (int)(wave_id / ((long long)nwaves * rows));
    const int i = row0 + r;
    const int t = query_pos(q_pos, b, i, T, S);
    const int s_hi = min(S, t + 1);  // causal end
    const int tile_step = nwaves * kKeyTile;
    float *out = scores + (size_t)b * batch_stride + (size_t)r * S;
    if (write_masked) {  // -inf past the causal end, over this wave's tiles
        for (int s0 = c * kKeyTile; s0 < S; s0 += tile_step)
            if (s0 + kKeyTile > s_hi && lane < kKeyTile && s0 + lane >= s_hi && s0 + lane < S)
                out[s0 + lane] = -INFINITY;
    }
    const int s_first = c * kKeyTile;
    if (s_first >= s_hi) return;
    const int ntiles = (s_hi - s_first + tile_step - 1) / tile_step;
    // Let the stores above drain: with only loads outstanding from here on,
    // each tile waits for its own loads and not for the whole pipeline.
    __builtin_amdgcn_s_waitcnt(0);

    const size_t qrow = ((size_t)b * T + i) * kIdxHeads;
    Op qa[2][KS];
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
        const uint8_t *qp = q_idx + ((qrow + tl * 32 + col) * kIdxDim + 64 * half) * EB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[tl][ks] = Tr::load(qp + ks * DPS * EB);
    }
    float wr[2][16];
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
        for (int rg = 0; rg < 16; ++rg)
            wr[tl][rg] = w[qrow + tl * 32 + 8 * (rg >> 2) + 4 * half + (rg & 3)];

    const uint8_t *kb_base = k_idx + (size_t)b * S * St::row_bytes;
    // The loads are unconditional: a key past the causal end re-reads the last
    // key row (one cache line per wave load; its column is never stored), so
    // the loop has no branch around a load.
    constexpr int Depth = Fp8 ? 4 : 2;
    u32x4 g[Depth][St::loads];
    auto load_tile = [&](u32x4 (&dst)[St::loads], int m) {
        const int s0 = s_first + m * tile_step;
#pragma unroll
        for (int j = 0; j < St::loads; ++j) {
            const int q = lane + 64 * j;
            const int key = min(s0 + q / St::pieces, s_hi - 1);
            dst[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                kb_base + (size_t)key * St::row_bytes + 16 * (q % St::pieces)));
        }
    };
    // issued in tile order (the scheduler may not reorder them), so the wait
    // for tile d counts only the loads behind it
#pragma unroll
    for (int d = 0; d < Depth; ++d) {
        load_tile(g[d], d);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Unrolled by Depth so register set d always holds tile d (mod Depth): no
    // register rotation, hence no wait on loads younger than the tile in use.
    // Tiles past the wave's last one (at most Depth - 1) are multiplied but
    // not kept.
    for (int m0 = 0; m0 < ntiles; m0 += Depth) {
#pragma unroll
        for (int d = 0; d < Depth; ++d) {
            const int m = m0 + d;
#pragma unroll
            for (int j = 0; j < St::loads; ++j) {
                const int q = lane + 64 * j;
                *reinterpret_cast<u32x4 *>(tile + (q / St::pieces) * St::pitch +
                                           (q % St::pieces) * 16) = g[d][j];
            }
            load_tile(g[d], m + Depth);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            Op kb[KS];
            const uint8_t *brow = tile + col * St::pitch + 64 * half * EB;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kb[ks] = Tr::load(brow + ks * DPS * EB);

            f32x16 acc0 = {}, acc1 = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                acc0 = Tr::mma(qa[0][ks], kb[ks], acc0);
                acc1 = Tr::mma(qa[1][ks], kb[ks], acc1);
            }
            const float all = sum_halves(weighted_relu_sum(acc0, acc1, wr));
            if (half == 0 && m < ntiles) stage[m * kKeyTile + col] = all;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
    // the wave's scores, two tiles per store instruction
    for (int e = lane; e < ntiles * kKeyTile; e += 64) {
        const int key = s_first + (e / kKeyTile) * tile_step + e % kKeyTile;
        if (key < s_hi) out[key] = stage[e];
    }
}

// ---------------------------------------------------------- prefill tile --
// Prefill: consecutive query rows read (almost) the same keys, so a workgroup
// owns 8 consecutive rows and a range of keys; each 128-key tile is brought
// into LDS once for all 8 rows (direct-to-LDS loads, issued two tiles ahead
// into a ring of three buffers) and every wave reads its B operands from
// there.  Row pitch = row + 16 bytes, so the operand reads are free of bank
// conflicts.  One barrier a tile: the longer the tile, the smaller the share
// of the per-barrier costs (the drain of the matrix pipe before it, the
// operand reads after it, the hand-over of the scores).
//
// Each query row is split over two waves (one 32-head tile each): 16 waves a
// workgroup, 4 per SIMD, at most 128 registers a wave.  Software pipeline
// inside a wave: a tile is four quarters of 32 keys; the products of a
// quarter go to one of two accumulator sets while the VALU reduces the other
// set (the previous quarter: ReLU, head weights), so the matrix pipe always
// has independent work next to the reduction, and the two sets alternate
// without copies.
//
// Waves 0..11 issue the tile loads, the same number every tile, and no other
// memory operation, so the wait for a tile's loads is one static vmcnt (loads
// complete in order among themselves; a store between them could complete
// early and satisfy the count).  Every wave parks its partial scores in LDS;
// waves 12..15, which issue no loads, add the two head tiles' partials and
// write the scores with bounds-checked buffer stores (keys outside a row's
// causal range get an offset past the buffer and are dropped).
constexpr int kPfRows = 8;                   // query rows per workgroup
constexpr int kPfKeys = 128;                 // keys per LDS tile
constexpr int kPfQuarters = kPfKeys / 32;    // 32-key product blocks a tile
constexpr int kPfRing = 3;                   // tile buffers; loads run two tiles ahead

// Raw buffer resource over `bytes` bytes at `base` (dword 3: the usual
// untyped-buffer configuration on gfx9); accesses at offsets >= bytes are
// dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
constexpr int kDropOffset = 0x7ffffff0;  // beyond every buffer here: the store is dropped

constexpr int kPfWaves = 2 * kPfRows;           // a wave per (row, 32-head tile)
constexpr int kPfStorers = kPfRows / 2;         // a storing wave per two rows
constexpr int kPfLoaders = kPfWaves - kPfStorers;
static_assert(kPfRows % 2 == 0, "storing waves take rows in pairs");
static_assert(kPfQuarters % 2 == 0, "the two accumulator sets alternate evenly over a tile");
constexpr int kPfMinWgs = 4 * 256 * 16 / kPfWaves;  // four rounds of 4 waves a SIMD
constexpr int kPfAhead = 4;  // operand fragments read ahead of their product

template <bool Fp8>
struct PrefillTile {
    static constexpr int row_bytes = kIdxDim * IdxTraits<Fp8>::elem_bytes;
    static constexpr int pitch = row_bytes + 16;
    static constexpr int slots = pitch / 16;
    static constexpr int loads = (kPfKeys * slots + 63) / 64;
    static constexpr int per_loader = (loads + kPfLoaders - 1) / kPfLoaders;
    static constexpr int bytes = per_loader * kPfLoaders * 1024;
};

// Byte offset, inside a tile's key rows, of the 16 bytes that lane `lane` of
// loading wave `wave` brings in with its m-th load; slots of the LDS row
// padding get an offset past every tile and are filled with zeros.
template <bool Fp8>
__device__ __forceinline__ uint32_t prefill_load_offset(int wave, int lane, int m) {
    typedef PrefillTile<Fp8> Pt;
    const int q = 64 * (wave + kPfLoaders * m) + lane;
    const int row = q / Pt::slots;
    const int piece = q - row * Pt::slots;
    const bool real = q < kPfKeys * Pt::slots && piece * 16 < Pt::row_bytes;
    return real ? (uint32_t)(row * Pt::row_bytes + piece * 16) : (uint32_t)kDropOffset;
}

// Buffer loads straight to LDS over the tile's rows: rows past the cache are
// outside the buffer and read as zeros (their scores are never stored).
template <bool Fp8>
__device__ __forceinline__ void prefill_issue_tile(uint8_t *buf, const uint8_t *kb_base,
                                                     int s0, int S, int wave,
                                                     const uint32_t *voff) {
    typedef PrefillTile<Fp8> Pt;
    typedef __attribute__((address_space(3))) void *lds_ptr;
    const __amdgpu_buffer_rsrc_t rs =
        raw_buffer(const_cast<uint8_t *>(kb_base) + (size_t)s0 * Pt::row_bytes,
                   (uint32_t)min(S - s0, kPfKeys) * (uint32_t)Pt::row_bytes);
#pragma unroll
    for (int m = 0; m < Pt::per_loader; ++m)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(buf + 1024 * (wave + kPfLoaders * m)),
                                                 16, voff[m], 0, 0, 0);
}

// Lanes 0..31 get lo summed over the two half-waves, lanes 32..63 get hi
// summed likewise (one lane swap: lanes 32..63 of the first operand trade
// places with lanes 0..31 of the second).
__device__ __forceinline__ float sum_pair_halves(float lo, float hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi),
                                                     false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool Fp8>
__global__ __launch_bounds__(kPfWaves * 64, 4) void indexer_prefill_kernel(
    const uint8_t *__restrict__ q_idx, const uint8_t *__restrict__ k_idx,
    const float *__restrict__ w, const int32_t *__restrict__ q_pos, int B, int T, int S,
    int row0, int rows, int kchunk, int nkc, float *__restrict__ scores, size_t batch_stride,
    int write_masked) {
    typedef IdxTraits<Fp8> Tr;
    typedef PrefillTile<Fp8> Pt;
    typedef typename Tr::operand Op;
    constexpr int EB = Tr::elem_bytes;
    constexpr int KS = Tr::ksteps;
    constexpr int DPS = Tr::dims_per_step;
    __shared__ __align__(16) uint8_t tile0[Pt::bytes];
    __shared__ __align__(16) uint8_t tile1[Pt::bytes];
    __shared__ __align__(16) uint8_t tile2[Pt::bytes];
    __shared__ int tmax_s[kPfRows];
    // [buffer][row][head tile][entry]; entry e of a tile's scores is key base + e,
    // base = the tile's first key - 32 (its first 32 entries hold the previous
    // tile's last quarter)
    __shared__ __align__(16) float staged[2][kPfRows][2][kPfKeys];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int col = lane & 31;
    const int rw = wave % kPfRows, ht = wave / kPfRows;  // row in the block, head tile
    const int nrb = (rows + kPfRows - 1) / kPfRows;
    const int id = blockIdx.x;
    const int kc = id % nkc;
    const int rb = nrb - 1 - (id / nkc) % nrb;  // last (longest) rows first
    const int b = id / (nkc * nrb);
    const int r = rb * kPfRows + rw;
    const bool live = r < rows;
    const int i = row0 + (live ? r : rows - 1);
    const int t = live ? query_pos(q_pos, b, i, T, S) : -1;
    if (lane == 0 && ht == 0) tmax_s[rw] = t;
    __syncthreads();
    int tmax = tmax_s[0];
#pragma unroll
    for (int v = 1; v < kPfRows; ++v) tmax = max(tmax, tmax_s[v]);

    const int k_begin = kc * kchunk;
    const int k_end = min(S, k_begin + kchunk);
    float *out = scores + (size_t)b * batch_stride + (size_t)(live ? r : 0) * S;
    if (live && write_masked && ht == 0) {
        for (int s = max(k_begin, t + 1) + lane; s < k_end; s += 64) out[s] = -INFINITY;
    }
    const int k_hi = min(k_end, tmax + 1);  // keys any row of the block needs
    if (k_begin >= k_hi) return;             // uniform over the workgroup

    // storing wave kPfLoaders + j: lane l adds and writes entries 4(l&31) ..
    // 4(l&31)+3 of row 2j + (l>>5)
    const bool storer = wave >= kPfLoaders;
    const int srow = storer ? 2 * (wave - kPfLoaders) + half : 0, spart = col;
    const int s_hi = min(k_end, tmax_s[srow] + 1);
    const int live_rows = min(kPfRows, rows - rb * kPfRows);
    const __amdgpu_buffer_rsrc_t oblk =
        raw_buffer(scores + (size_t)b * batch_stride + (size_t)rb * kPfRows * S,
                   (uint32_t)live_rows * (uint32_t)S * 4u);

    const uint8_t *kb_base = k_idx + (size_t)b * S * Pt::row_bytes;
    const int last_tile = k_begin + (k_hi - 1 - k_begin) / kPfKeys * kPfKeys;
    uint32_t voff[Pt::per_loader];
#pragma unroll
    for (int m = 0; m < Pt::per_loader; ++m) voff[m] = prefill_load_offset<Fp8>(wave, lane, m);
    auto issue = [&](uint8_t *buf, int s_tile) {
        prefill_issue_tile<Fp8>(buf, kb_base, min(s_tile, last_tile), S, wave, voff);
    };
    auto flush = [&](int sb, int base) {
        const float4 a = *reinterpret_cast<const float4 *>(&staged[sb][srow][0][4 * spart]);
        const float4 c = *reinterpret_cast<const float4 *>(&staged[sb][srow][1][4 * spart]);
        const float v[4] = {a.x + c.x, a.y + c.y, a.z + c.z, a.w + c.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = base + 4 * spart + e;
            const int off = key >= k_begin && key < s_hi ? (srow * S + key) * 4 : kDropOffset;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[e]), oblk, off, 0, 0);
        }
    };
    if (!storer) {
        issue(tile0, k_begin);
        issue(tile1, k_begin + kPfKeys);
    }

    const size_t qrow = ((size_t)b * T + i) * kIdxHeads + ht * 32;
    Op qa[KS];
    {
        const uint8_t *qp = q_idx + ((qrow + col) * kIdxDim + 64 * half) * EB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = Tr::load(qp + ks * DPS * EB);
    }
    float wr[16];
#pragma unroll
    for (int rg = 0; rg < 16; ++rg) wr[rg] = w[qrow + 8 * (rg >> 2) + 4 * half + (rg & 3)];

    constexpr int kAhead = Pt::per_loader;  // loads of the next tile, still in flight
    constexpr int kWaitThis = (kAhead & 15) | ((kAhead >> 4) << 14) | 0x70 | 0xF00;
    // products of the even quarters go to acc_a, of the odd ones to acc_b; the
    // last quarter of a tile is reduced during the first quarter of the next
    f32x16 acc_a = f32x16{}, acc_b = f32x16{};
    int pbase = k_begin - kPfKeys - 32;
    int sb = 0;
    // operand fragment f (quarter f/KS, k-step f%KS) of tile cur
    auto frag = [&](const uint8_t *cur, int f) -> Op {
        const int st = f / KS, ks = f % KS;
        return Tr::load(cur + (st * 32 + col) * Pt::pitch + 64 * half * EB + ks * DPS * EB);
    };
    static_assert(KS >= 2, "the reduction starts one product into a quarter");
    // element rg of the previous quarter is reduced after product red(rg) of
    // the current one: from the second product on, so the last product of the
    // previous quarter has finished before its accumulators are read
    auto red = [](int rg) { return 1 + rg * (KS - 1) / 16; };
    auto step = [&](auto is_storer, const int s0, const uint8_t *cur,
                    uint8_t *ahead2) __attribute__((always_inline)) {
        if (!is_storer) __builtin_amdgcn_s_waitcnt(kWaitThis);
        lds_barrier();
        if (is_storer) {
            if (s0 > k_begin) flush(sb ^ 1, pbase);
        } else {
            issue(ahead2, s0 + 2 * kPfKeys);
        }
        constexpr int NF = kPfQuarters * KS;
        constexpr int DA = kPfAhead < NF ? kPfAhead : NF;
        Op kb[NF];
#pragma unroll
        for (int f = 0; f < DA; ++f) kb[f] = frag(cur, f);
        float sums[kPfQuarters];  // [0]: previous tile's last quarter, [q]: quarter q-1
#pragma unroll
        for (int qt = 0; qt < kPfQuarters; ++qt) {
            f32x16 &dst = (qt & 1) ? acc_b : acc_a;
            const f32x16 &src = (qt & 1) ? acc_a : acc_b;
            float r0, r1;  // even and odd elements; both start after product red(0) = red(1)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int f = qt * KS + ks;
                if (f + DA < NF) kb[f + DA] = frag(cur, f + DA);
                dst = Tr::mma(qa[ks], kb[f], ks == 0 ? f32x16{} : dst);
#pragma unroll
                for (int rg = 0; rg < 16; ++rg) {
                    float &rr = (rg & 1) ? r1 : r0;
                    if (red(rg) != ks) continue;
                    const float x = wr[rg] * relu_bits(src[rg]);
                    rr = rg < 2 ? x : rr + x;
                }
                // The sums are materialised here, so the compiler cannot sink the
                // reduction below the remaining products: interleaved, the VALU
                // work of one wave runs while the matrix unit serves the others.
                if (ks >= red(1)) asm volatile("" : "+v"(r0), "+v"(r1));
                __builtin_amdgcn_sched_barrier(0);
            }
            sums[qt] = r0 + r1;
        }
        staged[sb][rw][ht][lane] = sum_pair_halves(sums[0], sums[1]);
        staged[sb][rw][ht][64 + lane] = sum_pair_halves(sums[2], sums[3]);
        pbase = s0 - 32;
        sb ^= 1;
    };
    auto walk = [&](auto is_storer) __attribute__((always_inline)) {
        for (int s0 = k_begin; s0 < k_hi; s0 += kPfRing * kPfKeys) {
            step(is_storer, s0, tile0, tile2);
            if (s0 + kPfKeys < k_hi) step(is_storer, s0 + kPfKeys, tile1, tile0);
            if (s0 + 2 * kPfKeys < k_hi) step(is_storer, s0 + 2 * kPfKeys, tile2, tile1);
        }
    };
    if (storer) walk(std::true_type{});
    else walk(std::false_type{});
    __builtin_amdgcn_s_waitcnt(0);  // the surplus tile loads of the last steps
    lds_barrier();
    if (storer) flush(sb ^ 1, pbase);
    float last = 0.0f;
#pragma unroll
    for (int rg = 0; rg < 16; ++rg) last = fmaf(wr[rg], relu_bits(acc_b[rg]), last);
    const float last_all = sum_pair_halves(last, 0.0f);
    lds_barrier();  // staged[sb] is free (its previous contents left two steps ago)
    staged[sb][rw][ht][lane] = last_all;  // keys pbase + kPfKeys + lane; the rest is dropped
    lds_barrier();
    if (storer) flush(sb, pbase + kPfKeys);
}

// ------------------------------------------------------------- generic ----
constexpr int kGenericThreads = 256;
constexpr int kGenericMaxQ = 16384;

__global__ __launch_bounds__(kGenericThreads) void indexer_generic_kernel(
    const void *__restrict__ q_idx, const void *__restrict__ k_idx, int dt,
    const float *__restrict__ w, const int32_t *__restrict__ q_pos, int B, int T, int S, int H,
    int D, int row0, float *__restrict__ scores, size_t batch_stride, int write_masked) {
    __shared__ float qs[kGenericMaxQ];
    __shared__ float ws[128];
    const int r = blockIdx.y;
    const int b = blockIdx.z;
    const int i = row0 + r;
    const int t = query_pos(q_pos, b, i, T, S);
    const int s = blockIdx.x * kGenericThreads + threadIdx.x;
    const int tile_first = blockIdx.x * kGenericThreads;
    if (tile_first > t && !write_masked) return;

    const size_t qrow = ((size_t)b * T + i) * H;
    for (int e = threadIdx.x; e < H * D; e += kGenericThreads)
        qs[e] = load_as_f32(q_idx, qrow * D + e, dt);
    for (int e = threadIdx.x; e < H; e += kGenericThreads) ws[e] = w[qrow + e];
    __syncthreads();
    if (s >= S) return;
    float *out = scores + (size_t)b * batch_stride + (size_t)r * S;
    if (s > t) {
        out[s] = -INFINITY;
        return;
    }
    const size_t krow = ((size_t)b * S + s) * D;
    float total = 0.0f;
    for (int j = 0; j < H; ++j) {
        float dot = 0.0f;
        for (int d = 0; d < D; ++d) dot = fmaf(qs[j * D + d], load_as_f32(k_idx, krow + d, dt), dot);
        total = fmaf(ws[j], fmaxf(dot, 0.0f), total);
    }
    out[s] = total;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t *p, size_t n) {
    for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < n; j += (size_t)gridDim.x * 256)
        p[j] = 0u;
}

}  // namespace

bool indexer_shape_supported(int H, int D) { return H >= 1 && D >= 1 && H <= 128 && H * D <= kGenericMaxQ; }

hipError_t launch_indexer(const void *q_idx, const void *k_idx, int idx_dtype, const float *w,
                          const int32_t *q_pos, int B, int T, int S, int H, int D, int row0,
                          int rows, float *scores, size_t batch_stride, bool write_masked,
                          uint32_t *clear, size_t clear_words, hipStream_t stream) {
    if (H == kIdxHeads && D == kIdxDim && idx_dtype != DSA_F32) {
        // key chunk per wave: long enough to amortise the query-block load,
        // short enough that a few query rows still give ~16 waves per CU (a
        // streaming kernel needs that many loads in flight)
        int chunk = kStreamMaxChunk;
        while (chunk > 128 && (long long)B * rows * ceil_div(S, chunk) < 2048) chunk >>= 1;
        const int nchunks = ceil_div(S, chunk);
        const long long waves = (long long)B * rows * nchunks;
        const int blocks = (int)((waves + 3) / 4);
        if (rows == 1) {  // each key is read by one query row: stream the cache
            if (idx_dtype == DSA_BF16)
                hipLaunchKernelGGL((indexer_stream_kernel<false>), dim3(blocks), dim3(256), 0,
                                   stream, static_cast<const uint8_t *>(q_idx),
                                   static_cast<const uint8_t *>(k_idx), w, q_pos, B, T, S, row0,
                                   rows, nchunks, scores, batch_stride, (int)write_masked, clear,
                                   clear_words);
            else
                hipLaunchKernelGGL((indexer_stream_kernel<true>), dim3(blocks), dim3(256), 0,
                                   stream, static_cast<const uint8_t *>(q_idx),
                                   static_cast<const uint8_t *>(k_idx), w, q_pos, B, T, S, row0,
                                   rows, nchunks, scores, batch_stride, (int)write_masked, clear,
                                   clear_words);
            return hipGetLastError();
        }
        if (rows >= kPfRows) {  // rows share key tiles: 8 rows a workgroup
            // Keys per workgroup: the whole causal row when the row blocks alone
            // give enough workgroups with work (each block then loads its query
            // rows once and pays its prologue once), halved while there are
            // fewer than kPfMinWgs of them.  Without explicit positions the rows
            // of this launch end at position S - T + row0 + rows - 1, so key
            // chunks past that hold no work (unless -inf must be written there).
            const long long nrb = (long long)B * ceil_div(rows, kPfRows);
            const long long keys_hi =
                q_pos ? S : std::min<long long>(S, (long long)(S - T) + row0 + rows);
            const long long keys_avg =
                q_pos ? S : std::max<long long>(1, (long long)(S - T) + row0 + rows / 2);
            int kchunk = 4096;
            while (kchunk < keys_hi) kchunk <<= 1;
            while (kchunk > 4096 && nrb * ((keys_avg + kchunk - 1) / kchunk) < kPfMinWgs)
                kchunk >>= 1;
            if (!write_masked) {
                // the same count of key ranges, made equal (whole tiles): with
                // power-of-two ranges a row block's last range was short, the
                // CUs that drew those finished early and others ran one more
                // full range, so a launch took as long as if the rows reached
                // the next multiple of the range
                const long long n0 = (keys_hi + kchunk - 1) / kchunk;
                kchunk = (int)(((keys_hi + n0 - 1) / n0 + kPfKeys - 1) / kPfKeys * kPfKeys);
            }
            const int nkc = write_masked ? ceil_div(S, kchunk)
                                         : (int)((keys_hi + kchunk - 1) / kchunk);
            const long long wgs = nrb * nkc;
            if (idx_dtype == DSA_BF16)
                hipLaunchKernelGGL((indexer_prefill_kernel<false>), dim3((unsigned)wgs),
                                   dim3(kPfWaves * 64), 0, stream,
                                   static_cast<const uint8_t *>(q_idx),
                                   static_cast<const uint8_t *>(k_idx), w, q_pos, B, T, S, row0,
                                   rows, kchunk, nkc, scores, batch_stride, (int)write_masked);
            else
                hipLaunchKernelGGL((indexer_prefill_kernel<true>), dim3((unsigned)wgs),
                                   dim3(kPfWaves * 64), 0, stream,
                                   static_cast<const uint8_t *>(q_idx),
                                   static_cast<const uint8_t *>(k_idx), w, q_pos, B, T, S, row0,
                                   rows, kchunk, nkc, scores, batch_stride, (int)write_masked);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess || !clear_words) return e;
            hipLaunchKernelGGL(fill_zero_kernel, dim3(min((size_t)1024, (clear_words + 255) / 256)),
                               dim3(256), 0, stream, clear, clear_words);
            return hipGetLastError();
        }
        if (idx_dtype == DSA_BF16)
            hipLaunchKernelGGL((indexer_mfma_kernel<false>), dim3(blocks), dim3(256), 0, stream,
                               static_cast<const uint8_t *>(q_idx),
                               static_cast<const uint8_t *>(k_idx), w, q_pos, B, T, S, row0,
                               rows, chunk, nchunks, scores, batch_stride, (int)write_masked,
                               clear, clear_words);
        else
            hipLaunchKernelGGL((indexer_mfma_kernel<true>), dim3(blocks), dim3(256), 0, stream,
                               static_cast<const uint8_t *>(q_idx),
                               static_cast<const uint8_t *>(k_idx), w, q_pos, B, T, S, row0,
                               rows, chunk, nchunks, scores, batch_stride, (int)write_masked,
                               clear, clear_words);
        return hipGetLastError();
    }
    if (clear_words) {
        hipLaunchKernelGGL(fill_zero_kernel, dim3(min((size_t)1024, (clear_words + 255) / 256)),
                           dim3(256), 0, stream, clear, clear_words);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    for (int r0 = 0; r0 < rows; r0 += kMaxGridY) {
        const int n = min(kMaxGridY, rows - r0);
        dim3 grid(ceil_div(S, kGenericThreads), n, B);
        hipLaunchKernelGGL(indexer_generic_kernel, grid, dim3(kGenericThreads), 0, stream, q_idx,
                           k_idx, idx_dtype, w, q_pos, B, T, S, H, D, row0 + r0,
                           scores + (size_t)r0 * S, batch_stride, (int)write_masked);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dsa
