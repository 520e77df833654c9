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
// Workgroup = 4 waves = one query row x 64 heads x one range of selected
// entries, walked 64 entries at a time:
//   gather  the 64 selected rows go straight from memory into one of two LDS
//           tile buffers (global_load_lds, 16 bytes a lane), so the next tile
//           is in flight while the current one is multiplied; the row pitch
//           carries one spare 16-byte slot against bank conflicts, and masked
//           entries load a valid row whose probability is then forced to 0;
//   S phase wave w computes S^T = C(32 keys) . Q^T(32 heads) over 576 dims for
//           key tile w/2 and head tile w%2 (v_mfma_f32_32x32x16_bf16), with
//           its 32x576 query block held in registers as the B operand;
//   softmax online, fp32: tile max exchanged through LDS, probabilities
//           written to LDS as bf16 [head][key];
//   PV phase wave w accumulates O[64 heads, dims 128w..128w+127] += P . V,
//           V read straight from the row-major tile with the LDS transpose
//           read (ds_read_b64_tr_b16) as the B operand.
// Decode rows split their entries over several workgroups; each writes a
// normalised partial output and its log-sum-exp, merged by a second kernel.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kHg = 64;            // heads per workgroup
constexpr int kKt = 64;            // selected entries per step
constexpr int kKsteps = kDqk / 16; // 36
constexpr int kRowPitch = kDqk * 2 + 16;   // bytes: 1168 (bank shift of 36 dwords)
constexpr int kPPitch = kKt * 2 + 16;      // bytes: 144
constexpr int kChunksPerRow = kDqk * 2 / 16;  // 72 chunks of 16 bytes
constexpr int kThreads = 256;
constexpr float kRescaleLog2 = 8.0f;  // reference-max slack, base-2 units

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kPitchChunks = kRowPitch / 16;            // 73 slots of 16 bytes a row
constexpr int kTileLoads = kKt * kPitchChunks / 64;      // 73 wave loads of 1 KB a tile
static_assert(kKt * kPitchChunks % 64 == 0, "a tile is a whole number of wave loads");

struct __align__(16) MlaSmem {
    uint8_t kv[2][kKt * kRowPitch];    // 2 x 74752, double-buffered tiles
    uint8_t p[kHg * kPPitch];          // 9216
    int32_t sel[2][kKt];
    float tile_max[2][kHg];            // per key tile, per head
    float corr[kHg];
    float lsum[2][kHg];
};

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

// Issue the loads of one tile: wave load j fills LDS bytes [1024j, 1024j+1024)
// of the tile, lane l the 16-byte slot q = 64j + l, i.e. row q / 73, slot
// q % 73.  Slot 72 is the pitch padding (loaded with chunk 0, never read).  A
// masked entry (-1) loads row 0; its probability is forced to 0.  Completion
// is awaited later with s_waitcnt.
__device__ __forceinline__ void issue_tile(uint8_t *tile, const int32_t *sel,
                                           const uint8_t *__restrict__ lat_b, int wave,
                                           int lane) {
    typedef __attribute__((address_space(3))) void *lds_ptr;
    constexpr int kStep = 64 * (kThreads / 64);  // slots between a wave's loads
    int q = 64 * wave + lane;
    int row = q / kPitchChunks;
    int c = q - row * kPitchChunks;
    for (int j = wave; j < kTileLoads; j += kThreads / 64) {
        const uint32_t s = (uint32_t)max(sel[row], 0);
        const uint8_t *src = lat_b + s * (uint64_t)(kDqk * 2) + (c < kChunksPerRow ? c * 16 : 0);
        __builtin_amdgcn_global_load_lds(src, (lds_ptr)(tile + 1024 * j), 16, 0, 0);
        row += kStep / kPitchChunks;
        c += kStep % kPitchChunks;
        if (c >= kPitchChunks) {
            c -= kPitchChunks;
            row += 1;
        }
    }
}

template <typename Tout>
__device__ __forceinline__ void store_out(Tout *p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t *p, float v) {
    *p = (uint16_t)f32_to_bf16_bits(v);
}

// grid: 1-D.  Work item = (head group, split, row, batch).  When the number
// of (row, split) units is a multiple of 8, the head groups of one unit get
// workgroup ids that are 8 apart, so they run on the same XCD (ids are dealt
// round-robin over the 8 XCDs) and the second gather of the same rows hits
// that XCD's L2.
template <typename Tout>
__global__ __launch_bounds__(kThreads, 1) void mla_attention_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ lat,
    const int32_t *__restrict__ idx, int T, int S, int H, int k, float scale, int row0,
    int rows, int B, int splits, int per_split, Tout *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ o_part, float *__restrict__ lse_part) {
    __shared__ MlaSmem sm;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int hgs = H / kHg;
    const int id = blockIdx.x;
    int hg, split, qidx;
    if ((rows * B * splits) % 8 == 0) {
        const int slot = id >> 3;
        hg = slot % hgs;
        const int unit = (slot / hgs) * 8 + (id & 7);
        qidx = unit / splits;
        split = unit % splits;
    } else {
        hg = id % hgs;
        split = (id / hgs) % splits;
        qidx = id / (hgs * splits);
    }
    const int r = qidx % rows;
    const int b = qidx / rows;
    const int i = row0 + r;
    const int head0 = hg * kHg;

    const int e_begin = split * per_split;
    const int e_end = min(k, e_begin + per_split);
    const int ntiles = (e_end - e_begin + kKt - 1) / kKt;
    const int32_t *sel_row = idx + ((size_t)b * T + i) * k;
    const uint8_t *lat_b = reinterpret_cast<const uint8_t *>(lat) + (size_t)b * S * (kDqk * 2);

    // ---- prologue: indices of tiles 0 and 1, loads of tile 0 in flight
    if (tid < kKt) {
        const int e = e_begin + tid;
        sm.sel[0][tid] = e < e_end ? sel_row[e] : -1;
        sm.sel[1][tid] = e + kKt < e_end ? sel_row[e + kKt] : -1;
    }
    __syncthreads();
    issue_tile(sm.kv[0], sm.sel[0], lat_b, wave, lane);

    // ---- S-phase role and its query block (B operand: 32 heads x 576 dims)
    const int kt = wave >> 1;  // key tile of the S phase
    const int ht = wave & 1;   // head tile of the S phase
    bf16x8 qb[kKsteps];
    {
        const uint16_t *qp = q + (((size_t)b * T + i) * H + head0 + ht * 32 + l32) * kDqk + 8 * half;
#pragma unroll
        for (int ks = 0; ks < kKsteps; ++ks)
            qb[ks] = *reinterpret_cast<const bf16x8 *>(qp + ks * 16);
    }

    // ---- PV-phase accumulators: 2 head tiles x 4 dim tiles of 32x32
    f32x16 o[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) o[a][c] = f32x16{};

    float m_run = -INFINITY;  // running max of head (head0 + 32*ht + l32), S-phase view
    float l_run = 0.0f;       // this wave's share of the running sum
    const float sl2 = scale * 1.4426950408889634f;  // logits in base-2 units
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        // loads of the next tile overlap this tile's arithmetic
        if (it + 1 < ntiles) issue_tile(sm.kv[buf ^ 1], sm.sel[buf ^ 1], lat_b, wave, lane);
        int next_sel = -1;
        if (tid < kKt) {
            const int e = e_begin + (it + 2) * kKt + tid;
            next_sel = e < e_end ? sel_row[e] : -1;
        }
        const uint8_t *kvt = sm.kv[buf];
        const int32_t *selt = sm.sel[buf];

        // ---- S^T = C . Q^T for (key tile kt, head tile ht)
        f32x16 sacc = {};
        const uint8_t *arow = kvt + (kt * 32 + l32) * kRowPitch + 16 * half;
#pragma unroll
        for (int ks = 0; ks < kKsteps; ++ks)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(arow + ks * 32), qb[ks], sacc,
                                                           0, 0, 0);
        // register rg holds key kt*32 + 8*(rg/4) + 4*half + rg%4, head ht*32 + l32
        float tmax = -INFINITY;
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
            const int key = kt * 32 + 8 * (rg >> 2) + 4 * half + (rg & 3);
            const float x = selt[key] >= 0 ? sacc[rg] * sl2 : -INFINITY;
            sacc[rg] = x;
            tmax = fmaxf(tmax, x);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        if (half == 0) sm.tile_max[kt][ht * 32 + l32] = tmax;
        __syncthreads();
        const float m_tile = fmaxf(sm.tile_max[0][ht * 32 + l32], sm.tile_max[1][ht * 32 + l32]);
        // Lazy rescaling: the reference max m_run only moves when the tile max
        // exceeds it by more than 2^8, so probabilities stay <= 256 and the
        // accumulators are rescaled only on those (rare) steps.  The softmax is
        // unchanged: numerator and denominator share the reference.
        float corr = 1.0f;
        if (m_tile > m_run + kRescaleLog2) {
            corr = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_tile);
            m_run = m_tile;
        }
        const float m_ref = m_run;
        float psum = 0.0f;
        uint8_t *prow = sm.p + (ht * 32 + l32) * kPPitch;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float pv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pv[j] = m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sacc[4 * g + j] - m_ref);
                psum += pv[j];
            }
            const bf16x4 pk = {(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3]};
            const int key = kt * 32 + 8 * g + 4 * half;
            *reinterpret_cast<bf16x4 *>(prow + key * 2) = pk;
        }
        l_run = l_run * corr + psum;
        if (kt == 0 && half == 0) sm.corr[ht * 32 + l32] = corr;
        __syncthreads();

        // ---- O[64 heads, 128 dims of this wave] = O * corr + P . V
        const int dv0 = wave * 128;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            float cr[16];
            bool any = false;
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                cr[rg] = sm.corr[a * 32 + 8 * (rg >> 2) + 4 * half + (rg & 3)];
                any |= cr[rg] != 1.0f;
            }
            if (__ballot(any)) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int rg = 0; rg < 16; ++rg) o[a][c][rg] *= cr[rg];
            }
        }
        // transpose-read lane address: row key0 + j/4, column col0 + 4*(j%4)
        const int trj = lane & 15;
        const int trg = lane >> 4;
        const uint8_t *vbase = kvt + (8 * (trg >> 1) + (trj >> 2)) * kRowPitch +
                               (dv0 + 16 * (trg & 1) + 4 * (trj & 3)) * 2;
#pragma unroll
        for (int ks = 0; ks < kKt / 16; ++ks) {
            bf16x8 pa[2], vb[4];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                pa[a] = lds_b128(sm.p + (a * 32 + l32) * kPPitch + (16 * ks + 8 * half) * 2);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint8_t *vp = vbase + 16 * ks * kRowPitch + 32 * c * 2;
                const bf16x4 lo = lds_tr16(vp);
                const bf16x4 hi = lds_tr16(vp + 4 * kRowPitch);
                vb[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int a = 0; a < 2; ++a)
                    o[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[a], vb[c], o[a][c], 0, 0,
                                                                      0);
        }
        __syncthreads();  // every wave is done with kv[buf], sel[buf], p
        if (tid < kKt) sm.sel[buf][tid] = next_sel;  // indices of tile it + 2
        __builtin_amdgcn_s_waitcnt(0);               // tile it + 1 has landed
        __syncthreads();
    }

    // ---- final normalisation: l per head = sum of both key-tile waves' shares
    const float l_wave = l_run + __shfl_xor(l_run, 32, 64);
    __syncthreads();
    if (half == 0) sm.lsum[kt][ht * 32 + l32] = l_wave;
    if (kt == 0 && half == 0) sm.tile_max[0][ht * 32 + l32] = m_run;  // reuse as final max
    __syncthreads();
    const int dv0 = wave * 128;
    const size_t rowq = ((size_t)b * T + i);
    const size_t prow = (size_t)qidx;  // row of this launch's split partials
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
            const int hl = a * 32 + 8 * (rg >> 2) + 4 * half + (rg & 3);
            const float l = sm.lsum[0][hl] + sm.lsum[1][hl];
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int d = dv0 + 32 * c + l32;
                const float v = o[a][c][rg] * inv;
                if (splits == 1)
                    store_out(out + (rowq * H + head0 + hl) * kDv + d, v);
                else
                    o_part[((prow * splits + split) * H + head0 + hl) * kDv + d] = v;
            }
        }
    }
    if (tid < kHg) {
        const float l = sm.lsum[0][tid] + sm.lsum[1][tid];
        const float m2 = sm.tile_max[0][tid];  // base-2 units
        const float ls = l > 0.0f ? (m2 + log2f(l)) * 0.6931471805599453f : -INFINITY;
        if (splits == 1) {
            if (lse) lse[rowq * H + head0 + tid] = ls;
        } else {
            lse_part[(prow * splits + split) * H + head0 + tid] = ls;
        }
    }
}

// Merge split partials: out = sum_s exp(lse_s - lse) o_s, lse = log sum exp lse_s.
// Two heads per workgroup, 4 dims per thread; the splits are read in batches
// of 8 whose loads are all issued before any is used (clamped indices, zero
// weight past the last split), so a row costs a few memory latencies rather
// than one per split.
constexpr int kCombineBatch = 8;

template <typename Tout>
__global__ __launch_bounds__(256) void mla_combine_kernel(
    const float *__restrict__ o_part, const float *__restrict__ lse_part, int T, int H,
    int row0, int rows, int splits, Tout *__restrict__ out, float *__restrict__ lse) {
    const int h = blockIdx.x * 2 + (threadIdx.x >> 7);
    const int d = (threadIdx.x & 127) * 4;
    const int r = blockIdx.y;
    const int b = blockIdx.z;
    const size_t rowq = (size_t)b * T + row0 + r;
    const size_t prow = (size_t)b * rows + r;  // row of the launch's split partials
    const float *lp = lse_part + prow * splits * H + h;  // split s at lp[s * H]
    float mx = -INFINITY;
    for (int s0 = 0; s0 < splits; s0 += kCombineBatch) {
        float ls[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) ls[j] = lp[(size_t)min(s0 + j, splits - 1) * H];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) mx = fmaxf(mx, ls[j]);
    }
    const float *op = o_part + (prow * splits * H + h) * kDv + d;  // split s at op[s * H * kDv]
    float wsum = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < splits; s0 += kCombineBatch) {
        float ls[kCombineBatch];
        f32x4 ov[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {
            const size_t sc = (size_t)min(s0 + j, splits - 1);
            ls[j] = lp[sc * H];
            ov[j] = *reinterpret_cast<const f32x4 *>(op + sc * H * kDv);
        }
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {
            const float wgt = (s0 + j < splits && mx != -INFINITY) ? __expf(ls[j] - mx) : 0.0f;
            wsum += wgt;
            acc += wgt * ov[j];
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    Tout *o = out + (rowq * H + h) * kDv + d;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out(o + e, acc[e] * inv);
    if (lse && d == 0) lse[rowq * H + h] = wsum > 0.0f ? mx + __logf(wsum) : -INFINITY;
}

// Entry splits per query row: enough workgroups to cover the CUs, but at least
// two tiles per split so the two-stage gather pipeline has work to overlap.
int mla_splits(int B, int rows, int H, int k) {
    const long long wgs = (long long)B * rows * (H / kHg);
    const int max_splits = ceil_div(k, 2 * kKt);
    long long s = (256 + wgs - 1) / wgs;
    if (s < 1) s = 1;
    if (s > max_splits) s = max_splits;
    return (int)s;
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
        const int splits = mla_splits(B, n, d.num_heads, k);
        if (splits > 1) {
            const size_t need = (size_t)B * n * splits * d.num_heads * (kDv + 1) * 4 + 256;
            total = need > total ? need : total;
        }
    }
    return total;
}

hipError_t launch_mla(const dsa_attn_desc_t &d, const void *q, const void *kv,
                      const int32_t *idx, int B, int T, int S, int row0, int rows, int k,
                      void *out, float *lse, void *workspace, hipStream_t stream) {
    const int H = d.num_heads;
    for (int r0 = 0; r0 < rows; r0 += kMaxGridY) {
        const int n = min(kMaxGridY, rows - r0);
        const int splits = mla_splits(B, n, H, k);
        const int per_split = ceil_div(ceil_div(k, splits), kKt) * kKt;
        const int used_splits = ceil_div(k, per_split);
        float *o_part = static_cast<float *>(workspace);
        float *lse_part = o_part + (size_t)B * n * used_splits * H * kDv;
        const long long nwg = (long long)(H / kHg) * used_splits * n * B;
        dim3 grid((unsigned)nwg);
        if (d.out_dtype == DSA_BF16)
            hipLaunchKernelGGL(mla_attention_kernel<uint16_t>, grid, dim3(kThreads), 0, stream,
                               static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv),
                               idx, T, S, H, k, d.scale, row0 + r0, n, B, used_splits, per_split,
                               static_cast<uint16_t *>(out), lse, o_part, lse_part);
        else
            hipLaunchKernelGGL(mla_attention_kernel<float>, grid, dim3(kThreads), 0, stream,
                               static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv),
                               idx, T, S, H, k, d.scale, row0 + r0, n, B, used_splits, per_split,
                               static_cast<float *>(out), lse, o_part, lse_part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (used_splits > 1) {
            dim3 cg(H / 2, n, B);
            if (d.out_dtype == DSA_BF16)
                hipLaunchKernelGGL(mla_combine_kernel<uint16_t>, cg, dim3(256), 0, stream, o_part,
                                   lse_part, T, H, row0 + r0, n, used_splits,
                                   static_cast<uint16_t *>(out), lse);
            else
                hipLaunchKernelGGL(mla_combine_kernel<float>, cg, dim3(256), 0, stream, o_part,
                                   lse_part, T, H, row0 + r0, n, used_splits,
                                   static_cast<float *>(out), lse);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace dsa
